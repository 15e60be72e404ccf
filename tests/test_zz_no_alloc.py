"""kv_int4_paged_decode_noalloc: the decode with the library's static per-GPU scratch in
place of a caller workspace (for callers that cannot allocate).  Through the C ABI, its
output must equal kv_int4_paged_decode's with a workspace bit for bit (same kernels, same
plan) and the oracle within 2e-3, on consecutive calls that share the static array, the
later ones smaller; a decode whose workspace exceeds the array is rejected before any HIP
call."""
import ctypes

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_harness import D, bf16_dev, decode_compare, to_dev


@pytest.fixture(scope="module")
def K():
    import int4_kv_cache_rotquant_amd as K
    K.lib()
    return K


def test_noalloc_rejects_oversized_before_any_hip_call(K):
    """Host-side only (no device memory touched): 1000 sequences of 5000 tokens, 64 query and
    8 KV heads, on the balanced grid need ~42 MB of scratch, more than the 32 MiB array."""
    L = K.lib()
    desc = K.CacheDesc(128, 8, 16, 64, 128, 0)
    bufs = K.CacheBuffers(0x10000, 0x20000, 0x30000, 0x40000)
    st = L.kv_int4_paged_decode_noalloc(ctypes.byref(desc), ctypes.byref(bufs), 0x1000, 1000, 64,
                                        0x2000, 400, 0x3000, 5000, 0.0, 0, 0x4000, None)
    assert st == K.KVRQ_EWORKSPACE and "static scratch" in K.last_error()
    st = L.kv_int4_paged_decode_noalloc(ctypes.byref(desc), ctypes.byref(bufs), 0, 2, 64,
                                        0x2000, 400, 0x3000, 5000, 0.0, 0, 0x4000, None)
    assert st == K.KVRQ_EINVAL


def _case(K, lens, Hkv, G, P, kb, vb, seed):
    rng = np.random.default_rng(seed)
    paging = W.assign_pages(np.random.default_rng(seed + 1), list(lens), P)
    T = int(sum(lens))
    k = W.make_rows(rng, T, Hkv, W.OutlierSpec.random(rng, Hkv))
    v = W.make_rows(rng, T, Hkv)
    slots = np.concatenate([paging.slots(s, 0, int(L)) for s, L in enumerate(lens)])
    cache = K.PagedInt4Cache(paging.num_pages, Hkv, P, kb, vb, fill=0)
    K.kv_rotquant_write(cache, bf16_dev(k), bf16_dev(v), to_dev(slots))
    orc = oracle.Cache(paging.num_pages, Hkv, P, fill=0)
    oracle.write(orc, k, v, slots, kb, vb)
    q = W.f32_to_bf16_bits(rng.standard_normal((len(lens), Hkv * G, D)).astype(np.float32))
    return cache, orc, q, paging.page_table(), np.array(lens, np.int32)


@pytest.mark.gpu
@pytest.mark.parametrize("split", [0, -1, 256])
def test_noalloc_matches_workspace_decode(K, split):
    """Two calls in a row on the shared static array, the second with fewer and shorter
    sequences: both equal the workspace decode exactly and the oracle within 2e-3."""
    import torch
    cases = [([3000, 17, 0, 900, 4500, 1200, 64, 2048], 2, 4, 16, 64, 0, 501),
             ([300, 1, 129], 2, 8, 32, 128, 128, 502)]
    for i, (lens, Hkv, G, P, kb, vb, seed) in enumerate(cases):
        cache, orc, q, tab, L = _case(K, lens, Hkv, G, P, kb, vb, seed)
        maxlen = int(L.max())
        qd, td, ld = bf16_dev(q), to_dev(tab), to_dev(L)
        ref = K.kv_int4_paged_decode(cache, qd, td, ld, maxlen, split_tokens=split)
        out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
        K.kv_int4_paged_decode_noalloc(cache, qd, td, ld, maxlen, out, split_tokens=split)
        torch.cuda.synchronize()
        a, b = out.cpu().numpy(), ref.cpu().numpy()
        assert np.array_equal(a, b), (split, i, float(np.nanmax(np.abs(a - b))))
        arrays = (orc.k_codes, orc.v_codes, orc.k_params, orc.v_params)
        decode_compare(a, oracle.decode(q, arrays, tab, L, Hkv, P, kb, vb), f"noalloc split {split} call {i}")
