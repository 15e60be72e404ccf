"""GPU parity of the 2-bit pools (K and/or V at 2 bits: the pages' open question,
wispaper.ai blog, section 5, limitations) through the C ABI:

* the write stores exactly the oracle's bytes and parameters (K 2-bit, V 2-bit, both),
  for plain and rotated rows, ragged token counts and page sizes 16 and 1;
* the decode, the extend and the fused decode step match the oracle within 2e-3 for
  every width mix, query groups 1..16 and forced split counts; the fused step's cache
  equals the separate write's byte for byte.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_harness import D, bf16_dev, decode_compare, gpu_cache_arrays, to_dev

pytestmark = pytest.mark.gpu
MIXES = [(2, 2), (4, 2), (2, 4)]


@pytest.fixture(scope="module")
def K():
    import int4_kv_cache_rotquant_amd as K
    K.lib()
    return K


def _caches(K, paging, Hkv, P, kb, vb, kbits, vbits, k, v, slots, fill=0):
    cache = K.PagedInt4Cache(paging.num_pages, Hkv, P, kb, vb, fill=fill, k_bits=kbits, v_bits=vbits)
    orc = oracle.Cache(paging.num_pages, Hkv, P, fill=fill, k_bits=kbits, v_bits=vbits)
    if len(slots):
        K.kv_rotquant_write(cache, bf16_dev(k), bf16_dev(v), to_dev(slots))
        oracle.write(orc, k, v, slots, kb, vb)
    return cache, orc


@pytest.mark.parametrize("kbits,vbits", MIXES)
@pytest.mark.parametrize("kb,vb,P", [(0, 0, 16), (128, 128, 16), (16, 64, 1), (64, 0, 16)])
def test_write_bit_exact(K, kbits, vbits, kb, vb, P):
    rng = np.random.default_rng(200 + kb + vb + P + kbits)
    T, Hkv = 333, 4
    paging = W.assign_pages(rng, [T], P, extra_pages=3)
    k = W.make_rows(rng, T, Hkv, W.OutlierSpec.random(rng, Hkv))
    v = W.make_rows(rng, T, Hkv, W.OutlierSpec.random(rng, Hkv))
    slots = paging.slots(0, 0, T)
    cache, orc = _caches(K, paging, Hkv, P, kb, vb, kbits, vbits, k, v, slots, fill=0xAA)
    got = gpu_cache_arrays(cache)
    want = (orc.k_codes, orc.v_codes, orc.k_params, orc.v_params)
    for g, w, name in zip(got, want, ("k_codes", "v_codes", "k_params", "v_params")):
        assert g.shape == w.shape, name
        assert np.array_equal(g, w), (name, int((g != w).sum()))


def _seqs(K, lens, Hkv, Hq, P, kb, vb, kbits, vbits, seed):
    rng = np.random.default_rng(seed)
    paging = W.assign_pages(np.random.default_rng(seed + 1), list(lens), P)
    T = int(sum(lens))
    k = W.make_rows(rng, T, Hkv, W.OutlierSpec.random(rng, Hkv))
    v = W.make_rows(rng, T, Hkv)
    slots = np.concatenate([paging.slots(s, 0, int(L)) for s, L in enumerate(lens)]).astype(np.int32)
    cache, orc = _caches(K, paging, Hkv, P, kb, vb, kbits, vbits, k, v, slots)
    return rng, paging, cache, orc


@pytest.mark.parametrize("kbits,vbits", MIXES)
@pytest.mark.parametrize("G,kb,vb", [(1, 128, 128), (4, 0, 0), (8, 64, 16), (16, 128, 0)])
def test_decode(K, kbits, vbits, G, kb, vb):
    import torch
    lens, Hkv, P = [1, 31, 200, 1000, 0, 77], 2, 16
    rng, paging, cache, orc = _seqs(K, lens, Hkv, Hkv * G, P, kb, vb, kbits, vbits, 300 + G + kb)
    q = W.f32_to_bf16_bits(rng.standard_normal((len(lens), Hkv * G, D)).astype(np.float32))
    tab, L = paging.page_table(), np.array(lens, np.int32)
    arrays = (orc.k_codes, orc.v_codes, orc.k_params, orc.v_params)
    ref = oracle.decode(q, arrays, tab, L, Hkv, P, kb, vb)
    for split in (0, 128):
        out = K.kv_int4_paged_decode(cache, bf16_dev(q), to_dev(tab), to_dev(L), int(L.max()),
                                     split_tokens=split)
        torch.cuda.synchronize()
        decode_compare(out.cpu().numpy(), ref, f"2-bit decode K{kbits}V{vbits} G{G} split {split}")


@pytest.mark.parametrize("kbits,vbits", MIXES)
def test_extend(K, kbits, vbits):
    import torch
    lens, news, Hkv, Hq, P = [300, 129, 64], [100, 129, 1], 2, 8, 16
    rng, paging, cache, orc = _seqs(K, lens, Hkv, Hq, P, 128, 0, kbits, vbits, 400 + kbits)
    qo = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    q = W.f32_to_bf16_bits(rng.standard_normal((int(qo[-1]), Hq, D)).astype(np.float32))
    tab, L = paging.page_table(), np.array(lens, np.int32)
    out = K.kv_int4_paged_extend(cache, bf16_dev(q), to_dev(qo), to_dev(tab), to_dev(L), int(L.max()),
                                 int(max(news)))
    torch.cuda.synchronize()
    arrays = (orc.k_codes, orc.v_codes, orc.k_params, orc.v_params)
    decode_compare(out.cpu().numpy(), oracle.extend(q, arrays, qo, tab, L, Hkv, P, 128, 0),
                   f"2-bit extend K{kbits}V{vbits}")


@pytest.mark.parametrize("kbits,vbits", MIXES)
def test_fused_step(K, kbits, vbits):
    import torch
    lens, Hkv, Hq, P, kb, vb = [40, 300, 1], 2, 8, 16, 128, 32
    rng = np.random.default_rng(500 + kbits)
    paging = W.assign_pages(np.random.default_rng(501), list(lens), P)
    pre = [L - 1 for L in lens]
    T = int(sum(pre))
    k = W.make_rows(rng, T, Hkv, W.OutlierSpec.random(rng, Hkv))
    v = W.make_rows(rng, T, Hkv)
    slots = np.concatenate([paging.slots(s, 0, n) for s, n in enumerate(pre)]).astype(np.int32)
    fused, orc = _caches(K, paging, Hkv, P, kb, vb, kbits, vbits, k, v, slots)
    ref, _ = _caches(K, paging, Hkv, P, kb, vb, kbits, vbits, k, v, slots)
    kn = W.make_rows(rng, len(lens), Hkv)
    vn = W.make_rows(rng, len(lens), Hkv)
    ns = np.array([paging.slots(s, L - 1, 1)[0] for s, L in enumerate(lens)], np.int32)
    q = W.f32_to_bf16_bits(rng.standard_normal((len(lens), Hq, D)).astype(np.float32))
    tab, L = paging.page_table(), np.array(lens, np.int32)
    out_f = K.kv_int4_paged_decode_step(fused, bf16_dev(kn), bf16_dev(vn), to_dev(ns), bf16_dev(q),
                                        to_dev(tab), to_dev(L), int(L.max()))
    K.kv_rotquant_write(ref, bf16_dev(kn), bf16_dev(vn), to_dev(ns))
    out_r = K.kv_int4_paged_decode(ref, bf16_dev(q), to_dev(tab), to_dev(L), int(L.max()))
    torch.cuda.synchronize()
    for a, b in zip(gpu_cache_arrays(fused), gpu_cache_arrays(ref)):
        assert np.array_equal(a, b)
    assert np.array_equal(out_f.cpu().numpy(), out_r.cpu().numpy())
    oracle.write(orc, kn, vn, ns, kb, vb)
    arrays = (orc.k_codes, orc.v_codes, orc.k_params, orc.v_params)
    decode_compare(out_f.cpu().numpy(), oracle.decode(q, arrays, tab, L, Hkv, P, kb, vb),
                   f"2-bit fused step K{kbits}V{vbits}")
