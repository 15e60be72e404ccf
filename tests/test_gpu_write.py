"""GPU parity of kv_rotquant_write against the oracle (bit-exact codes, parameters and
placement; codes within 1e-6 of a rounding boundary would be excused and counted).

Workloads follow the five configurations: the tiny case, the Qwen3-4B-like layer,
the 32768-token prefill chunk (every block size and plain INT4), the high-concurrency
decode step write (256 tokens, one per sequence, into a 3 GB pool) and a 16384-token
long-context chunk into a 1M-token pool.  Edge cases: every (K block, V block) pair,
ragged token counts, skipped slots, degenerate rows, strided inputs, page sizes 1 and
1024, an empty call.
"""
import numpy as np
import pytest

import workloads as W
from gpu_harness import D, log, run_write_case, to_dev, bf16_dev

pytestmark = pytest.mark.gpu

BLOCKS = [0, 16, 32, 64, 128]


@pytest.fixture(scope="module")
def K():
    import int4_kv_cache_rotquant_amd as K
    K.lib()
    return K


def test_tiny(K):
    w = W.tiny()
    k, v = w.kv()
    run_write_case(K, k, v, w.all_slots(), w.paging.num_pages, 1, 16, 128, 128, "tiny")


def test_qwen3_4b_like_all_tokens(K):
    w = W.qwen3_4b_like()
    k, v = w.kv()
    log(f"qwen3_4b_like: T={k.shape[0]}")
    run_write_case(K, k, v, w.all_slots(), w.paging.num_pages, 8, 16, 64, 0, "qwen3_4b_like")


@pytest.mark.parametrize("kb", [16, 32, 64, 128, 0])
def test_prefill_chunk_block_sweep(K, kb):
    w = W.prefill_chunk(kb)
    k, v = w.kv()
    run_write_case(K, k, v, w.all_slots(), w.paging.num_pages, 8, 64, kb, 0, f"prefill_chunk_b{kb}")


@pytest.mark.parametrize("kb", BLOCKS)
@pytest.mark.parametrize("vb", BLOCKS)
def test_block_pairs_ragged(K, kb, vb):
    rng = np.random.default_rng(100 + kb * 7 + vb)
    T, Hkv, P = 77, 3, 16
    out = W.OutlierSpec.random(rng, Hkv)
    k = W.make_rows(rng, T, Hkv, out)
    v = W.make_rows(rng, T, Hkv, W.OutlierSpec.random(rng, Hkv))
    paging = W.assign_pages(rng, [T], P, extra_pages=3)
    slots = paging.slots(0, 0, T)
    slots[rng.random(T) < 0.1] = -1
    run_write_case(K, k, v, slots, paging.num_pages, Hkv, P, kb, vb, f"pair_{kb}_{vb}")


def test_degenerate_and_extreme_rows(K):
    T, Hkv, P = 12, 2, 4
    x = np.zeros((T, Hkv, D), np.float32)
    x[1] = 1.5                                    # all equal
    x[2, :, ::3] = -0.0                           # zeros with negative zeros
    x[3] = np.linspace(-60000, 60000, D)          # near the fp16 range (scale ~ 8000)
    x[4, :, 7] = 1e4                              # one huge spike
    x[5] = 2.0 ** -20 * np.arange(D)              # tiny values (fp16 subnormal scale)
    x[6] = -1.0 + (np.arange(D) % 16) / 8.0       # on the grid
    x[7, :, 0] = -3.0                             # single negative spike
    rng = np.random.default_rng(5)
    x[8:] = rng.standard_normal((T - 8, Hkv, D)) * 100
    k = W.f32_to_bf16_bits(x)
    v = W.f32_to_bf16_bits(-x)
    slots = np.arange(T, dtype=np.int32)[::-1].copy()
    for kb, vb in [(0, 0), (16, 128), (128, 64), (32, 0)]:
        run_write_case(K, k, v, slots, 3, Hkv, P, kb, vb, f"degenerate_{kb}_{vb}")


def test_round_half_even_ties(K):
    """Plain rows whose codes all fall exactly on a half: (y - zero) * (1 / scale) is
    k + 0.5 for every non-extreme channel (scales 1, 2 and 0.5 are exact in fp16), so each
    code is decided by the round-half-to-even rule alone (0.5 -> 0, 1.5 -> 2, 2.5 -> 2)."""
    T, Hkv, P = 4, 1, 4
    x = np.zeros((T, Hkv, D), np.float32)
    half = np.arange(D) % 15 + 0.5                 # 0.5, 1.5, ..., 14.5
    x[0, 0] = half
    x[0, 0, :2] = [0.0, 15.0]                      # scale 1, zero 0
    x[1, 0] = half - 8.0
    x[1, 0, :2] = [-8.0, 7.0]                      # scale 1, zero -8
    x[2, 0] = 2.0 * half
    x[2, 0, :2] = [0.0, 30.0]                      # scale 2
    x[3, 0] = 0.5 * half
    x[3, 0, :2] = [0.0, 7.5]                       # scale 0.5
    k = W.f32_to_bf16_bits(x)
    v = W.f32_to_bf16_bits(x[::-1].copy())
    run_write_case(K, k, v, np.arange(T, dtype=np.int32), 1, Hkv, P, 0, 0, "ties")


def test_strided_input_and_page_sizes(K):
    rng = np.random.default_rng(6)
    T, Hkv = 50, 2
    k = W.make_rows(rng, T, Hkv, W.OutlierSpec.random(rng, Hkv))
    v = W.make_rows(rng, T, Hkv)
    for P in (1, 2, 1024):
        paging = W.assign_pages(rng, [T], P, extra_pages=1)
        slots = paging.slots(0, 0, T)
        run_write_case(K, k, v, slots, paging.num_pages, Hkv, P, 128, 32, f"P{P}")
    paging = W.assign_pages(rng, [T], 16)
    run_write_case(K, k, v, paging.slots(0, 0, T), paging.num_pages, Hkv, 16, 64, 64, "strided",
                   token_pad=24)


def test_empty_call_is_noop(K):
    import torch
    cache = K.PagedInt4Cache(2, 1, 16, 128, 128, fill=0xAA)
    e = torch.empty((0, 1, D), dtype=torch.bfloat16, device="cuda")
    K.kv_rotquant_write(cache, e, e, torch.empty(0, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert bool((cache.k_codes == 0xAA).all())


def test_decode_step_write_full_pool(K):
    """The high-concurrency step: 256 new tokens (one per sequence, pages scattered over a
    ~3 GB pool), exactly the launch the decode-step benchmark times."""
    import torch
    w = W.qwen3_32b_like_decode()
    rng = w.rng(10)
    T = w.num_seqs
    k = W.make_rows(rng, T, 8, w.k_out)
    v = W.make_rows(rng, T, 8)
    step = 37
    slots = np.array([w.paging.slots(s, int(L) + step, 1)[0] for s, L in enumerate(w.seq_lens)],
                     np.int32)
    log(f"decode-step write: pool pages {w.paging.num_pages}")
    cache = K.PagedInt4Cache(w.paging.num_pages, 8, 16, 128, 0, fill=0xAA)
    K.kv_rotquant_write(cache, bf16_dev(k), bf16_dev(v), to_dev(slots))
    torch.cuda.synchronize()
    # compare only the written cells (a 3 GB host copy of the pool is not needed): the
    # rest of the pool is checked through a sample of untouched pages
    import oracle
    pages = slots // 16
    offs = slots % 16
    sub = oracle.Cache(T, 8, 16)
    oracle.write(sub, k, v, (np.arange(T) * 16 + offs).astype(np.int32), 128, 0)
    pidx = torch.from_numpy(pages.astype(np.int64)).cuda()
    got_kc = cache.k_codes.index_select(0, pidx).cpu().numpy()
    got_vc = cache.v_codes.index_select(0, pidx).cpu().numpy()
    got_kp = cache.k_params.index_select(0, pidx).cpu().numpy().view(np.uint16)
    got_vp = cache.v_params.index_select(0, pidx).cpu().numpy().view(np.uint16)
    assert np.array_equal(got_kc, sub.k_codes) and np.array_equal(got_vc, sub.v_codes)
    assert np.array_equal(got_kp, sub.k_params) and np.array_equal(got_vp, sub.v_params)
    untouched = np.setdiff1d(np.arange(0, w.paging.num_pages, 997), pages)
    u = torch.from_numpy(untouched.astype(np.int64)).cuda()
    assert bool((cache.k_codes.index_select(0, u) == 0xAA).all())
    assert bool((cache.v_params.index_select(0, u).view(torch.uint8) == 0xAA).all())


def test_long_context_chunk(K):
    """A 16384-token chunk written into the 1M-token, 16384-page pool (page 64), as in the
    long-context fill; the chunk is the 40th of 64."""
    import torch
    w = W.long_context()
    chunk = 40
    C = w.notes["chunk"]
    rng = w.rng(100 + chunk)
    k = W.make_rows(rng, C, 8, w.k_out)
    v = W.make_rows(rng, C, 8, w.v_out)
    slots = w.paging.slots(0, chunk * C, C)
    cache = K.PagedInt4Cache(w.paging.num_pages, 8, 64, 128, 128, fill=0xAA)
    K.kv_rotquant_write(cache, bf16_dev(k), bf16_dev(v), to_dev(slots))
    torch.cuda.synchronize()
    import oracle
    pages = np.unique(slots // 64)
    remap = {int(p): i for i, p in enumerate(pages)}
    local = np.array([remap[int(s) // 64] * 64 + int(s) % 64 for s in slots], np.int32)
    sub = oracle.Cache(len(pages), 8, 64)
    oracle.write(sub, k, v, local, 128, 128)
    pidx = torch.from_numpy(pages.astype(np.int64)).cuda()
    for got, ref in ((cache.k_codes, sub.k_codes), (cache.v_codes, sub.v_codes)):
        assert np.array_equal(got.index_select(0, pidx).cpu().numpy(), ref)
    for got, ref in ((cache.k_params, sub.k_params), (cache.v_params, sub.v_params)):
        assert np.array_equal(got.index_select(0, pidx).cpu().numpy().view(np.uint16), ref)
    log(f"long-context chunk: {len(pages)} pages bit-exact")
