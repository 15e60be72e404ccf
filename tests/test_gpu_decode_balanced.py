"""GPU parity of the balanced decode grid (split_tokens = KVRQ_SPLIT_BALANCED, the automatic
choice for large batches): one resident round of workgroups, each taking an equal share of
the (sequence, KV head, 32-token tile) space, partials where a share starts or ends inside
a pair, merged by the last workgroup of the pair.  Checked against the oracle's fp64 decode
(<= 2e-3 absolute) and against the split grid on the same cache (<= 1e-4).

Covers fewer tiles than workgroups (one tile each), shares that cross many pair boundaries,
one pair spread over every workgroup (a merge of more than 64 partials), empty sequences,
G = 1, 2, 4, 8, 16 and every V rotation branch, page sizes 16..64, three calls on one
workspace (counters back at zero after each), the fused decode step and 2-bit pools.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_harness import D, bf16_dev, decode_compare, to_dev
from test_gpu_decode import _build, _ref, _run
from test_gpu_decode_step import _check_step, _setup

pytestmark = pytest.mark.gpu
BAL = -1


@pytest.fixture(scope="module")
def K():
    import int4_kv_cache_rotquant_amd as K
    K.lib()
    assert K.KVRQ_SPLIT_BALANCED == BAL
    return K


@pytest.mark.parametrize("G,kb,vb,P", [(1, 128, 128, 16), (2, 16, 64, 32), (4, 64, 0, 16),
                                       (8, 128, 0, 16), (16, 0, 32, 64)])
def test_few_tiles_ragged(K, G, kb, vb, P):
    """247 tiles per KV head: fewer tiles than workgroups, so each takes one tile and most
    pairs are merged from several partials."""
    Hkv = 2
    lens = [0, 1, 31, 32, 33, 500, 1021, 4096, 77, 2000]
    cache, orc, q, tab, L = _build(K, lens, Hkv, Hkv * G, P, kb, vb, seed=300 + G + kb + P)
    out = _run(K, cache, q, tab, L, split=BAL)
    assert np.all(out[0] == 0)
    decode_compare(out, _ref(orc, q, tab, L, Hkv, P, kb, vb), f"balanced few tiles G={G}")
    split = _run(K, cache, q, tab, L, split=256)
    assert float(np.abs(out - split).max()) <= 1e-4


def test_shares_cross_pairs(K):
    """40 sequences of 1..6000 tokens, 4 KV heads: ~15 tiles per workgroup, pairs of ~100
    tiles, so shares start and end inside pairs and cover several pairs each."""
    rng = np.random.default_rng(5)
    lens = [int(x) for x in rng.integers(1, 6000, size=40)]
    lens[7] = 0
    Hkv, G, P = 4, 8, 16
    cache, orc, q, tab, L = _build(K, lens, Hkv, Hkv * G, P, 128, 0, seed=301)
    out = _run(K, cache, q, tab, L, split=BAL)
    decode_compare(out, _ref(orc, q, tab, L, Hkv, P, 128, 0), "balanced 40 seqs")
    auto = _run(K, cache, q, tab, L, split=0)
    assert float(np.abs(out - auto).max()) <= 1e-4


def test_one_pair_over_every_workgroup(K):
    """One 200,000-token sequence, one KV head, 8 query heads: 6,250 tiles over every
    workgroup, one pair merged from hundreds of partials."""
    lens = [200000]
    cache, orc, q, tab, L = _build(K, lens, 1, 8, 64, 128, 128, seed=302)
    out = _run(K, cache, q, tab, L, split=BAL)
    decode_compare(out, _ref(orc, q, tab, L, 1, 64, 128, 128), "balanced one pair")


def test_calls_share_one_workspace(K):
    """Three calls with fresh queries on one zero-filled workspace: each matches the oracle
    and leaves the pair counters at zero; the output starts as NaN so no row is skipped."""
    import torch
    lens = [3000, 17, 0, 900, 4500]
    Hkv, G, P = 2, 4, 16
    cache, orc, q, tab, L = _build(K, lens, Hkv, Hkv * G, P, 64, 0, seed=303)
    n = K.kv_int4_paged_decode_workspace(cache, len(lens), Hkv * G, int(L.max()), BAL)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(9)
    for i in range(3):
        qi = W.f32_to_bf16_bits(rng.standard_normal(q.shape).astype(np.float32))
        out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
        K.kv_int4_paged_decode(cache, bf16_dev(qi), to_dev(tab), to_dev(L), int(L.max()), out=out,
                               split_tokens=BAL, workspace=ws)
        torch.cuda.synchronize()
        decode_compare(out.cpu().numpy(), _ref(orc, qi, tab, L, Hkv, P, 64, 0), f"balanced call {i}")
        assert int(ws[:16384 * 4].count_nonzero()) == 0, f"counters left set after call {i}"


@pytest.mark.parametrize("Hq,kb,vb", [(32, 128, 0), (128, 64, 128)])
def test_fused_step(K, Hq, kb, vb):
    """The fused decode step on the balanced grid: the cache equals the separate write, the
    output equals the balanced decode after it, both within 2e-3 of the oracle; two steps."""
    Hkv, P = 8, 16
    lens = [1, 127, 128, 129, 300, 513, 0, 64, 2500]
    caches, orc, paging, news = _setup(K, lens, Hkv, Hq, P, kb, vb, seed=310 + Hq, steps=2)
    for i in range(2):
        _check_step(K, caches, orc, paging, lens, news[i], Hkv, P, kb, vb, BAL,
                    f"balanced step {i} G{Hq // Hkv}", i=i)


@pytest.mark.parametrize("k_bits,v_bits", [(2, 4), (4, 2), (2, 2)])
def test_two_bit_pools(K, k_bits, v_bits):
    rng = np.random.default_rng(320 + k_bits * 4 + v_bits)
    lens = [700, 3, 2100, 0, 1500]
    Hkv, G, P, kb, vb = 2, 8, 16, 128, 64
    paging = W.assign_pages(np.random.default_rng(321), lens, P)
    T = int(sum(lens))
    k = W.make_rows(rng, T, Hkv, W.OutlierSpec.random(rng, Hkv))
    v = W.make_rows(rng, T, Hkv)
    slots = np.concatenate([paging.slots(s, 0, int(L)) for s, L in enumerate(lens)])
    cache = K.PagedInt4Cache(paging.num_pages, Hkv, P, kb, vb, fill=0, k_bits=k_bits, v_bits=v_bits)
    K.kv_rotquant_write(cache, bf16_dev(k), bf16_dev(v), to_dev(slots))
    orc = oracle.Cache(paging.num_pages, Hkv, P, fill=0, k_bits=k_bits, v_bits=v_bits)
    oracle.write(orc, k, v, slots, kb, vb)
    q = W.f32_to_bf16_bits(rng.standard_normal((len(lens), Hkv * G, D)).astype(np.float32))
    tab = paging.page_table()
    L = np.array(lens, np.int32)
    out = _run(K, cache, q, tab, L, split=BAL)
    ref = oracle.decode(q, (orc.k_codes, orc.v_codes, orc.k_params, orc.v_params), tab, L, Hkv, P,
                        kb, vb)
    decode_compare(out, ref, f"balanced {k_bits}/{v_bits}-bit")
