"""GPU parity of kv_int4_paged_extend (causal chunked-prefill attention over the rotated
INT4 cache) against the oracle's fp64 extend, max abs error <= 2e-3, through the C ABI.

Covers every query-head group size 1..16 (16, 8, 4, 2, 1 query rows per workgroup), pure
prefill (no prefix), single-token chunks, an empty chunk, rotation block pairs, ragged
lengths, forced split counts, and a Qwen3-4B-like batch of 256-token chunks.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_harness import DECODE_ATOL, bf16_dev, decode_compare, to_dev

pytestmark = pytest.mark.gpu
D = 128


@pytest.fixture(scope="module")
def K():
    import int4_kv_cache_rotquant_amd as K
    K.lib()
    return K


def _build(K, lens, news, Hkv, Hq, P, kb, vb, seed):
    rng = np.random.default_rng(seed)
    paging = W.assign_pages(np.random.default_rng(seed + 7), list(lens), P)
    T = int(sum(lens))
    k = W.make_rows(rng, T, Hkv, W.OutlierSpec.random(rng, Hkv))
    v = W.make_rows(rng, T, Hkv)
    slots = np.concatenate([paging.slots(s, 0, int(L)) for s, L in enumerate(lens)])
    cache = K.PagedInt4Cache(paging.num_pages, Hkv, P, kb, vb, fill=0)
    K.kv_rotquant_write(cache, bf16_dev(k), bf16_dev(v), to_dev(slots))
    orc = oracle.Cache(paging.num_pages, Hkv, P, fill=0)
    oracle.write(orc, k, v, slots, kb, vb)
    qo = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    q = W.f32_to_bf16_bits(rng.standard_normal((int(qo[-1]), Hq, D)).astype(np.float32))
    return cache, orc, q, qo, paging.page_table(), np.array(lens, np.int32)


def _run(K, cache, q, qo, tab, lens, news, split=0):
    import torch
    out = K.kv_int4_paged_extend(cache, bf16_dev(q), to_dev(qo), to_dev(tab), to_dev(lens),
                                 int(lens.max()), int(max(max(news), 1)), split_tokens=split)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _ref(orc, q, qo, tab, lens, Hkv, P, kb, vb):
    arrays = (orc.k_codes, orc.v_codes, orc.k_params, orc.v_params)
    return oracle.extend(q, arrays, qo, tab, lens, Hkv, P, kb, vb)


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_group_sizes(K, G):
    lens, news = [37, 16, 5, 200, 70, 0], [9, 16, 1, 64, 0, 0]
    Hkv = 2
    cache, orc, q, qo, tab, L = _build(K, lens, news, Hkv, Hkv * G, 16, 128, 0, seed=30 + G)
    out = _run(K, cache, q, qo, tab, L, news)
    decode_compare(out, _ref(orc, q, qo, tab, L, Hkv, 16, 128, 0), f"extend G={G}")


@pytest.mark.parametrize("kb,vb,P", [(0, 0, 16), (64, 64, 32), (16, 128, 64), (32, 0, 128)])
def test_blocks_and_pages(K, kb, vb, P):
    lens, news = [300, 129, 64], [100, 129, 33]
    cache, orc, q, qo, tab, L = _build(K, lens, news, 2, 8, P, kb, vb, seed=40 + kb + P)
    out = _run(K, cache, q, qo, tab, L, news)
    decode_compare(out, _ref(orc, q, qo, tab, L, 2, P, kb, vb), f"extend kb={kb} vb={vb} P={P}")


def test_long_prefix_one_split(K):
    """A 20k-token prefix walked in one split: each wave of a row block walks ~5k tokens, 300
    pages of 16, so its window of page ids (and the ids requested one move ahead) moves
    several times."""
    lens, news = [20000, 9000], [40, 33]
    Hkv, G = 2, 4
    cache, orc, q, qo, tab, L = _build(K, lens, news, Hkv, Hkv * G, 16, 64, 0, seed=61)
    out = _run(K, cache, q, qo, tab, L, news, split=32768)
    decode_compare(out, _ref(orc, q, qo, tab, L, Hkv, 16, 64, 0), "extend long prefix")


def test_split_counts_agree(K):
    lens, news = [1500, 700], [96, 31]
    cache, orc, q, qo, tab, L = _build(K, lens, news, 1, 8, 16, 128, 0, seed=50)
    ref = _ref(orc, q, qo, tab, L, 1, 16, 128, 0)
    outs = []
    for split in (128, 512, 2048, 0):
        out = _run(K, cache, q, qo, tab, L, news, split=split)
        decode_compare(out, ref, f"extend split {split}")
        outs.append(out)
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) < 1e-4


def test_qwen3_4b_like_chunks(K):
    rng = np.random.default_rng(60)
    news = [256] * 4
    lens = [int(x) + 256 for x in rng.integers(1024, 3073, size=4)]
    cache, orc, q, qo, tab, L = _build(K, lens, news, 8, 32, 16, 64, 0, seed=61)
    out = _run(K, cache, q, qo, tab, L, news)
    decode_compare(out, _ref(orc, q, qo, tab, L, 8, 16, 64, 0), "extend qwen3-4b-like")


def test_last_rows_match_the_decode(K):
    import torch
    lens, news = [333, 100], [40, 100]
    cache, orc, q, qo, tab, L = _build(K, lens, news, 2, 8, 16, 128, 128, seed=70)
    ext = _run(K, cache, q, qo, tab, L, news)
    last = qo[1:] - 1
    dec = K.kv_int4_paged_decode(cache, bf16_dev(q[last]), to_dev(tab), to_dev(L), int(L.max()))
    torch.cuda.synchronize()
    assert np.max(np.abs(ext[last] - dec.cpu().numpy())) < 1e-4


def test_every_prefix_as_a_decode(K):
    """The decode (query heads in pairs of MFMA halves) of each prefix 1..129 of one
    sequence, with the chunk's rows as queries, against the oracle and the extend; plain
    INT4 keys with outlier channels give peaked weights, the case where the f16 split of
    a weight must stay exact."""
    import torch
    lens, news = [300, 129, 64], [100, 129, 33]
    cache, orc, q, qo, tab, L = _build(K, lens, news, 2, 8, 16, 0, 0, seed=56)
    ext = _run(K, cache, q, qo, tab, L, news)
    rows = np.arange(qo[1], qo[2])
    ptab = np.repeat(tab[1:2], len(rows), axis=0)
    plens = np.arange(1, len(rows) + 1, dtype=np.int32)
    dec = K.kv_int4_paged_decode(cache, bf16_dev(q[rows]), to_dev(ptab), to_dev(plens), int(plens.max()))
    torch.cuda.synchronize()
    dec = dec.cpu().numpy()
    arrays = (orc.k_codes, orc.v_codes, orc.k_params, orc.v_params)
    decode_compare(dec, oracle.decode(q[rows], arrays, ptab, plens, 2, 16, 0, 0), "prefix decodes")
    assert np.max(np.abs(dec - ext[rows])) < DECODE_ATOL


def test_one_workspace_for_decode_and_extend(K):
    """One zero-filled workspace serves decode and extend calls in turn: the extend writes
    its partials after the decode's split counters and leaves those alone, so decode,
    extend, decode all match the oracle and the counters are zero after each call (the
    decode here merges its 12 splits inside the split launch)."""
    import torch
    lens, news = [1500, 700], [96, 31]
    cache, orc, q, qo, tab, L = _build(K, lens, news, 1, 8, 16, 128, 0, seed=80)
    arrays = (orc.k_codes, orc.v_codes, orc.k_params, orc.v_params)
    maxlen, total_q, max_q = int(L.max()), int(qo[-1]), int(max(news))
    nd = K.kv_int4_paged_decode_workspace(cache, len(lens), 8, maxlen, 128)
    ne = K.kv_int4_paged_extend_workspace(cache, len(lens), 8, total_q, max_q, maxlen, 128)
    ws = torch.zeros(max(nd, ne), dtype=torch.uint8, device="cuda")
    qd = q[qo[1:] - 1].copy()
    dref = oracle.decode(qd, arrays, tab, L, 1, 16, 128, 0)
    eref = _ref(orc, q, qo, tab, L, 1, 16, 128, 0)
    for step in ("decode", "extend", "decode"):
        if step == "decode":
            out = K.kv_int4_paged_decode(cache, bf16_dev(qd), to_dev(tab), to_dev(L), maxlen,
                                         split_tokens=128, workspace=ws)
            ref = dref
        else:
            out = K.kv_int4_paged_extend(cache, bf16_dev(q), to_dev(qo), to_dev(tab), to_dev(L),
                                         maxlen, max_q, split_tokens=128, workspace=ws)
            ref = eref
        torch.cuda.synchronize()
        assert int(ws[:16384 * 4].count_nonzero()) == 0, f"counters left set after the {step}"
        decode_compare(out.cpu().numpy(), ref, f"shared workspace: {step}")


@pytest.mark.parametrize("split", [0, 128])
def test_bad_qo_start_stays_inside_its_buffers(K, split):
    """qo_start is device data the host cannot check.  Entries beyond total_q, a decreasing
    pair and a negative start give unspecified rows but no access outside q, out or the
    workspace: both buffers sit inside guard bands that must come back untouched."""
    import torch
    lens, news = [300, 200, 150, 90], [20, 20, 20, 20]
    Hkv, G = 2, 4
    Hq = Hkv * G
    cache, orc, q, qo, tab, L = _build(K, lens, news, Hkv, Hq, 16, 64, 0, seed=77)
    total_q = int(qo[-1])
    guard = 4096
    for bad in ([0, 50, 30, 500, total_q], [-8, 10, 70, 75, total_q], [0, 79, 79, 79, 80]):
        bad = np.array(bad, np.int32)
        n_out = total_q * Hq * D
        big = torch.full((n_out + 2 * guard,), 12345.0, dtype=torch.float32, device="cuda")
        out = big[guard:guard + n_out].view(total_q, Hq, D)
        n_ws = K.kv_int4_paged_extend_workspace(cache, len(lens), Hq, total_q, 40, int(L.max()), split)
        ws_big = torch.full((max(n_ws, 16) + 2 * guard,), 0x5A, dtype=torch.uint8, device="cuda")
        ws = ws_big[guard:guard + max(n_ws, 16)]
        ws.zero_()
        K.kv_int4_paged_extend(cache, bf16_dev(q), to_dev(bad), to_dev(tab), to_dev(L), int(L.max()), 40,
                               out=out, split_tokens=split, workspace=ws)
        torch.cuda.synchronize()
        b = big.cpu().numpy()
        assert np.all(b[:guard] == 12345.0) and np.all(b[guard + n_out:] == 12345.0), bad
        w = ws_big.cpu().numpy()
        assert np.all(w[:guard] == 0x5A) and np.all(w[guard + max(n_ws, 16):] == 0x5A), bad
