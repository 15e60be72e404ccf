"""GPU parity of kv_int4_paged_decode against the oracle's fp64 decode (max abs error
<= 2e-3 on fp32 outputs).  The cache the oracle reads is written by the oracle from the
same seeded inputs (the write is bit-exact, checked in test_gpu_write.py).

Covers the tiny case (G=1), the Qwen3-4B-like layer (G=4, 16 ragged sequences, page 16
scattered), the high-concurrency workload (G=8, 256 log-normal sequences, 100 steps of
write + decode: steps 1, 50 and 100 checked in full and every step write byte for byte),
the 1M-token long context (G=8, K and V rotated: the whole fill byte for byte and all 64
query heads), split-count sweeps, page-table permutation invariance, GQA group sizes
1..16, page sizes 16..128, every block pair, lengths 0, 1, 15..33 and tail tiles,
caches of degenerate rows (zero and tiny scales, spiked keys) in decode and extend, the
in-kernel combine over calls that share one workspace, and the combine launch it falls
back to.
"""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_harness import D, DECODE_ATOL, bf16_dev, decode_compare, log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import int4_kv_cache_rotquant_amd as K
    K.lib()
    return K


def _build(K, lens, Hkv, Hq, P, kb, vb, seed, permute=True, k_out=True, extra_pages=0):
    rng = np.random.default_rng(seed)
    prng = np.random.default_rng(seed + 999)
    paging = W.assign_pages(prng if permute else None, list(lens), P, extra_pages=extra_pages)
    T = int(sum(lens))
    k = W.make_rows(rng, T, Hkv, W.OutlierSpec.random(rng, Hkv) if k_out else None)
    v = W.make_rows(rng, T, Hkv)
    slots = np.concatenate([paging.slots(s, 0, int(L)) for s, L in enumerate(lens)]) if T else \
        np.zeros(0, np.int32)
    q = W.f32_to_bf16_bits(rng.standard_normal((len(lens), Hq, D)).astype(np.float32))
    cache = K.PagedInt4Cache(paging.num_pages, Hkv, P, kb, vb, fill=0)
    if T:
        K.kv_rotquant_write(cache, bf16_dev(k), bf16_dev(v), to_dev(slots))
    orc = oracle.Cache(paging.num_pages, Hkv, P, fill=0)
    if T:
        oracle.write(orc, k, v, slots, kb, vb)
    tab = paging.page_table()
    return cache, orc, q, tab, np.array(lens, np.int32)


def _run(K, cache, q, tab, lens, split=0, sm_scale=0.0):
    import torch
    out = K.kv_int4_paged_decode(cache, bf16_dev(q), to_dev(tab), to_dev(lens),
                                 int(max(lens.max(), 1)), sm_scale=sm_scale, split_tokens=split)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _ref(orc, q, tab, lens, Hkv, P, kb, vb, sm_scale=0.0):
    arrays = (orc.k_codes, orc.v_codes, orc.k_params, orc.v_params)
    return oracle.decode(q, arrays, tab, lens, Hkv, P, kb, vb, sm_scale)


def test_tiny(K):
    w = W.tiny()
    k, v = w.kv()
    cache = K.PagedInt4Cache(w.paging.num_pages, 1, 16, 128, 128, fill=0)
    K.kv_rotquant_write(cache, bf16_dev(k), bf16_dev(v), to_dev(w.all_slots()))
    orc = oracle.Cache(w.paging.num_pages, 1, 16, fill=0)
    oracle.write(orc, k, v, w.all_slots(), 128, 128)
    tab = w.paging.page_table()
    out = _run(K, cache, w.q(), tab, w.seq_lens.astype(np.int32))
    decode_compare(out, _ref(orc, w.q(), tab, w.seq_lens, 1, 16, 128, 128), "tiny")


def test_qwen3_4b_like(K):
    w = W.qwen3_4b_like()
    k, v = w.kv()
    cache = K.PagedInt4Cache(w.paging.num_pages, 8, 16, 64, 0, fill=0)
    K.kv_rotquant_write(cache, bf16_dev(k), bf16_dev(v), to_dev(w.all_slots()))
    orc = oracle.Cache(w.paging.num_pages, 8, 16, fill=0)
    oracle.write(orc, k, v, w.all_slots(), 64, 0)
    tab = w.paging.page_table()
    lens = w.seq_lens.astype(np.int32)
    q = w.q()
    out = _run(K, cache, q, tab, lens)
    decode_compare(out, _ref(orc, q, tab, lens, 8, 16, 64, 0), "qwen3_4b_like")


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_group_sizes_and_tails(K, G):
    lens = [1, 15, 16, 17, 31, 32, 33, 100, 257]
    Hkv = 2
    cache, orc, q, tab, L = _build(K, lens, Hkv, Hkv * G, 16, 128, 0, seed=G)
    out = _run(K, cache, q, tab, L, split=128)
    decode_compare(out, _ref(orc, q, tab, L, Hkv, 16, 128, 0), f"G{G}")


@pytest.mark.parametrize("kb,vb", [(0, 0), (16, 16), (32, 64), (64, 128), (128, 128), (128, 32)])
def test_block_pairs(K, kb, vb):
    lens = [40, 300, 77]
    cache, orc, q, tab, L = _build(K, lens, 2, 8, 16, kb, vb, seed=kb + vb)
    out = _run(K, cache, q, tab, L)
    decode_compare(out, _ref(orc, q, tab, L, 2, 16, kb, vb), f"blocks_{kb}_{vb}")


@pytest.mark.parametrize("P", [16, 32, 64, 128])
def test_page_sizes(K, P):
    lens = [P - 3, 3 * P + 5, 500]
    cache, orc, q, tab, L = _build(K, lens, 1, 4, P, 64, 64, seed=P)
    out = _run(K, cache, q, tab, L, split=128 if P <= 32 else 256)
    decode_compare(out, _ref(orc, q, tab, L, 1, P, 64, 64), f"P{P}")


@pytest.mark.parametrize("split", [16384, 32768])
def test_long_walks_split_grid(K, split):
    """Splits of 16k and 32k tokens: each wave walks up to 8k tokens, 500 pages of 16, so its
    window of 128 page ids (and the ids it requests one move ahead) moves several times on
    the split grid (the large automatic decodes take the balanced grid instead)."""
    lens = [32000, 17001, 5003]
    Hkv, G, P = 2, 4, 16
    cache, orc, q, tab, L = _build(K, lens, Hkv, Hkv * G, P, 128, 0, seed=44)
    out = _run(K, cache, q, tab, L, split=split)
    decode_compare(out, _ref(orc, q, tab, L, Hkv, P, 128, 0), f"long walks split{split}")


def test_split_sweep_consistent(K):
    lens = [2049, 700, 33]
    cache, orc, q, tab, L = _build(K, lens, 2, 16, 16, 128, 128, seed=11)
    ref = _ref(orc, q, tab, L, 2, 16, 128, 128)
    outs = []
    for split in (128, 256, 512, 1024, 4096, 8192, 0):
        out = _run(K, cache, q, tab, L, split=split)
        decode_compare(out, ref, f"split{split}")
        outs.append(out)
    for o in outs[1:]:
        # only the fp32 summation order differs between split counts
        assert np.max(np.abs(o - outs[0])) < 1e-4


def test_combine_split_counts_around_64(K):
    """64 splits is the largest count combined one wave per query head; 65 takes the
    workgroup-per-head combine.  Both must agree with the oracle and with each other."""
    lens = [8192, 8191, 129]
    cache, orc, q, tab, L = _build(K, lens, 1, 8, 16, 64, 32, seed=21)
    ref = _ref(orc, q, tab, L, 1, 16, 64, 32)
    # one more (unused) page-table column so that max_seq_len 8193 is a valid bound
    tab = np.concatenate([tab, np.full((tab.shape[0], 1), -1, np.int32)], axis=1)
    outs = []
    for split, maxlen in ((128, 8192), (128, 8193)):   # 64 and 65 splits
        import torch
        out = K.kv_int4_paged_decode(cache, bf16_dev(q), to_dev(tab), to_dev(L), maxlen,
                                     split_tokens=split)
        torch.cuda.synchronize()
        out = out.cpu().numpy()
        decode_compare(out, ref, f"split{split}/maxlen{maxlen}")
        outs.append(out)
    assert np.max(np.abs(outs[0] - outs[1])) < 1e-5


def test_page_permutation_bit_identical(K):
    lens = [500, 129]
    c1, o1, q1, t1, L1 = _build(K, lens, 2, 8, 16, 128, 0, seed=12, permute=False)
    c2, o2, q2, t2, L2 = _build(K, lens, 2, 8, 16, 128, 0, seed=12, permute=True)
    assert np.array_equal(q1, q2)
    a = _run(K, c1, q1, t1, L1)
    b = _run(K, c2, q2, t2, L2)
    assert np.array_equal(a, b)
    decode_compare(a, _ref(o1, q1, t1, L1, 2, 16, 128, 0), "perm")


def test_zero_length_and_scale_override(K):
    lens = [0, 64, 1]
    cache, orc, q, tab, L = _build(K, lens, 1, 2, 16, 32, 0, seed=13, extra_pages=1)
    tab[0, 0] = 0  # a valid page, never read
    out = _run(K, cache, q, tab, L, sm_scale=0.3)
    assert np.all(out[0] == 0)
    decode_compare(out, _ref(orc, q, tab, L, 1, 16, 32, 0, sm_scale=0.3), "len0_scale")


def test_high_concurrency_sampled(K):
    """256 sequences with log-normal lengths (median 8192, clip [512, 32768]), Hq=64, Hkv=8,
    page 16 scattered over the ~3 GB pool: the full decode launch, with eight sequences
    (shortest, longest and six more) checked against the oracle."""
    import torch
    w = W.qwen3_32b_like_decode()
    lens = (w.seq_lens + 1).astype(np.int32)   # the step's new token is included
    S, Hkv, Hq, P = w.num_seqs, 8, 64, 16
    check = sorted(set([int(np.argmin(lens)), int(np.argmax(lens))] + list(range(0, S, 43))))[:8]
    cache = K.PagedInt4Cache(w.paging.num_pages, Hkv, P, 128, 0, fill=0)
    host_rows = {}
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed)
    for s in range(S):
        slots = w.paging.slots(s, 0, int(lens[s]))
        if s in check:
            rng = w.rng(1000 + s)
            k = W.make_rows(rng, int(lens[s]), Hkv, w.k_out)
            v = W.make_rows(rng, int(lens[s]), Hkv)
            host_rows[s] = (k, v, slots)
            kd, vd = bf16_dev(k), bf16_dev(v)
        else:
            kd = W.make_rows_torch(gen, int(lens[s]), Hkv, w.k_out, "cuda")
            vd = W.make_rows_torch(gen, int(lens[s]), Hkv, None, "cuda")
        K.kv_rotquant_write(cache, kd, vd, to_dev(slots))
    q = W.f32_to_bf16_bits(w.rng(3).standard_normal((S, Hq, D)).astype(np.float32))
    tab = w.paging.page_table()
    log(f"high-concurrency: total tokens {int(lens.sum())}, checking {check}")
    out = _run(K, cache, q, tab, lens)
    for s in check:
        k, v, slots = host_rows[s]
        pages = np.unique(slots // P)
        remap = {int(p): i for i, p in enumerate(pages)}
        local = np.array([remap[int(x) // P] * P + int(x) % P for x in slots], np.int32)
        orc = oracle.Cache(len(pages), Hkv, P, fill=0)
        oracle.write(orc, k, v, local, 128, 0)
        ltab = np.array([[remap[int(p)] for p in tab[s, :len(pages)]]], np.int32)
        ref = _ref(orc, q[s:s + 1], ltab, lens[s:s + 1], Hkv, P, 128, 0)
        decode_compare(out[s:s + 1], ref, f"hc_seq{s}_L{lens[s]}")
    torch.cuda.synchronize()


def test_high_concurrency_100_steps(K):
    """The Qwen3-32B-like workload over its 100 decode steps: 256 sequences of log-normal
    lengths (median 8192, clip [512, 32768]) filled on the device, Hq=64, Hkv=8, page 16
    scattered over the ~3 GB pool, K block 128, the automatic (balanced) plan.  Each step
    writes one new token per sequence (kv_rotquant_write) and decodes every sequence over
    it.  Steps 1, 50 and 100 are checked in full against the oracle (every sequence and
    query head, on the cache bytes the GPU wrote); after the last step the pool must equal
    the pool after the fill with the oracle's write of all 25,600 step rows applied, byte
    for byte (so every step write is exact and nothing else in the pool moved)."""
    import torch
    from gpu_harness import assert_write_ok, compare_write, gpu_cache_arrays
    w = W.qwen3_32b_like_decode()
    S, Hkv, Hq, P = w.num_seqs, 8, 64, 16
    steps = int(w.notes["steps"])
    cache = K.PagedInt4Cache(w.paging.num_pages, Hkv, P, 128, 0, fill=0)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed + 17)
    for s in range(S):
        L = int(w.seq_lens[s])
        K.kv_rotquant_write(cache, W.make_rows_torch(gen, L, Hkv, w.k_out, "cuda"),
                            W.make_rows_torch(gen, L, Hkv, None, "cuda"),
                            to_dev(w.paging.slots(s, 0, L)))
    base = gpu_cache_arrays(cache)
    q = W.f32_to_bf16_bits(w.rng(4).standard_normal((S, Hq, D)).astype(np.float32))
    tab = w.paging.page_table()
    ks, vs, sl = [], [], []
    for i in range(steps):
        slots = np.array([w.paging.slots(s, int(w.seq_lens[s]) + i, 1)[0] for s in range(S)],
                         np.int32)
        k = W.make_rows_torch(gen, S, Hkv, w.k_out, "cuda")
        v = W.make_rows_torch(gen, S, Hkv, None, "cuda")
        K.kv_rotquant_write(cache, k, v, to_dev(slots))
        ks.append(k.view(torch.int16).cpu().numpy().view(np.uint16))
        vs.append(v.view(torch.int16).cpu().numpy().view(np.uint16))
        sl.append(slots)
        lens = (w.seq_lens + i + 1).astype(np.int32)
        out = _run(K, cache, q, tab, lens)
        if i + 1 in (1, 50, steps):
            log(f"step {i + 1}: {int(lens.sum())} tokens")
            ref = oracle.decode(q, gpu_cache_arrays(cache), tab, lens, Hkv, P, 128, 0)
            decode_compare(out, ref, f"hc_step_{i + 1}")
    final = gpu_cache_arrays(cache)
    del cache
    torch.cuda.empty_cache()
    orc = oracle.Cache(w.paging.num_pages, Hkv, P, fill=0)
    orc.k_codes[...], orc.v_codes[...], orc.k_params[...], orc.v_params[...] = base
    del base
    k_all, v_all, s_all = np.concatenate(ks), np.concatenate(vs), np.concatenate(sl)
    oracle.write(orc, k_all, v_all, s_all, 128, 0)
    assert_write_ok(compare_write(final, orc, {"k": k_all, "v": v_all}, s_all, (128, 0)),
                    "hc_100_step_writes")


def test_long_context_full(K):
    """One 1,048,576-token sequence, Hq=64, Hkv=8, page 64 scattered, K and V rotated with
    block 128 and both with outlier channels: the fill by 64 writes of 16384 tokens is
    checked byte for byte against the oracle's write of the same rows (all 16.8M rows), and
    the decode of all 64 query heads against the oracle."""
    import torch
    from gpu_harness import assert_write_ok, compare_write, gpu_cache_arrays
    w = W.long_context()
    C, L, Hkv, Hq, P = w.notes["chunk"], 1 << 20, 8, 64, 64
    cache = K.PagedInt4Cache(w.paging.num_pages, Hkv, P, 128, 128, fill=0)
    kh = np.empty((L, Hkv, D), np.uint16)
    vh = np.empty((L, Hkv, D), np.uint16)
    slots = w.paging.slots(0, 0, L)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed)
    for c in range(L // C):
        k = W.make_rows_torch(gen, C, Hkv, w.k_out, "cuda")
        v = W.make_rows_torch(gen, C, Hkv, w.v_out, "cuda")
        K.kv_rotquant_write(cache, k, v, to_dev(slots[c * C:(c + 1) * C]))
        kh[c * C:(c + 1) * C] = k.view(torch.int16).cpu().numpy().view(np.uint16)
        vh[c * C:(c + 1) * C] = v.view(torch.int16).cpu().numpy().view(np.uint16)
    q = W.f32_to_bf16_bits(w.rng(3).standard_normal((1, Hq, D)).astype(np.float32))
    tab = w.paging.page_table()
    lens = np.array([L], np.int32)
    out = _run(K, cache, q, tab, lens)
    gpu = gpu_cache_arrays(cache)
    del cache
    torch.cuda.empty_cache()
    log("long context: oracle write of all 8 KV heads")
    orc = oracle.Cache(w.paging.num_pages, Hkv, P, fill=0)
    oracle.write(orc, kh, vh, slots, 128, 128)
    assert_write_ok(compare_write(gpu, orc, {"k": kh, "v": vh}, slots, (128, 128)),
                    "long_context_fill")
    del kh, vh
    log("long context: oracle decode of 64 query heads")
    ref = oracle.decode(q, (orc.k_codes, orc.v_codes, orc.k_params, orc.v_params), tab, lens,
                        Hkv, P, 128, 128)
    decode_compare(out, ref, "long_context_full")


@pytest.mark.parametrize("G,vb", [(4, 128), (16, 0), (8, 32)])
def test_single_split_writes_the_output(K, G, vb):
    """One split covering every sequence: the split kernel merges, normalises, rotates V
    back and writes the rows itself (no combine, no workspace); an empty sequence gets
    zero rows.  The output buffer starts as NaN so a row left unwritten fails."""
    import torch
    lens = [0, 5, 100, 128]
    Hkv = 2
    cache, orc, q, tab, L = _build(K, lens, Hkv, Hkv * G, 16, 128, vb, seed=900 + G)
    assert K.kv_int4_paged_decode_workspace(cache, len(lens), Hkv * G, 128, 128) == 0
    out = torch.full((len(lens), Hkv * G, D), float("nan"), dtype=torch.float32, device="cuda")
    K.kv_int4_paged_decode(cache, bf16_dev(q), to_dev(tab), to_dev(L), 128, out=out, split_tokens=128)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(got[0] == 0.0)
    decode_compare(got, _ref(orc, q, tab, L, Hkv, 16, 128, vb), f"single split G{G} vb{vb}")


@pytest.mark.parametrize("G", [4, 16])
def test_in_kernel_combine_reuses_its_workspace(K, G):
    """Up to 16 splits are merged inside the split launch: the last split of each (sequence,
    KV head) to finish, elected by a counter at the head of the workspace, combines the
    partials; a row of one split writes itself and an empty row gets zeros.  Three calls
    share one zero-filled workspace, each with fresh queries: every output matches the
    oracle (the output starts as NaN, so a row nobody writes fails) and the counters are
    zero again after every call."""
    import torch
    lens = [0, 1, 128, 129, 300, 700, 1000, 1025]   # 0, 1, 1, 2, 3, 6, 8 and 9 splits
    Hkv = 2
    cache, orc, q, tab, L = _build(K, lens, Hkv, Hkv * G, 16, 64, 128, seed=950 + G)
    maxlen = int(L.max())
    n = K.kv_int4_paged_decode_workspace(cache, len(lens), Hkv * G, maxlen, 128)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(951 + G)
    for call in range(3):
        qc = q if call == 0 else W.f32_to_bf16_bits(rng.standard_normal(q.shape).astype(np.float32))
        out = torch.full((len(lens), Hkv * G, D), float("nan"), dtype=torch.float32, device="cuda")
        K.kv_int4_paged_decode(cache, bf16_dev(qc), to_dev(tab), to_dev(L), maxlen, out=out,
                               split_tokens=128, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[:16384 * 4].count_nonzero()) == 0, f"counters left set after call {call}"
        got = out.cpu().numpy()
        assert np.all(got[0] == 0.0)
        decode_compare(got, _ref(orc, qc, tab, L, Hkv, 16, 64, 128), f"in-kernel combine G{G} call {call}")


@pytest.mark.parametrize("S", [600, 2050])
def test_combine_launch_beyond_the_counters(K, S):
    """The separate combine launch merges the splits of a grid too large for one round
    (600 sequences x 8 KV heads x 2 splits: counters exist, the launcher leaves them
    unused) and of more (sequence, KV head) pairs than the workspace holds counters
    (2,050 x 8 = 16,400 > 16,384).  Lengths 0..200 in splits of 128; 64 sampled sequences
    checked against the oracle."""
    rng = np.random.default_rng(960 + S)
    Hkv = 8
    lens = rng.integers(0, 201, S)
    lens[:4] = [0, 128, 129, 200]
    cache, orc, q, tab, L = _build(K, lens, Hkv, Hkv, 16, 128, 128, seed=961, k_out=False)
    out = _run(K, cache, q, tab, L, split=128)
    idx = np.concatenate([np.arange(4), np.sort(rng.choice(np.arange(4, S), 60, replace=False))])
    ref = _ref(orc, q[idx].copy(), tab[idx].copy(), L[idx].copy(), Hkv, 16, 128, 128)
    decode_compare(out[idx], ref, "combine launch beyond the counters")


def _degenerate_rows(rng, T, Hkv):
    """K and V rows of every degenerate kind the quantiser has, mixed with ordinary ones:
    all zero, constant (scale 0), a range far below the values (tiny scale), on the code
    grid, and K rows with one large channel (peaked scores that move the softmax maximum
    mid-sequence)."""
    k = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    kind = rng.integers(0, 6, size=T)
    for t in range(T):
        if kind[t] == 1:
            k[t] = 0.0
            v[t] = 0.0
        elif kind[t] == 2:
            k[t] = 1.5
            v[t] = -2.0
        elif kind[t] == 3:
            k[t] = 1.0 + 1e-3 * np.arange(D) / D
            v[t] = 3.0 - 1e-3 * np.arange(D) / D
        elif kind[t] == 4:
            v[t] = -1.0 + (np.arange(D) % 16) / 8.0
        elif kind[t] == 5:
            k[t, :, int(rng.integers(0, D))] = 40.0 * (1 + t % 3)
    return W.f32_to_bf16_bits(k), W.f32_to_bf16_bits(v)


@pytest.mark.parametrize("G,kb,vb", [(4, 128, 64), (8, 0, 0), (16, 64, 128)])
def test_degenerate_rows(K, G, kb, vb):
    """Decode and extend over caches full of zero-scale, tiny-scale and spiked rows."""
    import torch
    Hkv, P = 2, 16
    lens = np.array([37, 300, 129, 1], np.int32)
    rng = np.random.default_rng(77 + G)
    paging = W.assign_pages(np.random.default_rng(78), list(lens), P)
    T = int(lens.sum())
    k, v = _degenerate_rows(rng, T, Hkv)
    slots = np.concatenate([paging.slots(s, 0, int(L)) for s, L in enumerate(lens)])
    cache = K.PagedInt4Cache(paging.num_pages, Hkv, P, kb, vb, fill=0)
    K.kv_rotquant_write(cache, bf16_dev(k), bf16_dev(v), to_dev(slots))
    orc = oracle.Cache(paging.num_pages, Hkv, P, fill=0)
    oracle.write(orc, k, v, slots, kb, vb)
    tab = paging.page_table()
    arrays = (orc.k_codes, orc.v_codes, orc.k_params, orc.v_params)
    q = W.f32_to_bf16_bits(rng.standard_normal((len(lens), Hkv * G, D)).astype(np.float32))
    for split in (0, 128):
        out = _run(K, cache, q, tab, lens, split=split)
        decode_compare(out, _ref(orc, q, tab, lens, Hkv, P, kb, vb), f"degenerate decode G{G} split {split}")
    # extend: the last rows of each sequence (up to 40) as a chunk
    nq = np.minimum(lens, 40)
    qo = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    qx = W.f32_to_bf16_bits(rng.standard_normal((int(qo[-1]), Hkv * G, D)).astype(np.float32))
    out = K.kv_int4_paged_extend(cache, bf16_dev(qx), to_dev(qo), to_dev(tab), to_dev(lens),
                                 int(lens.max()), int(nq.max()))
    torch.cuda.synchronize()
    ref = oracle.extend(qx, arrays, qo, tab, lens, Hkv, P, kb, vb)
    decode_compare(out.cpu().numpy(), ref, f"degenerate extend G{G}")
