"""Pins of the oracle's fp64 paged decode.

Plain definition: softmax attention of the rotated query over the
de-quantised cache, rotated back through H_bV (wispaper.ai blog, section 3:
query rotated at inference, dot product unchanged; K and V both stored
rotated by the core formula).  Pinned by:

* an independent numpy brute force with explicit scipy Hadamard matrices;
* closed forms: one token -> H_bV v^; zero query -> mean of v^; two tokens
  with hand-computable scores;
* caches whose codes represent the rotated rows exactly, where the decode
  must equal exact attention over the unrotated K, V (catches a missing or
  wrong query rotation and a missing or wrong inverse V rotation);
* GQA head mapping, page-permutation invariance, scale override, empty
  sequences.
"""
import math

import numpy as np
import pytest

import workloads as W

D = 128


def _setup(seed, lens, Hkv, Hq, P, kb, vb, permute=True, outliers=True):
    rng = np.random.default_rng(seed)
    import oracle
    prng = np.random.default_rng(seed + 1000)
    paging = W.assign_pages(prng if permute else None, list(lens), P)
    out = W.OutlierSpec.random(rng, Hkv) if outliers else None
    T = int(sum(lens))
    k = W.make_rows(rng, T, Hkv, out)
    v = W.make_rows(rng, T, Hkv)
    slots = np.concatenate([paging.slots(s, 0, int(L)) for s, L in enumerate(lens)])
    cache = oracle.Cache(paging.num_pages, Hkv, P)
    oracle.write(cache, k, v, slots, kb, vb)
    q = W.f32_to_bf16_bits(rng.standard_normal((len(lens), Hq, D)).astype(np.float32))
    arrays = (cache.k_codes, cache.v_codes, cache.k_params, cache.v_params)
    return q, arrays, paging.page_table(), np.array(lens, np.int32), k, v


@pytest.mark.parametrize("kb,vb", [(128, 128), (64, 0), (0, 0), (16, 32)])
def test_c_oracle_matches_brute_force(oracle_mod, kb, vb):
    import oracle.brute as br
    lens = [1, 17, 64, 100]
    q, arrays, tab, L, _, _ = _setup(1, lens, 2, 8, 16, kb, vb)
    a = oracle_mod.decode(q, arrays, tab, L, 2, 16, kb, vb)
    b = br.decode(q, arrays, tab, L, 2, 16, kb, vb)
    assert np.max(np.abs(a - b)) < 1e-12


def test_tiny_workload_brute_force(oracle_mod):
    import oracle.brute as br
    w = W.tiny()
    k, v = w.kv()
    cache = oracle_mod.Cache(w.paging.num_pages, 1, 16)
    oracle_mod.write(cache, k, v, w.all_slots(), 128, 128)
    arrays = (cache.k_codes, cache.v_codes, cache.k_params, cache.v_params)
    a = oracle_mod.decode(w.q(), arrays, w.paging.page_table(), w.seq_lens, 1, 16, 128, 128)
    b = br.decode(w.q(), arrays, w.paging.page_table(), w.seq_lens, 1, 16, 128, 128)
    assert np.max(np.abs(a - b)) < 1e-12


@pytest.mark.parametrize("vb", [0, 16, 128])
def test_single_token_returns_rotated_back_value(oracle_mod, vb):
    import oracle.brute as br
    q, arrays, tab, L, _, _ = _setup(2, [1], 1, 4, 16, 128, vb)
    out = oracle_mod.decode(q, arrays, tab, L, 1, 16, 128, vb)
    kc, vc, kp, vp = arrays
    page = tab[0, 0]
    vhat = br.dequant_rows(vc[page, 0, 0][None], vp[page, 0, 0, 0], vp[page, 0, 0, 1])[0]
    expect = oracle_mod.rotate_f64(vhat, vb)
    for g in range(4):
        assert np.allclose(out[0, g], expect, atol=1e-14)


def test_zero_query_gives_mean_value(oracle_mod):
    import oracle.brute as br
    lens = [37]
    q, arrays, tab, L, _, _ = _setup(3, lens, 1, 1, 16, 64, 128)
    q[:] = 0
    out = oracle_mod.decode(q, arrays, tab, L, 1, 16, 64, 128)
    _, V = br.gather_seq(arrays, tab[0], 37, 16, 0)
    assert np.allclose(out[0, 0], oracle_mod.rotate_f64(V.mean(0), 128), atol=1e-13)


def test_two_tokens_hand_scores(oracle_mod):
    """Two plain-grid K rows that differ only in channel 0, and q = 2 e_0: the softmax
    weights follow in closed form from the de-quantised channel-0 values."""
    # each row: channel 1 = 1, channel 2 = 0, the rest 0.5 -> min 0, max 1, scale fp16(1/15);
    # channel 0 is 1 (code 15) in token 0 and 0 (code 0) in token 1.
    x = np.full((2, 1, D), 0.5, np.float32)
    x[:, 0, 1], x[:, 0, 2] = 1.0, 0.0
    x[0, 0, 0], x[1, 0, 0] = 1.0, 0.0
    k = W.f32_to_bf16_bits(x)
    v = W.f32_to_bf16_bits(np.stack([np.full((1, D), 2.0), np.full((1, D), -2.0)]).astype(np.float32))
    cache = oracle_mod.Cache(1, 1, 16)
    oracle_mod.write(cache, k, v, np.array([0, 1], np.int32), 0, 0)
    s = float(np.float16(np.float32(1) / np.float32(15)))
    k0 = 15 * s          # de-quantised channel 0 of token 0; token 1 de-quantises to 0 there
    q = np.zeros((1, 1, D), np.float32)
    q[0, 0, 0] = 2.0
    # the other channels are equal in both tokens and q is zero there
    arrays = (cache.k_codes, cache.v_codes, cache.k_params, cache.v_params)
    for sm in (0.0, 0.25):
        out = oracle_mod.decode(W.f32_to_bf16_bits(q), arrays, np.array([[0]], np.int32),
                                np.array([2], np.int32), 1, 16, 0, 0, sm_scale=sm)
        scale = 1 / math.sqrt(D) if sm == 0 else sm
        p0 = 1.0 / (1.0 + math.exp(-scale * 2.0 * k0))
        assert np.allclose(out[0, 0], p0 * 2.0 + (1 - p0) * -2.0, atol=1e-12)


def _ongrid_pair(rng, n):
    """bf16 rows x whose 16-block rotation lies exactly on the grid (-1 + c/8)."""
    import oracle.brute as br
    c = rng.integers(0, 16, size=(n, D))
    c[:, 0], c[:, 1] = 0, 15
    y = -1.0 + c / 8.0
    x = y @ br.hadamard_blockdiag(D, 16).T
    xb = W.f32_to_bf16_bits(x.astype(np.float32))
    assert np.array_equal(W.bf16_bits_to_f32(xb).astype(np.float64), x)
    return xb, x


def test_exactly_represented_cache_equals_plain_attention(oracle_mod):
    """When the codes represent H k and H v exactly, the decode must equal ordinary attention
    over the unrotated k and v: pins the query rotation and the inverse V rotation."""
    rng = np.random.default_rng(4)
    L = 40
    kb_, kx = _ongrid_pair(rng, L)
    vb_, vx = _ongrid_pair(rng, L)
    cache = oracle_mod.Cache(4, 1, 16)
    oracle_mod.write(cache, kb_[:, None], vb_[:, None], np.arange(L, dtype=np.int32), 16, 16)
    qb = W.f32_to_bf16_bits(rng.standard_normal((1, 2, D)).astype(np.float32))
    qf = W.bf16_bits_to_f32(qb).astype(np.float64)
    arrays = (cache.k_codes, cache.v_codes, cache.k_params, cache.v_params)
    out = oracle_mod.decode(qb, arrays, np.arange(4, dtype=np.int32)[None], np.array([L], np.int32),
                            1, 16, 16, 16)
    for g in range(2):
        sc = (kx @ qf[0, g]) / math.sqrt(D)
        p = np.exp(sc - sc.max())
        p /= p.sum()
        assert np.allclose(out[0, g], p @ vx, atol=1e-12)


def test_gqa_head_mapping(oracle_mod):
    """Query head g reads KV head g // (Hq/Hkv)."""
    lens = [50]
    q, arrays, tab, L, _, _ = _setup(5, lens, 2, 6, 16, 32, 0)
    out = oracle_mod.decode(q, arrays, tab, L, 2, 16, 32, 0)
    for h in range(2):
        sub = tuple(a[:, h:h + 1].copy() for a in arrays)
        single = oracle_mod.decode(q[:, 3 * h:3 * h + 3].copy(), sub, tab, L, 1, 16, 32, 0)
        assert np.allclose(out[:, 3 * h:3 * h + 3], single, atol=1e-15)


def test_page_permutation_invariance(oracle_mod):
    lens = [70, 33]
    qa, aa, ta, La, _, _ = _setup(6, lens, 1, 2, 16, 128, 0, permute=False)
    qb, ab, tb, Lb, _, _ = _setup(6, lens, 1, 2, 16, 128, 0, permute=True)
    # same seed -> same values; only the physical pages differ
    assert np.array_equal(qa, qb)
    oa = oracle_mod.decode(qa, aa, ta, La, 1, 16, 128, 0)
    ob = oracle_mod.decode(qb, ab, tb, Lb, 1, 16, 128, 0)
    assert np.array_equal(oa, ob)


def test_empty_sequence_gives_zeros(oracle_mod):
    q, arrays, tab, L, _, _ = _setup(7, [20, 5], 1, 1, 16, 0, 0)
    L[1] = 0
    out = oracle_mod.decode(q, arrays, tab, L, 1, 16, 0, 0)
    assert np.all(out[1] == 0) and np.any(out[0] != 0)


def test_decode_close_to_unquantised_attention_with_rotation(oracle_mod):
    """Quality direction (not a parity pin): with outlier K, the BDR cache keeps attention
    closer to the unquantised result than plain INT4 does."""
    rng = np.random.default_rng(8)
    L, Hkv, Hq = 256, 1, 4
    out = W.OutlierSpec.random(rng, Hkv)
    k = W.make_rows(rng, L, Hkv, out)
    v = W.make_rows(rng, L, Hkv)
    q = W.f32_to_bf16_bits(rng.standard_normal((1, Hq, D)).astype(np.float32) * 3)
    kf = W.bf16_bits_to_f32(k[:, 0]).astype(np.float64)
    vf = W.bf16_bits_to_f32(v[:, 0]).astype(np.float64)
    qf = W.bf16_bits_to_f32(q[0]).astype(np.float64)
    sc = qf @ kf.T / math.sqrt(D)
    p = np.exp(sc - sc.max(1, keepdims=True))
    ref = (p / p.sum(1, keepdims=True)) @ vf
    errs = {}
    for kb in (0, 128):
        cache = oracle_mod.Cache(16, Hkv, 16)
        oracle_mod.write(cache, k, v, np.arange(L, dtype=np.int32), kb, 0)
        arrays = (cache.k_codes, cache.v_codes, cache.k_params, cache.v_params)
        o = oracle_mod.decode(q, arrays, np.arange(16, dtype=np.int32)[None], np.array([L], np.int32),
                              Hkv, 16, kb, 0)
        errs[kb] = np.abs(o[0] - ref).max()
    assert errs[128] < errs[0]
