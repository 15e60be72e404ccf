"""Pins of the oracle's 2-bit variant (the pages leave 2-bit open: wispaper.ai blog,
section 5, limitations), read as the INT4 quantiser with 3 levels and four codes per byte.

* a row worked by hand (tests/golden/int2_row_by_hand.json);
* on-grid rows, plain and through a 16-block rotation, give their grid codes exactly;
* the error bound |y - (c s + z)| <= s/2 (+ fp16 slack), codes 0 and 3 both present;
* the C oracle equals an independent numpy re-derivation (oracle/brute.py) for every
  block, for K and V at 2 bits and for mixed widths;
* the decode equals a numpy brute force with explicit matrices for mixed widths, and
  2-bit V with an exactly representable cache equals exact attention.
"""
import json
import os

import numpy as np
import pytest

import workloads as W

D = 128


def _codes2(c):
    c = np.asarray(c, np.uint8)
    return (c[..., 0::4] | (c[..., 1::4] << 2) | (c[..., 2::4] << 4) | (c[..., 3::4] << 6)).astype(np.uint8)


def test_hand_worked_row(oracle_mod):
    path = os.path.join(os.path.dirname(__file__), "golden", "int2_row_by_hand.json")
    with open(path) as f:
        g = json.load(f)
    xb = W.f32_to_bf16_bits(np.array(g["x"], np.float32))
    codes, params, _, _ = oracle_mod.quant_row(xb, 0, bits=2)
    assert len(codes) == g["num_bytes"]
    assert [int(v) for v in codes[:len(g["bytes_head"])]] == g["bytes_head"]
    assert all(int(v) == 228 for v in codes[2:])
    assert float(np.uint16(params[0]).view(np.float16)) == g["scale"]
    assert float(np.uint16(params[1]).view(np.float16)) == g["zero"]


@pytest.mark.parametrize("b", [0, 16])
def test_on_grid_rows_are_exact(oracle_mod, b):
    import oracle.brute as br
    rng = np.random.default_rng(40 + b)
    for _ in range(32):
        c = rng.integers(0, 4, size=D)
        c[rng.choice(D, 2, replace=False)] = [0, 3]
        y = -2.0 + c * 0.25
        x = y if b == 0 else y @ br.hadamard_blockdiag(D, b).T
        xb = W.f32_to_bf16_bits(x.astype(np.float32))
        assert np.array_equal(W.bf16_bits_to_f32(xb).astype(np.float64), x)
        codes, params, vpre, yo = oracle_mod.quant_row(xb, b, bits=2)
        assert np.array_equal(yo.astype(np.float64), y)
        assert params[0] == np.float16(0.25).view(np.uint16)
        assert params[1] == np.float16(-2.0).view(np.uint16)
        assert np.array_equal(codes, _codes2(c))
        assert np.array_equal(vpre, c.astype(np.float32))


@pytest.mark.parametrize("b", [0, 32, 128])
def test_error_bound_and_range(oracle_mod, b):
    import oracle.brute as br
    rng = np.random.default_rng(50 + b)
    x = W.make_rows(rng, 200, 1, W.OutlierSpec.random(rng, 1))[:, 0]
    for i in range(200):
        codes, params, _, y = oracle_mod.quant_row(x[i], b, bits=2)
        s = float(np.uint16(params[0]).view(np.float16))
        z = float(np.uint16(params[1]).view(np.float16))
        q = br.unpack_codes(codes, 2)
        y64 = y.astype(np.float64)
        mn, mx = y64.min(), y64.max()
        slack = max(abs(mn - z), abs(mx - (z + 3 * s)))
        err = np.abs(y64 - (q * s + z))
        assert np.all(err <= s / 2 + slack + 4 * np.spacing(np.float32(max(abs(mn), abs(mx)))))
        if slack < s / 4:
            assert q.min() == 0 and q.max() == 3
        assert params[0] == np.float16(np.float32(np.float32(mx) - np.float32(mn)) / np.float32(3)).view(np.uint16)


def test_degenerate_row(oracle_mod):
    codes, params, _, _ = oracle_mod.quant_row(W.f32_to_bf16_bits(np.full(D, -0.5, np.float32)), 0, bits=2)
    assert params[0] == 0 and params[1] == np.float16(-0.5).view(np.uint16) and np.all(codes == 0)


@pytest.mark.parametrize("b", [0, 16, 64, 128])
@pytest.mark.parametrize("kbits,vbits", [(2, 2), (4, 2), (2, 4)])
def test_write_matches_numpy_rederivation(oracle_mod, b, kbits, vbits):
    import oracle.brute as br
    rng = np.random.default_rng(60 + b + kbits)
    x = W.make_rows(rng, 300, 2, W.OutlierSpec.random(rng, 2))
    cache = oracle_mod.Cache(300 // 16 + 1, 2, 16, k_bits=kbits, v_bits=vbits)
    oracle_mod.write(cache, x, x, np.arange(300, dtype=np.int32), b, b)
    for bits, codes_arr, params_arr in ((kbits, cache.k_codes, cache.k_params),
                                        (vbits, cache.v_codes, cache.v_params)):
        codes, s16, z16, _ = br.quantize_rows(x, b, bits)
        rb = D * bits // 8
        got_c = codes_arr.reshape(-1, 2, 16, rb).transpose(0, 2, 1, 3).reshape(-1, 2, rb)[:300]
        got_p = params_arr.reshape(-1, 2, 16, 2).transpose(0, 2, 1, 3).reshape(-1, 2, 2)[:300]
        assert np.array_equal(got_c, codes)
        assert np.array_equal(got_p[..., 0], s16) and np.array_equal(got_p[..., 1], z16)


@pytest.mark.parametrize("kbits,vbits,kb,vb", [(2, 2, 128, 128), (4, 2, 64, 0), (2, 4, 0, 16)])
def test_decode_and_extend_match_brute_force(oracle_mod, kbits, vbits, kb, vb):
    import oracle.brute as br
    rng = np.random.default_rng(70 + kbits + vb)
    lens, Hkv, Hq, P = [37, 5, 64], 2, 8, 16
    paging = W.assign_pages(rng, lens, P)
    T = sum(lens)
    k = W.make_rows(rng, T, Hkv, W.OutlierSpec.random(rng, Hkv))
    v = W.make_rows(rng, T, Hkv)
    slots = np.concatenate([paging.slots(s, 0, L) for s, L in enumerate(lens)])
    cache = oracle_mod.Cache(paging.num_pages, Hkv, P, k_bits=kbits, v_bits=vbits)
    oracle_mod.write(cache, k, v, slots, kb, vb)
    arrays = (cache.k_codes, cache.v_codes, cache.k_params, cache.v_params)
    q = W.f32_to_bf16_bits(rng.standard_normal((3, Hq, D)).astype(np.float32))
    L = np.array(lens, np.int32)
    tab = paging.page_table()
    got = oracle_mod.decode(q, arrays, tab, L, Hkv, P, kb, vb)
    ref = br.decode(q, arrays, tab, L, Hkv, P, kb, vb)
    assert np.max(np.abs(got - ref)) < 1e-10
    qo = np.array([0, 4, 5, 9], np.int32)
    qe = W.f32_to_bf16_bits(rng.standard_normal((9, Hq, D)).astype(np.float32))
    got = oracle_mod.extend(qe, arrays, qo, tab, L, Hkv, P, kb, vb)
    ref = br.extend(qe, arrays, qo, tab, L, Hkv, P, kb, vb)
    assert np.max(np.abs(got - ref)) < 1e-10


def test_exactly_representable_two_bit_cache_equals_attention(oracle_mod):
    """K and V rows on a 2-bit grid (plain): the decode equals exact softmax attention
    over those rows, which catches a wrong code position or width in the reader."""
    rng = np.random.default_rng(80)
    L, Hq = 20, 2
    ck = rng.integers(0, 4, size=(L, D))
    cv = rng.integers(0, 4, size=(L, D))
    ck[:, :2] = [0, 3]
    cv[:, :2] = [0, 3]
    kr = -1.0 + 0.5 * ck
    vr = -0.25 + 0.125 * cv
    cache = oracle_mod.Cache(2, 1, 16, k_bits=2, v_bits=2)
    oracle_mod.write(cache, W.f32_to_bf16_bits(kr[:, None].astype(np.float32)),
                     W.f32_to_bf16_bits(vr[:, None].astype(np.float32)), np.arange(L, dtype=np.int32), 0, 0)
    arrays = (cache.k_codes, cache.v_codes, cache.k_params, cache.v_params)
    qb = W.f32_to_bf16_bits(rng.standard_normal((1, Hq, D)).astype(np.float32))
    qf = W.bf16_bits_to_f32(qb).astype(np.float64)[0]
    got = oracle_mod.decode(qb, arrays, np.array([[0, 1]], np.int32), np.array([L], np.int32), 1, 16, 0, 0)
    for g in range(Hq):
        sc = kr @ qf[g] / np.sqrt(D)
        p = np.exp(sc - sc.max())
        assert np.allclose(got[0, g], p @ vr / p.sum(), atol=1e-12)
