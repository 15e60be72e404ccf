"""Pins of the oracle's token-wise INT4 encoding.

The pages name the scheme (token-wise INT4 after the block rotation:
fugumt.com abstract; wispaper.ai blog, section 3 core formula) and leave the
quantiser's details open.  The reading used (asymmetric min/max, 16 levels,
fp16 scale and zero per token per head, codes computed from the stored
fp16 parameters, round half to even, even channel in the low nibble) is
pinned here by:

* numpy's binary16 conversion (library routine) for the hand-written
  fp16 <-> fp32 conversions;
* constructed rows that lie exactly on a known grid, whose codes, scale,
  zero and bytes are known in closed form -- in the plain path and through a
  16-block rotation (x = H y is exact for dyadic y);
* the error bound |y - (q s + z)| <= s/2 (+ the fp16 rounding of the
  parameters), the 0..15 range and the use of both end codes;
* degenerate rows;
* an independent vectorised numpy re-derivation (``oracle/brute.py``).
"""
import numpy as np
import pytest

import workloads as W

D = 128


# ---------------------------------------------------------------- fp16 formats
def test_f16_to_f32_all_patterns(oracle_mod):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = oracle_mod.f16_bits_to_f32(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _f32_edge_values():
    vals = []
    # every fp16 value, the midpoints between neighbours and one fp32 ulp around them
    h = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    mids = (h[:-1] + h[1:]) / 2
    for m in (h, mids):
        m32 = m.astype(np.float32)
        vals += [m32, np.nextafter(m32, np.float32(np.inf)), np.nextafter(m32, np.float32(0))]
    vals.append(np.array([65504, 65519.99, 65520, 65536, 1e30, 2.0 ** -24, 2.0 ** -25,
                          2.0 ** -25 * 1.0000001, 2.0 ** -26, 1e-30, 0.0], np.float32))
    v = np.concatenate(vals).astype(np.float32)
    return np.concatenate([v, -v])


def test_f32_to_f16_rne_against_numpy(oracle_mod):
    x = _f32_edge_values()
    rng = np.random.default_rng(7)
    rnd = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 12, 100000))).astype(np.float32)
    x = np.concatenate([x, rnd])
    ref = x.astype(np.float16).view(np.uint16)
    got = oracle_mod.f32_to_f16_bits(x)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- on-grid rows
def _ongrid_rotated_domain(rng, n, s_exp=-3, z=-1.0):
    """Codes c (with 0 and 15 present per row) and y = z + c*2^s_exp, exact."""
    c = rng.integers(0, 16, size=(n, D))
    c[:, rng.integers(0, D, n)] = 0
    for i in range(n):
        a, b = rng.choice(D, 2, replace=False)
        c[i, a], c[i, b] = 0, 15
    y = z + c.astype(np.float64) * 2.0 ** s_exp
    return c, y


def _expected_bytes(c):
    c = c.astype(np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def test_plain_path_on_grid_is_exact(oracle_mod):
    rng = np.random.default_rng(10)
    c, y = _ongrid_rotated_domain(rng, 64)
    xb = W.f32_to_bf16_bits(y.astype(np.float32))
    assert np.array_equal(W.bf16_bits_to_f32(xb).astype(np.float64), y)   # bf16-exact
    for i in range(64):
        codes, params, vpre, _ = oracle_mod.quant_row(xb[i], 0)
        assert params[0] == np.float16(0.125).view(np.uint16)
        assert params[1] == np.float16(-1.0).view(np.uint16)
        assert np.array_equal(codes, _expected_bytes(c[i:i + 1])[0])
        assert np.array_equal(vpre, c[i].astype(np.float32))


def test_rotated_path_on_grid_is_exact(oracle_mod):
    """x = H_16 y with y on the grid: the oracle must return exactly the grid codes."""
    import oracle.brute as br
    rng = np.random.default_rng(11)
    c, y = _ongrid_rotated_domain(rng, 64)
    H = br.hadamard_blockdiag(D, 16)
    x = y @ H.T
    xb = W.f32_to_bf16_bits(x.astype(np.float32))
    assert np.array_equal(W.bf16_bits_to_f32(xb).astype(np.float64), x)   # dyadic, bf16-exact
    for i in range(64):
        codes, params, vpre, yo = oracle_mod.quant_row(xb[i], 16)
        assert np.array_equal(yo.astype(np.float64), y[i])
        assert params[0] == np.float16(0.125).view(np.uint16)
        assert params[1] == np.float16(-1.0).view(np.uint16)
        assert np.array_equal(codes, _expected_bytes(c[i:i + 1])[0])


def test_hand_worked_row():
    """A tiny fixture in tests/golden with codes worked out by hand (see the file)."""
    import oracle
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "plain_row_by_hand.json")
    with open(path) as f:
        g = json.load(f)
    x = np.array(g["x"], np.float32)
    xb = W.f32_to_bf16_bits(x)
    codes, params, _, _ = oracle.quant_row(xb, 0)
    assert [int(v) for v in codes[:len(g["bytes_head"])]] == g["bytes_head"]
    assert float(np.uint16(params[0]).view(np.float16)) == g["scale"]
    assert float(np.uint16(params[1]).view(np.float16)) == g["zero"]


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("b", [0, 16, 32, 64, 128])
def test_error_bound_and_range(oracle_mod, b):
    rng = np.random.default_rng(12 + b)
    out = W.OutlierSpec.random(rng, 1)
    x = W.make_rows(rng, 300, 1, out)[:, 0]
    for i in range(300):
        codes, params, vpre, y = oracle_mod.quant_row(x[i], b)
        s = float(np.uint16(params[0]).view(np.float16))
        z = float(np.uint16(params[1]).view(np.float16))
        q = np.empty(D, np.int64)
        q[0::2] = codes & 15
        q[1::2] = codes >> 4
        assert q.min() >= 0 and q.max() <= 15
        y64 = y.astype(np.float64)
        mn, mx = y64.min(), y64.max()
        slack = max(abs(mn - z), abs(mx - (z + 15 * s)))
        err = np.abs(y64 - (q * s + z))
        assert np.all(err <= s / 2 + slack + 4 * np.spacing(np.float32(max(abs(mn), abs(mx)))))
        if slack < s / 4:
            assert q.min() == 0 and q.max() == 15
        # scale is the fp16 rounding of (mx - mn)/15 computed in fp32
        assert params[0] == np.float16(np.float32(np.float32(mx) - np.float32(mn)) / np.float32(15)).view(np.uint16)
        assert params[1] == np.float16(np.float32(mn)).view(np.uint16)


def test_degenerate_rows(oracle_mod):
    # all-equal row, plain: scale 0, codes 0, zero = the value
    xb = W.f32_to_bf16_bits(np.full(D, 1.5, np.float32))
    codes, params, _, _ = oracle_mod.quant_row(xb, 0)
    assert params[0] == 0 and params[1] == np.float16(1.5).view(np.uint16)
    assert np.all(codes == 0)
    # all-zero row with negative zeros mixed in: zero stored as +0
    x = np.zeros(D, np.float32)
    x[::3] = -0.0
    for b in (0, 16, 128):
        codes, params, _, _ = oracle_mod.quant_row(W.f32_to_bf16_bits(x), b)
        assert params[0] == 0 and params[1] == 0 and np.all(codes == 0)
    # constant row through a rotation is not degenerate: (c sqrt(b), 0, ...) per block
    codes, params, _, y = oracle_mod.quant_row(xb, 16)
    assert params[0] != 0
    assert np.allclose(y[::16], 1.5 * 4) and np.all(np.delete(y, np.arange(0, D, 16)) == 0)


@pytest.mark.parametrize("b", [0, 16, 32, 64, 128])
def test_c_oracle_matches_numpy_rederivation(oracle_mod, b):
    import oracle.brute as br
    rng = np.random.default_rng(20 + b)
    out = W.OutlierSpec.random(rng, 4)
    x = W.make_rows(rng, 500, 4, out)
    codes, s16, z16, vpre = br.quantize_rows(x, b)
    cache = oracle_mod.Cache(500 * 4 // 16 + 1, 4, 16)
    slots = np.arange(500, dtype=np.int32)
    kv, _ = oracle_mod.write(cache, x, x, slots, b, b, want_vpre=True)
    got_c = cache.k_codes.reshape(-1, 4, 16, 64).transpose(0, 2, 1, 3).reshape(-1, 4, 64)[:500]
    got_p = cache.k_params.reshape(-1, 4, 16, 2).transpose(0, 2, 1, 3).reshape(-1, 4, 2)[:500]
    assert np.array_equal(got_c, codes)
    assert np.array_equal(got_p[..., 0], s16)
    assert np.array_equal(got_p[..., 1], z16)
    assert np.array_equal(kv, vpre)


def test_rotation_lowers_quantisation_error_on_outliers(oracle_mod):
    """Direction of the pages' claim (outlier channels stretch the token grid; the
    rotation spreads them): relative MSE with BDR is well below plain INT4."""
    import oracle.brute as br
    rng = np.random.default_rng(30)
    out = W.OutlierSpec.random(rng, 8)
    x = W.make_rows(rng, 512, 8, out)
    xf = W.bf16_bits_to_f32(x).astype(np.float64)
    err = {}
    for b in (0, 16, 64, 128):
        codes, s16, z16, _ = br.quantize_rows(x, b)
        deq = br.dequant_rows(codes, s16, z16) @ br.hadamard_blockdiag(D, b)   # back to x basis
        err[b] = np.mean((deq - xf) ** 2) / np.mean(xf ** 2)
    assert err[128] < err[0] / 4
    assert err[64] < err[0] / 4
    assert err[16] < err[0]


@pytest.mark.parametrize("bits", [4, 2])
def test_codes_from_given_params(oracle_mod, bits):
    """The write's last steps under parameters from elsewhere (what a checker needs when an
    encoder's fp16 scale or zero lands one ulp off at a rounding midpoint): equal to the numpy
    re-derivation for the row's own parameters and for every one-ulp neighbour of them, and
    exact on a row built on the grid of arbitrary given parameters."""
    import oracle.brute as br
    rng = np.random.default_rng(60 + bits)
    x = W.make_rows(rng, 64, 1, W.OutlierSpec.random(rng, 1))[:, 0]
    for b in (0, 64):
        for row in x[:16]:
            codes, params, _, y = oracle_mod.quant_row(row, b, bits)
            got, _ = oracle_mod.codes_from_params(y, params, bits)
            assert np.array_equal(got, codes)
            for ds, dz in ((1, 0), (-1, 0), (0, 1), (0, -1), (1, 1)):
                p = (int(params[0]) + ds, int(params[1]) + dz)
                got, vpre = oracle_mod.codes_from_params(y, p, bits)
                ref, vref = br.codes_for_params(y, np.uint16(p[0]), np.uint16(p[1]), bits)
                assert np.array_equal(got, ref) and np.array_equal(vpre, vref)
    # on the grid of s = 0.375, z = -2.5 (both exact binary16): y = z + c s gives back c
    levels = (1 << bits) - 1
    c = rng.integers(0, levels + 1, size=D)
    y = (np.float32(-2.5) + c.astype(np.float32) * np.float32(0.375)).astype(np.float32)
    s16 = int(np.float16(0.375).view(np.uint16))
    z16 = int(np.float16(-2.5).view(np.uint16))
    got, vpre = oracle_mod.codes_from_params(y, (s16, z16), bits)
    assert np.array_equal(br.unpack_codes(got[None], bits)[0], c)
    assert np.array_equal(vpre, c.astype(np.float32))
    # a zero scale gives all-zero codes
    got, vpre = oracle_mod.codes_from_params(y, (0, z16), bits)
    assert np.all(got == 0) and np.all(vpre == 0)
