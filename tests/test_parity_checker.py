"""The write parity checker (gpu_harness.compare_write) pinned on the CPU: a "GPU" cache is
the oracle's own cache with a planted difference, and the checker must count it and excuse it
exactly when the rules allow.

  * codes: a differing code is excused only if it differs by one and its pre-round value
    lies within 1e-6 relative of the boundary between the two codes (an exact tie k + 1/2
    flipped to its other neighbour is excused; any other flip is not);
  * parameters: a differing fp16 scale or zero is excused only if the oracle's fp32 value
    lies within 1e-6 relative of the fp16 midpoint between the two, and that row's codes
    must then be the ones the GPU's own parameters give, re-derived by the oracle;
  * placement: a byte changed outside every written slot is a placement mismatch.

No GPU is used: the planted mistakes live in copies of the oracle's arrays."""
import numpy as np
import pytest

import oracle
from gpu_harness import _codes, assert_write_ok, compare_write

D = 128


def _bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest even (finite inputs)."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _write(k, v, slots, num_pages, Hkv, P, kb, vb):
    orc = oracle.Cache(num_pages, Hkv, P)
    oracle.write(orc, k, v, slots, kb, vb)
    gpu = [a.copy() for a in (orc.k_codes, orc.v_codes, orc.k_params, orc.v_params)]
    return orc, gpu


def _small_case(seed=3, kb=128, vb=0):
    rng = np.random.default_rng(seed)
    T, Hkv, P, num_pages = 20, 2, 16, 4
    k = _bf16(rng.standard_normal((T, Hkv, D)).astype(np.float32))
    v = _bf16(rng.standard_normal((T, Hkv, D)).astype(np.float32))
    slots = rng.permutation(num_pages * P)[:T].astype(np.int32)
    slots[5] = -1                                   # a skipped token
    orc, gpu = _write(k, v, slots, num_pages, Hkv, P, kb, vb)
    return orc, gpu, {"k": k, "v": v}, slots, (kb, vb), P


def _cell(slots, t, P):
    s = int(slots[t])
    return s // P, s % P


def test_identical_cache_passes():
    orc, gpu, rows, slots, blocks, P = _small_case()
    rep = compare_write(tuple(gpu), orc, rows, slots, blocks)
    assert all(v == 0 for v in rep.values())
    assert_write_ok(rep, "identical")


@pytest.mark.parametrize("delta", [1, 2])
def test_code_flip_off_boundary_is_not_excused(delta):
    orc, gpu, rows, slots, blocks, P = _small_case()
    page, off = _cell(slots, 7, P)
    _, _, vpre, _ = oracle.quant_row(rows["k"][7, 1], blocks[0])
    codes = _codes(gpu[0][page, 1, off][None], 4)[0]
    # the channel farthest from a rounding boundary k + 1/2
    d = int(np.argmax(np.abs(vpre - np.floor(vpre) - 0.5)))
    new = codes.copy()
    new[d] = codes[d] + delta if codes[d] + delta <= 15 else codes[d] - delta
    packed = (new[0::2] | (new[1::2] << 4)).astype(np.uint8)
    gpu[0][page, 1, off] = packed
    rep = compare_write(tuple(gpu), orc, rows, slots, blocks)
    assert rep["code_mismatch"] == 1 and rep["code_excused"] == 0
    with pytest.raises(AssertionError):
        assert_write_ok(rep, "planted")


def test_tie_flip_is_excused_and_counted():
    """A plain row with min 0 and max 15 has scale 1 and zero 0, so a value k + 1/2 is an exact
    tie: the oracle rounds it to the even code; the odd neighbour is excused, and counted."""
    T, Hkv, P, num_pages = 1, 1, 16, 1
    x = np.zeros((T, Hkv, D), np.float32)
    x[0, 0, 0], x[0, 0, 1] = 0.0, 15.0
    x[0, 0, 2:] = np.arange(D - 2) % 15 + 0.5          # every k + 1/2 in 0.5 .. 14.5
    k = _bf16(x)
    v = _bf16(np.ones((T, Hkv, D), np.float32))
    slots = np.array([3], np.int32)
    orc, gpu = _write(k, v, slots, num_pages, Hkv, P, 0, 0)
    codes = _codes(gpu[0][0, 0, 3][None], 4)[0]
    assert codes[2] == 0 and codes[3] == 2                # 0.5 -> 0, 1.5 -> 2 (half to even)
    new = codes.copy()
    new[2], new[3] = 1, 1                                 # the other neighbours
    gpu[0][0, 0, 3] = (new[0::2] | (new[1::2] << 4)).astype(np.uint8)
    rep = compare_write(tuple(gpu), orc, {"k": k, "v": v}, slots, (0, 0))
    assert rep["code_mismatch"] == 2 and rep["code_excused"] == 2
    assert_write_ok(rep, "ties")


def test_placement_outside_written_slots_is_caught():
    orc, gpu, rows, slots, blocks, P = _small_case()
    written = {int(s) for s in slots if s >= 0}
    free = next(s for s in range(4 * P) if s not in written)
    gpu[1][free // P, 0, free % P, 0] ^= 0x11            # a V code byte of an unwritten slot
    rep = compare_write(tuple(gpu), orc, rows, slots, blocks)
    assert rep["placement_mismatch"] == 1
    with pytest.raises(AssertionError):
        assert_write_ok(rep, "placement")


def test_param_off_midpoint_is_not_excused():
    orc, gpu, rows, slots, blocks, P = _small_case()
    page, off = _cell(slots, 9, P)
    gpu[2][page, 0, off, 0] += 1                          # scale one fp16 ulp up
    rep = compare_write(tuple(gpu), orc, rows, slots, blocks)
    assert rep["param_mismatch"] == 1 and rep["param_excused"] == 0
    with pytest.raises(AssertionError):
        assert_write_ok(rep, "param")


def _midpoint_row(b=128, tries=60000, seed=11):
    """A bf16 row (outlier channels, rotated by b) whose fp32 scale lies within 1e-6 relative
    of an fp16 rounding midpoint, and whose codes under the two roundings differ."""
    rng = np.random.default_rng(seed)
    for _ in range(tries):
        x = rng.standard_normal(D).astype(np.float32)
        x[rng.choice(D, 3, replace=False)] *= rng.uniform(10, 30, 3).astype(np.float32)
        xb = _bf16(x)
        codes, params, vpre, y = oracle.quant_row(xb, b)
        mn, mx = np.float32(y.min()), np.float32(y.max())
        s32 = np.float32((mx - mn) / np.float32(15))
        s16 = np.uint16(params[0])
        a = float(s16.view(np.float16))
        nb = np.uint16(s16 + 1) if float(s32) > a else np.uint16(s16 - 1)
        mid = (a + float(nb.view(np.float16))) / 2
        if abs(float(s32) - mid) > 1e-6 * abs(mid):
            continue
        other = np.array([nb, params[1]], np.uint16)
        codes_o, _ = oracle.codes_from_params(y, other)
        if not np.array_equal(codes_o, codes):
            return xb, params, other, codes, codes_o
    pytest.skip("no midpoint row in the search")


def test_param_at_midpoint_is_excused_and_codes_rederived():
    xb, params, other, codes, codes_o = _midpoint_row()
    T, Hkv, P, num_pages = 1, 1, 16, 1
    k = xb.reshape(T, Hkv, D)
    v = _bf16(np.ones((T, Hkv, D), np.float32))
    slots = np.array([0], np.int32)
    orc, gpu = _write(k, v, slots, num_pages, Hkv, P, 128, 0)
    # the GPU rounded the scale the other way and coded with it: excused, codes agree
    gpu[2][0, 0, 0] = other
    gpu[0][0, 0, 0] = codes_o
    rep = compare_write(tuple(gpu), orc, {"k": k, "v": v}, slots, (128, 0))
    assert rep["param_mismatch"] == 1 and rep["param_excused"] == 1
    assert rep["code_mismatch"] == rep["code_excused"]
    assert_write_ok(rep, "midpoint")
    # the same parameters with the oracle's own codes: the row's codes disagree with the
    # GPU's parameters, which the re-derivation catches
    gpu[0][0, 0, 0] = codes
    rep = compare_write(tuple(gpu), orc, {"k": k, "v": v}, slots, (128, 0))
    assert rep["param_excused"] == 1 and rep["code_mismatch"] > 0


def test_decode_compare_bounds():
    """gpu_harness.decode_compare: 2e-3 absolute per element, and per output row
    ||err|| <= 1e-3 ||ref|| + 1e-4; planted errors beyond either bound fail."""
    from gpu_harness import decode_compare
    rng = np.random.default_rng(5)
    ref = rng.standard_normal((3, 4, D)) * 0.5
    ok = ref + rng.uniform(-1e-5, 1e-5, ref.shape)
    decode_compare(ok.astype(np.float32), ref, "noise")
    one = ok.copy()
    one[1, 2, 7] += 3e-3                                   # one element past 2e-3
    with pytest.raises(AssertionError):
        decode_compare(one.astype(np.float32), ref, "element")
    row = ok.copy()
    # every channel of one row 1.5e-3 off: each element within 2e-3, the row norm not
    row[2, 1] += 1.5e-3 * np.sign(rng.standard_normal(D))
    assert np.abs(row - ref).max() < 2e-3
    assert np.linalg.norm(row[2, 1] - ref[2, 1]) > 1e-3 * np.linalg.norm(ref[2, 1]) + 1e-4
    with pytest.raises(AssertionError):
        decode_compare(row.astype(np.float32), ref, "row")
    bad = ok.copy()
    bad[0, 0, 0] = np.nan
    with pytest.raises(AssertionError):
        decode_compare(bad.astype(np.float32), ref, "nan")
