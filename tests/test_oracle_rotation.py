"""Pins of the oracle's rotation (block-diagonal Hadamard, BDR).

The pages define the rotation only in words and one garbled formula
(wispaper.ai blog, section 2 block-diagonal bullet: blocks of 16..128
channels rotated independently; section 3 core formula K~ = quant(K H_blk);
section 3 consequence 3: rotating the query keeps the dot product).  These
tests tie the oracle to things outside itself:

* ``scipy.linalg.hadamard`` (a library routine) for the matrix, its order
  and its normalisation;
* closed forms: unit vectors, spikes, constant blocks, the first row;
* the invariant (H q).(H k) = q.k and H H^T = I;
* a rounding-error bound between the fp32 butterflies and the exact fp64
  product.
"""
import numpy as np
import pytest
import scipy.linalg

BLOCKS = [16, 32, 64, 128]
D = 128


def test_rb_is_nearest_binary32(oracle_mod):
    for b in BLOCKS:
        r = oracle_mod.rb(b)
        exact = 1.0 / np.sqrt(np.float64(b))
        ulp = np.spacing(np.float32(r))
        assert abs(np.float64(r) - exact) <= 0.5 * np.float64(ulp)
    assert oracle_mod.rb(16) == np.float32(0.25)
    assert oracle_mod.rb(64) == np.float32(0.125)


@pytest.mark.parametrize("b", BLOCKS)
def test_unit_vectors_give_hadamard_columns(oracle_mod, b):
    """FWHT(e_j) equals column j of the block-diagonal scipy Hadamard / sqrt(b), bit for bit."""
    Hb = scipy.linalg.hadamard(b).astype(np.float64) / np.sqrt(b)
    ref = scipy.linalg.block_diag(*([Hb] * (D // b))).astype(np.float32)
    eye = np.eye(D, dtype=np.float32)
    y = oracle_mod.fwht_f32(eye, b)          # row j = transform of e_j
    assert np.array_equal(y, ref.T)
    # the exact fp64 rotation by definition gives the same matrix
    y64 = oracle_mod.rotate_f64(np.eye(D), b)
    assert np.allclose(y64, scipy.linalg.block_diag(*([Hb] * (D // b))).T, atol=0, rtol=1e-15)


@pytest.mark.parametrize("b", BLOCKS)
def test_matrix_is_symmetric_orthonormal(oracle_mod, b):
    M = oracle_mod.rotate_f64(np.eye(D), b)
    assert np.allclose(M, M.T, atol=1e-15)
    assert np.allclose(M @ M.T, np.eye(D), atol=1e-13)
    # the transform is its own inverse
    x = np.random.default_rng(1).standard_normal((4, D))
    assert np.allclose(oracle_mod.rotate_f64(oracle_mod.rotate_f64(x, b), b), x, atol=1e-13)


@pytest.mark.parametrize("b", BLOCKS)
def test_query_key_dot_product_invariant(oracle_mod, b):
    """(H q).(H k) = q.k : the equivalence the pages rely on for the query rotation."""
    rng = np.random.default_rng(2)
    q = rng.standard_normal((64, D))
    k = rng.standard_normal((64, D)) * np.where(rng.random(D) < 0.03, 25.0, 1.0)
    lhs = np.einsum("nd,nd->n", oracle_mod.rotate_f64(q, b), oracle_mod.rotate_f64(k, b))
    rhs = np.einsum("nd,nd->n", q, k)
    scale = np.einsum("nd,nd->n", np.abs(q), np.abs(k))
    assert np.all(np.abs(lhs - rhs) <= 1e-13 * scale)
    # the fp32 butterflies keep it to fp32 accuracy
    lhs32 = np.einsum("nd,nd->n", oracle_mod.fwht_f32(q.astype(np.float32), b).astype(np.float64),
                      oracle_mod.fwht_f32(k.astype(np.float32), b).astype(np.float64))
    rhs32 = np.einsum("nd,nd->n", q.astype(np.float32).astype(np.float64),
                      k.astype(np.float32).astype(np.float64))
    assert np.all(np.abs(lhs32 - rhs32) <= 1e-5 * scale)


@pytest.mark.parametrize("b", BLOCKS)
def test_spike_spreads_evenly(oracle_mod, b):
    """An outlier A e_j spreads to +-A/sqrt(b) over its block and nowhere else."""
    for j in (0, 5, b - 1, D - 1):
        A = 32.0
        x = np.zeros(D, np.float32)
        x[j] = A
        y = oracle_mod.fwht_f32(x, b)
        blk = j // b
        inside = np.zeros(D, bool)
        inside[blk * b:(blk + 1) * b] = True
        assert np.all(np.abs(y[inside]) == np.float32(A) * oracle_mod.rb(b))
        assert np.all(y[~inside] == 0)


@pytest.mark.parametrize("b", BLOCKS)
def test_constant_block_and_first_row(oracle_mod, b):
    """Sylvester order: row 0 is all ones, so y_0 = sum(x)/sqrt(b); a constant block maps to
    (c sqrt(b), 0, ..., 0)."""
    x = np.full(D, 3.0, np.float32)
    y = oracle_mod.rotate_f64(x.astype(np.float64), b)
    for blk in range(D // b):
        assert y[blk * b] == pytest.approx(3.0 * np.sqrt(b), rel=1e-15)
        assert np.allclose(y[blk * b + 1:(blk + 1) * b], 0, atol=1e-12)
    rng = np.random.default_rng(3)
    x = rng.standard_normal(D)
    y = oracle_mod.rotate_f64(x, b)
    for blk in range(D // b):
        assert y[blk * b] == pytest.approx(x[blk * b:(blk + 1) * b].sum() / np.sqrt(b), rel=1e-12)


@pytest.mark.parametrize("b", BLOCKS)
def test_fp32_butterflies_within_rounding_of_exact(oracle_mod, b):
    """fp32 FWHT vs exact fp64 product: error bounded by (log2 b + 1) roundings of the largest
    partial sum of the block."""
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((256, D)) * np.where(rng.random(D) < 0.03, 20.0, 1.0)).astype(np.float32)
    y32 = oracle_mod.fwht_f32(x, b).astype(np.float64)
    y64 = oracle_mod.rotate_f64(x.astype(np.float64), b)
    stages = int(np.log2(b)) + 1
    absx = np.abs(x.astype(np.float64)).reshape(256, D // b, b).sum(-1)   # per block
    bound = np.repeat(absx, b, axis=1) * stages * 2.0 ** -24 * 2
    assert np.all(np.abs(y32 - y64) <= bound)


def test_plain_mode_is_identity(oracle_mod):
    x = np.random.default_rng(5).standard_normal((3, D)).astype(np.float32)
    assert np.array_equal(oracle_mod.fwht_f32(x, 0), x)
    assert np.array_equal(oracle_mod.rotate_f64(x.astype(np.float64), 0), x.astype(np.float64))
