"""Pins of the oracle's paged placement.

The pages require uniform fixed-size pages and contiguous, coalesced
accesses (wispaper.ai blog, section 1 pain points: PagedAttention pages,
channel-wise jumps; fugumt.com abstract: paged memory layouts).  The layout
read from that (one (page, head) tile holds the page's tokens contiguously,
codes [page][Hkv][P][D/2] and fp16 (scale, zero) [page][Hkv][P][2]; slot =
page * P + offset; negative slot = skip) is pinned by hand-placed cases.
"""
import numpy as np

import workloads as W

D = 128


def _rows(seed, T, Hkv):
    return W.make_rows(np.random.default_rng(seed), T, Hkv)


def test_single_slot_lands_where_the_formula_says(oracle_mod):
    """P=2, Hkv=2, slot 5 -> page 2, offset 1: bytes at [2][h][1] and nowhere else."""
    k, v = _rows(1, 1, 2), _rows(2, 1, 2)
    cache = oracle_mod.Cache(4, 2, 2)
    oracle_mod.write(cache, k, v, np.array([5], np.int32), 0, 0)
    for h in range(2):
        ck, pk, _, _ = oracle_mod.quant_row(k[0, h], 0)
        cv, pv, _, _ = oracle_mod.quant_row(v[0, h], 0)
        assert np.array_equal(cache.k_codes[2, h, 1], ck)
        assert np.array_equal(cache.v_codes[2, h, 1], cv)
        assert np.array_equal(cache.k_params[2, h, 1], pk)
        assert np.array_equal(cache.v_params[2, h, 1], pv)
    mask = np.ones((4, 2, 2), bool)
    mask[2, :, 1] = False
    assert np.all(cache.k_codes[mask] == 0xAA) and np.all(cache.v_codes[mask] == 0xAA)
    assert np.all(cache.k_params[mask] == 0xAAAA) and np.all(cache.v_params[mask] == 0xAAAA)


def test_identity_pages_equal_contiguous_array(oracle_mod):
    """Identity page table: for each head, the pages concatenate to the token-ordered rows."""
    T, Hkv, P = 96, 3, 16
    k, v = _rows(3, T, Hkv), _rows(4, T, Hkv)
    cache = oracle_mod.Cache(T // P, Hkv, P)
    oracle_mod.write(cache, k, v, np.arange(T, dtype=np.int32), 32, 0)
    for h in range(Hkv):
        flat = cache.k_codes[:, h].reshape(T, D // 2)
        for t in range(0, T, 7):
            assert np.array_equal(flat[t], oracle_mod.quant_row(k[t, h], 32)[0])


def test_negative_slots_are_skipped(oracle_mod):
    T, Hkv, P = 32, 2, 16
    k, v = _rows(5, T, Hkv), _rows(6, T, Hkv)
    slots = np.arange(T, dtype=np.int32)
    slots[::3] = -1
    cache = oracle_mod.Cache(2, Hkv, P)
    oracle_mod.write(cache, k, v, slots, 128, 128)
    for t in range(T):
        page, off = divmod(t, P)
        if slots[t] < 0:
            assert np.all(cache.k_codes[page, :, off] == 0xAA)
            assert np.all(cache.v_params[page, :, off] == 0xAAAA)
        else:
            assert not np.all(cache.k_codes[page, :, off] == 0xAA)


def test_permuted_pages_move_bytes_only(oracle_mod):
    """The same tokens under a permuted page assignment give the same bytes, moved page-wise."""
    T, Hkv, P = 64, 2, 16
    k, v = _rows(7, T, Hkv), _rows(8, T, Hkv)
    perm = np.array([3, 0, 2, 1], np.int32)
    ident = oracle_mod.Cache(4, Hkv, P)
    moved = oracle_mod.Cache(4, Hkv, P)
    t = np.arange(T)
    oracle_mod.write(ident, k, v, t.astype(np.int32), 64, 0)
    oracle_mod.write(moved, k, v, (perm[t // P] * P + t % P).astype(np.int32), 64, 0)
    for lp in range(4):
        assert np.array_equal(moved.k_codes[perm[lp]], ident.k_codes[lp])
        assert np.array_equal(moved.v_params[perm[lp]], ident.v_params[lp])


def test_slot_outside_pool_is_an_error(oracle_mod):
    import pytest
    cache = oracle_mod.Cache(2, 1, 16)
    k = _rows(9, 1, 1)
    with pytest.raises(ValueError):
        oracle_mod.write(cache, k, k, np.array([32], np.int32), 0, 0)


def test_workload_page_tables_are_consistent():
    for name in ("tiny", "qwen3_4b_like", "prefill_chunk"):
        w = W.WORKLOADS[name]()
        tab = w.paging.page_table()
        used = np.concatenate(w.paging.seq_pages)
        assert len(np.unique(used)) == len(used)               # no page shared
        assert used.min() >= 0 and used.max() < w.paging.num_pages
        slots = w.all_slots()
        assert len(np.unique(slots)) == len(slots)             # slots unique per call
        s0 = w.paging.slots(0, 0, int(w.seq_lens[0]))
        assert np.array_equal(s0 // w.page_size, tab[0][np.arange(len(s0)) // w.page_size])
