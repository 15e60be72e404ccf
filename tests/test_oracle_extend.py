"""The oracle's extend (chunked prefill) attention, pinned to an independent numpy brute
force with an explicit causal mask, to the decode at each chunk's last row, and to
causality (later tokens never change earlier rows)."""
import numpy as np
import pytest

import oracle
from oracle import brute
import workloads as W

D = 128


def _case(seed, lens, news, Hkv, Hq, P, kb, vb):
    rng = np.random.default_rng(seed)
    paging = W.assign_pages(rng, list(lens), P)
    T = int(sum(lens))
    k = W.make_rows(rng, T, Hkv, W.OutlierSpec.random(rng, Hkv))
    v = W.make_rows(rng, T, Hkv)
    slots = np.concatenate([paging.slots(s, 0, int(L)) for s, L in enumerate(lens)])
    cache = oracle.Cache(paging.num_pages, Hkv, P, fill=0)
    oracle.write(cache, k, v, slots, kb, vb)
    qo = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    q = W.f32_to_bf16_bits(rng.standard_normal((int(qo[-1]), Hq, D)).astype(np.float32))
    arrays = (cache.k_codes, cache.v_codes, cache.k_params, cache.v_params)
    return arrays, q, qo, paging.page_table(), np.array(lens, np.int32)


@pytest.mark.parametrize("kb,vb", [(0, 0), (128, 0), (64, 32), (16, 128)])
def test_extend_matches_brute_force(kb, vb):
    lens, news = [37, 16, 5, 64], [9, 16, 1, 3]          # prefix 0 (pure prefill) included
    arrays, q, qo, tab, L = _case(3, lens, news, 2, 4, 16, kb, vb)
    got = oracle.extend(q, arrays, qo, tab, L, 2, 16, kb, vb)
    ref = brute.extend(q, arrays, qo, tab, L, 2, 16, kb, vb)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_last_row_is_the_decode():
    lens, news = [50, 33, 17], [7, 33, 2]
    arrays, q, qo, tab, L = _case(4, lens, news, 1, 2, 16, 128, 128)
    got = oracle.extend(q, arrays, qo, tab, L, 1, 16, 128, 128)
    last = qo[1:] - 1
    dec = oracle.decode(q[last], arrays, tab, L, 1, 16, 128, 128)
    np.testing.assert_allclose(got[last], dec, rtol=0, atol=1e-13)


def test_causal_rows_ignore_later_tokens():
    lens, news = [40], [40]
    arrays, q, qo, tab, L = _case(5, lens, news, 1, 1, 16, 64, 0)
    a = oracle.extend(q, arrays, qo, tab, L, 1, 16, 64, 0)
    kc, vc, kp, vp = [x.copy() for x in arrays]
    # scramble the codes of positions 30..39: rows 0..29 must not change
    for t in range(30, 40):
        page, off = tab[0][t // 16], t % 16
        kc[page, 0, off] ^= 0x5A
        vc[page, 0, off] ^= 0xA5
    b = oracle.extend(q, (kc, vc, kp, vp), qo, tab, L, 1, 16, 64, 0)
    assert np.array_equal(a[:30], b[:30])
    assert not np.allclose(a[30:], b[30:])


def test_rejects_chunk_longer_than_sequence():
    arrays, q, qo, tab, L = _case(6, [10], [10], 1, 1, 16, 0, 0)
    with pytest.raises(ValueError):
        oracle.extend(q, arrays, qo, tab, np.array([9], np.int32), 1, 16, 0, 0)
