"""GPU checks of kv_int4_paged_decode_step (the write of one new token per sequence fused
into the decode that reads it), through the C ABI.

* the cache after the fused step is bit-identical to kv_rotquant_write of the same rows,
  and the output equals kv_int4_paged_decode after that write;
* the output matches the oracle (its write, then its decode) within 2e-3;
* covered: the new token in every split position (forced 128-token splits), sequences of
  one token (only the new one), an empty sequence and a negative slot (nothing written),
  query groups 4 (two MFMA halves per head) and 16, K/V block pairs that take every V
  rotation branch, and two steps in a row.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_harness import D, bf16_dev, decode_compare, gpu_cache_arrays, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import int4_kv_cache_rotquant_amd as K
    K.lib()
    return K


def _setup(K, lens, Hkv, Hq, P, kb, vb, seed, steps=1):
    """Prefix of lens[s] - 1 tokens written; returns both GPU caches (identical), the
    oracle cache, the paging and per-step new rows."""
    rng = np.random.default_rng(seed)
    paging = W.assign_pages(np.random.default_rng(seed + 1), [max(int(L) + steps - 1, 1) for L in lens], P)
    pre = [max(int(L) - 1, 0) for L in lens]
    T = int(sum(pre))
    k = W.make_rows(rng, T, Hkv, W.OutlierSpec.random(rng, Hkv))
    v = W.make_rows(rng, T, Hkv)
    slots = np.concatenate([paging.slots(s, 0, n) for s, n in enumerate(pre)]).astype(np.int32)
    caches = []
    for _ in range(2):
        c = K.PagedInt4Cache(paging.num_pages, Hkv, P, kb, vb, fill=0)
        if T:
            K.kv_rotquant_write(c, bf16_dev(k), bf16_dev(v), to_dev(slots))
        caches.append(c)
    orc = oracle.Cache(paging.num_pages, Hkv, P, fill=0)
    if T:
        oracle.write(orc, k, v, slots, kb, vb)
    S = len(lens)
    news = [(W.make_rows(rng, S, Hkv, W.OutlierSpec.random(rng, Hkv)), W.make_rows(rng, S, Hkv),
             W.f32_to_bf16_bits(rng.standard_normal((S, Hq, D)).astype(np.float32)))
            for _ in range(steps)]
    return caches, orc, paging, news


def _step_slots(paging, lens, i):
    return np.array([paging.slots(s, int(L) - 1 + i, 1)[0] if L > 0 else -1
                     for s, L in enumerate(lens)], np.int32)


def _check_step(K, caches, orc, paging, lens, new, Hkv, P, kb, vb, split, label, i=0,
                slot_override=None, workspaces=(None, None)):
    import torch
    kn, vn, q = new
    L = np.array([int(x) + i if x > 0 else 0 for x in lens], np.int32)
    slots = _step_slots(paging, lens, i) if slot_override is None else slot_override
    tab = paging.page_table()
    maxlen = int(max(L.max(), 1))
    fused, ref = caches
    out_f = K.kv_int4_paged_decode_step(fused, bf16_dev(kn), bf16_dev(vn), to_dev(slots), bf16_dev(q),
                                        to_dev(tab), to_dev(L), maxlen, split_tokens=split,
                                        workspace=workspaces[0])
    K.kv_rotquant_write(ref, bf16_dev(kn), bf16_dev(vn), to_dev(slots))
    out_r = K.kv_int4_paged_decode(ref, bf16_dev(q), to_dev(tab), to_dev(L), maxlen, split_tokens=split,
                                   workspace=workspaces[1])
    torch.cuda.synchronize()
    for a, b, name in zip(gpu_cache_arrays(fused), gpu_cache_arrays(ref), ("kc", "vc", "kp", "vp")):
        assert np.array_equal(a, b), (label, name, int((a != b).sum()))
    out_f, out_r = out_f.cpu().numpy(), out_r.cpu().numpy()
    assert np.array_equal(out_f, out_r), (label, float(np.abs(out_f - out_r).max()))
    keep = slots >= 0
    oracle.write(orc, kn[keep], vn[keep], slots[keep], kb, vb)
    arrays = (orc.k_codes, orc.v_codes, orc.k_params, orc.v_params)
    decode_compare(out_f, oracle.decode(q, arrays, tab, L, Hkv, P, kb, vb), label)


@pytest.mark.parametrize("Hq,kb,vb", [(32, 128, 0), (32, 0, 16), (128, 64, 128), (32, 32, 32),
                                      (128, 16, 64)])
def test_matches_write_then_decode(K, Hq, kb, vb):
    Hkv, P = 8, 16
    lens = [1, 127, 128, 129, 300, 513, 0, 64]
    caches, orc, paging, news = _setup(K, lens, Hkv, Hq, P, kb, vb, seed=100 + Hq + kb + vb)
    _check_step(K, caches, orc, paging, lens, news[0], Hkv, P, kb, vb, 128, f"step G{Hq // Hkv} {kb}/{vb}")


def test_automatic_splits_and_two_steps(K):
    Hkv, Hq, P, kb, vb = 2, 16, 32, 128, 128
    lens = [5, 1000, 4097, 2048]
    caches, orc, paging, news = _setup(K, lens, Hkv, Hq, P, kb, vb, seed=7, steps=2)
    for i in range(2):
        _check_step(K, caches, orc, paging, lens, news[i], Hkv, P, kb, vb, 0, f"step {i}", i=i)


def test_negative_slot_writes_nothing(K):
    Hkv, Hq, P, kb, vb = 2, 8, 16, 128, 0
    lens = [40, 77]
    caches, orc, paging, news = _setup(K, lens, Hkv, Hq, P, kb, vb, seed=9)
    slots = _step_slots(paging, lens, 0)
    slots[1] = -1
    before = gpu_cache_arrays(caches[0])
    _check_step(K, caches, orc, paging, lens, news[0], Hkv, P, kb, vb, 0, "negative slot",
                slot_override=slots)
    after = gpu_cache_arrays(caches[0])
    page, off = divmod(int(_step_slots(paging, lens, 0)[1]), P)
    assert np.array_equal(before[0][page, :, off], after[0][page, :, off])
    assert np.array_equal(before[2][page, :, off], after[2][page, :, off])


def test_steps_in_a_row_on_one_workspace(K):
    """The serving loop: four fused steps in a row, each on the same zero-filled workspace
    (and the reference decode on another), rows of 0 to 9 splits of 128 tokens merged
    inside the split launch; every step matches the separate write and decode bit for bit
    and the oracle within 2e-3, and leaves the split counters at zero."""
    import torch
    Hkv, Hq, P, kb, vb = 2, 8, 16, 64, 128
    lens = [0, 1, 127, 128, 300, 1021]
    steps = 4
    caches, orc, paging, news = _setup(K, lens, Hkv, Hq, P, kb, vb, seed=11, steps=steps)
    n = K.kv_int4_paged_decode_workspace(caches[0], len(lens), Hq, max(lens) + steps, 128)
    ws = (torch.zeros(n, dtype=torch.uint8, device="cuda"),
          torch.zeros(n, dtype=torch.uint8, device="cuda"))
    for i in range(steps):
        _check_step(K, caches, orc, paging, lens, news[i], Hkv, P, kb, vb, 128, f"shared step {i}",
                    i=i, workspaces=ws)
        for w in ws:
            assert int(w[:16384 * 4].count_nonzero()) == 0, f"counters left set after step {i}"
