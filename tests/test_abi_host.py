"""Host-side checks of the C-ABI library (no GPU needed, no kernel launched).

* the library loads and exports exactly the functions ``include/kvrq.h`` declares;
* every invalid argument returns the right status and a message, before any HIP call;
* the page pool: identity and seeded orders, all-or-nothing growth, release and reuse,
  page-table export with -1 padding, slot arithmetic.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def K():
    import int4_kv_cache_rotquant_amd as K
    if not os.path.exists(K.LIB_PATH):
        from int4_kv_cache_rotquant_amd import build
        build.build()
    K.lib()
    return K


def _declared():
    with open(os.path.join(ROOT, "include", "kvrq.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^KVRQ_API [^;(]*?\b(\w+)\s*\(", text, re.M)))


def test_exports_match_header(K):
    names = _declared()
    assert "kv_rotquant_write" in names and "kv_int4_paged_decode" in names
    L = K.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", K.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    c_exports = {e for e in exported if not e.startswith("_Z") and not e.startswith("__hip")}
    assert c_exports == set(names), c_exports ^ set(names)


def _desc(K, **kw):
    d = dict(head_dim=128, num_kv_heads=8, page_size=16, num_pages=64, k_block=128, v_block=0)
    d.update(kw)
    return K.CacheDesc(**d)


def _bufs(K, aligned=True):
    base = 0x10000 if aligned else 0x10004
    return K.CacheBuffers(base, base + 0x100000, base + 0x200000, base + 0x300000)


def _write(K, desc, bufs, k=0x40000000, v=0x50000000, T=4, ks=1024, vs=1024, slots=0x60000000):
    L = K.lib()
    return L.kv_rotquant_write(ctypes.byref(desc) if desc is not None else None,
                               ctypes.byref(bufs) if bufs is not None else None, k, v, T, ks, vs,
                               slots, None)


def test_write_validation(K):
    E = K
    cases = [
        (dict(desc=None), E.KVRQ_EINVAL, "descriptor"),
        (dict(desc=_desc(K, head_dim=64)), E.KVRQ_EUNSUPPORTED, "head_dim"),
        (dict(desc=_desc(K, num_kv_heads=0)), E.KVRQ_EINVAL, "num_kv_heads"),
        (dict(desc=_desc(K, page_size=24)), E.KVRQ_EUNSUPPORTED, "page_size"),
        (dict(desc=_desc(K, page_size=2048)), E.KVRQ_EUNSUPPORTED, "page_size"),
        (dict(desc=_desc(K, num_pages=0)), E.KVRQ_EINVAL, "num_pages"),
        (dict(desc=_desc(K, k_block=8)), E.KVRQ_EUNSUPPORTED, "blocks"),
        (dict(desc=_desc(K, v_block=256)), E.KVRQ_EUNSUPPORTED, "blocks"),
        (dict(bufs=None), E.KVRQ_EINVAL, "buffers"),
        (dict(bufs=K.CacheBuffers(0, 0x1000, 0x2000, 0x3000)), E.KVRQ_EINVAL, "NULL"),
        (dict(bufs=_bufs(K, aligned=False)), E.KVRQ_EINVAL, "aligned"),
        (dict(T=-1), E.KVRQ_EINVAL, "num_tokens"),
        (dict(T=1 << 31), E.KVRQ_EUNSUPPORTED, "num_tokens"),
        (dict(k=0), E.KVRQ_EINVAL, "non-NULL"),
        (dict(slots=0), E.KVRQ_EINVAL, "non-NULL"),
        (dict(ks=1000), E.KVRQ_EINVAL, "strides"),
        (dict(ks=1028), E.KVRQ_EINVAL, "multiples of 8"),
        (dict(k=0x40000008), E.KVRQ_EINVAL, "aligned"),
        (dict(slots=0x60000002), E.KVRQ_EINVAL, "aligned"),
    ]
    for kw, status, word in cases:
        desc = kw.pop("desc", _desc(K))
        bufs = kw.pop("bufs", _bufs(K))
        st = _write(K, desc, bufs, **kw)
        assert st == status, (kw, K.status_str(st), K.last_error())
        assert word in K.last_error(), (word, K.last_error())
    # an empty call is valid and launches nothing
    assert _write(K, _desc(K), _bufs(K), T=0) == K.KVRQ_OK


def test_decode_validation(K):
    L = K.lib()
    size = ctypes.c_size_t()

    def ws(desc, S=4, Hq=64, maxlen=1000, split=0):
        return L.kv_int4_paged_decode_workspace(ctypes.byref(desc), S, Hq, maxlen, split, ctypes.byref(size))

    assert ws(_desc(K), maxlen=5000) == K.KVRQ_OK and size.value > 0
    # one split covers 1000 tokens: no partials, no workspace
    assert ws(_desc(K)) == K.KVRQ_OK and size.value == 0
    assert ws(_desc(K), Hq=60) == K.KVRQ_EINVAL
    assert ws(_desc(K), Hq=8 * 17) == K.KVRQ_EUNSUPPORTED
    assert ws(_desc(K, page_size=8)) == K.KVRQ_EUNSUPPORTED
    assert ws(_desc(K), split=48) == K.KVRQ_EINVAL
    assert ws(_desc(K), split=96) == K.KVRQ_EINVAL
    assert ws(_desc(K), maxlen=-1) == K.KVRQ_EINVAL
    # workspace size grows with the number of splits
    ws(_desc(K), split=256)
    small = size.value
    ws(_desc(K), split=128)
    assert size.value > small
    # a 1M-token sequence (enough work for several rounds of split workgroups) takes the
    # balanced decode: 64 KiB of split counters, then partials of 128 + 2 floats per query
    # head of a KV head and slot, with 2048 + S * Hkv slots (a workgroup's share starts and
    # ends at most one partial per pair)
    counters = 16384 * 4
    assert ws(_desc(K), S=1, maxlen=1 << 20) == K.KVRQ_OK
    assert size.value == counters + (2048 + 1 * 8) * 8 * (128 + 2) * 4
    # a forced split size is kept as given
    assert ws(_desc(K), S=1, maxlen=1 << 20, split=4096) == K.KVRQ_OK
    assert size.value == counters + 1 * 64 * 256 * (128 + 2) * 4
    # the balanced grid on request, for any shape that fits it (at most 1024 sequences);
    # below 2^22 tokens of work the automatic plan keeps split workgroups
    assert ws(_desc(K), S=4, maxlen=1000, split=K.KVRQ_SPLIT_BALANCED) == K.KVRQ_OK
    assert size.value == counters + (2048 + 4 * 8) * 8 * (128 + 2) * 4
    assert ws(_desc(K), S=1025, maxlen=1000, split=K.KVRQ_SPLIT_BALANCED) == K.KVRQ_EUNSUPPORTED
    assert ws(_desc(K), S=1025, maxlen=1000) == K.KVRQ_OK
    assert ws(_desc(K), split=-2) == K.KVRQ_EINVAL
    # the extend has no balanced grid
    assert L.kv_int4_paged_extend_workspace(ctypes.byref(_desc(K)), 1, 64, 16, 16, 64,
                                            K.KVRQ_SPLIT_BALANCED, ctypes.byref(size)) == \
        K.KVRQ_EUNSUPPORTED

    def dec(desc=None, q=0x1000, S=2, Hq=64, tab=0x2000, maxp=400, lens=0x3000, maxlen=5000,
            scale=0.0, split=0, out=0x4000, wsp=0x5000, wsb=1 << 30):
        desc = desc or _desc(K)
        return L.kv_int4_paged_decode(ctypes.byref(desc), ctypes.byref(_bufs(K)), q, S, Hq, tab, maxp,
                                      lens, maxlen, scale, split, out, wsp, wsb, None)

    assert dec(S=0) == K.KVRQ_OK
    assert dec(q=0) == K.KVRQ_EINVAL
    assert dec(q=0x1004) == K.KVRQ_EINVAL
    assert dec(maxp=10) == K.KVRQ_EINVAL            # 10 pages of 16 < 5000 tokens
    assert dec(scale=float("nan")) == K.KVRQ_EINVAL
    assert dec(wsb=16) == K.KVRQ_EWORKSPACE
    assert "workspace" in K.last_error()
    assert dec(wsp=0) == K.KVRQ_EWORKSPACE


def test_decode_step_validation(K):
    L = K.lib()

    def step(k=0x10000, v=0x20000, ks=1024, vs=1024, slots=0x30000, S=2, q=0x1000, wsb=1 << 30,
             lens=0x3000, out=0x4000):
        return L.kv_int4_paged_decode_step(ctypes.byref(_desc(K)), ctypes.byref(_bufs(K)), k, v, ks, vs,
                                           slots, q, S, 64, 0x2000, 400, lens, 5000, 0.0, 0, out,
                                           0x5000, wsb, None)

    assert step(S=0) == K.KVRQ_OK
    assert step(k=0) == K.KVRQ_EINVAL and "non-NULL" in K.last_error()
    assert step(slots=0) == K.KVRQ_EINVAL
    assert step(ks=1000) == K.KVRQ_EINVAL and "strides" in K.last_error()
    assert step(vs=1028) == K.KVRQ_EINVAL
    assert step(v=0x20008) == K.KVRQ_EINVAL and "aligned" in K.last_error()
    assert step(slots=0x30002) == K.KVRQ_EINVAL
    assert step(q=0) == K.KVRQ_EINVAL
    assert step(wsb=16) == K.KVRQ_EWORKSPACE


def test_extend_validation(K):
    L = K.lib()
    size = ctypes.c_size_t()

    def ws(desc=None, S=4, Hq=64, total_q=40, max_q=16, maxlen=1000, split=0):
        desc = desc or _desc(K)
        return L.kv_int4_paged_extend_workspace(ctypes.byref(desc), S, Hq, total_q, max_q, maxlen,
                                                split, ctypes.byref(size))

    assert ws() == K.KVRQ_OK and size.value > 0
    # the decode's layout: 64 KiB of split counters (left alone), then the partials
    base = size.value - 16384 * 4
    assert ws(total_q=80) == K.KVRQ_OK and size.value == 16384 * 4 + 2 * base   # per query row and head
    assert ws(Hq=60) == K.KVRQ_EINVAL
    assert ws(total_q=-1) == K.KVRQ_EINVAL
    assert ws(max_q=0) == K.KVRQ_EINVAL                 # rows but no row per sequence
    assert ws(total_q=0, max_q=0) == K.KVRQ_OK
    assert ws(max_q=1001) == K.KVRQ_EINVAL              # a chunk longer than the sequence
    assert "max_q_len" in K.last_error()
    assert ws(split=48) == K.KVRQ_EINVAL

    def ext(q=0x1000, total_q=40, S=4, Hq=64, qo=0x6000, tab=0x2000, maxp=100, lens=0x3000,
            maxlen=1000, max_q=16, scale=0.0, split=0, out=0x4000, wsp=0x5000, wsb=1 << 30):
        return L.kv_int4_paged_extend(ctypes.byref(_desc(K)), ctypes.byref(_bufs(K)), q, total_q, S,
                                      Hq, qo, tab, maxp, lens, maxlen, max_q, scale, split, out, wsp,
                                      wsb, None)

    assert ext(S=0) == K.KVRQ_OK and ext(total_q=0) == K.KVRQ_OK   # nothing to launch
    assert ext(qo=0) == K.KVRQ_EINVAL
    assert ext(qo=0x6002) == K.KVRQ_EINVAL
    assert ext(out=0x4004) == K.KVRQ_EINVAL
    assert ext(maxp=10) == K.KVRQ_EINVAL
    assert ext(scale=float("inf")) == K.KVRQ_EINVAL
    assert ext(wsb=16) == K.KVRQ_EWORKSPACE


def test_helper_validation(K):
    L = K.lib()
    assert L.kvrq_device_copy(0x1000, 0x2000, 0, None) == K.KVRQ_OK
    assert L.kvrq_device_copy(0x1000, 0x2000, 24, None) == K.KVRQ_EINVAL
    assert L.kvrq_device_copy(0, 0x2000, 32, None) == K.KVRQ_EINVAL
    assert L.kvrq_device_read(0x1000, 0, 0x2000, None) == K.KVRQ_OK
    assert L.kvrq_device_read(0x1000, 24, 0x2000, None) == K.KVRQ_EINVAL
    assert L.kvrq_device_read(0x1008, 32, 0x2000, None) == K.KVRQ_EINVAL
    assert L.kvrq_device_read(0x1000, 32, 0x2002, None) == K.KVRQ_EINVAL
    assert L.kvrq_device_read(0, 32, 0x2000, None) == K.KVRQ_EINVAL
    assert L.kvrq_device_read(0x1000, 32, 0, None) == K.KVRQ_EINVAL
    d = _desc(K)
    assert L.kvrq_bf16_paged_write(ctypes.byref(d), 0, 0x1000, 0x2000, 0x3000, 4, 1024, 1024,
                                   0x4000, None) == K.KVRQ_EINVAL


def test_paged_read_validation(K):
    """kvrq_paged_read checks its arguments on the host before any launch."""
    L = K.lib()
    d, b = _desc(K), _bufs(K)

    def call(desc=d, bufs=b, pages=0x7000, n=4, wgs=2, sink=0x8000, pattern=0):
        return L.kvrq_paged_read(ctypes.byref(desc), ctypes.byref(bufs), pages, n, pattern, wgs, sink,
                                 None)

    assert call(n=0) == K.KVRQ_OK                       # nothing to read: no launch
    assert call(n=-1) == K.KVRQ_EINVAL
    assert call(wgs=0) == K.KVRQ_EINVAL
    assert call(wgs=5) == K.KVRQ_EINVAL
    assert call(pages=0) == K.KVRQ_EINVAL
    assert call(sink=0) == K.KVRQ_EINVAL
    assert call(sink=0x8002) == K.KVRQ_EINVAL
    assert call(desc=_desc(K, page_size=8)) == K.KVRQ_EUNSUPPORTED      # 8 heads x 8 tokens
    assert call(desc=_desc(K, page_size=8), pattern=1) == K.KVRQ_EUNSUPPORTED   # 16-token blocks
    assert call(pattern=4) == K.KVRQ_EINVAL
    assert call(pattern=-1) == K.KVRQ_EINVAL
    assert call(desc=_desc(K, k_bits=2)) == K.KVRQ_EUNSUPPORTED
    assert call(bufs=K.CacheBuffers(0, 0x1000, 0x2000, 0x3000)) == K.KVRQ_EINVAL
    assert call(desc=_desc(K, head_dim=64)) == K.KVRQ_EUNSUPPORTED


def test_status_strings(K):
    for st, name in [(0, "KVRQ_OK"), (1, "KVRQ_EINVAL"), (2, "KVRQ_EUNSUPPORTED"), (3, "KVRQ_ENOPAGES"),
                     (4, "KVRQ_EHIP"), (5, "KVRQ_EWORKSPACE"), (99, "KVRQ_UNKNOWN")]:
        assert K.status_str(st) == name


def test_cache_sizes(K):
    kb, vb, pb = K.kvrq_cache_sizes(_desc(K))
    assert kb == vb == 64 * 8 * 16 * 64 and pb == 64 * 8 * 16 * 4
    # the footprint the pages call "a quarter of the space": 68 B vs 256 B per token-head
    assert (kb + pb) / (64 * 8 * 16) == 68
    # 2-bit pools: 32-byte rows (mixed widths allowed)
    kb, vb, pb = K.kvrq_cache_sizes(_desc(K, k_bits=4, v_bits=2))
    assert kb == 64 * 8 * 16 * 64 and vb == 64 * 8 * 16 * 32
    with pytest.raises(K.KvrqError) as e:
        K.kvrq_cache_sizes(_desc(K, k_bits=3))
    assert e.value.status == K.KVRQ_EUNSUPPORTED
    # (page, head, token) cells are 32-bit indexes in the kernels: 2^32 cells at most
    kb, vb, pb = K.kvrq_cache_sizes(_desc(K, num_kv_heads=64, page_size=1024, num_pages=1 << 16))
    assert kb == (1 << 32) * 64
    with pytest.raises(K.KvrqError) as e:
        K.kvrq_cache_sizes(_desc(K, num_kv_heads=65, page_size=1024, num_pages=1 << 16))
    assert e.value.status == K.KVRQ_EINVAL and "2^32" in str(e.value)


def test_pool_identity_order_and_slots(K):
    p = K.Pool(num_pages=8, page_size=16, max_seqs=3, max_pages_per_seq=4)
    p.seq_extend(0, 20)
    p.seq_extend(1, 16)
    tab, lens = p.page_table()
    assert list(tab[0]) == [0, 1, -1, -1] and list(tab[1]) == [2, -1, -1, -1]
    assert list(tab[2]) == [-1] * 4 and list(lens) == [20, 16, 0]
    assert list(p.slots(0, 14, 4)) == [14, 15, 16, 17]
    assert list(p.slots(1, 0, 2)) == [32, 33]
    assert p.free_pages() == 5


def test_pool_seeded_permutation_deterministic(K):
    a = K.Pool(64, 16, 1, 64, shuffle_seed=1234)
    b = K.Pool(64, 16, 1, 64, shuffle_seed=1234)
    c = K.Pool(64, 16, 1, 64, shuffle_seed=99)
    for p in (a, b, c):
        p.seq_extend(0, 64 * 16)
    ta, tb, tc = a.page_table()[0][0], b.page_table()[0][0], c.page_table()[0][0]
    assert np.array_equal(ta, tb) and not np.array_equal(ta, tc)
    assert sorted(ta) == list(range(64)) and not np.array_equal(ta, np.arange(64))


def test_pool_all_or_nothing_and_reuse(K):
    p = K.Pool(num_pages=4, page_size=16, max_seqs=2, max_pages_per_seq=3)
    p.seq_extend(0, 40)                       # 3 pages
    before = p.page_table()
    with pytest.raises(K.KvrqError) as e:
        p.seq_extend(1, 33)                   # needs 3, only 1 free
    assert e.value.status == K.KVRQ_ENOPAGES
    after = p.page_table()
    assert np.array_equal(before[0], after[0]) and p.free_pages() == 1 and p.seq_len(1) == 0
    with pytest.raises(K.KvrqError) as e:
        p.seq_extend(0, 49)                   # beyond max_pages_per_seq
    assert e.value.status == K.KVRQ_ENOPAGES
    with pytest.raises(K.KvrqError) as e:
        p.seq_extend(0, 10)                   # shrinking is not allowed
    assert e.value.status == K.KVRQ_EINVAL
    p.seq_release(0)
    assert p.free_pages() == 4 and p.seq_len(0) == 0
    p.seq_extend(1, 33)
    assert sorted(p.page_table()[0][1][:3]) == sorted(set(p.page_table()[0][1][:3]))
    with pytest.raises(K.KvrqError):
        p.slots(1, 30, 4)                     # beyond the length
    with pytest.raises(K.KvrqError):
        p.seq_extend(5, 1)


def test_pool_invalid_create(K):
    with pytest.raises(K.KvrqError) as e:
        K.Pool(0, 16, 1, 1)
    assert e.value.status == K.KVRQ_EINVAL
    with pytest.raises(K.KvrqError) as e:
        K.Pool(4, 12, 1, 1)
    assert e.value.status == K.KVRQ_EUNSUPPORTED
