"""The C ABI under HIP graph capture (torch.cuda.CUDAGraph on torch's current stream): a
serving loop replays a recorded decode step instead of paying the host's launch overhead
per call.  The entry points enqueue kernels only (no memset, copy or allocation on the
stream), so a step records as plain kernel nodes.

Each case records one step once (after an eager warm-up of the same calls) and replays it
three times, with eager calls of the library and device synchronisations between the
replays.  Every replay must reproduce the eager step bit for bit: the outputs (filled with
NaN before each replay, so a row left unwritten fails) and the cache bytes.  The eager
step itself matches the oracle (its write, then its fp64 decode) within 2e-3.

Cases: a new token's write followed by the decode, the fused decode step, and the decode
that allocates nothing; each on the split grid (automatic and 128-token splits, the
in-kernel combine) and on the balanced grid with its combine launch.  And a chunk's write
followed by its causal extend, in one split and in forced 128-token splits.
"""
import numpy as np
import pytest

import oracle
from gpu_harness import bf16_dev, decode_compare, gpu_cache_arrays, to_dev
from test_gpu_decode_step import _setup, _step_slots

pytestmark = pytest.mark.gpu
BAL = -1
LENS = [1, 127, 300, 513, 0, 2000, 64, 4100]
HKV, HQ, P, KB, VB = 2, 8, 16, 128, 0


@pytest.fixture(scope="module")
def K():
    import int4_kv_cache_rotquant_amd as K
    K.lib()
    assert K.KVRQ_SPLIT_BALANCED == BAL
    return K


def _inputs(paging, new):
    kn, vn, q = new
    L = np.array(LENS, np.int32)
    slots = _step_slots(paging, LENS, 0)
    dev = dict(kn=bf16_dev(kn), vn=bf16_dev(vn), slots=to_dev(slots), q=bf16_dev(q),
               tab=to_dev(paging.page_table()), L=to_dev(L))
    return dev, int(max(L.max(), 1)), slots, L


def _workspace(K, cache, maxlen, split):
    import torch
    n = K.kv_int4_paged_decode_workspace(cache, len(LENS), HQ, maxlen, split)
    return torch.zeros(max(n, 16), dtype=torch.uint8, device="cuda")


def _record(body):
    """An eager warm-up of ``body`` on a side stream, then ``body`` recorded into a graph."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        body()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    torch.cuda.synchronize()
    return g


def _replay_and_compare(g, out_g, out_e, graph_cache, eager_cache, eager_work, label):
    import torch
    for r in range(3):
        out_g.fill_(float("nan"))
        eager_work()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), (label, r, float((out_g - out_e).abs().nan_to_num(9.0).max()))
        for a, b, name in zip(gpu_cache_arrays(graph_cache), gpu_cache_arrays(eager_cache),
                              ("kc", "vc", "kp", "vp")):
            assert np.array_equal(a, b), (label, r, name, int((a != b).sum()))


def _oracle_check(orc, paging, new, slots, L, out_e, label):
    kn, vn, q = new
    keep = slots >= 0
    oracle.write(orc, kn[keep], vn[keep], slots[keep], KB, VB)
    arrays = (orc.k_codes, orc.v_codes, orc.k_params, orc.v_params)
    decode_compare(out_e.cpu().numpy(), oracle.decode(q, arrays, paging.page_table(), L, HKV, P, KB, VB),
                   label)


@pytest.mark.parametrize("split", [0, 128, BAL])
def test_write_then_decode(K, split):
    import torch
    (gc, ec), orc, paging, news = _setup(K, LENS, HKV, HQ, P, KB, VB, seed=4100 + split)
    d, maxlen, slots, L = _inputs(paging, news[0])
    ws_g, ws_e = _workspace(K, gc, maxlen, split), _workspace(K, ec, maxlen, split)
    K.kv_rotquant_write(ec, d["kn"], d["vn"], d["slots"])
    out_e = K.kv_int4_paged_decode(ec, d["q"], d["tab"], d["L"], maxlen, split_tokens=split, workspace=ws_e)
    torch.cuda.synchronize()
    out_g = torch.empty_like(out_e)
    other = torch.empty_like(out_e)
    q2 = torch.flip(d["q"], dims=[1]).contiguous()

    def body():
        K.kv_rotquant_write(gc, d["kn"], d["vn"], d["slots"])
        K.kv_int4_paged_decode(gc, d["q"], d["tab"], d["L"], maxlen, out=out_g, split_tokens=split,
                               workspace=ws_g)

    g = _record(body)
    _replay_and_compare(g, out_g, out_e, gc, ec,
                        lambda: K.kv_int4_paged_decode(ec, q2, d["tab"], d["L"], maxlen, out=other,
                                                       split_tokens=split, workspace=ws_e),
                        f"write+decode split={split}")
    _oracle_check(orc, paging, news[0], slots, L, out_e, f"graph write+decode split={split}")


@pytest.mark.parametrize("split", [0, 128, BAL])
def test_fused_step(K, split):
    import torch
    (gc, ec), orc, paging, news = _setup(K, LENS, HKV, HQ, P, KB, VB, seed=4200 + split)
    d, maxlen, slots, L = _inputs(paging, news[0])
    ws_g, ws_e = _workspace(K, gc, maxlen, split), _workspace(K, ec, maxlen, split)
    out_e = K.kv_int4_paged_decode_step(ec, d["kn"], d["vn"], d["slots"], d["q"], d["tab"], d["L"], maxlen,
                                        split_tokens=split, workspace=ws_e)
    torch.cuda.synchronize()
    out_g = torch.empty_like(out_e)
    other = torch.empty_like(out_e)

    def body():
        K.kv_int4_paged_decode_step(gc, d["kn"], d["vn"], d["slots"], d["q"], d["tab"], d["L"], maxlen,
                                    out=out_g, split_tokens=split, workspace=ws_g)

    g = _record(body)
    # the eager work between replays rewrites the same rows into the eager cache
    _replay_and_compare(g, out_g, out_e, gc, ec,
                        lambda: K.kv_int4_paged_decode_step(ec, d["kn"], d["vn"], d["slots"], d["q"],
                                                            d["tab"], d["L"], maxlen, out=other,
                                                            split_tokens=split, workspace=ws_e),
                        f"fused step split={split}")
    _oracle_check(orc, paging, news[0], slots, L, out_e, f"graph fused step split={split}")


@pytest.mark.parametrize("split", [0, BAL])
def test_noalloc_decode(K, split):
    import torch
    (gc, ec), orc, paging, news = _setup(K, LENS, HKV, HQ, P, KB, VB, seed=4300 + split)
    d, maxlen, slots, L = _inputs(paging, news[0])
    for c in (gc, ec):
        K.kv_rotquant_write(c, d["kn"], d["vn"], d["slots"])
    out_e = torch.empty((len(LENS), HQ, 128), dtype=torch.float32, device="cuda")
    K.kv_int4_paged_decode_noalloc(ec, d["q"], d["tab"], d["L"], maxlen, out_e, split_tokens=split)
    torch.cuda.synchronize()
    ws = _workspace(K, ec, maxlen, split)
    ref = K.kv_int4_paged_decode(ec, d["q"], d["tab"], d["L"], maxlen, split_tokens=split, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out_e, ref), "noalloc and workspace decodes differ"
    out_g = torch.empty_like(out_e)
    other = torch.empty_like(out_e)
    q2 = torch.flip(d["q"], dims=[1]).contiguous()

    def body():
        K.kv_int4_paged_decode_noalloc(gc, d["q"], d["tab"], d["L"], maxlen, out_g, split_tokens=split)

    g = _record(body)
    # eager calls of the same entry point between replays share the static scratch, one at a time
    _replay_and_compare(g, out_g, out_e, gc, ec,
                        lambda: K.kv_int4_paged_decode_noalloc(ec, q2, d["tab"], d["L"], maxlen, other,
                                                               split_tokens=split),
                        f"noalloc split={split}")
    _oracle_check(orc, paging, news[0], slots, L, out_e, f"graph noalloc split={split}")


@pytest.mark.parametrize("split", [0, 128])
def test_chunk_write_then_extend(K, split):
    """A chunk of new tokens per sequence written, then its causal extend over prefix + chunk."""
    import torch
    import workloads as W
    lens, news = [300, 129, 64, 1000], [100, 129, 33, 7]
    rng = np.random.default_rng(4400 + split)
    paging = W.assign_pages(np.random.default_rng(4401 + split), lens, P)
    T = int(sum(lens))
    k = W.make_rows(rng, T, HKV, W.OutlierSpec.random(rng, HKV))
    v = W.make_rows(rng, T, HKV)
    slots = np.concatenate([paging.slots(s, 0, int(L)) for s, L in enumerate(lens)]).astype(np.int32)
    chunk = np.concatenate([np.arange(int(L) - n, int(L)) + off for L, n, off in
                            zip(lens, news, np.concatenate([[0], np.cumsum(lens)[:-1]]))])
    prefix = np.setdiff1d(np.arange(T), chunk)
    caches = [K.PagedInt4Cache(paging.num_pages, HKV, P, KB, VB, fill=0) for _ in range(2)]
    for c in caches:
        K.kv_rotquant_write(c, bf16_dev(k[prefix]), bf16_dev(v[prefix]), to_dev(slots[prefix]))
    gc, ec = caches
    qo = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    q = W.f32_to_bf16_bits(rng.standard_normal((int(qo[-1]), HQ, 128)).astype(np.float32))
    L = np.array(lens, np.int32)
    d = dict(kc=bf16_dev(k[chunk]), vc=bf16_dev(v[chunk]), sc=to_dev(slots[chunk]), q=bf16_dev(q),
             qo=to_dev(qo), tab=to_dev(paging.page_table()), L=to_dev(L))
    maxlen, maxq = int(L.max()), int(max(news))

    def ws():
        n = K.kv_int4_paged_extend_workspace(gc, len(lens), HQ, int(qo[-1]), maxq, maxlen, split)
        return torch.zeros(max(n, 16), dtype=torch.uint8, device="cuda")

    ws_g, ws_e = ws(), ws()
    K.kv_rotquant_write(ec, d["kc"], d["vc"], d["sc"])
    out_e = K.kv_int4_paged_extend(ec, d["q"], d["qo"], d["tab"], d["L"], maxlen, maxq,
                                   split_tokens=split, workspace=ws_e)
    torch.cuda.synchronize()
    out_g = torch.empty_like(out_e)
    other = torch.empty_like(out_e)
    q2 = torch.flip(d["q"], dims=[1]).contiguous()

    def body():
        K.kv_rotquant_write(gc, d["kc"], d["vc"], d["sc"])
        K.kv_int4_paged_extend(gc, d["q"], d["qo"], d["tab"], d["L"], maxlen, maxq, out=out_g,
                               split_tokens=split, workspace=ws_g)

    g = _record(body)
    _replay_and_compare(g, out_g, out_e, gc, ec,
                        lambda: K.kv_int4_paged_extend(ec, q2, d["qo"], d["tab"], d["L"], maxlen, maxq,
                                                       out=other, split_tokens=split, workspace=ws_e),
                        f"chunk write+extend split={split}")
    orc = oracle.Cache(paging.num_pages, HKV, P, fill=0)
    oracle.write(orc, k, v, slots, KB, VB)
    arrays = (orc.k_codes, orc.v_codes, orc.k_params, orc.v_params)
    decode_compare(out_e.cpu().numpy(), oracle.extend(q, arrays, qo, paging.page_table(), L, HKV, P, KB, VB),
                   f"graph chunk write+extend split={split}")
