"""ctypes binding of ``libkvrq.so`` (declared in ``include/kvrq.h``).

Argument marshalling only: every step of the hot path runs in the library's
HIP kernels.  PyTorch provides device memory and the current HIP stream.
The functions keep the C names; tensors stand in for the raw pointers.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libkvrq.so")

KVRQ_OK, KVRQ_EINVAL, KVRQ_EUNSUPPORTED, KVRQ_ENOPAGES, KVRQ_EHIP, KVRQ_EWORKSPACE = range(6)
KVRQ_SPLIT_BALANCED = -1      # split_tokens of the decode calls: the balanced grid
HEAD_DIM = 128


class KvrqError(RuntimeError):
    def __init__(self, status: int, name: str, message: str):
        super().__init__(f"{name}: {message}")
        self.status = status


class CacheDesc(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("k_block", ctypes.c_int32), ("v_block", ctypes.c_int32),
                ("k_bits", ctypes.c_int32), ("v_bits", ctypes.c_int32)]


class CacheBuffers(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("k_params", ctypes.c_void_p), ("v_params", ctypes.c_void_p)]


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load the HIP library; fails loudly if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m int4_kv_cache_rotquant_amd.build` (there is no fallback)")
    # torch carries its own HIP runtime under the soname the library links against; load
    # torch first so that the library binds to that one copy (a second copy loaded before
    # torch would not see the device memory torch allocates)
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    st = ctypes.c_int32
    sig = {
        "kvrq_status_str": (ctypes.c_char_p, [st]),
        "kvrq_last_error": (ctypes.c_char_p, []),
        "kvrq_cache_sizes": (st, [P, P, P, P]),
        "kvrq_pool_create": (st, [i32, i32, i32, i32, ctypes.c_uint64, P]),
        "kvrq_pool_destroy": (None, [P]),
        "kvrq_seq_extend": (st, [P, i32, i32]),
        "kvrq_seq_release": (st, [P, i32]),
        "kvrq_seq_len": (i32, [P, i32]),
        "kvrq_slots": (st, [P, i32, i32, i32, P]),
        "kvrq_page_table": (st, [P, P, P]),
        "kvrq_pool_free_pages": (i32, [P]),
        "kv_rotquant_write": (st, [P, P, P, P, i64, i64, i64, P, P]),
        "kv_int4_paged_decode_workspace": (st, [P, i32, i32, i32, i32, P]),
        "kv_int4_paged_decode": (st, [P, P, P, i32, i32, P, i32, P, i32, ctypes.c_float, i32, P, P,
                                      sz, P]),
        "kv_int4_paged_decode_noalloc": (st, [P, P, P, i32, i32, P, i32, P, i32, ctypes.c_float,
                                              i32, P, P]),
        "kv_int4_paged_decode_step": (st, [P, P, P, P, i64, i64, P, P, i32, i32, P, i32, P, i32,
                                           ctypes.c_float, i32, P, P, sz, P]),
        "kv_int4_paged_extend_workspace": (st, [P, i32, i32, i32, i32, i32, i32, P]),
        "kv_int4_paged_extend": (st, [P, P, P, i32, i32, i32, P, P, i32, P, i32, i32, ctypes.c_float,
                                      i32, P, P, sz, P]),
        "kvrq_bf16_paged_write": (st, [P, P, P, P, P, i64, i64, i64, P, P]),
        "kvrq_device_copy": (st, [P, P, sz, P]),
        "kvrq_device_read": (st, [P, sz, P, P]),
        "kvrq_paged_read": (st, [P, P, P, i64, i32, i32, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(status: int) -> None:
    if status != KVRQ_OK:
        L = lib()
        raise KvrqError(status, L.kvrq_status_str(status).decode(), L.kvrq_last_error().decode())


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def status_str(status: int) -> str:
    return lib().kvrq_status_str(status).decode()


def last_error() -> str:
    return lib().kvrq_last_error().decode()


# --------------------------------------------------------------------- cache
def kvrq_cache_sizes(desc: CacheDesc) -> Tuple[int, int, int]:
    """(K codes bytes, V codes bytes, params bytes of one pool)."""
    kb, vb, pb = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().kvrq_cache_sizes(ctypes.byref(desc), ctypes.byref(kb), ctypes.byref(vb),
                                  ctypes.byref(pb)))
    return kb.value, vb.value, pb.value


class PagedInt4Cache:
    """One layer's INT4 (or 2-bit: ``k_bits``/``v_bits`` = 2) cache: descriptor + four torch
    device tensors."""

    def __init__(self, num_pages: int, num_kv_heads: int, page_size: int, k_block: int,
                 v_block: int, device="cuda", fill: Optional[int] = None, k_bits: int = 4,
                 v_bits: int = 4):
        import torch
        self.desc = CacheDesc(HEAD_DIM, num_kv_heads, page_size, num_pages, k_block, v_block,
                              k_bits, v_bits)
        k_bytes, v_bytes, params_bytes = kvrq_cache_sizes(self.desc)
        shape_p = (num_pages, num_kv_heads, page_size, 2)
        self.k_codes = torch.empty((num_pages, num_kv_heads, page_size, HEAD_DIM * k_bits // 8),
                                   dtype=torch.uint8, device=device)
        self.v_codes = torch.empty((num_pages, num_kv_heads, page_size, HEAD_DIM * v_bits // 8),
                                   dtype=torch.uint8, device=device)
        self.k_params = torch.empty(shape_p, dtype=torch.int16, device=device)
        self.v_params = torch.empty(shape_p, dtype=torch.int16, device=device)
        if fill is not None:
            for t in (self.k_codes, self.v_codes, self.k_params, self.v_params):
                t.view(torch.uint8).fill_(fill)
        assert self.k_codes.numel() == k_bytes and self.v_codes.numel() == v_bytes
        assert self.k_params.numel() * 2 == params_bytes
        self.buffers = CacheBuffers(self.k_codes.data_ptr(), self.v_codes.data_ptr(),
                                    self.k_params.data_ptr(), self.v_params.data_ptr())

    @property
    def num_kv_heads(self) -> int:
        return self.desc.num_kv_heads

    @property
    def page_size(self) -> int:
        return self.desc.page_size


# --------------------------------------------------------------------- hot path
def kv_rotquant_write(cache: PagedInt4Cache, k, v, slot_mapping, stream=None) -> None:
    """Fused BDR + token-wise INT4 write of bf16 ``k, v`` [T][Hkv][128] at int32 ``slot_mapping``."""
    import torch
    T = int(slot_mapping.shape[0])
    for name, t in (("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != HEAD_DIM:
            raise ValueError(f"{name} must be bf16 [T][Hkv][128] with contiguous heads")
        if t.shape[0] != T:
            raise ValueError(f"{name} has {t.shape[0]} tokens, slot_mapping {T}")
    if slot_mapping.dtype != torch.int32:
        raise ValueError("slot_mapping must be int32")
    _check(lib().kv_rotquant_write(ctypes.byref(cache.desc), ctypes.byref(cache.buffers), _ptr(k),
                                   _ptr(v), T, k.stride(0), v.stride(0), _ptr(slot_mapping),
                                   _stream(stream)))


def kv_int4_paged_decode_workspace(cache: PagedInt4Cache, num_seqs: int, num_q_heads: int,
                                   max_seq_len: int, split_tokens: int = 0) -> int:
    n = ctypes.c_size_t()
    _check(lib().kv_int4_paged_decode_workspace(ctypes.byref(cache.desc), num_seqs, num_q_heads,
                                                max_seq_len, split_tokens, ctypes.byref(n)))
    return n.value


def kv_int4_paged_decode(cache: PagedInt4Cache, q, page_table, seq_lens, max_seq_len: int,
                         out=None, sm_scale: float = 0.0, split_tokens: int = 0, workspace=None,
                         stream=None):
    """Paged INT4 decode of bf16 ``q`` [S][Hq][128]; returns fp32 ``out`` [S][Hq][128].

    A ``workspace`` passed in must have been zero-filled before its first use (its leading
    split counters); the calls leave it so.  Without one, a zeroed workspace is allocated.
    """
    import torch
    S, Hq, D = q.shape
    if q.dtype != torch.bfloat16 or not q.is_contiguous() or D != HEAD_DIM:
        raise ValueError("q must be contiguous bf16 [S][Hq][128]")
    if page_table.dtype != torch.int32 or not page_table.is_contiguous() or page_table.shape[0] != S:
        raise ValueError("page_table must be contiguous int32 [S][max_pages]")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (S,):
        raise ValueError("seq_lens must be int32 [S]")
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.float32, device=q.device)
    if workspace is None:
        n = kv_int4_paged_decode_workspace(cache, S, Hq, max_seq_len, split_tokens)
        workspace = torch.zeros(max(n, 16), dtype=torch.uint8, device=q.device)
    _check(lib().kv_int4_paged_decode(
        ctypes.byref(cache.desc), ctypes.byref(cache.buffers), _ptr(q), S, Hq, _ptr(page_table),
        int(page_table.shape[1]), _ptr(seq_lens), int(max_seq_len), float(sm_scale), int(split_tokens),
        _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def kv_int4_paged_decode_noalloc(cache: PagedInt4Cache, q, page_table, seq_lens, max_seq_len: int,
                                 out, sm_scale: float = 0.0, split_tokens: int = 0, stream=None):
    """kv_int4_paged_decode with the library's static per-GPU scratch instead of a workspace:
    writes fp32 ``out`` [S][Hq][128] (caller-allocated) and allocates nothing."""
    import torch
    S, Hq, D = q.shape
    if q.dtype != torch.bfloat16 or not q.is_contiguous() or D != HEAD_DIM:
        raise ValueError("q must be contiguous bf16 [S][Hq][128]")
    if page_table.dtype != torch.int32 or not page_table.is_contiguous() or page_table.shape[0] != S:
        raise ValueError("page_table must be contiguous int32 [S][max_pages]")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (S,):
        raise ValueError("seq_lens must be int32 [S]")
    if out.dtype != torch.float32 or tuple(out.shape) != (S, Hq, D) or not out.is_contiguous():
        raise ValueError("out must be contiguous fp32 [S][Hq][128]")
    _check(lib().kv_int4_paged_decode_noalloc(
        ctypes.byref(cache.desc), ctypes.byref(cache.buffers), _ptr(q), S, Hq, _ptr(page_table),
        int(page_table.shape[1]), _ptr(seq_lens), int(max_seq_len), float(sm_scale),
        int(split_tokens), _ptr(out), _stream(stream)))
    return out


def kv_int4_paged_decode_step(cache: PagedInt4Cache, k_new, v_new, new_slots, q, page_table, seq_lens,
                              max_seq_len: int, out=None, sm_scale: float = 0.0, split_tokens: int = 0,
                              workspace=None, stream=None):
    """Write one new token per sequence (bf16 ``k_new``/``v_new`` [S][Hkv][128] into
    ``new_slots`` [S]) and decode ``q`` over it, in one pass; returns fp32 ``out``."""
    import torch
    S, Hq, D = q.shape
    if q.dtype != torch.bfloat16 or not q.is_contiguous() or D != HEAD_DIM:
        raise ValueError("q must be contiguous bf16 [S][Hq][128]")
    for t in (k_new, v_new):
        if t.dtype != torch.bfloat16 or t.dim() != 3 or t.shape[0] != S or t.stride(2) != 1 or \
                t.stride(1) != HEAD_DIM:
            raise ValueError("k_new and v_new must be bf16 [S][Hkv][128] with contiguous heads")
    if new_slots.dtype != torch.int32 or new_slots.shape != (S,):
        raise ValueError("new_slots must be int32 [S]")
    if page_table.dtype != torch.int32 or not page_table.is_contiguous() or page_table.shape[0] != S:
        raise ValueError("page_table must be contiguous int32 [S][max_pages]")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (S,):
        raise ValueError("seq_lens must be int32 [S]")
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.float32, device=q.device)
    if workspace is None:
        n = kv_int4_paged_decode_workspace(cache, S, Hq, max_seq_len, split_tokens)
        workspace = torch.zeros(max(n, 16), dtype=torch.uint8, device=q.device)
    _check(lib().kv_int4_paged_decode_step(
        ctypes.byref(cache.desc), ctypes.byref(cache.buffers), _ptr(k_new), _ptr(v_new),
        k_new.stride(0), v_new.stride(0), _ptr(new_slots), _ptr(q), S, Hq, _ptr(page_table),
        int(page_table.shape[1]), _ptr(seq_lens), int(max_seq_len), float(sm_scale),
        int(split_tokens), _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return out


def kv_int4_paged_extend_workspace(cache: PagedInt4Cache, num_seqs: int, num_q_heads: int,
                                   total_q: int, max_q_len: int, max_seq_len: int,
                                   split_tokens: int = 0) -> int:
    n = ctypes.c_size_t()
    _check(lib().kv_int4_paged_extend_workspace(ctypes.byref(cache.desc), num_seqs, num_q_heads,
                                                total_q, max_q_len, max_seq_len, split_tokens,
                                                ctypes.byref(n)))
    return n.value


def kv_int4_paged_extend(cache: PagedInt4Cache, q, qo_start, page_table, seq_lens,
                         max_seq_len: int, max_q_len: int, out=None, sm_scale: float = 0.0,
                         split_tokens: int = 0, workspace=None, stream=None):
    """Causal extend attention of bf16 ``q`` [total_q][Hq][128] (rows qo_start[s]..
    qo_start[s+1]-1 = the last tokens of sequence s); returns fp32 ``out`` like ``q``."""
    import torch
    total_q, Hq, D = q.shape
    S = seq_lens.shape[0]
    if q.dtype != torch.bfloat16 or not q.is_contiguous() or D != HEAD_DIM:
        raise ValueError("q must be contiguous bf16 [total_q][Hq][128]")
    if qo_start.dtype != torch.int32 or qo_start.shape != (S + 1,):
        raise ValueError("qo_start must be int32 [S+1]")
    if page_table.dtype != torch.int32 or not page_table.is_contiguous() or page_table.shape[0] != S:
        raise ValueError("page_table must be contiguous int32 [S][max_pages]")
    if seq_lens.dtype != torch.int32:
        raise ValueError("seq_lens must be int32 [S]")
    if out is None:
        out = torch.empty((total_q, Hq, D), dtype=torch.float32, device=q.device)
    if workspace is None:
        n = kv_int4_paged_extend_workspace(cache, S, Hq, total_q, max_q_len, max_seq_len,
                                           split_tokens)
        workspace = torch.zeros(max(n, 16), dtype=torch.uint8, device=q.device)
    _check(lib().kv_int4_paged_extend(
        ctypes.byref(cache.desc), ctypes.byref(cache.buffers), _ptr(q), total_q, S, Hq,
        _ptr(qo_start), _ptr(page_table), int(page_table.shape[1]), _ptr(seq_lens),
        int(max_seq_len), int(max_q_len), float(sm_scale), int(split_tokens), _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


# --------------------------------------------------------------------- measurement helpers
def kvrq_bf16_paged_write(desc: CacheDesc, k_cache, v_cache, k, v, slot_mapping, stream=None) -> None:
    T = int(slot_mapping.shape[0])
    _check(lib().kvrq_bf16_paged_write(ctypes.byref(desc), _ptr(k_cache), _ptr(v_cache), _ptr(k),
                                       _ptr(v), T, k.stride(0), v.stride(0), _ptr(slot_mapping),
                                       _stream(stream)))


def kvrq_device_copy(dst, src, nbytes: Optional[int] = None, stream=None) -> None:
    n = nbytes if nbytes is not None else src.numel() * src.element_size()
    _check(lib().kvrq_device_copy(_ptr(dst), _ptr(src), n, _stream(stream)))


def kvrq_device_read(src, sink, nbytes: Optional[int] = None, stream=None) -> None:
    n = nbytes if nbytes is not None else src.numel() * src.element_size()
    _check(lib().kvrq_device_read(_ptr(src), n, _ptr(sink), _stream(stream)))


def kvrq_paged_read(cache: PagedInt4Cache, pages, sink, wgs_per_cu: int = 2, pattern: int = 0,
                    stream=None) -> None:
    """Page-gather read of the pages listed in the int32 device tensor ``pages`` (K and V codes
    and parameters of every KV head), in list order; nothing is written.  ``pattern`` 0: whole
    pages per wave; 1: per (page, KV head) block with the decode's load shapes and depth; 2: as 1
    with 16-byte V loads; 3: as 1 with four tiles in flight."""
    import torch
    if pages.dtype != torch.int32 or not pages.is_contiguous():
        raise ValueError("pages must be a contiguous int32 tensor")
    _check(lib().kvrq_paged_read(ctypes.byref(cache.desc), ctypes.byref(cache.buffers), _ptr(pages),
                                 int(pages.numel()), pattern, wgs_per_cu, _ptr(sink), _stream(stream)))


# --------------------------------------------------------------------- host page pool
class Pool:
    """Host page allocator + page table (``kvrq_pool_*``)."""

    def __init__(self, num_pages: int, page_size: int, max_seqs: int, max_pages_per_seq: int,
                 shuffle_seed: int = 0):
        self._h = ctypes.c_void_p()
        _check(lib().kvrq_pool_create(num_pages, page_size, max_seqs, max_pages_per_seq,
                                      shuffle_seed, ctypes.byref(self._h)))
        self.num_pages, self.page_size = num_pages, page_size
        self.max_seqs, self.max_pages_per_seq = max_seqs, max_pages_per_seq

    def close(self):
        if self._h:
            lib().kvrq_pool_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def seq_extend(self, seq: int, new_len: int) -> None:
        _check(lib().kvrq_seq_extend(self._h, seq, new_len))

    def seq_release(self, seq: int) -> None:
        _check(lib().kvrq_seq_release(self._h, seq))

    def seq_len(self, seq: int) -> int:
        return lib().kvrq_seq_len(self._h, seq)

    def free_pages(self) -> int:
        return lib().kvrq_pool_free_pages(self._h)

    def slots(self, seq: int, first_pos: int, count: int):
        import numpy as np
        out = np.zeros(count, np.int32)
        _check(lib().kvrq_slots(self._h, seq, first_pos, count, out.ctypes.data_as(ctypes.c_void_p)))
        return out

    def page_table(self):
        import numpy as np
        tab = np.zeros((self.max_seqs, self.max_pages_per_seq), np.int32)
        lens = np.zeros(self.max_seqs, np.int32)
        _check(lib().kvrq_page_table(self._h, tab.ctypes.data_as(ctypes.c_void_p),
                                     lens.ctypes.data_as(ctypes.c_void_p)))
        return tab, lens
