"""CPU oracle for the rotated INT4 paged KV cache -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the product
library (``int4_kv_cache_rotquant_amd``) and never imports it.

Two independent implementations live here:

* ``kvrq_oracle.c`` (loaded through ctypes): the canonical fp32 write
  encoding and an fp64 paged decode, written from the SAW-INT4 pages
  (wispaper.ai blog, sections 2-3; fugumt.com abstract).
* ``brute.py``: numpy brute force with explicit Hadamard matrices from
  ``scipy.linalg.hadamard``, used to cross-check the C code on small inputs.

Every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py`` against closed forms, library routines,
invariants and brute force; see the list of pins in each test module.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvrq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkvrq_oracle.so")

GCC_FLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
             "-std=c11", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (plain C, OpenMP, no contraction)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.kvrq_oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.kvrq_oracle_bf16_to_f32.restype = ctypes.c_float
        L.kvrq_oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.kvrq_oracle_f16_to_f32.restype = ctypes.c_float
        L.kvrq_oracle_f32_to_f16.argtypes = [ctypes.c_float]
        L.kvrq_oracle_f32_to_f16.restype = ctypes.c_uint16
        L.kvrq_oracle_rb.argtypes = [i32]
        L.kvrq_oracle_rb.restype = ctypes.c_float
        L.kvrq_oracle_fwht_f32.argtypes = [P, i32, i32]
        L.kvrq_oracle_fwht_f32.restype = None
        L.kvrq_oracle_rotate_f64.argtypes = [P, P, i32, i32]
        L.kvrq_oracle_rotate_f64.restype = None
        L.kvrq_oracle_codes_from_params.argtypes = [P, i32, i32, ctypes.c_uint16, ctypes.c_uint16,
                                                    P, P]
        L.kvrq_oracle_codes_from_params.restype = i32
        L.kvrq_oracle_quant_row.argtypes = [P, i32, i32, i32, P, P, P, P]
        L.kvrq_oracle_quant_row.restype = i32
        L.kvrq_oracle_write.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32, P, P, i64,
                                        i64, P, P, P, P, P, P, P]
        L.kvrq_oracle_write.restype = i32
        L.kvrq_oracle_decode.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32, i32, P, P,
                                         i32, P, f64, P, P, P, P, P]
        L.kvrq_oracle_decode.restype = i32
        L.kvrq_oracle_extend.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32, i32, P, P,
                                         P, i32, P, ctypes.c_double, P, P, P, P, P]
        L.kvrq_oracle_extend.restype = i32
        _lib = L
    return _lib


def set_threads(n: int) -> int:
    """Threads the oracle's OpenMP loops use from this thread on (its runtime's
    omp_set_num_threads); returns the count in force."""
    lib()
    gomp = ctypes.CDLL("libgomp.so.1")
    gomp.omp_set_num_threads.argtypes = [ctypes.c_int]
    gomp.omp_get_max_threads.restype = ctypes.c_int
    gomp.omp_set_num_threads(max(1, int(n)))
    return int(gomp.omp_get_max_threads())


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ------------------------------------------------------------------ formats
def f32_to_f16_bits(x) -> np.ndarray:
    """Elementwise binary32 -> binary16 bits (round to nearest even)."""
    x = np.ascontiguousarray(x, np.float32)
    f = lib().kvrq_oracle_f32_to_f16
    return np.array([f(float(v)) for v in x.ravel()], np.uint16).reshape(x.shape)


def f16_bits_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, np.uint16)
    f = lib().kvrq_oracle_f16_to_f32
    return np.array([f(int(v)) for v in h.ravel()], np.float32).reshape(h.shape)


def rb(b: int) -> np.float32:
    return np.float32(lib().kvrq_oracle_rb(b))


# ------------------------------------------------------------------ rotation
def fwht_f32(x: np.ndarray, b: int) -> np.ndarray:
    """Canonical fp32 block FWHT (times r_b) along the last axis."""
    y = np.array(x, dtype=np.float32, copy=True, order="C")
    n = y.shape[-1]
    flat = y.reshape(-1, n)
    for row in flat:
        lib().kvrq_oracle_fwht_f32(_p(row), n, b)
    return flat.reshape(y.shape)


def rotate_f64(x: np.ndarray, b: int) -> np.ndarray:
    """Exact block rotation by its definition, fp64, along the last axis."""
    x = np.ascontiguousarray(x, np.float64)
    n = x.shape[-1]
    flat = x.reshape(-1, n)
    out = np.empty_like(flat)
    for i in range(flat.shape[0]):
        lib().kvrq_oracle_rotate_f64(_p(flat[i]), _p(out[i]), n, b)
    return out.reshape(x.shape)


# ------------------------------------------------------------------ write
def quant_row(x_bf16: np.ndarray, b: int, bits: int = 4):
    """One row -> (codes uint8[D*bits/8], (s16, z16) uint16[2], vpre f32[D], y f32[D])."""
    x = np.ascontiguousarray(x_bf16, np.uint16)
    D = x.shape[0]
    codes = np.zeros(D * bits // 8, np.uint8)
    params = np.zeros(2, np.uint16)
    vpre = np.zeros(D, np.float32)
    y = np.zeros(D, np.float32)
    rc = lib().kvrq_oracle_quant_row(_p(x), D, b, bits, _p(codes), _p(params), _p(vpre), _p(y))
    if rc:
        raise ValueError("bad row shape")
    return codes, params, vpre, y


def codes_from_params(y: np.ndarray, params, bits: int = 4):
    """Codes of the rotated fp32 row ``y`` under given (s16, z16) bits (the write's steps 6-7
    with those parameters) -> (codes uint8[D*bits/8], vpre f32[D])."""
    y = np.ascontiguousarray(y, np.float32)
    D = y.shape[0]
    codes = np.zeros(D * bits // 8, np.uint8)
    vpre = np.zeros(D, np.float32)
    rc = lib().kvrq_oracle_codes_from_params(_p(y), D, bits, int(params[0]), int(params[1]),
                                             _p(codes), _p(vpre))
    if rc:
        raise ValueError("bad row shape")
    return codes, vpre


class Cache:
    """Host copy of one layer's paged INT4 (or 2-bit) cache (oracle side)."""

    def __init__(self, num_pages: int, num_kv_heads: int, page_size: int, head_dim: int = 128,
                 fill: int = 0xAA, k_bits: int = 4, v_bits: int = 4):
        self.num_pages, self.Hkv, self.P, self.D = num_pages, num_kv_heads, page_size, head_dim
        self.k_bits, self.v_bits = k_bits, v_bits
        shape_p = (num_pages, num_kv_heads, page_size, 2)
        self.k_codes = np.full((num_pages, num_kv_heads, page_size, head_dim * k_bits // 8), fill,
                               np.uint8)
        self.v_codes = np.full((num_pages, num_kv_heads, page_size, head_dim * v_bits // 8), fill,
                               np.uint8)
        self.k_params = np.full(shape_p, fill * 0x101, np.uint16)
        self.v_params = np.full(shape_p, fill * 0x101, np.uint16)


def write(cache: Cache, k: np.ndarray, v: np.ndarray, slots: np.ndarray, k_block: int,
          v_block: int, want_vpre: bool = False) -> Optional[Tuple[np.ndarray, np.ndarray]]:
    """Encode tokens ``k, v`` (bf16 bits [T][Hkv][D]) into ``cache`` at ``slots``."""
    k = np.ascontiguousarray(k, np.uint16)
    v = np.ascontiguousarray(v, np.uint16)
    slots = np.ascontiguousarray(slots, np.int32)
    T, Hkv, D = k.shape
    assert v.shape == k.shape and Hkv == cache.Hkv and D == cache.D and slots.shape == (T,)
    kv = vv = None
    if want_vpre:
        kv = np.zeros((T, Hkv, D), np.float32)
        vv = np.zeros((T, Hkv, D), np.float32)
    rc = lib().kvrq_oracle_write(T, Hkv, D, cache.P, cache.num_pages, k_block, v_block,
                                 cache.k_bits, cache.v_bits, _p(k),
                                 _p(v), Hkv * D, Hkv * D, _p(slots), _p(cache.k_codes),
                                 _p(cache.v_codes), _p(cache.k_params), _p(cache.v_params),
                                 _p(kv), _p(vv))
    if rc:
        raise ValueError("slot outside the page pool")
    return (kv, vv) if want_vpre else None


# ------------------------------------------------------------------ decode
def code_bits(codes: np.ndarray, head_dim: int) -> int:
    """Code width of a pool from its row bytes: D/2 -> 4 bits, D/4 -> 2 bits."""
    bits = codes.shape[-1] * 8 // head_dim
    if bits not in (2, 4) or codes.shape[-1] * 8 != bits * head_dim:
        raise ValueError(f"code rows of {codes.shape[-1]} bytes fit no supported width")
    return bits


def decode(q: np.ndarray, cache_arrays, page_table: np.ndarray, seq_lens: np.ndarray,
           num_kv_heads: int, page_size: int, k_block: int, v_block: int,
           sm_scale: float = 0.0) -> np.ndarray:
    """fp64 attention; ``cache_arrays`` = (k_codes, v_codes, k_params, v_params); the
    code widths follow from the code arrays' row bytes (D/2: 4 bits, D/4: 2 bits)."""
    q = np.ascontiguousarray(q, np.uint16)
    S, Hq, D = q.shape
    kc, vc, kp, vp = [np.ascontiguousarray(a) for a in cache_arrays]
    kbits, vbits = code_bits(kc, D), code_bits(vc, D)
    num_pages = kc.shape[0]
    page_table = np.ascontiguousarray(page_table, np.int32)
    seq_lens = np.ascontiguousarray(seq_lens, np.int32)
    out = np.zeros((S, Hq, D), np.float64)
    rc = lib().kvrq_oracle_decode(S, Hq, num_kv_heads, D, page_size, num_pages, k_block, v_block,
                                  kbits, vbits, _p(q), _p(page_table), page_table.shape[1], _p(seq_lens),
                                  float(sm_scale), _p(kc), _p(vc), _p(kp), _p(vp), _p(out))
    if rc == 1:
        raise ValueError("bad decode shapes")
    if rc == 2:
        raise ValueError("page id outside the pool")
    return out


def extend(q: np.ndarray, cache_arrays, qo_start: np.ndarray, page_table: np.ndarray,
           seq_lens: np.ndarray, num_kv_heads: int, page_size: int, k_block: int, v_block: int,
           sm_scale: float = 0.0) -> np.ndarray:
    """fp64 causal extend attention: ``q`` [total_q][Hq][D] bf16 bits; the rows
    qo_start[s]..qo_start[s+1]-1 are the last tokens of sequence s (of seq_lens[s])."""
    q = np.ascontiguousarray(q, np.uint16)
    total_q, Hq, D = q.shape
    kc, vc, kp, vp = [np.ascontiguousarray(a) for a in cache_arrays]
    kbits, vbits = code_bits(kc, D), code_bits(vc, D)
    num_pages = kc.shape[0]
    qo_start = np.ascontiguousarray(qo_start, np.int32)
    page_table = np.ascontiguousarray(page_table, np.int32)
    seq_lens = np.ascontiguousarray(seq_lens, np.int32)
    S = seq_lens.shape[0]
    if qo_start.shape != (S + 1,) or qo_start[-1] != total_q:
        raise ValueError("qo_start must have S+1 entries ending at total_q")
    out = np.zeros((total_q, Hq, D), np.float64)
    rc = lib().kvrq_oracle_extend(S, Hq, num_kv_heads, D, page_size, num_pages, k_block,
                                  v_block, kbits, vbits, _p(q), _p(qo_start), _p(page_table),
                                  page_table.shape[1], _p(seq_lens), float(sm_scale), _p(kc),
                                  _p(vc), _p(kp), _p(vp), _p(out))
    if rc == 1:
        raise ValueError("bad extend shapes")
    if rc == 2:
        raise ValueError("page id outside the pool")
    return out
