"""numpy brute force for small inputs -- TEST INFRASTRUCTURE ONLY.

A second, independent implementation used to cross-check ``kvrq_oracle.c``:

* the rotation is an explicit block-diagonal matrix built from
  ``scipy.linalg.hadamard(b) / sqrt(b)`` (Sylvester order), the block design
  of the SAW-INT4 pages (wispaper.ai blog, section 2, block-diagonal bullet);
* binary16 conversion is numpy's own ``astype(np.float16)``;
* attention is the textbook softmax over explicit matrices in fp64
  (wispaper.ai blog, section 3: query rotated at inference so that the
  rotated-space dot product equals the original one).

The fp32 write here re-derives the same encoding with vectorised numpy
operations (stage by stage over whole arrays), so that an indexing or
format mistake in the C code shows up as a mismatch.
"""
from __future__ import annotations

import numpy as np
import scipy.linalg


def hadamard_blockdiag(D: int, b: int) -> np.ndarray:
    """Orthonormal block-diagonal Hadamard matrix, fp64 [D][D]; b = 0 -> identity."""
    if b <= 1:
        return np.eye(D)
    Hb = scipy.linalg.hadamard(b).astype(np.float64) / np.sqrt(b)
    return scipy.linalg.block_diag(*([Hb] * (D // b)))


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def fwht_f32_vec(x: np.ndarray, b: int) -> np.ndarray:
    """fp32 butterflies over the last axis, widths 1, 2, ..., b/2, then * fp32(1/sqrt(b))."""
    y = np.array(x, np.float32, copy=True)
    if b <= 1:
        return y
    D = y.shape[-1]
    lead = y.shape[:-1]
    blocks = y.reshape(*lead, D // b, b)
    h = 1
    while h < b:
        v = blocks.reshape(*lead, D // b, b // (2 * h), 2, h)
        u = v[..., 0, :].copy()
        w = v[..., 1, :].copy()
        v[..., 0, :] = u + w
        v[..., 1, :] = u - w
        h *= 2
    r = np.float32(1.0 / np.sqrt(np.float64(b)))
    return (blocks * r).reshape(y.shape)


def codes_for_params(y: np.ndarray, s16_bits, z16_bits, bits: int = 4):
    """Rotated fp32 rows [..., D] and binary16 (scale, zero) bit patterns [...] -> (codes uint8
    [..., D*bits/8], vpre f32): the quantiser's last steps for parameters given from outside."""
    levels = (1 << bits) - 1
    s16 = np.asarray(s16_bits, np.uint16).view(np.float16)
    z16 = np.asarray(z16_bits, np.uint16).view(np.float16)
    sf = s16.astype(np.float32)[..., None]
    zf = z16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        inv = np.float32(1.0) / sf
        v = (np.asarray(y, np.float32) - zf) * inv
    zero = (s16.view(np.uint16) & 0x7FFF) == 0
    v = np.where(zero[..., None], np.float32(0.0), v).astype(np.float32)
    q = np.clip(np.rint(v), 0, levels).astype(np.uint8)
    per = 8 // bits
    codes = np.zeros(q.shape[:-1] + (q.shape[-1] // per,), np.uint8)
    for j in range(per):
        codes |= (q[..., j::per] << (bits * j)).astype(np.uint8)
    return codes, v


def quantize_rows(x_bf16: np.ndarray, b: int, bits: int = 4):
    """Rows [..., D] -> (codes uint8 [..., D*bits/8], s16 bits, z16 bits, vpre f32); 2^bits - 1
    levels, channel d at bit (d*bits) % 8 of byte d*bits/8."""
    levels = (1 << bits) - 1
    y = fwht_f32_vec(bf16_to_f32(x_bf16), b)
    mn = y.min(axis=-1) + np.float32(0.0)
    mx = y.max(axis=-1) + np.float32(0.0)
    scale32 = (mx - mn) / np.float32(levels)
    s16 = scale32.astype(np.float16).view(np.uint16)
    z16 = mn.astype(np.float16).view(np.uint16)
    codes, v = codes_for_params(y, s16, z16, bits)
    return codes, s16, z16, v


def unpack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Codes [..., D*bits/8] -> integer codes [..., D]."""
    c = np.asarray(codes, np.uint8)
    per = 8 // bits
    q = np.empty(c.shape[:-1] + (per * c.shape[-1],), np.int64)
    for j in range(per):
        q[..., j::per] = (c >> (bits * j)) & ((1 << bits) - 1)
    return q


def dequant_rows(codes: np.ndarray, s16: np.ndarray, z16: np.ndarray, bits: int = 4) -> np.ndarray:
    """Codes [..., D*bits/8] with fp16 bits (s, z) -> fp64 values q*s + z."""
    q = unpack_codes(codes, bits).astype(np.float64)
    s = np.asarray(s16, np.uint16).view(np.float16).astype(np.float64)[..., None]
    z = np.asarray(z16, np.uint16).view(np.float16).astype(np.float64)[..., None]
    return q * s + z


def gather_seq(cache_arrays, page_table_row: np.ndarray, L: int, page_size: int, h: int):
    """Dequantised K and V rows (fp64 [L][D]) of one sequence and KV head."""
    kc, vc, kp, vp = cache_arrays
    t = np.arange(L)
    pages = np.asarray(page_table_row)[t // page_size]
    off = t % page_size
    D = 128
    K = dequant_rows(kc[pages, h, off], kp[pages, h, off, 0], kp[pages, h, off, 1],
                     kc.shape[-1] * 8 // D)
    V = dequant_rows(vc[pages, h, off], vp[pages, h, off, 0], vp[pages, h, off, 1],
                     vc.shape[-1] * 8 // D)
    return K, V


def decode(q_bf16: np.ndarray, cache_arrays, page_table: np.ndarray, seq_lens, num_kv_heads: int,
           page_size: int, k_block: int, v_block: int, sm_scale: float = 0.0) -> np.ndarray:
    """fp64 attention with explicit matrices; returns [S][Hq][D]."""
    q = bf16_to_f32(q_bf16).astype(np.float64)
    S, Hq, D = q.shape
    G = Hq // num_kv_heads
    if sm_scale <= 0:
        sm_scale = 1.0 / np.sqrt(D)
    HK = hadamard_blockdiag(D, k_block)
    HV = hadamard_blockdiag(D, v_block)
    out = np.zeros((S, Hq, D))
    for s in range(S):
        L = int(seq_lens[s])
        if L <= 0:
            continue
        for h in range(num_kv_heads):
            K, V = gather_seq(cache_arrays, page_table[s], L, page_size, h)
            qs = q[s, h * G:(h + 1) * G] @ HK.T          # rotated queries [G][D]
            scores = sm_scale * (qs @ K.T)                # [G][L]
            scores -= scores.max(axis=1, keepdims=True)
            p = np.exp(scores)
            p /= p.sum(axis=1, keepdims=True)
            out[s, h * G:(h + 1) * G] = (p @ V) @ HV.T    # back to the unrotated basis
    return out


def extend(q_bf16: np.ndarray, cache_arrays, qo_start, page_table: np.ndarray, seq_lens,
           num_kv_heads: int, page_size: int, k_block: int, v_block: int,
           sm_scale: float = 0.0) -> np.ndarray:
    """fp64 causal extend attention with explicit matrices and an explicit mask: the n
    query rows of sequence s are its last n positions; row i sees tokens 0..L-n+i."""
    q = bf16_to_f32(q_bf16).astype(np.float64)
    total_q, Hq, D = q.shape
    G = Hq // num_kv_heads
    if sm_scale <= 0:
        sm_scale = 1.0 / np.sqrt(D)
    HK = hadamard_blockdiag(D, k_block)
    HV = hadamard_blockdiag(D, v_block)
    out = np.zeros((total_q, Hq, D))
    for s in range(len(seq_lens)):
        r0, r1 = int(qo_start[s]), int(qo_start[s + 1])
        n, L = r1 - r0, int(seq_lens[s])
        if n == 0:
            continue
        pos = L - n + np.arange(n)                              # query positions
        mask = np.arange(L)[None, :] <= pos[:, None]            # [n][L], causal
        for h in range(num_kv_heads):
            K, V = gather_seq(cache_arrays, page_table[s], L, page_size, h)
            for g in range(h * G, (h + 1) * G):
                qs = q[r0:r1, g] @ HK.T                         # [n][D]
                scores = sm_scale * (qs @ K.T)
                scores = np.where(mask, scores, -np.inf)
                scores -= scores.max(axis=1, keepdims=True)
                p = np.exp(scores)
                p /= p.sum(axis=1, keepdims=True)
                out[r0:r1, g] = (p @ V) @ HV.T
    return out
