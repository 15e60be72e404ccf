"""Seeded synthetic inputs for the rotated INT4 paged KV cache.

This module is shared by the product tests, the oracle tests and the
benchmark.  It holds ONLY random-number generation and bookkeeping of
shapes, lengths and page assignments: no rotation, no quantisation and no
attention arithmetic lives here.

The recipes stand in for the models and serving sweeps the SAW-INT4 pages
measure on (Qwen3-4B/8B/32B, GLM-4.7 and request-rate sweeps; wispaper.ai
blog, section 4 "experiments and results"), which are not available: the
head geometry follows those models, values are N(0,1) with a few strong
outlier channels in K -- the structure the pages blame for the failure of
naive INT4 (wispaper.ai blog, section 2 "core intuition").

Conventions shared by every consumer:
  * bf16 tensors are carried as uint16 bit patterns, fp32 -> bf16 by
    round-to-nearest-even of the fp32 bit pattern;
  * a slot is ``page * page_size + offset``; a negative slot means "skip";
  * page tables are int32 ``[num_seqs][max_pages_per_seq]`` padded with -1.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np

BASE_SEED = 20260421
HEAD_DIM = 128


# --------------------------------------------------------------------------
# bf16 helpers (input encoding only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even.

    Inputs are finite by construction, so NaN handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# outlier channel recipe
# --------------------------------------------------------------------------
@dataclasses.dataclass
class OutlierSpec:
    """Per-head channel multipliers applied to every token of K (or V).

    ``mult[h, d]`` is 1 except on the chosen outlier channels.
    """
    mult: np.ndarray  # float32 [Hkv][D]

    @staticmethod
    def none(num_kv_heads: int, head_dim: int = HEAD_DIM) -> "OutlierSpec":
        return OutlierSpec(np.ones((num_kv_heads, head_dim), np.float32))

    @staticmethod
    def fixed(num_kv_heads: int, channels, factor: float,
              head_dim: int = HEAD_DIM) -> "OutlierSpec":
        m = np.ones((num_kv_heads, head_dim), np.float32)
        m[:, list(channels)] = factor
        return OutlierSpec(m)

    @staticmethod
    def random(rng: np.random.Generator, num_kv_heads: int, frac: float = 0.02,
               lo: float = 10.0, hi: float = 30.0,
               head_dim: int = HEAD_DIM) -> "OutlierSpec":
        """ceil(frac*D) channels per head, each scaled by U(lo, hi)."""
        n = int(math.ceil(frac * head_dim))
        m = np.ones((num_kv_heads, head_dim), np.float32)
        for h in range(num_kv_heads):
            ch = rng.choice(head_dim, size=n, replace=False)
            m[h, ch] = rng.uniform(lo, hi, size=n).astype(np.float32)
        return OutlierSpec(m)


def make_rows(rng: np.random.Generator, num_tokens: int, num_kv_heads: int,
              outliers: Optional[OutlierSpec] = None,
              head_dim: int = HEAD_DIM) -> np.ndarray:
    """bf16 bits ``[T][Hkv][D]``: N(0,1) times the per-head channel multipliers."""
    x = rng.standard_normal((num_tokens, num_kv_heads, head_dim), dtype=np.float32)
    if outliers is not None:
        x *= outliers.mult[None, :, :]
    return f32_to_bf16_bits(x)


def make_rows_torch(gen, num_tokens: int, num_kv_heads: int, outliers: Optional[OutlierSpec],
                    device, head_dim: int = HEAD_DIM):
    """Device-side generator with the same distribution as :func:`make_rows`.

    Used where host generation of the full tensor would be too slow (the
    multi-GB long-context and high-concurrency fills).  Values differ from the
    numpy generator; tests that compare against the oracle copy the sampled
    rows back to the host.
    """
    import torch
    x = torch.randn((num_tokens, num_kv_heads, head_dim), generator=gen, device=device,
                    dtype=torch.float32)
    if outliers is not None:
        x *= torch.from_numpy(outliers.mult).to(device)[None]
    return x.to(torch.bfloat16)


# --------------------------------------------------------------------------
# paging bookkeeping
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Paging:
    page_size: int
    num_pages: int
    seq_pages: List[np.ndarray]   # physical page ids per sequence, in logical order

    def page_table(self, max_pages: Optional[int] = None) -> np.ndarray:
        mp = max_pages if max_pages is not None else max(len(p) for p in self.seq_pages)
        tab = np.full((len(self.seq_pages), mp), -1, np.int32)
        for s, pages in enumerate(self.seq_pages):
            tab[s, :len(pages)] = pages
        return tab

    def slots(self, seq: int, first_pos: int, count: int) -> np.ndarray:
        pos = np.arange(first_pos, first_pos + count, dtype=np.int64)
        pages = self.seq_pages[seq][pos // self.page_size].astype(np.int64)
        return (pages * self.page_size + pos % self.page_size).astype(np.int32)


def assign_pages(rng: Optional[np.random.Generator], capacities: List[int], page_size: int,
                 extra_pages: int = 0) -> Paging:
    """Give each sequence ``ceil(capacity/page_size)`` pages.

    With ``rng`` the physical ids are a random permutation of the pool
    (scattered pages); without it they are handed out in order (identity).
    """
    need = [int(math.ceil(c / page_size)) for c in capacities]
    total = int(sum(need)) + extra_pages
    order = np.arange(total, dtype=np.int32) if rng is None else rng.permutation(total).astype(np.int32)
    out, k = [], 0
    for n in need:
        out.append(order[k:k + n].copy())
        k += n
    return Paging(page_size, total, out)


def lognormal_lengths(rng: np.random.Generator, n: int, median: float, sigma: float,
                      lo: int, hi: int) -> np.ndarray:
    x = np.exp(math.log(median) + sigma * rng.standard_normal(n))
    return np.clip(np.round(x), lo, hi).astype(np.int64)


# --------------------------------------------------------------------------
# the workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    name: str
    num_kv_heads: int
    num_q_heads: int
    page_size: int
    k_block: int
    v_block: int
    seq_lens: np.ndarray            # tokens written / attended per sequence
    paging: Paging
    k_out: OutlierSpec
    v_out: OutlierSpec
    seed: int
    head_dim: int = HEAD_DIM
    notes: Dict[str, object] = dataclasses.field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return len(self.seq_lens)

    @property
    def total_tokens(self) -> int:
        return int(self.seq_lens.sum())

    def rng(self, stream: int) -> np.random.Generator:
        """Independent seeded stream ``stream`` of this workload."""
        return np.random.Generator(np.random.PCG64([self.seed, stream]))

    # host-side full inputs (small and medium workloads)
    def all_slots(self) -> np.ndarray:
        return np.concatenate([self.paging.slots(s, 0, int(L)) for s, L in enumerate(self.seq_lens)])

    def kv(self) -> Tuple[np.ndarray, np.ndarray]:
        T = self.total_tokens
        k = make_rows(self.rng(1), T, self.num_kv_heads, self.k_out, self.head_dim)
        v = make_rows(self.rng(2), T, self.num_kv_heads, self.v_out, self.head_dim)
        return k, v

    def q(self) -> np.ndarray:
        r = self.rng(3)
        x = r.standard_normal((self.num_seqs, self.num_q_heads, self.head_dim), dtype=np.float32)
        return f32_to_bf16_bits(x)


def tiny() -> Workload:
    """1 sequence x 64 tokens, 1 KV head; K channels {5,37,70,101} x20; blocks 128/128."""
    seed = BASE_SEED + 0
    paging = assign_pages(None, [64], 16)
    return Workload("tiny", 1, 1, 16, 128, 128, np.array([64]), paging,
                    OutlierSpec.fixed(1, (5, 37, 70, 101), 20.0), OutlierSpec.none(1), seed)


def qwen3_4b_like() -> Workload:
    """Hq=32, Hkv=8, 16 sequences of U{1024..4096} tokens, page 16 scattered; K block 64, V plain."""
    seed = BASE_SEED + 1
    rng = np.random.Generator(np.random.PCG64([seed, 0]))
    lens = rng.integers(1024, 4096, size=16, endpoint=True)
    k_out = OutlierSpec.random(rng, 8)
    paging = assign_pages(rng, list(lens), 16)
    return Workload("qwen3_4b_like", 8, 32, 16, 64, 0, lens, paging, k_out, OutlierSpec.none(8), seed)


def prefill_chunk(k_block: int = 128) -> Workload:
    """One sequence, 32768-token chunk, Hkv=8, page 64 scattered; K block swept, V plain."""
    seed = BASE_SEED + 2
    rng = np.random.Generator(np.random.PCG64([seed, 0]))
    k_out = OutlierSpec.random(rng, 8)
    v_out = OutlierSpec.random(rng, 8)
    paging = assign_pages(rng, [32768], 64)
    return Workload("prefill_chunk", 8, 8, 64, k_block, 0, np.array([32768]), paging,
                    k_out, v_out, seed, notes={"k_block_sweep": [16, 32, 64, 128, 0]})


def qwen3_32b_like_decode(num_steps: int = 100) -> Workload:
    """Hq=64, Hkv=8, 256 sequences, log-normal lengths (median 8192, sigma 1, clip
    [512, 32768]); page 16 scattered, pool sized for ``num_steps`` more tokens each;
    K block 128, V plain."""
    seed = BASE_SEED + 3
    rng = np.random.Generator(np.random.PCG64([seed, 0]))
    lens = lognormal_lengths(rng, 256, 8192.0, 1.0, 512, 32768)
    k_out = OutlierSpec.random(rng, 8)
    paging = assign_pages(rng, [int(L) + num_steps for L in lens], 16)
    return Workload("qwen3_32b_like_decode", 8, 64, 16, 128, 0, lens, paging, k_out,
                    OutlierSpec.none(8), seed, notes={"steps": num_steps})


def small_batch_decode(num_steps: int = 100) -> Workload:
    """Latency-bound decode steps: Hq=32, Hkv=8, 4 sequences of 4096 tokens, page 16
    scattered, pool sized for ``num_steps`` more tokens each; K block 128, V plain."""
    seed = BASE_SEED + 6
    rng = np.random.Generator(np.random.PCG64([seed, 0]))
    lens = np.full(4, 4096, np.int64)
    k_out = OutlierSpec.random(rng, 8)
    paging = assign_pages(rng, [int(L) + num_steps for L in lens], 16)
    return Workload("small_batch_decode", 8, 32, 16, 128, 0, lens, paging, k_out,
                    OutlierSpec.none(8), seed, notes={"steps": num_steps})


def long_context() -> Workload:
    """One sequence of 1,048,576 tokens, Hkv=8, Hq=64, page 64 scattered, blocks 128/128,
    filled by 64 writes of 16384 tokens."""
    seed = BASE_SEED + 4
    rng = np.random.Generator(np.random.PCG64([seed, 0]))
    k_out = OutlierSpec.random(rng, 8)
    v_out = OutlierSpec.random(rng, 8)
    paging = assign_pages(rng, [1 << 20], 64)
    return Workload("long_context", 8, 64, 64, 128, 128, np.array([1 << 20]), paging,
                    k_out, v_out, seed, notes={"chunk": 16384})


def chunked_prefill() -> Workload:
    """Qwen3-4B-like heads (Hq=32, Hkv=8), 8 sequences with prefixes of U{1024..6144}
    tokens already cached, each extended by a 1024-token chunk: the chunk is written, then
    its rows attend causally over prefix + chunk.  Page 16 scattered; K block 64, V plain."""
    seed = BASE_SEED + 5
    rng = np.random.Generator(np.random.PCG64([seed, 0]))
    chunk = 1024
    prefix = rng.integers(1024, 6144, size=8, endpoint=True)
    k_out = OutlierSpec.random(rng, 8)
    lens = prefix + chunk
    paging = assign_pages(rng, list(lens), 16)
    return Workload("chunked_prefill", 8, 32, 16, 64, 0, lens, paging, k_out, OutlierSpec.none(8),
                    seed, notes={"chunk": chunk, "prefix": prefix})


WORKLOADS = {
    "tiny": tiny,
    "qwen3_4b_like": qwen3_4b_like,
    "prefill_chunk": prefill_chunk,
    "qwen3_32b_like_decode": qwen3_32b_like_decode,
    "long_context": long_context,
    "chunked_prefill": chunked_prefill,
    "small_batch_decode": small_batch_decode,
}
