#!/usr/bin/env python3
"""Benchmark of the rotated INT4 paged KV-cache hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
kv_rotquant_write of the batch's new tokens (rotation + INT4 quantisation +
paged store) and kv_int4_paged_decode over the cache (query rotation, page
walk, de-quantised attention, split-K combine, inverse V rotation).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--variant ...]

Workloads (sizes of the SAW-INT4 serving shapes; synthetic data):
  qwen3_32b_like_decode  (default) Hq=64, Hkv=8, 256 log-normal sequences
                         (~2.94M tokens), page 16 scattered, K block 128, V
                         plain; a step writes 1 token per sequence and decodes
                         all sequences over L+1; --variant fused does both in
                         one kv_int4_paged_decode_step call
  qwen3_4b_like          Hq=32, Hkv=8, 16 sequences of U{1024..4096} tokens,
                         page 16 scattered, K block 64, V plain; a step writes
                         every token, then decodes every sequence
  prefill_chunk          32768-token chunk write, Hkv=8, page 64 scattered;
                         --variant bdr (K block --k-block) | plain | bf16
  small_batch_decode     the same step for 4 sequences of 4096 tokens, Hq=32,
                         Hkv=8 (latency-bound; --variant fused as above)
  long_context           1M-token sequence, Hq=64, Hkv=8, page 64, blocks
                         128/128; a step is the 64-chunk fill plus one decode
  chunked_prefill        Hq=32, Hkv=8, 8 sequences with cached prefixes, each
                         extended by a 1024-token chunk: write + causal extend

Prints ONE JSON line.  ``value`` is KV tokens/s over the timed steps: the KV
tokens the step's decode attends (each token = all KV heads of K and V; the
step's own write included in the time), or, for a step with no decode, the
tokens it writes; wall clock between two device synchronisations, inputs
already in HBM.  ``rates`` gives each kernel's own rate from HIP events on its
stream: the write's tokens written / write time and the decode's tokens
attended / decode time.  The ``roofline`` object covers the kernel with the
largest share of the step time: algorithmic bytes per launch / its mean launch
time.  ``cpu_baseline`` times the CPU oracle on a bounded sample of the same
workload in the same unit (rank 0, N=1 only).  ``--graph`` (decode-step
workloads) adds a ``graph`` object: the workload's distinct steps recorded once
into a HIP graph and replayed, i.e. the step without the host's per-call launch
overhead, which a small batch's kernels are shorter than.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

HBM_PEAK_GBPS = 8000.0
# attention at MFMA peak: half the flops on int8 (5.0 POP/s dense), half on f16 (2.5 PFLOP/s)
MFMA_ATTENTION_PEAK_TFLOPS = 1.0 / (0.5 / 5000.0 + 0.5 / 2500.0)
D = 128


# Default (timed steps, warmup steps) per workload: the warmup keeps the GPU busy long enough
# for its clocks to settle (a 5-step warmup read the chunked-prefill extend 18% slow and the
# Qwen3-32B-like decode 7% slow), and the timed region lasts a few hundred milliseconds.
DEFAULT_STEPS = {
    "tiny": (1000, 1000),
    "qwen3_4b_like": (3000, 3000),            # ~0.073 ms per step
    "prefill_chunk": (4000, 4000),            # ~0.05 ms
    "qwen3_32b_like_decode": (400, 400),      # ~0.65 ms
    "long_context": (150, 150),               # ~1.9 ms
    "chunked_prefill": (250, 250),            # ~1.3 ms
    "small_batch_decode": (10000, 10000),     # ~0.02 ms
}


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: per workload, about 0.2-0.4 s of GPU time)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default: per workload, as long as the timed ones: "
                         "MI355X clocks ramp up over the first few hundred milliseconds of load)")
    ap.add_argument("--workload", default="qwen3_32b_like_decode", choices=sorted(W.WORKLOADS))
    ap.add_argument("--variant", default="bdr", choices=["bdr", "plain", "bf16", "fused"],
                    help="prefill_chunk: fused BDR write, plain INT4 write, or bf16 paged copy; "
                         "qwen3_32b_like_decode: fused = write + decode in one call")
    ap.add_argument("--k-block", type=int, default=None, help="override the workload's K block")
    ap.add_argument("--k-bits", type=int, default=4, choices=[4, 2], help="K code width")
    ap.add_argument("--v-bits", type=int, default=4, choices=[4, 2], help="V code width")
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--graph", action="store_true",
                    help="decode-step workloads: also time the steps replayed from a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle sample time")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="oracle threads (0: every core of the process's affinity)")
    ap.add_argument("--bdr-vs-plain", action="store_true",
                    help="also time the 32k prefill-chunk write with BDR-128 and plain INT4 "
                         "(always on for the default workload)")
    ap.add_argument("--paged-ceiling", action="store_true",
                    help="only measure the decode's pages read in the decode's order with no "
                         "arithmetic (kvrq_paged_read), the decode alone and a streaming read of "
                         "as many bytes, each after a cache-evicting read; print one JSON line")
    ap.add_argument("--ceilings", action="store_true",
                    help="only measure the size-matched streaming-read and copy ceilings and print "
                         "them as one JSON line")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="(accepted for older scripts: the 1 GiB copy probe always runs)")
    ap.add_argument("--counters", default=None,
                    help="JSON with FETCH_SIZE/WRITE_SIZE per launch (see --parse-counters); "
                         "default: profiles/hbm_counters.<workload>[.<variant>].json if present")
    ap.add_argument("--parse-counters", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT_JSON"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) and exit")
    ap.add_argument("--profiled-args", default="",
                    help="with --parse-counters: the bench.py arguments the two --pmc runs used")
    args = ap.parse_args(argv)
    steps, warmup = DEFAULT_STEPS[args.workload]
    if args.steps is None:
        args.steps = steps
    if args.warmup is None:
        args.warmup = warmup
    if args.counters is None:
        args.counters = os.path.join(ROOT, "profiles", f"hbm_counters.{workload_tag(args)}.json")
    return args


def workload_tag(args) -> str:
    """Name of the measured configuration, used for the counter summary files."""
    tag = args.workload
    if args.variant != "bdr":
        tag += "." + args.variant
    elif args.k_block is not None:
        tag += f".k{args.k_block}"
    if (args.k_bits, args.v_bits) != (4, 4):
        tag += f".k{args.k_bits}v{args.v_bits}bit"
    return tag


def kernel_source_hash() -> str:
    """Hash of the kernel sources with comments and blank space removed: counter figures
    taken on other code are not reported as this code's traffic."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "int4_kv_cache_rotquant_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(csrc, name)) as f:
                text = f.read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            text = re.sub(r"//[^\n]*", "", text)
            h.update(name.encode() + re.sub(r"\s+", " ", text).strip().encode())
    return h.hexdigest()[:16]


class HipEvent:
    """A HIP timing event recorded on the stream the kernels are launched on (torch's
    current stream, which the bindings use by default).

    Created with hipEventDisableSystemFence: a default event performs a system-scope
    release (an L2 write-back) when it is recorded, which adds several microseconds to
    every bracketed kernel; a fence-free event times the kernel, not the fence."""
    FLAGS = 0x20000000          # hipEventDisableSystemFence
    _hip = None

    @classmethod
    def hip(cls):
        if cls._hip is None:
            import ctypes
            h = ctypes.CDLL("libamdhip64.so")
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                              ctypes.c_void_p]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = h
        return cls._hip

    def __init__(self, torch):
        import ctypes
        self.torch = torch
        self.ev = ctypes.c_void_p()
        st = self.hip().hipEventCreateWithFlags(ctypes.byref(self.ev), self.FLAGS)
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {st}")

    def record(self):
        st = self.hip().hipEventRecord(self.ev, self.torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed: {st}")

    def elapsed_time(self, end) -> float:
        import ctypes
        ms = ctypes.c_float()
        st = self.hip().hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {st}")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.ev:
            self._hip.hipEventDestroy(self.ev)


class Setup:
    """Device buffers and one-step closure for a workload."""

    def __init__(self, args, K, torch):
        self.args, self.K, self.torch = args, K, torch
        self.w = W.WORKLOADS[args.workload]()
        self.dev = "cuda"
        self.gen = torch.Generator(device=self.dev)
        self.gen.manual_seed(self.w.seed)
        self.kernels = {}          # name -> algorithmic bytes per launch
        getattr(self, "setup_" + args.workload)()

    # -- helpers
    def rows(self, T, Hkv, out):
        return W.make_rows_torch(self.gen, T, Hkv, out, self.dev)

    def dev_i32(self, a):
        return self.torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(self.dev)

    def kv_row_bytes(self):
        """Cache bytes of one (token, head) K row plus V row: codes and (scale, zero)."""
        return D * (self.args.k_bits + self.args.v_bits) // 8 + 2 * 4

    def new_cache(self, num_pages, Hkv, P, kb, vb):
        return self.K.PagedInt4Cache(num_pages, Hkv, P, kb, vb, k_bits=self.args.k_bits,
                                     v_bits=self.args.v_bits)

    def write_bytes(self, T, Hkv):
        return T * (Hkv * (2 * 2 * D + self.kv_row_bytes()) + 4)

    def decode_bytes(self, lens, Hkv, Hq, P):
        lens = np.asarray(lens, np.int64)
        return int(lens.sum() * Hkv * self.kv_row_bytes() + len(lens) * Hq * (2 * D + 4 * D)
                   + np.ceil(lens / P).sum() * 4 + len(lens) * 4)

    # -- qwen3_4b_like: write everything, decode every sequence; 3 rotating buffer sets
    def setup_qwen3_4b_like(self):
        K, torch, w = self.K, self.torch, self.w
        kb = self.args.k_block if self.args.k_block is not None else w.k_block
        self.kb, self.vb = kb, w.v_block
        T, Hkv, Hq = w.total_tokens, w.num_kv_heads, w.num_q_heads
        self.sets = []
        for i in range(3):
            cache = self.new_cache(w.paging.num_pages, Hkv, w.page_size, kb, w.v_block)
            k, v = self.rows(T, Hkv, w.k_out), self.rows(T, Hkv, w.v_out)
            q = torch.randn((w.num_seqs, Hq, D), generator=self.gen, device=self.dev).to(torch.bfloat16)
            self.sets.append((cache, k, v, q))
        self.slots = self.dev_i32(w.all_slots())
        self.tab = self.dev_i32(w.paging.page_table())
        self.lens = self.dev_i32(w.seq_lens)
        self.maxlen = int(w.seq_lens.max())
        self.out = torch.empty((w.num_seqs, Hq, D), dtype=torch.float32, device=self.dev)
        n = K.kv_int4_paged_decode_workspace(self.sets[0][0], w.num_seqs, Hq, self.maxlen,
                                             self.args.split_tokens)
        self.ws = torch.zeros(n, dtype=torch.uint8, device=self.dev)
        self.kernels = {"kv_rotquant_write": self.write_bytes(T, Hkv),
                        "kv_int4_paged_decode": self.decode_bytes(w.seq_lens, Hkv, Hq, w.page_size)}
        self.rate_tokens = {"kv_rotquant_write": T, "kv_int4_paged_decode": int(w.seq_lens.sum())}
        self.tokens_per_step = int(w.seq_lens.sum())
        self.config = {"workload": w.name, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
                       "num_seqs": w.num_seqs, "tokens_written": T,
                       "tokens_attended": int(w.seq_lens.sum()), "page_size": w.page_size,
                       "k_block": kb, "v_block": w.v_block}

    def step_qwen3_4b_like(self, i, ev):
        K = self.K
        cache, k, v, q = self.sets[i % len(self.sets)]
        ev[0].record()
        K.kv_rotquant_write(cache, k, v, self.slots)
        ev[1].record()
        K.kv_int4_paged_decode(cache, q, self.tab, self.lens, self.maxlen, out=self.out,
                               split_tokens=self.args.split_tokens, workspace=self.ws)
        ev[2].record()

    # -- prefill chunk: one 32768-token write per step; 4 rotating buffer sets
    def setup_prefill_chunk(self):
        K, torch, w = self.K, self.torch, self.w
        kb = self.args.k_block if self.args.k_block is not None else 128
        variant = self.args.variant
        if variant == "plain":
            kb = 0
        self.kb, self.vb = kb, 0
        T, Hkv = w.total_tokens, w.num_kv_heads
        self.sets = []
        for i in range(4):
            k, v = self.rows(T, Hkv, w.k_out), self.rows(T, Hkv, w.v_out)
            if variant == "bf16":
                shape = (w.paging.num_pages, Hkv, w.page_size, D)
                cache = (torch.empty(shape, dtype=torch.bfloat16, device=self.dev),
                         torch.empty(shape, dtype=torch.bfloat16, device=self.dev))
            else:
                cache = self.new_cache(w.paging.num_pages, Hkv, w.page_size, kb, 0)
            self.sets.append((cache, k, v))
        self.slots = self.dev_i32(w.all_slots())
        self.desc = K.CacheDesc(D, Hkv, w.page_size, w.paging.num_pages, 0, 0)
        name = "kvrq_bf16_paged_write" if variant == "bf16" else "kv_rotquant_write"
        nbytes = T * (Hkv * 2 * (2 * D + 2 * D) + 4) if variant == "bf16" else self.write_bytes(T, Hkv)
        self.kernels = {name: nbytes}
        self.rate_tokens = {name: T}
        self.tokens_per_step = T
        self.config = {"workload": w.name, "variant": variant, "num_kv_heads": Hkv, "head_dim": D,
                       "tokens_written": T, "page_size": w.page_size, "k_block": kb, "v_block": 0}

    def step_prefill_chunk(self, i, ev):
        K = self.K
        cache, k, v = self.sets[i % len(self.sets)]
        ev[0].record()
        if self.args.variant == "bf16":
            K.kvrq_bf16_paged_write(self.desc, cache[0], cache[1], k, v, self.slots)
        else:
            K.kv_rotquant_write(cache, k, v, self.slots)
        ev[1].record()

    # -- high-concurrency decode: prefix filled untimed; step i writes token L+i, decodes L+i+1
    def setup_qwen3_32b_like_decode(self):
        K, torch, w = self.K, self.torch, self.w
        kb = self.args.k_block if self.args.k_block is not None else w.k_block
        self.kb, self.vb = kb, w.v_block
        S, Hkv, Hq, P = w.num_seqs, w.num_kv_heads, w.num_q_heads, w.page_size
        self.cache = self.new_cache(w.paging.num_pages, Hkv, P, kb, w.v_block)
        chunk = 1 << 16
        all_slots = w.all_slots()
        for s0 in range(0, len(all_slots), chunk):
            sl = all_slots[s0:s0 + chunk]
            K.kv_rotquant_write(self.cache, self.rows(len(sl), Hkv, w.k_out),
                                self.rows(len(sl), Hkv, w.v_out), self.dev_i32(sl))
        n_steps = w.notes["steps"]
        self.new_k = [self.rows(S, Hkv, w.k_out) for _ in range(min(n_steps, 8))]
        self.new_v = [self.rows(S, Hkv, w.v_out) for _ in range(min(n_steps, 8))]
        self.step_slots = [self.dev_i32([w.paging.slots(s, int(L) + i, 1)[0]
                                         for s, L in enumerate(w.seq_lens)]) for i in range(n_steps)]
        self.step_lens = [self.dev_i32(w.seq_lens + i + 1) for i in range(n_steps)]
        self.q = torch.randn((S, Hq, D), generator=self.gen, device=self.dev).to(torch.bfloat16)
        self.tab = self.dev_i32(w.paging.page_table())
        self.maxlen = int(w.seq_lens.max()) + n_steps
        self.out = torch.empty((S, Hq, D), dtype=torch.float32, device=self.dev)
        n = K.kv_int4_paged_decode_workspace(self.cache, S, Hq, self.maxlen, self.args.split_tokens)
        self.ws = torch.zeros(n, dtype=torch.uint8, device=self.dev)
        # timed step i decodes over seq_lens + j + 1 (j = i mod n_steps): the algorithmic bytes
        # and tokens are averaged over exactly the timed steps
        js = [(self.args.warmup + i) % n_steps for i in range(self.args.steps)]
        dec_bytes = float(np.mean([self.decode_bytes(w.seq_lens + j + 1, Hkv, Hq, P) for j in js]))
        attended = float(np.mean([int(w.seq_lens.sum()) + S * (j + 1) for j in js]))
        if self.args.variant == "fused":
            self.kernels = {"kv_int4_paged_decode_step": round(self.write_bytes(S, Hkv) + dec_bytes)}
            self.rate_tokens = {"kv_int4_paged_decode_step": attended}
        else:
            self.kernels = {"kv_rotquant_write": self.write_bytes(S, Hkv),
                            "kv_int4_paged_decode": round(dec_bytes)}
            self.rate_tokens = {"kv_rotquant_write": S, "kv_int4_paged_decode": attended}
        self.tokens_per_step = attended
        self.tokens_by_step = [int(w.seq_lens.sum()) + S * (j + 1) for j in range(n_steps)]
        self.n_steps_max = n_steps
        self.config = {"workload": w.name, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
                       "num_seqs": S, "tokens_written": S, "tokens_attended_mean": round(attended),
                       "page_size": P, "k_block": kb, "v_block": w.v_block,
                       "variant": "fused" if self.args.variant == "fused" else "write+decode"}

    # -- small-batch decode steps: the same step as the high-concurrency one
    setup_small_batch_decode = setup_qwen3_32b_like_decode

    def step_qwen3_32b_like_decode(self, i, ev):
        K = self.K
        j = i % self.n_steps_max
        if self.args.variant == "fused":
            ev[0].record()
            K.kv_int4_paged_decode_step(self.cache, self.new_k[j % len(self.new_k)],
                                        self.new_v[j % len(self.new_v)], self.step_slots[j], self.q,
                                        self.tab, self.step_lens[j], self.maxlen, out=self.out,
                                        split_tokens=self.args.split_tokens, workspace=self.ws)
            ev[1].record()
            return
        ev[0].record()
        K.kv_rotquant_write(self.cache, self.new_k[j % len(self.new_k)], self.new_v[j % len(self.new_v)],
                            self.step_slots[j])
        ev[1].record()
        K.kv_int4_paged_decode(self.cache, self.q, self.tab, self.step_lens[j], self.maxlen,
                               out=self.out, split_tokens=self.args.split_tokens, workspace=self.ws)
        ev[2].record()

    def step_small_batch_decode(self, i, ev):
        self.step_qwen3_32b_like_decode(i, ev)

    # -- long context: 64 chunk writes + one decode
    def setup_long_context(self):
        K, torch, w = self.K, self.torch, self.w
        Hkv, Hq, P, C = w.num_kv_heads, w.num_q_heads, w.page_size, w.notes["chunk"]
        self.kb, self.vb = w.k_block, w.v_block
        L = w.total_tokens
        self.cache = self.new_cache(w.paging.num_pages, Hkv, P, w.k_block, w.v_block)
        self.chunks_k = [self.rows(C, Hkv, w.k_out) for _ in range(4)]
        self.chunks_v = [self.rows(C, Hkv, w.v_out) for _ in range(4)]
        self.chunk_slots = [self.dev_i32(w.paging.slots(0, c * C, C)) for c in range(L // C)]
        self.q = torch.randn((1, Hq, D), generator=self.gen, device=self.dev).to(torch.bfloat16)
        self.tab = self.dev_i32(w.paging.page_table())
        self.lens = self.dev_i32([L])
        self.out = torch.empty((1, Hq, D), dtype=torch.float32, device=self.dev)
        n = K.kv_int4_paged_decode_workspace(self.cache, 1, Hq, L, self.args.split_tokens)
        self.ws = torch.zeros(n, dtype=torch.uint8, device=self.dev)
        self.kernels = {"kv_rotquant_write": self.write_bytes(C, Hkv),
                        "kv_int4_paged_decode": self.decode_bytes([L], Hkv, Hq, P)}
        self.launch_count = {"kv_rotquant_write": L // C, "kv_int4_paged_decode": 1}
        self.rate_tokens = {"kv_rotquant_write": C, "kv_int4_paged_decode": L}
        self.tokens_per_step = L
        self.config = {"workload": w.name, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
                       "context": L, "chunk": C, "page_size": P, "k_block": w.k_block,
                       "v_block": w.v_block}

    def step_long_context(self, i, ev):
        K = self.K
        ev[0].record()
        for c, sl in enumerate(self.chunk_slots):
            K.kv_rotquant_write(self.cache, self.chunks_k[c % 4], self.chunks_v[c % 4], sl)
        ev[1].record()
        K.kv_int4_paged_decode(self.cache, self.q, self.tab, self.lens, int(self.w.total_tokens),
                               out=self.out, split_tokens=self.args.split_tokens, workspace=self.ws)
        ev[2].record()

    # -- chunked prefill: prefixes written untimed; a step writes every sequence's chunk and
    #    runs the causal extend of the chunk rows over prefix + chunk
    def setup_chunked_prefill(self):
        K, torch, w = self.K, self.torch, self.w
        kb = self.args.k_block if self.args.k_block is not None else w.k_block
        self.kb, self.vb = kb, w.v_block
        S, Hkv, Hq, P = w.num_seqs, w.num_kv_heads, w.num_q_heads, w.page_size
        C, prefix = w.notes["chunk"], w.notes["prefix"]
        self.cache = self.new_cache(w.paging.num_pages, Hkv, P, kb, w.v_block)
        pre = np.concatenate([w.paging.slots(s, 0, int(L)) for s, L in enumerate(prefix)])
        for s0 in range(0, len(pre), 1 << 16):
            sl = pre[s0:s0 + (1 << 16)]
            K.kv_rotquant_write(self.cache, self.rows(len(sl), Hkv, w.k_out),
                                self.rows(len(sl), Hkv, w.v_out), self.dev_i32(sl))
        T = S * C
        self.sets = [(self.rows(T, Hkv, w.k_out), self.rows(T, Hkv, w.v_out),
                      torch.randn((T, Hq, D), generator=self.gen, device=self.dev).to(torch.bfloat16))
                     for _ in range(2)]
        self.slots = self.dev_i32(np.concatenate([w.paging.slots(s, int(L), C)
                                                  for s, L in enumerate(prefix)]))
        self.qo = self.dev_i32(np.arange(S + 1) * C)
        self.tab = self.dev_i32(w.paging.page_table())
        self.lens = self.dev_i32(w.seq_lens)
        self.maxlen = int(w.seq_lens.max())
        self.out = torch.empty((T, Hq, D), dtype=torch.float32, device=self.dev)
        n = K.kv_int4_paged_extend_workspace(self.cache, S, Hq, T, C, self.maxlen, self.args.split_tokens)
        self.ws = torch.zeros(n, dtype=torch.uint8, device=self.dev)
        # attended (row, key) pairs: row i of a chunk at position prefix + i sees prefix + i + 1
        pairs = int(sum(C * int(L) + C * (C + 1) // 2 for L in prefix))
        self.kernels = {"kv_rotquant_write": self.write_bytes(T, Hkv),
                        "kv_int4_paged_extend": int(w.seq_lens.sum() * Hkv * self.kv_row_bytes()
                                                    + T * Hq * (2 * D + 4 * D)
                                                    + np.ceil(w.seq_lens / P).sum() * 4)}
        # QK^T and PV: 2 D flops each per (row, head, key)
        self.kernel_flops = {"kv_int4_paged_extend": pairs * Hq * 4 * D}
        self.rate_tokens = {"kv_rotquant_write": T, "kv_int4_paged_extend": T}
        self.tokens_per_step = T
        self.unit = "prefill tokens/s"
        self.config = {"workload": w.name, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
                       "num_seqs": S, "chunk": C, "prefix_tokens": int(prefix.sum()),
                       "attended_pairs": pairs, "page_size": P, "k_block": kb, "v_block": w.v_block}

    def step_chunked_prefill(self, i, ev):
        K = self.K
        k, v, q = self.sets[i % len(self.sets)]
        C = self.w.notes["chunk"]
        ev[0].record()
        K.kv_rotquant_write(self.cache, k, v, self.slots)
        ev[1].record()
        K.kv_int4_paged_extend(self.cache, q, self.qo, self.tab, self.lens, self.maxlen, C,
                               out=self.out, split_tokens=self.args.split_tokens, workspace=self.ws)
        ev[2].record()

    # -- tiny
    def setup_tiny(self):
        K, torch, w = self.K, self.torch, self.w
        self.kb, self.vb = w.k_block, w.v_block
        k, v = w.kv()
        self.cache = K.PagedInt4Cache(w.paging.num_pages, 1, 16, 128, 128)
        self.k = torch.from_numpy(k.view(np.int16)).view(torch.bfloat16).to(self.dev)
        self.v = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).to(self.dev)
        self.q = torch.from_numpy(w.q().view(np.int16)).view(torch.bfloat16).to(self.dev)
        self.slots = self.dev_i32(w.all_slots())
        self.tab = self.dev_i32(w.paging.page_table())
        self.lens = self.dev_i32(w.seq_lens)
        self.kernels = {"kv_rotquant_write": self.write_bytes(64, 1),
                        "kv_int4_paged_decode": self.decode_bytes([64], 1, 1, 16)}
        self.rate_tokens = {"kv_rotquant_write": 64, "kv_int4_paged_decode": 64}
        self.tokens_per_step = 64
        self.config = {"workload": w.name, "num_q_heads": 1, "num_kv_heads": 1, "head_dim": D,
                       "tokens_written": 64, "tokens_attended": 64, "page_size": 16,
                       "k_block": 128, "v_block": 128}

    def step_tiny(self, i, ev):
        K = self.K
        ev[0].record()
        K.kv_rotquant_write(self.cache, self.k, self.v, self.slots)
        ev[1].record()
        K.kv_int4_paged_decode(self.cache, self.q, self.tab, self.lens, 64)
        ev[2].record()

    def step(self, i, ev):
        getattr(self, "step_" + self.args.workload)(i, ev)


class _NoEvent:
    def record(self):
        pass


def measure_graph(s, args, torch):
    """The decode step replayed from a HIP graph: the workload's distinct steps (write +
    decode, or the fused step) recorded once into one torch.cuda.CUDAGraph on the current
    stream, after an eager warm-up, then replayed until about ``args.steps`` steps have run;
    wall clock between two device synchronisations.  Each step's kernels are the eager
    ones; what the graph removes is the host's per-call launch overhead."""
    if not hasattr(s, "tokens_by_step"):
        return {"skipped": "graph replay covers the decode-step workloads"}
    n = s.n_steps_max
    noev = [_NoEvent()] * 3
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for j in range(n):
            s.step(j, noev)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for j in range(n):
            s.step(j, noev)
    torch.cuda.synchronize()
    reps = max(1, round(args.steps / n))
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    steps = reps * n
    tokens = float(np.mean(s.tokens_by_step))
    return {"recorded_steps": n, "replays": reps, "steps": steps,
            "ms_per_step": round(el / steps * 1e3, 4),
            "value": round(tokens * steps / el, 1), "unit": "KV tokens/s"}


# ------------------------------------------------------------------ CPU oracle baseline
def cpu_baseline(args):
    """Time the oracle (as it stands) on a bounded sample of the same workload, in the unit of
    ``value``: KV tokens attended per second of write + decode (tokens written per second for
    the write-only workload, prefill tokens per second for the extend)."""
    import oracle
    oracle.build(force=False)
    cores = oracle.set_threads(args.cpu_threads or len(os.sched_getaffinity(0)))
    w = W.WORKLOADS[args.workload]()
    kb = args.k_block if args.k_block is not None else w.k_block
    if args.workload == "prefill_chunk" and args.variant == "plain":
        kb = 0
    rng = w.rng(77)
    threads = f"OMP threads={cores}"
    if args.workload == "chunked_prefill":
        return cpu_baseline_extend(args, w, kb, rng, cores, threads)
    if args.workload in ("qwen3_32b_like_decode", "small_batch_decode"):
        return cpu_baseline_steps(args, w, kb, rng, cores, threads)
    # sample: up to 8 sequences (long context: 65536 tokens) of the workload's own shapes
    if args.workload == "long_context":
        lens = np.array([65536])
    else:
        lens = w.seq_lens[:8]
    paging = W.assign_pages(rng, list(lens), w.page_size)
    T = int(lens.sum())
    k = W.make_rows(rng, T, w.num_kv_heads, w.k_out)
    v = W.make_rows(rng, T, w.num_kv_heads, w.v_out)
    slots = np.concatenate([paging.slots(s, 0, int(L)) for s, L in enumerate(lens)])
    q = W.f32_to_bf16_bits(rng.standard_normal((len(lens), w.num_q_heads, D)).astype(np.float32))
    tab = paging.page_table()
    decode = args.workload != "prefill_chunk"
    reps, t_total, tokens = 0, 0.0, 0
    while t_total < args.cpu_seconds and reps < 1000:
        cache = oracle.Cache(paging.num_pages, w.num_kv_heads, w.page_size, k_bits=args.k_bits,
                             v_bits=args.v_bits)
        t0 = time.perf_counter()
        oracle.write(cache, k, v, slots, kb, w.v_block)
        if decode:
            oracle.decode(q, (cache.k_codes, cache.v_codes, cache.k_params, cache.v_params), tab,
                          lens.astype(np.int32), w.num_kv_heads, w.page_size, kb, w.v_block)
        t_total += time.perf_counter() - t0
        tokens += T       # each token written once and (with a decode) attended once
        reps += 1
    what = f"{reps} x (write {T} tokens" + (f" + decode {len(lens)} sequences)" if decode else ")")
    return {"value": tokens / t_total, "unit": "KV tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{what}, {args.workload} shapes, {threads}", "seconds": round(t_total, 3)}


def cpu_baseline_steps(args, w, kb, rng, cores, threads):
    """Decode steps on a sample of the workload's sequences (their prefixes written untimed):
    each timed rep writes one new token per sampled sequence and decodes the sampled sequences
    over it, as a GPU step does for all of them."""
    import oracle
    lens = w.seq_lens[:8].astype(np.int64)
    steps = 4 * int(w.notes["steps"])    # cap on timed reps; the time target normally ends it
    paging = W.assign_pages(rng, [int(L) + steps for L in lens], w.page_size)
    cache = oracle.Cache(paging.num_pages, w.num_kv_heads, w.page_size, k_bits=args.k_bits,
                         v_bits=args.v_bits)
    for s, L in enumerate(lens):
        oracle.write(cache, W.make_rows(rng, int(L), w.num_kv_heads, w.k_out),
                     W.make_rows(rng, int(L), w.num_kv_heads, w.v_out), paging.slots(s, 0, int(L)),
                     kb, w.v_block)
    q = W.f32_to_bf16_bits(rng.standard_normal((len(lens), w.num_q_heads, D)).astype(np.float32))
    tab = paging.page_table()
    reps, t_total, tokens = 0, 0.0, 0
    while t_total < args.cpu_seconds and reps < steps:
        k = W.make_rows(rng, len(lens), w.num_kv_heads, w.k_out)
        v = W.make_rows(rng, len(lens), w.num_kv_heads, w.v_out)
        slots = np.array([paging.slots(s, int(L) + reps, 1)[0] for s, L in enumerate(lens)], np.int32)
        cur = (lens + reps + 1).astype(np.int32)
        t0 = time.perf_counter()
        oracle.write(cache, k, v, slots, kb, w.v_block)
        oracle.decode(q, (cache.k_codes, cache.v_codes, cache.k_params, cache.v_params), tab, cur,
                      w.num_kv_heads, w.page_size, kb, w.v_block)
        t_total += time.perf_counter() - t0
        tokens += int(cur.sum())
        reps += 1
    return {"value": tokens / t_total, "unit": "KV tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{reps} steps x (write 1 token + decode) of {len(lens)} sequences of "
                      f"{args.workload} ({int(lens.sum())} cached tokens), {threads}",
            "seconds": round(t_total, 3)}


def cpu_baseline_extend(args, w, kb, rng, cores, threads):
    """Oracle write of a chunk + causal extend, on the workload's first sequence with a
    256-token chunk (prefix as in the workload)."""
    import oracle
    C = 256
    prefix = int(w.notes["prefix"][0])
    L = prefix + C
    paging = W.assign_pages(rng, [L], w.page_size)
    k = W.make_rows(rng, L, w.num_kv_heads, w.k_out)
    v = W.make_rows(rng, L, w.num_kv_heads, w.v_out)
    slots = paging.slots(0, 0, L)
    q = W.f32_to_bf16_bits(rng.standard_normal((C, w.num_q_heads, D)).astype(np.float32))
    tab = paging.page_table()
    qo = np.array([0, C], np.int32)
    cache = oracle.Cache(paging.num_pages, w.num_kv_heads, w.page_size, k_bits=args.k_bits,
                         v_bits=args.v_bits)
    oracle.write(cache, k[:prefix], v[:prefix], slots[:prefix], kb, w.v_block)   # untimed prefix
    reps, t_total = 0, 0.0
    while t_total < args.cpu_seconds and reps < 1000:
        t0 = time.perf_counter()
        oracle.write(cache, k[prefix:], v[prefix:], slots[prefix:], kb, w.v_block)
        oracle.extend(q, (cache.k_codes, cache.v_codes, cache.k_params, cache.v_params), qo, tab,
                      np.array([L], np.int32), w.num_kv_heads, w.page_size, kb, w.v_block)
        t_total += time.perf_counter() - t0
        reps += 1
    return {"value": reps * C / t_total, "unit": "prefill tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{reps} x (write {C} tokens + extend {C} rows over {L} tokens), "
                      f"chunked_prefill shapes, {threads}",
            "seconds": round(t_total, 3)}


# ------------------------------------------------------------------ counters
def parse_counter_dirs(fetch_dir, write_dir, out_json, profiled_args=""):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) per kernel from two rocprofv3 --pmc
    runs, plus the calibration copy's values, into ``out_json``."""
    import csv
    import glob

    def load(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        acc = {}
        for fn in files:
            with open(fn) as f:
                for row in csv.DictReader(f):
                    if row.get("Counter_Name") != counter:
                        continue
                    name = row.get("Kernel_Name", "")
                    if "kvrq::" not in name:          # torch's set-up kernels are not ours
                        continue
                    acc.setdefault(name, []).append(float(row["Counter_Value"]))
        return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}

    fetch = load(fetch_dir, "FETCH_SIZE")
    write = load(write_dir, "WRITE_SIZE")
    out = {"kernel_hash": kernel_source_hash(), "fetch_kib": {}, "write_kib": {},
           "commands": [f"rocprofv3 --pmc {c} --output-format csv -d <{c}_DIR> -o run -- "
                        f"python bench.py {profiled_args}".rstrip() for c in ("FETCH_SIZE", "WRITE_SIZE")]
           + [f"python bench.py --parse-counters <FETCH_SIZE_DIR> <WRITE_SIZE_DIR> <OUT> "
              f"--profiled-args '{profiled_args}'"]}
    for k, (m, n) in fetch.items():
        out["fetch_kib"][k] = {"mean": m, "dispatches": n}
    for k, (m, n) in write.items():
        out["write_kib"][k] = {"mean": m, "dispatches": n}
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    print(json.dumps(out, indent=1, sort_keys=True))


def traffic_from_counters(path, kernel_symbols, copy_bytes):
    """HBM bytes per launch of the first of ``kernel_symbols`` that the counters summary holds,
    scaled by the plain copy kernel's counter-to-byte factor; None if absent or taken on other
    kernel sources."""
    if not path or not os.path.exists(path):
        return None, None
    with open(path) as f:
        c = json.load(f)
    if c.get("kernel_hash") != kernel_source_hash():
        return None, "stale"

    def pick(table, sub):
        for name, v in table.items():
            if sub in name:
                return v["mean"]
        return None

    f_k = w_k = None
    for sym in kernel_symbols:
        f_k, w_k = pick(c["fetch_kib"], sym), pick(c["write_kib"], sym)
        if f_k is not None:
            break
    f_c, w_c = pick(c["fetch_kib"], "device_copy_kernel"), pick(c["write_kib"], "device_copy_kernel")
    if None in (f_k, w_k, f_c, w_c):
        return None, "incomplete"
    fetch_factor = copy_bytes / (f_c * 1024.0)      # true bytes per counted byte (reads)
    write_factor = copy_bytes / (w_c * 1024.0)
    return f_k * 1024.0 * fetch_factor + w_k * 1024.0 * write_factor, \
        {"fetch_factor": fetch_factor, "write_factor": write_factor}


# ------------------------------------------------------------------ ceilings
def measure_ceilings(torch, K, reps=20):
    """Streaming-read (kvrq_device_read) and plain-copy (kvrq_device_copy) rates at the sizes
    the kernels move per launch: a short kernel pays its ramp-up and drain, so a 134 MB read
    is the fair ceiling of a write that reads 134 MB, not a 2 GiB one.  Between runs a 1 GiB
    read evicts the 256 MB Infinity Cache without leaving dirty lines (a fill would, and their
    write-back would slow the next run).  A copy below ~256 MB is flattered: its writes stay
    in the Infinity Cache and reach HBM only after the kernel ends."""
    big = torch.ones((2 << 30) // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty((1 << 30) // 4, dtype=torch.int32, device="cuda")
    flush = torch.ones((1 << 30) // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")

    def timed(fn):
        ts = []
        for _ in range(reps):
            K.kvrq_device_read(flush, sink)
            e0, e1 = HipEvent(torch), HipEvent(torch)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts)) * 1e-3

    out = {"read": {}, "copy": {}, "reps": reps, "statistic": "median"}
    for mb in (42.5, 85, 134, 170, 268, 1024, 2048):
        n = int(mb * 1e6) // 4096 * 4096
        t = timed(lambda: K.kvrq_device_read(big, sink, nbytes=n))
        out["read"][f"{mb:g}MB"] = {"us": round(t * 1e6, 2), "gbps": round(n / t / 1e9, 1)}
    for mb in (42.5, 85, 134, 512):
        n = int(mb * 1e6) // 4096 * 4096
        t = timed(lambda: K.kvrq_device_copy(dst, big, nbytes=n))
        out["copy"][f"{mb:g}MB"] = {"us": round(t * 1e6, 2), "gbps_rw": round(2 * n / t / 1e9, 1)}
    return out


# ------------------------------------------------------------------ page-gather ceiling
def measure_paged_ceiling(s, torch, K, reps=20):
    """The decode's own pages read in the decode's order (kvrq_paged_read: each sequence's
    page-table entries in order, whole pages of K and V codes and parameters, nothing
    computed) against the decode of the same lengths and a streaming read of as many bytes,
    each timed alone after a 1 GiB read that evicts the Infinity Cache, median of `reps`."""
    w = s.w
    if w.name == "long_context":
        lens = np.array([w.total_tokens], dtype=np.int64)
        maxlen, lens_dev = int(w.total_tokens), s.lens
    elif w.name in ("qwen3_32b_like_decode", "small_batch_decode"):
        lens = w.seq_lens.astype(np.int64) + 1
        maxlen, lens_dev = s.maxlen, s.step_lens[0]
    else:
        raise SystemExit("--paged-ceiling measures the decode workloads (qwen3_32b_like_decode, "
                         "small_batch_decode, long_context)")
    P = w.page_size
    tab = w.paging.page_table()
    pages = np.concatenate([tab[i, :(int(L) + P - 1) // P] for i, L in enumerate(lens)]).astype(np.int32)
    pages_dev = s.dev_i32(pages)
    page_bytes = w.num_kv_heads * P * 136
    read_bytes = int(len(pages)) * page_bytes
    dec_bytes = s.decode_bytes(lens, w.num_kv_heads, w.num_q_heads, P)
    flush = torch.ones((1 << 30) // 4, dtype=torch.int32, device="cuda")
    big = torch.ones(read_bytes // 4 + 1024, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")

    def timed(fn):
        fn()
        ts = []
        for _ in range(reps):
            K.kvrq_device_read(flush, sink)
            e0, e1 = HipEvent(torch), HipEvent(torch)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts)) * 1e-3

    out = {"workload": w.name, "pages": int(len(pages)), "page_bytes": page_bytes,
           "read_bytes": read_bytes, "decode_algorithmic_bytes": int(dec_bytes), "reps": reps,
           "statistic": "median", "paged_read": {}}
    for wg in (1, 2, 3, 4):
        t = timed(lambda: K.kvrq_paged_read(s.cache, pages_dev, sink, wgs_per_cu=wg))
        out["paged_read"][f"{wg}_wgs_per_cu"] = {"us": round(t * 1e6, 2),
                                                 "gbps": round(read_bytes / t / 1e9, 1)}
    # the same bytes per (page, KV head) block as the decode reads them, two workgroups per
    # CU: with the decode's load shapes and two tiles in flight per wave, with whole-line V,
    # and with the decode's shapes and four tiles in flight
    for pat, name in ((1, "decode_shapes"), (2, "decode_blocks_full_line_v"),
                      (3, "decode_shapes_four_tiles")):
        t = timed(lambda: K.kvrq_paged_read(s.cache, pages_dev, sink, wgs_per_cu=2, pattern=pat))
        out["paged_read"][name] = {"us": round(t * 1e6, 2), "gbps": round(read_bytes / t / 1e9, 1)}
    t = timed(lambda: K.kvrq_device_read(big, sink, nbytes=read_bytes // 16 * 16))
    out["streaming_read"] = {"us": round(t * 1e6, 2), "gbps": round(read_bytes / t / 1e9, 1)}
    t = timed(lambda: K.kv_int4_paged_decode(s.cache, s.q, s.tab, lens_dev, maxlen, out=s.out,
                                             split_tokens=s.args.split_tokens, workspace=s.ws))
    out["decode"] = {"us": round(t * 1e6, 2), "algorithmic_gbps": round(dec_bytes / t / 1e9, 1)}
    best = min(v["us"] for v in out["paged_read"].values())
    out["decode_vs_paged_read"] = round(best / out["decode"]["us"], 4)
    out["decode_vs_decode_shapes"] = round(out["paged_read"]["decode_shapes"]["us"] / out["decode"]["us"], 4)
    return out


# ------------------------------------------------------------------ BDR against plain INT4
def measure_bdr_vs_plain(args, torch, K, steps=1000, warmup=1000):
    """The prefill-chunk workload's write (32768 tokens, 8 KV heads, page 64, permuted pages,
    four rotating input sets, back-to-back launches as in `--workload prefill_chunk`) with the
    BDR-128 rotation on K and as plain INT4 (no rotation): the pages' claim is a rotated
    write as fast as the plain one.  Mean HIP-event time per launch over the timed steps of
    each, after as many warm-up steps."""
    out = {"workload": "prefill_chunk", "steps": steps, "warmup": warmup, "statistic": "mean"}
    for variant in ("bdr", "plain"):
        va = argparse.Namespace(**dict(vars(args), workload="prefill_chunk", variant=variant,
                                       k_block=None, k_bits=4, v_bits=4))
        su = Setup(va, K, torch)
        evs = [[HipEvent(torch), HipEvent(torch)] for _ in range(steps)]
        warm = [HipEvent(torch), HipEvent(torch)]
        for i in range(warmup):
            su.step(i, warm)
        for i in range(steps):
            su.step(i, evs[i])
        torch.cuda.synchronize()
        us = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) * 1e3
        nbytes = su.kernels["kv_rotquant_write"]
        out[f"{variant}_k_block"] = su.kb
        out[f"{variant}_us"] = round(us, 2)
        out[f"{variant}_hbm_frac"] = round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
        del su
    out["overhead"] = round(out["bdr_us"] / out["plain_us"] - 1.0, 4)
    return out


# ------------------------------------------------------------------ main
def main():
    args = parse_args()
    if args.parse_counters:
        parse_counter_dirs(*args.parse_counters, profiled_args=args.profiled_args)
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the rotated INT4 KV-cache path shards by KV head or by "
              "sequence with no exchange, and it is measured on a single MI355X only "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2

    import torch
    import int4_kv_cache_rotquant_amd as K
    K.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.ceilings:
        print(json.dumps(measure_ceilings(torch, K)))
        return 0
    s = Setup(args, K, torch)
    torch.cuda.synchronize()
    if args.paged_ceiling:
        print(json.dumps(measure_paged_ceiling(s, torch, K)))
        return 0

    copy_bytes = 1 << 30
    n_ev = 3
    evs = [[HipEvent(torch) for _ in range(n_ev)] for _ in range(args.steps)]
    warm = [HipEvent(torch) for _ in range(n_ev)]
    for i in range(args.warmup):
        s.step(i, warm)
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for i in range(args.steps):
        s.step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    graph = measure_graph(s, args, torch) if args.graph else None

    # the measured copy ceiling, after the timed steps (clocks settled): a plain 1 GiB device
    # copy, median of five; its counter figures also calibrate the HBM byte counters
    src = torch.empty(copy_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        K.kvrq_device_copy(dst, src)
    copy_ms = []
    for _ in range(5):
        e0, e1 = HipEvent(torch), HipEvent(torch)
        e0.record()
        K.kvrq_device_copy(dst, src)
        e1.record()
        torch.cuda.synchronize()
        copy_ms.append(e0.elapsed_time(e1))
    copy_gbps = 2 * copy_bytes / (float(np.median(copy_ms)) * 1e-3) / 1e9
    del src, dst
    # the measured read ceiling: a 2 GiB non-temporal streaming read (kvrq_device_read, eight
    # waves per CU), median of five; the decode is a read-only kernel
    read_bytes = 2 << 30
    rsrc = torch.ones(read_bytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    K.kvrq_device_read(rsrc, sink)
    read_ms = []
    for _ in range(5):
        e0, e1 = HipEvent(torch), HipEvent(torch)
        e0.record()
        K.kvrq_device_read(rsrc, sink)
        e1.record()
        torch.cuda.synchronize()
        read_ms.append(e0.elapsed_time(e1))
    read_gbps = read_bytes / (float(np.median(read_ms)) * 1e-3) / 1e9
    del rsrc, sink

    names = list(s.kernels)
    per_kernel = {}
    for j, name in enumerate(names):
        ms = [evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)]
        launches = getattr(s, "launch_count", {}).get(name, 1)
        mean_ms = float(np.mean(ms)) / launches
        per_kernel[name] = {"mean_us": round(mean_ms * 1e3, 3),
                            "median_us": round(float(np.median(ms)) / launches * 1e3, 3),
                            "algorithmic_bytes": s.kernels[name],
                            "algorithmic_gbps": round(s.kernels[name] / (mean_ms * 1e-3) / 1e9, 1),
                            "launches_per_step": launches}
    flops = getattr(s, "kernel_flops", {})
    for name, f in flops.items():
        per_kernel[name]["algorithmic_flops"] = f
        per_kernel[name]["algorithmic_tflops"] = round(f / (per_kernel[name]["mean_us"] * 1e-6) / 1e12, 1)
    dominant = max(names, key=lambda n: per_kernel[n]["mean_us"] * per_kernel[n]["launches_per_step"])
    dk = per_kernel[dominant]
    # the decode runs either the balanced persistent kernel or the split kernel, whichever
    # the plan chose for the workload; the counters hold the one that ran
    decode_kernels = ("decode_balanced_kernel", "decode_split_kernel")
    symbol = {"kv_rotquant_write": ("rotquant_write_kernel",), "kv_int4_paged_decode": decode_kernels,
              "kv_int4_paged_decode_step": decode_kernels,
              "kv_int4_paged_extend": ("decode_split_kernel",),
              "kvrq_bf16_paged_write": ("bf16_paged_write_kernel",)}[dominant]
    traffic, traffic_note = traffic_from_counters(args.counters, symbol, copy_bytes)
    if dominant in flops:
        # dense attention: QK^T on int8 MFMA (5.0 POP/s), PV on f16 MFMA (2.5 PFLOP/s), half
        # the flops each, so the time at peak is that of 3.33 PFLOP/s
        achieved = dk["algorithmic_tflops"]
        roofline = {"bound": "mfma", "kernel": dominant, "achieved": achieved,
                    "peak": MFMA_ATTENTION_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / MFMA_ATTENTION_PEAK_TFLOPS, 4),
                    "traffic": None if traffic is None else round(traffic), "traffic_note": traffic_note}
    else:
        achieved = dk["algorithmic_gbps"]
        roofline = {"bound": "hbm", "kernel": dominant, "achieved": achieved, "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                    "traffic": None if traffic is None else round(traffic), "traffic_note": traffic_note,
                    "frac_of_copy_probe": round(achieved / copy_gbps, 4),
                    "frac_of_read_probe": round(achieved / read_gbps, 4)}

    ms_per_step = elapsed / args.steps * 1e3
    value = s.tokens_per_step * args.steps / elapsed
    # each kernel's own rate: tokens it writes (write) or attends (decode, extend) per second
    rates = {}
    for name in names:
        pk = per_kernel[name]
        rates[name] = {"tokens_per_launch": round(s.rate_tokens[name]),
                       "tokens_per_s": round(s.rate_tokens[name] / (pk["mean_us"] * 1e-6), 1),
                       "hbm_frac": round(pk["algorithmic_gbps"] / HBM_PEAK_GBPS, 4)}
    result = {
        "metric": "KV tokens/s and achieved HBM GB/s (% of peak) for rotquant write + INT4 decode",
        "value": round(value, 1),
        "unit": getattr(s, "unit", "KV tokens/s"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in; write fp32; decode int8 MFMA (int4 codes x 21-bit query grid, exact "
                 "i32) + f16 MFMA (PV, hi/lo weights), fp32 accumulate; int4 + fp16 cache",
        "data": "synthetic (seeded N(0,1) with outlier channels; no model weights)",
        "config": dict(s.config, **({"k_bits": args.k_bits, "v_bits": args.v_bits}
                                    if (args.k_bits, args.v_bits) != (4, 4) else {})),
        "kernels": per_kernel,
        "rates": rates,
        "roofline": roofline,
        "hbm_gbps_step": round(sum(per_kernel[n]["algorithmic_bytes"] * per_kernel[n]["launches_per_step"]
                                   for n in names) / (ms_per_step * 1e-3) / 1e9, 1),
        "copy_probe_gbps": round(copy_gbps, 1),
        "read_probe_gbps": round(read_gbps, 1),
        "kernel_hash": kernel_source_hash(),
    }
    if graph is not None:
        result["graph"] = graph
    if args.workload == "qwen3_32b_like_decode" or args.bdr_vs_plain:
        # the write-side claim, next to the headline decode step
        result["bdr_vs_plain"] = measure_bdr_vs_plain(args, torch, K)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args)
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
