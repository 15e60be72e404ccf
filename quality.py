#!/usr/bin/env python3
"""Synthetic quality ablation of the rotated INT4 paged KV cache on the GPU.

SAW-INT4 reports that naive token-wise INT4 breaks down on keys with outlier channels,
that block-diagonal Hadamard rotation (BDR) recovers the accuracy, that rotating K alone
is the better trade-off, and that a 128 block balances accuracy and speed (wispaper.ai
blog, sections 2 and 4: the core intuition and the ablation bullets).  It leaves open
whether the rotation keeps 2-bit codes accurate, perhaps with mixed widths (section 5,
limitations); the 2-bit rows measure that too.  This harness
measures the same directions without models: for each (K block, V block, outlier
strength) it writes one seeded synthetic K/V set through ``kv_rotquant_write``, decodes
one query per sequence and query head with ``kv_int4_paged_decode``, and compares the
output with exact softmax attention over the unquantised bf16 K and V, computed on the
host in float64 from its plain definition.

    python quality.py [--seqs 8] [--len 2048] [--json]

Prints a markdown table (one row per configuration): the mean and maximum relative L2
error of the attention output over all (sequence, query head) rows.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

D = 128

# (label, K block, V block, K bits, V bits)
ROTATIONS = [
    ("plain INT4", 0, 0, 4, 4),
    ("BDR-16 K", 16, 0, 4, 4),
    ("BDR-32 K", 32, 0, 4, 4),
    ("BDR-64 K", 64, 0, 4, 4),
    ("BDR-128 K", 128, 0, 4, 4),
    ("BDR-128 K+V", 128, 128, 4, 4),
    # the pages' open question (wispaper.ai blog, section 5, limitations): does the
    # rotation keep 2 bits accurate, and does mixing widths help?
    ("plain 2-bit", 0, 0, 2, 2),
    ("BDR-128 K+V 2-bit", 128, 128, 2, 2),
    ("BDR-128 K 4-bit, V 2-bit", 128, 0, 4, 2),
    ("BDR-128 K+V, K 4-bit, V 2-bit", 128, 128, 4, 2),
    ("BDR-128 K 2-bit, V 4-bit", 128, 0, 2, 4),
]

# (label, outlier fraction, low factor, high factor); fraction 0 = none
OUTLIERS = [
    ("none", 0.0, 1.0, 1.0),
    ("2% x U(10,30)", 0.02, 10.0, 30.0),
    ("2% x U(50,100)", 0.02, 50.0, 100.0),
]


def reference_attention(q, k, v, lens, group, sm_scale):
    """Exact softmax attention in float64 from the bf16 inputs.

    q [S][Hq][D], k/v [T][Hkv][D] (sequences back to back), lens [S]; query head g of a
    sequence attends over that sequence's tokens with KV head g // group."""
    S, Hq, _ = q.shape
    out = np.zeros((S, Hq, D), np.float64)
    t0 = 0
    for s in range(S):
        L = int(lens[s])
        ks = k[t0:t0 + L]
        vs = v[t0:t0 + L]
        for g in range(Hq):
            h = g // group
            sc = ks[:, h, :] @ q[s, g] * sm_scale
            p = np.exp(sc - sc.max())
            out[s, g] = (p / p.sum()) @ vs[:, h, :]
        t0 += L
    return out


def run(args):
    import torch
    import int4_kv_cache_rotquant_amd as K
    K.lib()
    rng = np.random.Generator(np.random.PCG64([args.seed, 0]))
    S, L, Hkv, Hq, P = args.seqs, args.len, args.kv_heads, args.q_heads, 16
    group = Hq // Hkv
    lens = np.full(S, L, np.int64)
    paging = W.assign_pages(rng, [L] * S, P)
    slots = torch.from_numpy(np.concatenate([paging.slots(s, 0, L) for s in range(S)])).cuda()
    tab = torch.from_numpy(paging.page_table()).cuda()
    lens_dev = torch.from_numpy(lens.astype(np.int32)).cuda()
    q_bits = W.f32_to_bf16_bits(rng.standard_normal((S, Hq, D)).astype(np.float32))
    q = W.bf16_bits_to_f32(q_bits).astype(np.float64)
    q_dev = torch.from_numpy(q_bits.view(np.int16)).cuda().view(torch.bfloat16)
    sm_scale = 1.0 / math.sqrt(D)
    rows = []
    for o_label, frac, lo, hi in OUTLIERS:
        k_out = W.OutlierSpec.random(rng, Hkv, frac, lo, hi) if frac > 0 else None
        k_bits = W.make_rows(rng, S * L, Hkv, k_out)
        v_bits = W.make_rows(rng, S * L, Hkv)
        ref = reference_attention(q, W.bf16_bits_to_f32(k_bits).astype(np.float64),
                                  W.bf16_bits_to_f32(v_bits).astype(np.float64), lens, group,
                                  sm_scale)
        k_dev = torch.from_numpy(k_bits.view(np.int16)).cuda().view(torch.bfloat16)
        v_dev = torch.from_numpy(v_bits.view(np.int16)).cuda().view(torch.bfloat16)
        for r_label, kb, vb, kbits, vbits in ROTATIONS:
            cache = K.PagedInt4Cache(paging.num_pages, Hkv, P, kb, vb, k_bits=kbits, v_bits=vbits)
            K.kv_rotquant_write(cache, k_dev, v_dev, slots)
            out = K.kv_int4_paged_decode(cache, q_dev, tab, lens_dev, L).double().cpu().numpy()
            num = np.linalg.norm(out - ref, axis=-1)
            den = np.linalg.norm(ref, axis=-1)
            rel = num / den
            row = {"outliers": o_label, "rotation": r_label, "k_block": kb, "v_block": vb,
                   "k_bits": kbits, "v_bits": vbits,
                   "mean_rel_err": float(rel.mean()), "max_rel_err": float(rel.max()),
                   "max_abs_err": float(np.abs(out - ref).max())}
            rows.append(row)
            if args.json:
                print(json.dumps(row), flush=True)
    return rows


def table(rows):
    lines = ["| K outliers | rotation | mean rel. error | max rel. error |", "|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {r['outliers']} | {r['rotation']} | {r['mean_rel_err']:.4f} | "
                     f"{r['max_rel_err']:.4f} |")
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--seqs", type=int, default=8)
    ap.add_argument("--len", type=int, default=2048)
    ap.add_argument("--kv-heads", type=int, default=8)
    ap.add_argument("--q-heads", type=int, default=32)
    ap.add_argument("--seed", type=int, default=20260421 + 7)
    ap.add_argument("--json", action="store_true", help="also print one JSON line per row")
    args = ap.parse_args(argv)
    rows = run(args)
    print(table(rows))
    return 0


if __name__ == "__main__":
    sys.exit(main())
