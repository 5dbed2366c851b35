"""Where the scheme's error against exact attention comes from, per workload.

TEST INFRASTRUCTURE (oracle side only): runs the CPU oracle's attn_breakdown with one
approximation of the scheme switched on at a time -- INT8 Q/K scores, P rounded to its
P.V format, V quantised -- then all of them, and prints relative L1 and cosine against
exact attention on sampled query rows of each workload.

    python -m oracle.error_breakdown [--per-head 8]
"""
from __future__ import annotations

import argparse
import math
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth_inputs as si  # noqa: E402

WORKLOADS = [
    ("tiny (C1)", si.workload("tiny")),
    ("llm_prefill (C2)", si.workload("llm_prefill")),
    ("llm_prefill causal (C2)", si.workload("llm_prefill", causal=True)),
    ("video_dit (C3)", si.workload("video_dit")),
    ("seq_sweep N8192 (C4)", si.workload("seq_sweep")),
    ("gqa D128 (C5)", si.workload("gqa")),
    ("gqa D96 (C5)", si.workload("gqa", D=96)),
]
PARTS = [("Q/K INT8 only", oracle.PART_QK), ("P only", oracle.PART_P), ("V only", oracle.PART_V),
         ("all (the scheme)", oracle.PART_QK | oracle.PART_P | oracle.PART_V)]


def metrics(a, b):
    return float(np.abs(a - b).sum() / np.abs(b).sum()), float(a.ravel() @ b.ravel() / np.linalg.norm(a) /
                                                                  np.linalg.norm(b))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--per-head", type=int, default=8)
    args = ap.parse_args()
    print("| workload | P.V | " + " | ".join(f"{n}: rel L1 / cos" for n, _ in PARTS) + " |")
    print("|---|---|" + "---|" * len(PARTS))
    for name, w in WORKLOADS:
        q, k, v = si.make_qkv(w)
        qf, kf, vf = (oracle.to_hnd_f32(t, w.layout) for t in (q, k, v))
        Q = oracle.quantize(qf, kf, vf, w.pv == "fp8")
        sm = float(np.float32(1 / math.sqrt(w.D)))
        rows = oracle.sample_rows(w.B, w.Hq, w.Nq, per_head=args.per_head, seed=11)
        ex = oracle.attn_exact(qf, kf, vf, w.causal, sm, rows)
        cells = []
        for _, parts in PARTS:
            got = oracle.attn_breakdown(qf, kf, vf, Q, w.causal, sm, rows, parts)
            rl1, cos = metrics(got, ex)
            cells.append(f"{rl1:.4f} / {cos:.6f}")
        print(f"| {name} | {w.pv.upper()} | " + " | ".join(cells) + " |", flush=True)


if __name__ == "__main__":
    main()
