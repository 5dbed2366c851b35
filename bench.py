#!/usr/bin/env python3
"""Benchmark: SageAttention-style quantized attention forward on one MI355X.

One step = the whole hot path over one batch resident in HBM:
    sage_quant_qkv (K mean, INT8 Q/K, V operand in one call)  ->  sage_attn_fwd.
Metric (the kernel-throughput sweep of the SageAttention pages): effective TOPS =
4*B*H*Nq*Nkv*D / t, halved when causal.  `value` uses the whole step time; the
attention-kernel-only rate (the pages' convention, quantisation excluded) is reported
beside it, with a roofline against the dense INT8/FP8 matrix-core peak.

Workload: B=4, H=32, D=128, bf16 q/k/v ~ N(0,1), HND, INT8 QK^T + FP8-e4m3 P.V with the
"fp16+fp32" accumulation name (on gfx950 the P.V products chain through the fp32
accumulator), non-causal, N=8192 (the sweep covers N = 1K..32K, causal and
non-causal).  Every other workload (tiny, LLM prefill, video DiT, GQA at D128 / D96) is
timed after it, each with its own CPU-oracle baseline.  Prints ONE JSON line on stdout.

    python bench.py [--steps K] [--warmup W] [--n 8192] [--no-sweep] [--no-cpu] [--no-configs]
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective attention TOPS at D=128 vs N (1K–32K); % of INT8/FP8 MFMA peak"
PEAK_TOPS = 5000.0        # MI355X dense INT8 / FP8 matrix-core peak (TOPS)
PEAK_HBM_GBS = 8000.0
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "attn_fwd_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # defaults sized past the ~100 ms over which the shader clock ramps up under load
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--n", type=int, default=8192, help="sequence length of the headline point")
    p.add_argument("--causal", action="store_true", help="headline point causal")
    p.add_argument("--no-sweep", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--sweep-steps", type=int, default=10)
    p.add_argument("--mxfp4", action="store_true", help="time the MXFP4 variant also with --no-sweep")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="also run a plain device copy of this many MiB (HBM counter calibration)")
    p.add_argument("--no-configs", action="store_true", help="skip the per-workload points")
    p.add_argument("--configs-only", action="store_true",
                   help="only the per-workload points (one JSON line with them; for profiling)")
    p.add_argument("--cpu-full", action="store_true",
                   help="CPU baselines of the per-workload points on every query row (minutes)")
    return p.parse_args()


def kernel_source_hash() -> str:
    """Hash of the attention kernel's source with comments and blank lines removed, so
    that profiled counters stay attached to the code they were taken on."""
    h = hashlib.sha256()
    for f in ("attn_fwd.hip", "common.hpp"):
        with open(os.path.join(ROOT, "quantized_attention_04_amd", "csrc", f)) as fh:
            text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines())
        h.update("\n".join(ln for ln in lines if ln).encode())
    return h.hexdigest()[:16]


class Runner:
    """Preallocated buffers for one workload; step() enqueues the three C-ABI calls."""

    def __init__(self, qa, torch, q, k, v, w, gran: str = "block"):
        self.qa, self.torch, self.w, self.gran = qa, torch, w, gran
        self.q, self.k, self.v = q, k, v
        dev = q.device
        L = qa.lib()
        nws = L.sage_quant_qkv_workspace_bytes(w.B, w.Hkv, w.Nkv, w.D, 1 if w.pv == "fp8" else 0)
        self.ws = torch.empty(max(8, nws), dtype=torch.uint8, device=dev)
        self.qk, self.vq = qa.quant_qkv(q, k, v, w.layout, w.pv, workspace=self.ws, gran=gran)
        self.out = qa.attn_fwd(self.qk, self.vq, w.torch_dtype, w.layout, w.causal, None, w.accum)

    def quant(self):
        qa, w = self.qa, self.w
        qa.quant_qkv(self.q, self.k, self.v, w.layout, w.pv, workspace=self.ws, out_qk=self.qk, out_v=self.vq,
                     gran=self.gran)

    def attn(self):
        qa, w = self.qa, self.w
        qa.attn_fwd(self.qk, self.vq, w.torch_dtype, w.layout, w.causal, None, w.accum, out=self.out)

    def step(self):
        self.quant()
        self.attn()

    def time(self, steps: int, warmup: int, ramp_s: float = 0.0):
        """(ms per step, ms per attention launch, ms per quant pair), HIP events on the launch stream.
        ramp_s: before the warmup steps, untimed steps for at least this long (at most 500 steps),
        so that the shader clock has left its idle level whatever the warmup count."""
        torch = self.torch
        if ramp_s > 0:
            t_end = time.perf_counter() + ramp_s
            for _ in range(500):
                self.step()
                torch.cuda.synchronize()
                if time.perf_counter() >= t_end:
                    break
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
               torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for a, b, c in ev:
            a.record()
            self.quant()
            b.record()
            self.attn()
            c.record()
        t1.record()
        torch.cuda.synchronize()
        total = t0.elapsed_time(t1)
        attn = [b.elapsed_time(c) for a, b, c in ev]
        quant = [a.elapsed_time(b) for a, b, c in ev]
        self.attn_min = min(attn)
        return total / steps, sum(attn) / steps, sum(quant) / steps, sorted(attn)[len(attn) // 2]

    def graph_times(self, reps: int = 10, replays: int = 5):
        """(attention ms, quantisation ms, step ms) per call, each from a HIP graph of
        `reps` back-to-back calls replayed `replays` times: GPU time with no host gaps
        between launches (short kernels otherwise wait on the Python wrappers)."""
        return (graph_ms(self.torch, self.attn, reps, replays), graph_ms(self.torch, self.quant, reps, replays),
                graph_ms(self.torch, self.step, reps, replays))

    def fused_q_graph_times(self, reps: int = 10, replays: int = 5):
        """(attention ms, quantisation ms, step ms) of the schedule with Q quantised in the
        attention prologue: sage_quant_kv, then sage_attn_fwd_fused_q (the same codes and
        the same output as the step above), each from a HIP graph as graph_times."""
        qa, w = self.qa, self.w
        if not hasattr(self, "kq"):
            self.kq, self.vq2 = qa.quant_kv(self.k, self.v, w.layout, w.pv, workspace=self.ws)
            self.out2 = qa.attn_fwd_fused_q(self.q, self.kq, self.vq2, w.layout, w.causal, None, w.accum)

        def quant():
            qa.quant_kv(self.k, self.v, w.layout, w.pv, workspace=self.ws, out_k=self.kq, out_v=self.vq2)

        def attn():
            qa.attn_fwd_fused_q(self.q, self.kq, self.vq2, w.layout, w.causal, None, w.accum, out=self.out2)

        def step():
            quant()
            attn()
        return (graph_ms(self.torch, attn, reps, replays), graph_ms(self.torch, quant, reps, replays),
                graph_ms(self.torch, step, reps, replays))

    def time_graph(self, steps: int, warmup: int) -> float:
        """ms per step with the step (same kernels, same buffers) captured once into a HIP
        graph and replayed: the launch rate no longer depends on the Python wrappers."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.step()
        for _ in range(warmup):
            graph.replay()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(steps):
            graph.replay()
        t1.record()
        torch.cuda.synchronize()
        del graph
        return t0.elapsed_time(t1) / steps


def graph_ms(torch, fn, reps: int = 10, replays: int = 5) -> float:
    """ms per call of fn, from a captured HIP graph of `reps` calls (median of `replays`
    timed replays after two warm-up replays)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(reps):
            fn()
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(replays):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        graph.replay()
        t1.record()
        torch.cuda.synchronize()
        ts.append(t0.elapsed_time(t1) / reps)
    del graph
    return sorted(ts)[len(ts) // 2]


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the path has no multi-GPU code "
                                   f"(asked for --gpus {args.gpus}); one GPU's share of a sharded run is the same "
                                   "kernels on fewer heads or sequences"}))
        sys.exit(2)

    import numpy as np
    import torch

    import quantized_attention_04_amd as qa
    import synth_inputs as si

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    qa.lib()
    if args.configs_only:
        print(json.dumps({"configs": config_points(qa, torch, np, si, dev, args)}), flush=True)
        return

    nmax = max([args.n] + ([] if args.no_sweep else list(si.SWEEP_N)))
    base = si.workload("seq_sweep", Nq=nmax, Nkv=nmax)
    # Inputs: the seq_sweep recipe (seeded randn, cast to bf16), drawn on the GPU for
    # speed; shorter sequences are the leading tokens of the longest draw.
    g = torch.Generator(device=dev).manual_seed(base.seed)
    t = time.perf_counter()
    full = [torch.randn(base.B, base.Hq, nmax, base.D, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
            for _ in range(3)]
    torch.cuda.synchronize()
    log(f"[bench] inputs B{base.B} H{base.Hq} N{nmax} D{base.D} drawn in {time.perf_counter() - t:.1f}s")

    if args.calib_copy_mib:
        # a plain copy kernel of known size: its FETCH_SIZE / WRITE_SIZE counters give the
        # scale factor for converting the attention kernel's counters into HBM bytes
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {args.calib_copy_mib} MiB done")
        del src, dst

    def inputs_for(n):
        if n == nmax:
            return full
        return [x[:, :, :n].contiguous() for x in full]

    # ---------------------------------------------------------------- headline point
    w = base.with_(Nq=args.n, Nkv=args.n, causal=args.causal)
    q, k, v = inputs_for(args.n)
    r = Runner(qa, torch, q, k, v, w)
    log(f"[bench] headline {w}")
    # the shader clock ramps up over the first ~100 ms of load: 0.3 s of untimed steps first
    ms_step, ms_attn, ms_quant, ms_attn_med = r.time(args.steps, args.warmup, ramp_s=0.3)
    ms_graph = r.time_graph(args.steps, 5)
    ops = w.ops()
    value = ops / (ms_step * 1e-3) / 1e12
    attn_tops = ops / (ms_attn * 1e-3) / 1e12
    # roofline of the dominant kernel (attention): algorithmic MFMA work per launch =
    # 4*B*H*Nq*Nkv*Dp (halved when causal); Dp = D = 128 here.
    Dp = qa.padded_dim(w.D)
    alg_ops = 4.0 * w.B * w.Hq * w.Nq * w.Nkv * Dp / (2 if w.causal else 1)
    achieved = alg_ops / (ms_attn * 1e-3) / 1e12
    traffic = None
    cycles = None
    src_hash = kernel_source_hash()
    if os.path.exists(PROFILE_TRAFFIC):
        try:
            with open(PROFILE_TRAFFIC) as fh:
                pt = json.load(fh)
            key = f"B{w.B}_H{w.Hq}_N{w.Nq}_D{w.D}_{'causal' if w.causal else 'noncausal'}"
            if pt.get("kernel_source_sha256_16") == src_hash:
                traffic = pt.get("workloads", {}).get(key)
                cycles = pt.get("shader_cycles_per_launch", {}).get(key)
        except (OSError, ValueError):
            traffic = cycles = None
    # quantisation kernels: HBM-bound; algorithmic bytes = one read of q, k, v (bf16)
    # + one write of the int8 / fp8 codes and the scales
    elems = w.B * w.Hq * w.Nq * w.D
    quant_bytes = elems * 2 * 3 + elems * (1 + 1 + 1) + 4 * (2 * w.B * w.Hq * math.ceil(w.Nq / 64) + w.B * w.Hq * Dp)
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+fp8e4m3",
        "data": "synthetic (seeded randn, bf16, drawn on the GPU)",
        "config": {"workload": f"seq_sweep B{w.B} H{w.Hq} N{w.Nq} D{w.D} bf16 HND "
                               f"{'causal' if w.causal else 'non-causal'} INT8-QK FP8-PV fp16+fp32-accum",
                   "B": w.B, "H": w.Hq, "N": w.Nq, "D": w.D, "causal": w.causal, "layout": w.layout,
                   "pv": w.pv, "accum": w.accum},
        # the same step replayed from a captured HIP graph (no Python between launches)
        "graph_ms_per_step": round(ms_graph, 4),
        "graph_step_tops": round(ops / (ms_graph * 1e-3) / 1e12, 2),
        "attn_kernel_tops": round(attn_tops, 2),
        "attn_kernel_ms": round(ms_attn, 4),
        "attn_kernel_ms_median": round(ms_attn_med, 4),
        "attn_kernel_ms_min": round(r.attn_min, 4),
        "quant_ms": round(ms_quant, 4),
        "quant_GBps": round(quant_bytes / (ms_quant * 1e-3) / 1e9, 1),
        # dense INT8 (QK^T) + FP8 (P.V) matrix-core operations: tera-operations per second
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TOPS, "unit": "TOP/s",
                     "frac": round(achieved / PEAK_TOPS, 4), "traffic": traffic,
                     "kernel": "attn_fwd_kernel<128, fp8, noncausal, bf16 out>",
                     "alg_ops_per_launch": alg_ops, "kernel_source_sha256_16": src_hash},
    }
    if cycles:
        # the same fraction against 256 CUs x 8192 ops per clock at the clock the launch ran
        # at: the launch's shader cycles come from the counters (GRBM_GUI_ACTIVE / 8 XCDs,
        # hash-checked like traffic) and are a property of the compute-bound kernel, so the
        # time cancels; the clock this box's launches ran at is then cycles / time
        result["roofline"]["frac_per_clock"] = round(alg_ops / (cycles * 256 * 8192), 4)
        result["roofline"]["shader_cycles_per_launch"] = cycles
        result["roofline"]["implied_sclk_ghz"] = round(cycles / (ms_attn * 1e-3) / 1e9, 3)
    log(f"[bench] step {ms_step:.3f} ms  attn {ms_attn:.3f} ms ({attn_tops:.0f} TOPS, "
        f"{100 * achieved / PEAK_TOPS:.1f}% of peak)  quant {ms_quant:.3f} ms")
    del r

    # ---------------------------------------------------------------- per-thread granularity
    # the same workload with one Q scale per token and one K scale per 32 keys
    if not args.no_sweep:
        rt = Runner(qa, torch, q, k, v, w, gran="thread")
        st, at, qt, _ = rt.time(args.sweep_steps, 3)
        result["thread_gran"] = {"workload": "the headline workload with per-token Q and per-32-key K scales",
                                 "step_tops": round(ops / (st * 1e-3) / 1e12, 1),
                                 "attn_tops": round(ops / (at * 1e-3) / 1e12, 1),
                                 "attn_ms": round(at, 4), "quant_ms": round(qt, 4)}
        log(f"[bench] thread granularity: attn {at:.3f} ms = {result['thread_gran']['attn_tops']} TOPS, "
            f"quant {qt:.3f} ms")
        del rt

    # ---------------------------------------------------------------- sweep
    if not args.no_sweep:
        sweep = []
        for causal in (False, True):
            for n in si.SWEEP_N:
                ws = base.with_(Nq=n, Nkv=n, causal=causal)
                qs, ks, vs = inputs_for(n)
                rs = Runner(qa, torch, qs, ks, vs, ws)
                st, _, _, _ = rs.time(args.sweep_steps, 3)  # eager steps (host wrappers between launches)
                at, qt, gt = rs.graph_times()
                fa, fq, fs = rs.fused_q_graph_times()
                o = ws.ops()
                sweep.append({"N": n, "causal": causal, "step_tops": round(o / (gt * 1e-3) / 1e12, 1),
                              "eager_step_tops": round(o / (st * 1e-3) / 1e12, 1),
                              "attn_tops": round(o / (at * 1e-3) / 1e12, 1),
                              "attn_frac_of_peak": round(o / (at * 1e-3) / 1e12 / PEAK_TOPS, 4),
                              "attn_ms": round(at, 4), "quant_ms": round(qt, 4), "step_ms": round(gt, 4),
                              # Q quantised in the attention prologue (sage_quant_kv + sage_attn_fwd_fused_q)
                              "fused_q": {"step_tops": round(o / (fs * 1e-3) / 1e12, 1), "step_ms": round(fs, 4),
                                          "attn_ms": round(fa, 4), "quant_ms": round(fq, 4)}})
                log(f"[bench] sweep N={n} causal={causal}: attn {at:.3f} ms = {sweep[-1]['attn_tops']} TOPS, "
                    f"step {sweep[-1]['step_tops']} TOPS (graph), eager step {sweep[-1]['eager_step_tops']}; "
                    f"fused-Q step {sweep[-1]['fused_q']['step_tops']} TOPS (quant {fq:.3f} ms, attn {fa:.3f} ms)")
                del rs, qs, ks, vs
                torch.cuda.empty_cache()
        result["sweep"] = sweep

    # ---------------------------------------------------------------- packed variable-length batch
    if not args.no_sweep:
        result["varlen"] = varlen_point(qa, torch, np, si, dev, args.sweep_steps)

    # ---------------------------------------------------------------- microscaling FP4 variant
    if not args.no_sweep or args.mxfp4:
        result["mxfp4"] = mxfp4_points(qa, torch, q, k, v, w, args.sweep_steps)

    # ---------------------------------------------------------------- CPU baseline (the oracle, untuned)
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(w, full, np, torch)
    del full, q, k, v
    torch.cuda.empty_cache()

    # ---------------------------------------------------------------- every workload family
    if not args.no_configs:
        result["configs"] = config_points(qa, torch, np, si, dev, args)

    print(json.dumps(result), flush=True)


def varlen_point(qa, torch, np, si, dev, steps):
    """sageattn_varlen on a packed batch: 16 causal prefill sequences of seeded mixed
    lengths (256 .. 8192 tokens), GQA 32/8, D=128, bf16, INT8 QK + FP16 P.V (the
    README's varlen kernel).  Inputs drawn on the GPU."""
    rng = np.random.default_rng(41)
    lens = tuple(int(x) for x in rng.integers(256, 8193, size=16))
    w = si.VarlenWorkload("varlen_prefill", lens, lens, 32, 8, 128, causal=True, pv="fp16", seed=41)
    g = torch.Generator(device=dev).manual_seed(w.seed)
    tq = sum(lens)
    q = torch.randn(tq, w.Hq, w.D, generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn(tq, w.Hkv, w.D, generator=g, device=dev).to(torch.bfloat16)
    v = torch.randn(tq, w.Hkv, w.D, generator=g, device=dev).to(torch.bfloat16)
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device=dev)
    mx = max(lens)
    qk, vq = qa.quant_qkv_varlen(q, k, v, cu, cu, mx, mx, w.pv)
    ws = torch.empty(max(8, qa.lib().sage_quant_qkv_varlen_workspace_bytes(16, w.Hkv, tq, w.D, 0)), dtype=torch.uint8,
                     device=dev)
    out = qa.attn_fwd_varlen(qk, vq, torch.bfloat16, True)

    def quant():
        qa.quant_qkv_varlen(q, k, v, cu, cu, mx, mx, w.pv, workspace=ws, out_qk=qk, out_v=vq)

    def attn():
        qa.attn_fwd_varlen(qk, vq, torch.bfloat16, True, out=out)

    for _ in range(3):
        quant()
        attn()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for a, b, c in ev:
        a.record()
        quant()
        b.record()
        attn()
        c.record()
    torch.cuda.synchronize()
    at = sum(b.elapsed_time(c) for a, b, c in ev) / steps
    st = sum(a.elapsed_time(c) for a, b, c in ev) / steps
    # sageattn_varlen's own schedule: Q quantised in the attention prologue, graph-timed
    kq, vq2 = qa.quant_kv_varlen(k, v, cu, mx, w.pv, workspace=ws)
    out2 = torch.empty_like(q)

    def fstep():
        qa.quant_kv_varlen(k, v, cu, mx, w.pv, workspace=ws, out_k=kq, out_v=vq2)
        qa.attn_fwd_varlen_fused_q(q, cu, mx, kq, vq2, True, out=out2)
    fs = graph_ms(torch, fstep, reps=3, replays=3)
    ops = w.ops()
    res = {"workload": f"{w.name}: 16 causal sequences, {tq} tokens (lengths {min(lens)}..{max(lens)}), "
                       f"H{w.Hq}/{w.Hkv} D{w.D} bf16 INT8-QK FP16-PV",
           "attn_tops": round(ops / (at * 1e-3) / 1e12, 1), "attn_ms": round(at, 4),
           "step_tops": round(ops / (st * 1e-3) / 1e12, 1), "step_ms": round(st, 4),
           "fused_q_step_tops": round(ops / (fs * 1e-3) / 1e12, 1), "fused_q_step_ms": round(fs, 4)}
    log(f"[bench] varlen: attn {at:.3f} ms = {res['attn_tops']} TOPS, step {res['step_tops']} TOPS, "
        f"fused-Q step {res['fused_q_step_tops']} TOPS")
    return res


MXFP4_PEAK_TOPS = 10100.0  # dense FP4 matrix-core peak of MI355X


def mxfp4_points(qa, torch, q, k, v, w, steps):
    """The microscaling FP4 variant (quant_mxfp4 + attn_fwd_mxfp4, preallocated) on the
    headline workload, non-causal and causal; HIP events on the launch stream."""
    L = qa.lib()
    ws = torch.empty(max(8, L.sage_quant_mxfp4_workspace_bytes(w.B, w.Hkv, w.Nkv, w.D)), dtype=torch.uint8,
                     device=q.device)
    mq = qa.quant_mxfp4(q, k, v, w.layout, workspace=ws)
    out = torch.empty_like(q)
    res = {"workload": f"B{w.B} H{w.Hq} N{w.Nq} D{w.D} bf16 HND, MXFP4 Q/K/V/P (blocks of 32, E8M0 scales)",
           "peak_tops_fp4": MXFP4_PEAK_TOPS, "points": []}
    for causal in (False, True):
        wc = w.with_(causal=causal)

        def quant():
            qa.quant_mxfp4(q, k, v, w.layout, workspace=ws, out=mq)

        def attn():
            qa.attn_fwd_mxfp4(mq, w.torch_dtype, w.layout, causal, None, out=out)

        for _ in range(3):
            quant()
            attn()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for a, b, c in ev:
            a.record()
            quant()
            b.record()
            attn()
            c.record()
        torch.cuda.synchronize()
        at = sum(b.elapsed_time(c) for a, b, c in ev) / steps
        qt = sum(a.elapsed_time(b) for a, b, c in ev) / steps
        o = wc.ops()
        # Q quantised in the attention prologue (quant_mxfp4_kv + attn_fwd_mxfp4_fused_q), graph-timed
        mk = qa.quant_mxfp4_kv(k, v, w.layout, workspace=ws)
        out2 = torch.empty_like(q)

        def fstep():
            qa.quant_mxfp4_kv(k, v, w.layout, workspace=ws, out=mk)
            qa.attn_fwd_mxfp4_fused_q(q, mk, w.layout, causal, None, out=out2)
        fs = graph_ms(torch, fstep, reps=3, replays=3)
        res["points"].append({"causal": causal, "attn_ms": round(at, 4), "quant_ms": round(qt, 4),
                              "attn_tops": round(o / (at * 1e-3) / 1e12, 1),
                              "step_tops": round(o / ((at + qt) * 1e-3) / 1e12, 1),
                              "attn_frac_of_fp4_peak": round(o / (at * 1e-3) / 1e12 / MXFP4_PEAK_TOPS, 4),
                              "fused_q_step_ms": round(fs, 4), "fused_q_step_tops": round(o / (fs * 1e-3) / 1e12, 1)})
        log(f"[bench] mxfp4 causal={causal}: attn {at:.3f} ms = {res['points'][-1]['attn_tops']} TOPS, "
            f"quant {qt:.3f} ms; fused-Q step {fs:.3f} ms = {res['points'][-1]['fused_q_step_tops']} TOPS")
    return res


def cpu_baseline(w, full, np, torch):
    """Time the CPU oracle (emulation mode) on a bounded sample of the headline workload:
    quantisation of the full tensors plus attention for sampled query rows, extrapolated
    linearly in rows to the whole step."""
    import oracle
    n = w.Nq
    t = time.perf_counter()
    qf, kf, vf = (np.ascontiguousarray(x[:, :, :n].float().cpu().numpy()) for x in full)
    log(f"[cpu] host copies {time.perf_counter() - t:.1f}s; oracle threads {oracle.threads()}")
    t = time.perf_counter()
    Q = oracle.quantize(qf, kf, vf, w.pv == "fp8")
    t_quant = time.perf_counter() - t
    sm = float(np.float32(1 / math.sqrt(w.D)))
    # calibrate, then size the sample to ~15 s of attention work
    probe = oracle.sample_rows(w.B, w.Hq, n, per_head=4, seed=7)
    t = time.perf_counter()
    oracle.attn_emulate(Q, w.causal, sm, probe)
    per_row = (time.perf_counter() - t) / len(probe)
    per_head = int(max(8, min(n, 15.0 / max(per_row, 1e-9) / (w.B * w.Hq))))
    rows = oracle.sample_rows(w.B, w.Hq, n, per_head=per_head, seed=8)
    t = time.perf_counter()
    oracle.attn_emulate(Q, w.causal, sm, rows)
    t_rows = time.perf_counter() - t
    total_rows = w.B * w.Hq * n
    t_full = t_quant + t_rows * total_rows / len(rows)
    val = w.ops() / t_full / 1e12
    log(f"[cpu] quant {t_quant:.2f}s, {len(rows)} rows in {t_rows:.2f}s -> full step ~{t_full:.0f}s")
    return {"value": round(val, 6), "unit": "TOPS", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"emulation-mode oracle: full quantisation ({t_quant:.2f}s) + {len(rows)} of {total_rows} "
                      f"query rows ({t_rows:.2f}s), extrapolated linearly in rows to one whole step "
                      f"({t_full:.1f}s)",
            "seconds_measured": round(t_quant + t_rows, 2), "cpu_model": cpu_model()}


# The other workloads the benchmark sweep stands beside (seeded host inputs, the same
# bytes the parity tests use).  Ceiling in effective TOPS: with FP16 P.V the P.V half
# runs at the FP16 matrix rate (half the INT8/FP8 rate), so at most 2/3 of the 5.0 POPS
# peak; a padded head dim (96 -> 128) spends uncounted work on the padding.
CONFIGS = [
    ("tiny B1 H2 N256 D64 fp16 HND non-causal FP16-PV", "tiny", {}, 2 / 3),
    ("llm_prefill B1 H8 N2048 D128 fp16 HND non-causal FP16-PV", "llm_prefill", {}, 2 / 3),
    ("llm_prefill B1 H8 N2048 D128 fp16 HND causal FP16-PV", "llm_prefill", {"causal": True}, 2 / 3),
    ("video_dit B1 H24 N17776 D64 bf16 NHD non-causal FP8-PV (K channel offset)", "video_dit", {}, 1.0),
    ("gqa B2 H32/8 N8192 D128 bf16 NHD causal FP16-PV", "gqa", {}, 2 / 3),
    ("gqa B2 H32/8 N8192 D96 (padded to 128) bf16 NHD causal FP16-PV", "gqa", {"D": 96}, 0.5),
]


def config_points(qa, torch, np, si, dev, args):
    """Per workload: attention (with the library's key-range split choice, as sageattn
    does), quantisation and the whole step timed from HIP graphs of back-to-back calls,
    effective TOPS,
    fraction of the 5.0 POPS peak and of the P.V mode's ceiling, quantisation GB/s, and
    the CPU oracle on the machine's host (every row for the small workloads, a bounded
    sample extrapolated in rows for the large ones)."""
    import oracle
    out = []
    for label, fam, kw, ceil in CONFIGS:
        w = si.workload(fam, **kw)
        q, k, v = si.make_qkv(w)
        dq, dk, dv = (t.to(dev) for t in (q, k, v))
        L = qa.lib()
        ws = torch.empty(max(8, L.sage_quant_qkv_workspace_bytes(w.B, w.Hkv, w.Nkv, w.D, 1 if w.pv == "fp8" else 0)),
                         dtype=torch.uint8, device=dev)
        qk, vq = qa.quant_qkv(dq, dk, dv, w.layout, w.pv, workspace=ws)
        splits = qa.split_choice(qk, w.pv, w.causal)
        aws = torch.empty(max(16, qa.split_workspace_bytes(qk, splits)), dtype=torch.uint8, device=dev)
        o = qa.attn_fwd(qk, vq, w.torch_dtype, w.layout, w.causal, None, w.accum, splits=splits, workspace=aws)

        def quant():
            qa.quant_qkv(dq, dk, dv, w.layout, w.pv, workspace=ws, out_qk=qk, out_v=vq)

        def attn():
            qa.attn_fwd(qk, vq, w.torch_dtype, w.layout, w.causal, None, w.accum, out=o, splits=splits, workspace=aws)

        def step():
            quant()
            attn()

        # without a split, sageattn's schedule: Q quantised in the attention prologue
        if splits == 1:
            kq, vq2 = qa.quant_kv(dk, dv, w.layout, w.pv, workspace=ws)
            o2 = qa.attn_fwd_fused_q(dq, kq, vq2, w.layout, w.causal, None, w.accum)

        def fstep():
            qa.quant_kv(dk, dv, w.layout, w.pv, workspace=ws, out_k=kq, out_v=vq2)
            qa.attn_fwd_fused_q(dq, kq, vq2, w.layout, w.causal, None, w.accum, out=o2)

        t_end = time.perf_counter() + 0.2
        while time.perf_counter() < t_end:
            step()
            torch.cuda.synchronize()
        # GPU time per call from HIP graphs of back-to-back calls (these launches are short
        # enough that host wrappers between eager launches would show in the timings)
        at = graph_ms(torch, attn)
        qt = graph_ms(torch, quant)
        stp = graph_ms(torch, step)
        fst = graph_ms(torch, fstep) if splits == 1 else None
        ops = w.ops()
        Dp = qa.padded_dim(w.D)
        elems_q, elems_kv = w.B * w.Hq * w.Nq * w.D, w.B * w.Hkv * w.Nkv * w.D
        qbytes = (elems_q + 2 * elems_kv) * 2 + elems_q + elems_kv + elems_kv * (1 if w.pv == "fp8" else 2) + 4 * (
            w.B * w.Hq * math.ceil(w.Nq / 64) + w.B * w.Hkv * math.ceil(w.Nkv / 64) + w.B * w.Hkv * (Dp + w.D))
        tops = ops / (at * 1e-3) / 1e12
        pt = {"workload": label, "attn_ms_median": round(at, 4), "attn_tops": round(tops, 1),
              "attn_frac_of_peak": round(tops / PEAK_TOPS, 4), "mode_ceiling_frac": round(ceil, 4),
              "attn_frac_of_mode_ceiling": round(tops / (PEAK_TOPS * ceil), 4),
              "key_range_splits": splits, "quant_ms_median": round(qt, 4),
              "quant_GBps": round(qbytes / (qt * 1e-3) / 1e9, 1),
              "step_ms": round(stp, 4), "step_tops": round(ops / (stp * 1e-3) / 1e12, 1),
              "fused_q_step_ms": None if fst is None else round(fst, 4),
              "fused_q_step_tops": None if fst is None else round(ops / (fst * 1e-3) / 1e12, 1)}
        log(f"[bench] {label}: attn {at * 1e3:.1f} us = {tops:.1f} TOPS ({100 * tops / PEAK_TOPS:.1f}% of peak, "
            f"{100 * pt['attn_frac_of_mode_ceiling']:.1f}% of the mode ceiling), splits {splits}, "
            f"quant {qt * 1e3:.1f} us = {pt['quant_GBps']} GB/s, step {stp * 1e3:.1f} us"
            + ("" if fst is None else f", fused-Q step {fst * 1e3:.1f} us"))
        del dq, dk, dv, qk, vq, o, ws, aws
        if splits == 1:
            del kq, vq2, o2
        torch.cuda.empty_cache()
        if not args.no_cpu:
            pt["cpu_baseline"] = config_cpu_baseline(oracle, np, w, q, k, v, full=args.cpu_full)
        out.append(pt)
    return out


def config_cpu_baseline(oracle, np, w, q, k, v, full: bool):
    """The emulation-mode oracle on the host: full quantisation, then attention on every
    query row when that is at most ~2e10 multiply-adds (or --cpu-full), else on a seeded
    sample sized to ~3 s and extrapolated linearly in rows."""
    t = time.perf_counter()
    qf, kf, vf = (oracle.to_hnd_f32(x, w.layout) for x in (q, k, v))
    Q = oracle.quantize(qf, kf, vf, w.pv == "fp8")
    t_quant = time.perf_counter() - t
    sm = float(np.float32(1 / math.sqrt(w.D)))
    total_rows = w.B * w.Hq * w.Nq
    macs = 2.0 * total_rows * w.Nkv * w.D / (2 if w.causal else 1)
    if full or macs <= 2e10:
        rows = oracle.all_rows(w.B, w.Hq, w.Nq)
        kind = "every query row"
    else:
        probe = oracle.sample_rows(w.B, w.Hq, w.Nq, per_head=2, seed=7)
        t = time.perf_counter()
        oracle.attn_emulate(Q, w.causal, sm, probe)
        per_row = (time.perf_counter() - t) / len(probe)
        per_head = int(max(4, min(w.Nq, 3.0 / max(per_row, 1e-9) / (w.B * w.Hq))))
        rows = oracle.sample_rows(w.B, w.Hq, w.Nq, per_head=per_head, seed=8)
        kind = "sampled rows, extrapolated"
    t = time.perf_counter()
    oracle.attn_emulate(Q, w.causal, sm, rows)
    t_rows = time.perf_counter() - t
    t_full = t_quant + t_rows * total_rows / len(rows)
    return {"value": round(w.ops() / t_full / 1e12, 6), "unit": "TOPS", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"{kind}: quantisation {t_quant:.2f}s + {len(rows)} of {total_rows} rows {t_rows:.2f}s "
                      f"-> one whole pass {t_full:.1f}s", "cpu_model": cpu_model()}


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), for the oracle baseline."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
