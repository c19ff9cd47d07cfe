#!/usr/bin/env python3
"""Benchmark of the ThriftAttention prefill hot path on one MI355X.

One step = thrift_quantize -> thrift_select -> thrift_attn_fwd over one batch
of seeded synthetic inputs already resident in HBM (default workload: B=1,
Hq=32, Hkv=8, N=131072, d=128, causal, bf16 inputs, FP16 fraction 0.05).

Prints one JSON line:
  value      attention flops of the step (4 d per causally valid query-key
             pair, F = 4 d B Hq N(N+1)/2) / measured step time, in TFLOP/s;
  roofline   the fused attention call thrift_attn_fwd, which is three
             launches on one stream (attn_f16_kernel: FP16 blocks per head;
             attn_fwd_kernel: FP4 blocks per GQA group, finishing each row;
             attn_redo_kernel: exits at once unless an FP4 workgroup flagged
             an overflow): achieved = F / the call's average duration (HIP
             events on its stream), peak = the FP16/MXFP4 MFMA roofline
             weighted by the flops in FP16 and FP4 tiles
             (F16 / 2516.6 TF/s + F4 / 10066 TF/s), traffic = HBM bytes per
             call (all three kernels) from the committed rocprofv3 counter
             summary when it was taken on the current kernel source, else null;
  cpu_baseline  the CPU oracle's attention on a bounded row sample of the
             same workload, on this host's cores;
  kernels    quantize / select / attention times and algorithmic GB/s;
  quality    planted-needle check: error of frac=0.05 and of frac=0 against
             frac=1 (all-FP16) output;
  roofline_alu  the dominant kernel (attn_fwd_kernel, FP4 tiles) against
             the bound it runs into, full-rate VALU issue: 5.5 issue slots per
             FP4 score / its duration (HIP events the library records between
             its kernels), peak 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz;
  alt_rowsum_weights  the attention call under the other row-sum reading
             (thrift_attn_fwd_wsum: normalised by the quantized weights, the
             FP4 row sums from one more MFMA), timed alone over the same
             steps, with its own quality figures;
  alt_rowsum_weights_expfree  the same reading with FP4 P codes taken
             without an exponential (thrift_attn_fwd_ex, rowsum 2).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--frac F]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_F16 = 2516.6  # TFLOP/s, dense FP16 MFMA, MI355X
PEAK_F4 = 10066.0  # TFLOP/s, dense MXFP4 MFMA, MI355X
PEAK_HBM = 8000.0  # GB/s, MI355X HBM3E
# full-rate wave64 VALU issue of the chip: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
# (fp32 vector 157.3 TFLOP/s counts an fma as 2 and packed ops as 2 more)
PEAK_VALU = 256 * 4 * 16 * 2.4e9 / 1e12  # T lane-ops/s
# full-rate VALU issue slots per FP4 score: fma (s*c - M) 1, v_exp_f32 2 (half
# rate), row-sum add 1, group max 1/2 (max3), FP4 convert 1 (half rate, 2 codes)
VALU_SLOTS_PER_FP4_SCORE = 5.5
METRIC = "attention TFLOPs/s at frac=0.05 + % of FP16/MXFP4 MFMA roofline, N=128K"
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "attn_fwd_long_128k_traffic.txt")
ATTN_SRC = os.path.join(ROOT, "fp16_long_context_amd", "csrc", "attn_fwd.hip")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def attn_flops(w) -> float:
    N = w.N
    pairs = N * (N + 1) // 2
    return 4.0 * w.d * w.B * w.Hq * pairs


def fp16_tile_flops(w, n16, frac) -> float:
    """4d x causally valid pairs inside FP16 tiles (diagonal tiles hold 2080)."""
    nb = w.N // 64
    tiles16 = int(n16.sum().item())
    diag16 = w.B * w.Hq * nb if round(frac * 1e6) > 0 else 0  # the diagonal block is always kept in FP16
    return 4.0 * w.d * ((tiles16 - diag16) * 4096 + diag16 * 2080)


def quantize_bytes(w) -> float:
    elems = w.B * (w.Hq + 2 * w.Hkv) * w.N * w.d
    return elems * (2 + 2 + 0.5 + 1 / 32)


def select_bytes(w) -> float:
    nb = w.N // 64
    reads = 2.0 * w.B * (w.Hq + w.Hkv) * w.N * w.d
    lists = 4.0 * w.B * w.Hq * nb * (nb + 1) // 2 + 4.0 * w.B * w.Hq * nb
    return reads + lists


def read_traffic():
    """HBM bytes per attention call (its three kernels) from the committed
    counter summary, if it was measured on the current kernel source."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    txt = open(TRAFFIC_SUMMARY).read()
    m_sha = re.search(r"source_sha256:\s*([0-9a-f]{64})", txt)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not (m_sha and m_b):
        return None
    sha = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
    return float(m_b.group(1)) if sha == m_sha.group(1) else None


def cpu_baseline(x, w, frac, budget_s=12.0):
    """Oracle attention on sampled rows of query head 0 (its lists come from the
    oracle's own quantize/select of that head and its KV head)."""
    import numpy as np

    if "OMP_NUM_THREADS" not in os.environ:
        os.environ["OMP_NUM_THREADS"] = str(len(os.sched_getaffinity(0)))
    import oracle
    from fp16_long_context_amd import synth

    q, k, v = x["q"][:1, :1], x["k"][:1, :1], x["v"][:1, :1]
    dt = "fp16" if w.dtype == "fp16" else "bf16"
    qz = oracle.quantize(synth.bits(q), synth.bits(k), synth.bits(v), dt)
    sel = oracle.select(qz["q16"], qz["k16"], frac, True)
    g = np.random.default_rng(7)
    done_rows, done_flops, t_used = 0, 0.0, 0.0
    n = 16
    while t_used < budget_s:
        rows = g.integers(0, w.N, n)
        t0 = time.perf_counter()
        oracle.attn_rows(qz, sel, rows, True)
        dt_s = time.perf_counter() - t0
        t_used += dt_s
        done_rows += n
        done_flops += float(4.0 * w.d * (rows + 1).sum())
        rate = dt_s / n
        n = int(max(16, min(4096, (budget_s - t_used) / max(rate, 1e-6))))
    return {
        "value": done_flops / t_used / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.threads(),
        "kind": "oracle",
        "sample": f"oracle attention on {done_rows} random query rows of head (b=0, h=0) of the {w.name} workload "
                  f"({done_flops / 1e9:.1f} GFLOP algorithmic, {t_used:.1f} s), after the oracle's own quantize "
                  f"and select of that head; value = algorithmic flops / time",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long_128k")
    ap.add_argument("--frac", type=float, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-quality", action="store_true")
    ap.add_argument("--no-alt", action="store_true",
                    help="skip the timing and quality of the attention normalised by the quantized weights")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="only run a device copy of this many MiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(sharding over (batch, KV-head group) is a design note only).", file=sys.stderr)
        sys.exit(2)

    import torch

    from fp16_long_context_amd import binding, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": n, "launches": 3}))
        return

    t0 = time.perf_counter()
    x = synth.generate(args.workload)
    w = x["w"]
    frac = w.frac if args.frac is None else args.frac
    log(f"generated {w.name} in {time.perf_counter() - t0:.1f}s")
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    qz = binding.alloc_quantized(w.B, w.Hq, w.Hkv, w.N, w.d, dev)
    ents = binding.list_entries(w.B, w.Hq, w.N, True)
    idx = torch.empty(ents, dtype=torch.int32, device=dev)
    n16 = torch.empty((w.B, w.Hq, w.N // 64), dtype=torch.int32, device=dev)
    s = binding.make_shape(w.B, w.Hq, w.Hkv, w.N, w.d)
    ws = torch.empty(int(binding.lib().thrift_select_workspace_bytes(s)), dtype=torch.uint8, device=dev)
    out = torch.empty((w.B, w.Hq, w.N, w.d), dtype=torch.float32, device=dev)
    aws = torch.empty(binding.attn_workspace_bytes(w.B, w.Hq, w.Hkv, w.N, w.d), dtype=torch.uint8, device=dev)

    def step(evs=None):
        # evs: before quantize, before select, then the attention call's own
        # four events (before, between and after its three kernels)
        if evs:
            evs[0].record()
        binding.quantize(q, k, v, out=qz)
        if evs:
            evs[1].record()
        binding.select(qz["q16"], qz["k16"], frac, True, workspace=ws, idx=idx, n16=n16)
        binding.attn_fwd(qz, idx, n16, True, out=out, workspace=aws, events=evs[2:6] if evs else None)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e_start.record()
    for i in range(args.steps):
        step(evs[i])
    e_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = e_start.elapsed_time(e_end) / args.steps
    t_q = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    t_s = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    t_a = sum(e[2].elapsed_time(e[5]) for e in evs) / args.steps
    t_as = sorted(e[2].elapsed_time(e[5]) for e in evs)
    t_f16 = sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps
    t_f4 = sum(e[3].elapsed_time(e[4]) for e in evs) / args.steps
    t_redo = sum(e[4].elapsed_time(e[5]) for e in evs) / args.steps
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step (wall {1e3 * wall / args.steps:.3f}), "
        f"quantize {t_q:.3f} select {t_s:.3f} attn {t_a:.3f} ms")

    F = attn_flops(w)
    F16 = fp16_tile_flops(w, n16, frac)
    F4 = F - F16
    t_roof = F16 / (PEAK_F16 * 1e12) + F4 / (PEAK_F4 * 1e12)
    peak = F / t_roof / 1e12
    achieved = F / (t_a * 1e-3) / 1e12
    traffic = read_traffic()
    result = {
        "metric": METRIC,
        "value": round(F / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16+mxfp4",
        "data": f"synthetic: seeded {w.name} generator",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d, "block": 64,
                   "causal": True, "frac": frac, "in_dtype": w.dtype, "out_dtype": "f32"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1), "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "fp16_flop_share": round(F16 / F, 5),
                     "kernel": "thrift_attn_fwd = attn_f16_kernel + attn_fwd_kernel + attn_redo_kernel"},
        "kernels": {
            "quantize_ms": round(t_q, 4), "quantize_GBps": round(quantize_bytes(w) / (t_q * 1e-3) / 1e9, 1),
            "select_ms": round(t_s, 4), "select_GBps": round(select_bytes(w) / (t_s * 1e-3) / 1e9, 1),
            "attn_ms": round(t_a, 4), "attn_ms_median": round(t_as[len(t_as) // 2], 4),
            "attn_ms_min": round(t_as[0], 4), "attn_TFLOPs": round(achieved, 2), "hbm_peak_GBps": PEAK_HBM,
            "attn_f16_kernel_ms": round(t_f16, 4), "attn_fwd_kernel_ms": round(t_f4, 4),
            "attn_redo_kernel_ms": round(t_redo, 4),
        },
        # the dominant kernel (FP4 tiles) against its own bound, the VALU:
        # algorithmic work = the softmax's full-rate issue slots per FP4 score
        "roofline_alu": {"bound": "alu", "kernel": "attn_fwd_kernel",
                         "achieved": round(VALU_SLOTS_PER_FP4_SCORE * (F4 / (4 * w.d)) / (t_f4 * 1e-3) / 1e12, 2),
                         "peak": round(PEAK_VALU, 2), "unit": "T VALU lane-ops/s",
                         "frac": round(VALU_SLOTS_PER_FP4_SCORE * (F4 / (4 * w.d)) / (t_f4 * 1e-3) / 1e12 / PEAK_VALU, 4),
                         "fp4_scores": F4 / (4 * w.d), "slots_per_score": VALU_SLOTS_PER_FP4_SCORE},
    }
    alt = (("alt_rowsum_weights", "weights", "thrift_attn_fwd_wsum"),
           ("alt_rowsum_weights_expfree", "log", "thrift_attn_fwd_ex rowsum 2"))
    if not args.no_alt:
        # the same attention call under the other row-sum reading: normalised
        # by the quantized weights (thrift_attn_fwd_wsum), and the same with
        # exp-free FP4 codes; each timed alone on the same lists and inputs,
        # with the FP4 kernel's own time from the call's events
        for key, rs, entry in alt:
            for _ in range(2):
                binding.attn_fwd(qz, idx, n16, True, out=out, workspace=aws, rowsum=rs)
            torch.cuda.synchronize()
            aev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
            for i in range(args.steps):
                binding.attn_fwd(qz, idx, n16, True, out=out, workspace=aws, rowsum=rs, events=aev[i])
            torch.cuda.synchronize()
            t_w = sum(e[0].elapsed_time(e[3]) for e in aev) / args.steps
            t_w4 = sum(e[1].elapsed_time(e[2]) for e in aev) / args.steps
            result[key] = {
                "entry": entry, "attn_ms": round(t_w, 4), "attn_fwd_kernel_ms": round(t_w4, 4),
                "attn_TFLOPs": round(F / (t_w * 1e-3) / 1e12, 2),
                "roofline_frac": round(F / (t_w * 1e-3) / 1e12 / peak, 4)}
            log(f"attention, row-sum reading {rs}: {t_w:.3f} ms (FP4 kernel {t_w4:.3f} ms)")
    if not args.no_quality:
        result["quality"] = quality(binding, torch, qz, w, x["needles"], frac, dev)
        log(f"quality {result['quality']}")
        if not args.no_alt:
            from fp16_long_context_amd.quality import errors

            for key, rs, _ in alt:
                result[key]["quality"] = errors(binding, torch, qz, w, x["needles"], frac, rs)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(x, w, frac)
        log(f"cpu baseline {result['cpu_baseline']['value']:.3e} TFLOP/s on {result['cpu_baseline']['cores']} threads")
    print(json.dumps(result), flush=True)


def quality(binding, torch, qz, w, needles, frac, dev):
    """Planted-needle check: relative Frobenius error of frac and of frac=0
    against frac=1, over all rows and over the rows that look up a needle."""
    from fp16_long_context_amd.quality import errors

    return errors(binding, torch, qz, w, needles, frac)


if __name__ == "__main__":
    main()
