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
             attn_redo_kernel: reads the FP4 workgroups' overflow flags and
             redoes the flagged ones): achieved = F / the call's average duration (HIP
             events on its stream), peak = the FP16/MXFP4 MFMA roofline
             weighted by the flops in FP16 and FP4 tiles
             (F16 / 2516.6 TF/s + F4 / 10066 TF/s), traffic = HBM bytes per
             call (all three kernels) from the committed rocprofv3 counter
             summary when it was taken on the current kernel source, else null;
  cpu_baseline  the CPU oracle's attention on a bounded row sample of the
             same workload, on this host's cores;
  kernels    quantize / select / attention times and algorithmic GB/s, and
             the HBM rate a plain kernel reaches on the quantizer's byte mix;
  quality    planted-needle check: error of frac=0.05 and of frac=0 against
             frac=1 (all-FP16) output;
  roofline_alu  the dominant kernel (attn_fwd_kernel, FP4 tiles) against
             the bound it runs into, VALU issue: achieved = FP4 block-waves
             (one wave's 32 query rows x 64 keys) per second over its
             duration (HIP events the library records between its kernels);
             peak = 1024 SIMDs x 2.4 GHz / the VALU issue cycles of one
             block-wave (measured instruction costs x the walk's instruction
             mix), i.e. with every MFMA hidden under VALU work; also the same
             against VALU + MFMA cycles (no overlap);
  clock      the GPU's shader clock (sysfs pp_dpm_sclk) and board power
             sampled during the timed steps;
  configs_timed  quantize / select / attention times of the other workloads
             (16K, the 64K fraction sweep, 4 x 32K), a few steps each;
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
# Issue cost in SIMD cycles of the instructions of one FP4 block-wave (one
# wave's 32 query rows x 64 keys of the FP4 walk), measured at 3 waves per
# SIMD by the isa_costs program built next to the library (its output and
# command: profiles/isa_costs_gfx950.txt).  The block's VALU mix is that of
# the compiled walk of attn_fwd_kernel (row-sum reading 0).
VALU_CYCLES = {"v_fma_f32": 2.83, "v_exp_f32": 9.99, "v_add_f32": 2.83, "v_cvt_scalef32_pk_fp4_f32": 8.42,
               "v_max3_f32": 4.72, "v_max_f32": 5.73, "integer": 2.87}
FP4_BLOCK_VALU = {"v_fma_f32": 32, "v_exp_f32": 32, "v_add_f32": 32, "v_cvt_scalef32_pk_fp4_f32": 16,
                  "v_max3_f32": 14, "v_max_f32": 3, "integer": 6}
FP4_BLOCK_MFMAS = 8  # 4 for S, 4 for P.V, v_mfma_scale_f32_32x32x64_f8f6f4
MFMA_F4_CYCLES = 32.0  # 2 x 32 x 32 x 64 flops at the dense MXFP4 peak per SIMD (10066 TF/s / 1024 / 2.4 GHz)
SIMDS, NOMINAL_GHZ = 1024, 2.4
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


class ClockSampler:
    """Samples the GPU's current shader clock (sysfs pp_dpm_sclk: the line
    marked '*') and board power (hwmon power1_input) on a thread while the
    timed steps run; None where the files cannot be read."""

    def __init__(self, period_s: float = 0.005):
        import glob

        cards = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.sclk = cards[0] if cards else None
        pw = sorted(glob.glob(os.path.join(os.path.dirname(cards[0]), "hwmon", "hwmon*", "power1_input"))) if cards else []
        self.power = pw[0] if pw else None
        self.period = period_s
        self.mhz, self.watts = [], []
        self._stop = None
        self._thread = None

    def read_mhz(self):
        try:
            for line in open(self.sclk).read().splitlines():
                if line.strip().endswith("*"):
                    m = re.search(r"(\d+)\s*[Mm]hz", line)
                    return float(m.group(1)) if m else None
        except (OSError, TypeError):
            return None
        return None

    def read_watts(self):
        try:
            return float(open(self.power).read().strip()) * 1e-6
        except (OSError, TypeError, ValueError):
            return None

    def start(self):
        import threading

        self._stop = threading.Event()

        def run():
            while not self._stop.is_set():
                f, p = self.read_mhz(), self.read_watts()
                if f is not None:
                    self.mhz.append(f)
                if p is not None:
                    self.watts.append(p)
                self._stop.wait(self.period)

        self._thread = threading.Thread(target=run, daemon=True)
        self._thread.start()

    def stop(self):
        if self._thread:
            self._stop.set()
            self._thread.join()

    def summary(self, before_mhz):
        mean = lambda v: round(sum(v) / len(v), 1) if v else None  # noqa: E731
        return {"source": "sysfs pp_dpm_sclk (current level) and hwmon power1_input, sampled every "
                          f"{self.period * 1e3:.0f} ms during the timed steps",
                "before_MHz": before_mhz, "under_load_MHz_mean": mean(self.mhz),
                "under_load_MHz_min": min(self.mhz) if self.mhz else None,
                "under_load_MHz_max": max(self.mhz) if self.mhz else None,
                "samples": len(self.mhz), "power_W_mean": mean(self.watts)}


def fp4_block_waves(w, n16) -> float:
    """Block-waves of the FP4 path: causally valid tiles not on an FP16 list,
    two 32-row waves each."""
    nb = w.N // 64
    tiles = w.B * w.Hq * nb * (nb + 1) // 2
    return 2.0 * (tiles - int(n16.sum().item()))


def roofline_alu(w, n16, t_f4_ms):
    valu = sum(VALU_CYCLES[k] * n for k, n in FP4_BLOCK_VALU.items())
    mfma = FP4_BLOCK_MFMAS * MFMA_F4_CYCLES
    bw = fp4_block_waves(w, n16)
    achieved = bw / (t_f4_ms * 1e-3) / 1e9
    peak = SIMDS * NOMINAL_GHZ * 1e9 / valu / 1e9
    peak_serial = SIMDS * NOMINAL_GHZ * 1e9 / (valu + mfma) / 1e9
    return {"bound": "alu", "kernel": "attn_fwd_kernel", "unit": "G FP4 block-waves/s",
            "achieved": round(achieved, 4), "peak": round(peak, 4), "frac": round(achieved / peak, 4),
            "peak_valu_plus_mfma": round(peak_serial, 4), "frac_valu_plus_mfma": round(achieved / peak_serial, 4),
            "block_waves": bw, "valu_cycles_per_block_wave": round(valu, 1),
            "mfma_cycles_per_block_wave": mfma, "clock_GHz": NOMINAL_GHZ}


def copy_ceiling(w):
    """The HBM rate a plain kernel reaches on the quantizer's byte mix: the
    isa_costs program (built next to the library) in its hbm mode, reading
    the bf16 inputs' bytes and writing the FP16 + MXFP4 outputs' bytes with
    16-byte accesses; run as a child process."""
    import subprocess

    elems = w.B * (w.Hq + 2 * w.Hkv) * w.N * w.d
    rb, wb = 2 * elems, int(elems * (2 + 0.5 + 1 / 32))
    exe = os.path.join(ROOT, "fp16_long_context_amd", "isa_costs")
    try:
        r = subprocess.run([exe, "hbm", str(rb), str(wb)], capture_output=True, text=True, timeout=120)
        out = json.loads(r.stdout.strip().splitlines()[-1])
    except (OSError, ValueError, IndexError, subprocess.SubprocessError) as e:
        return {"GBps": None, "error": f"{type(e).__name__}: {e}"}
    out["what"] = ("one plain kernel reading the quantizer's input bytes and writing its output bytes "
                   "(16-byte accesses): the HBM ceiling for that mix")
    return out

def time_workload(torch, binding, synth, name, fracs, dev, steps=4, warmup=2):
    """Quantize / select / attention times of one workload at each FP16
    fraction, inputs resident in HBM, HIP events on the library's stream."""
    x = synth.generate(name)
    w = x["w"]
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    del x
    qz = binding.alloc_quantized(w.B, w.Hq, w.Hkv, w.N, w.d, dev)
    idx = torch.empty(binding.list_entries(w.B, w.Hq, w.N, True), dtype=torch.int32, device=dev)
    n16 = torch.empty((w.B, w.Hq, w.N // 64), dtype=torch.int32, device=dev)
    s = binding.make_shape(w.B, w.Hq, w.Hkv, w.N, w.d)
    ws = torch.empty(int(binding.lib().thrift_select_workspace_bytes(s)), dtype=torch.uint8, device=dev)
    out = torch.empty((w.B, w.Hq, w.N, w.d), dtype=torch.float32, device=dev)
    aws = torch.empty(binding.attn_workspace_bytes(w.B, w.Hq, w.Hkv, w.N, w.d), dtype=torch.uint8, device=dev)
    res = {}
    F = attn_flops(w)
    for frac in fracs:
        def step(evs=None):
            if evs:
                evs[0].record()
            binding.quantize(q, k, v, out=qz)
            if evs:
                evs[1].record()
            binding.select(qz["q16"], qz["k16"], frac, True, workspace=ws, idx=idx, n16=n16)
            if evs:
                evs[2].record()
            binding.attn_fwd(qz, idx, n16, True, out=out, workspace=aws)
            if evs:
                evs[3].record()

        for _ in range(warmup):
            step()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        for i in range(steps):
            step(evs[i])
        torch.cuda.synchronize()
        t = [sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps for j in range(3)]
        F16 = fp16_tile_flops(w, n16, frac)
        t_roof = F16 / (PEAK_F16 * 1e12) + (F - F16) / (PEAK_F4 * 1e12)
        res[f"frac={frac:g}"] = {
            "quantize_ms": round(t[0], 4), "select_ms": round(t[1], 4), "attn_ms": round(t[2], 4),
            "ms_per_step": round(sum(t), 4), "TFLOPs_per_step": round(F / (sum(t) * 1e-3) / 1e12, 2),
            "attn_TFLOPs": round(F / (t[2] * 1e-3) / 1e12, 2),
            "attn_roofline_frac": round(t_roof / (t[2] * 1e-3), 4), "fp16_flop_share": round(F16 / F, 5)}
    del q, k, v, qz, idx, n16, ws, out, aws
    torch.cuda.empty_cache()
    return {"config": {"B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d, "in_dtype": w.dtype},
            "steps": steps, "warmup": warmup, "by_frac": res}


def cpu_model() -> str:
    """The host CPU as /proc/cpuinfo names it (model name, family/model
    numbers, clock and cache of the first CPU), else the platform's name."""
    try:
        info = {}
        for line in open("/proc/cpuinfo"):
            if not line.strip():
                break  # the first CPU's fields only
            k, _, v = line.partition(":")
            info.setdefault(k.strip(), v.strip())
        if "model name" in info:
            extra = [f"family {info[k1]} model {info[k2]}" for k1, k2 in [("cpu family", "model")]
                     if k1 in info and k2 in info]
            extra += [f"{info[k]} MHz" for k in ["cpu MHz"] if k in info]
            extra += [f"cache {info[k]}" for k in ["cache size"] if k in info]
            return info["model name"] + (f" ({', '.join(extra)})" if extra else "")
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def cpu_baseline(x, w, frac, budget_s=12.0):
    """The oracle on a bounded sample of the workload: its quantize and select
    of query head 0 and that head's KV head, then its attention on random
    rows of that head until the time budget is spent.  value = the sampled
    rows' algorithmic attention flops / their time.  The full-problem time is
    an extrapolation, labelled as such: quantize time x (heads quantized in
    all) / 3, select time x query heads, attention at the sampled flop rate."""
    import numpy as np

    if "OMP_NUM_THREADS" not in os.environ:
        os.environ["OMP_NUM_THREADS"] = str(len(os.sched_getaffinity(0)))
    import oracle
    from fp16_long_context_amd import synth

    q, k, v = x["q"][:1, :1], x["k"][:1, :1], x["v"][:1, :1]
    dt = "fp16" if w.dtype == "fp16" else "bf16"
    t0 = time.perf_counter()
    qz = oracle.quantize(synth.bits(q), synth.bits(k), synth.bits(v), dt)
    t_q = time.perf_counter() - t0
    t0 = time.perf_counter()
    sel = oracle.select(qz["q16"], qz["k16"], frac, True)
    t_s = time.perf_counter() - t0
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
    flop_rate = done_flops / t_used
    full_q = t_q * w.B * (w.Hq + 2 * w.Hkv) / 3.0
    full_s = t_s * w.B * w.Hq
    full_a = attn_flops(w) / flop_rate
    return {
        "value": flop_rate / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.threads(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"oracle attention on {done_rows} random query rows of head (b=0, h=0) of the {w.name} workload "
                  f"({done_flops / 1e9:.1f} GFLOP algorithmic, {t_used:.1f} s), after the oracle's own quantize "
                  f"({t_q:.2f} s, 3 heads) and select ({t_s:.2f} s, 1 query head) of that head; "
                  f"value = algorithmic flops / time",
        "extrapolated_full_step_s": {
            "what": "EXTRAPOLATION, not measured: quantize x heads/3, select x query heads, "
                    "attention = all algorithmic flops at the sampled rate",
            "quantize": round(full_q, 1), "select": round(full_s, 1), "attention": round(full_a, 1),
            "total": round(full_q + full_s + full_a, 1)},
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
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the HBM ceiling run on the quantizer's byte mix (a child process)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip timing the other workloads (16K, the 64K fraction sweep, 4 x 32K)")
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
    clock = ClockSampler()
    before_mhz = clock.read_mhz()  # after the warmup steps
    torch.cuda.synchronize()
    clock.start()
    w0 = time.perf_counter()
    e_start.record()
    for i in range(args.steps):
        step(evs[i])
    e_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    clock.stop()
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
        # the dominant kernel (FP4 tiles) against its own bound, VALU issue
        "roofline_alu": roofline_alu(w, n16, t_f4),
        "clock": clock.summary(before_mhz),
    }
    log(f"clock under load {result['clock']['under_load_MHz_mean']} MHz "
        f"({result['clock']['samples']} samples), power {result['clock']['power_W_mean']} W")
    if not args.no_ceiling:
        result["kernels"]["quantize_copy_ceiling"] = copy_ceiling(w)
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
    if not args.no_configs:
        # the other workloads, each timed on its own seeded inputs
        result["configs_timed"] = {}
        for name, fracs in (("llama8b_16k", (0.05,)), ("sweep_64k", (0.0, 0.01, 0.05, 0.2, 1.0)),
                            ("batched_32k", (0.05,))):
            t0 = time.perf_counter()
            result["configs_timed"][name] = time_workload(torch, binding, synth, name, fracs, dev)
            log(f"{name}: " + ", ".join(f"{f} attn {r['attn_ms']:.3f} ms" for f, r in
                                      result["configs_timed"][name]["by_frac"].items())
                + f" ({time.perf_counter() - t0:.1f} s)")
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
