"""Seeded synthetic inputs for the prefill workloads.

This module only draws numbers: it holds none of the attention method's
arithmetic and is shared by the tests, the smoke check and the benchmark so
that the GPU library and the CPU oracle see the same arrays.

The paper evaluates on long-context benchmarks with trained models that are
not available here; these generators stand in for them with the shapes of
the workloads (Llama-8B-shaped GQA layers, 16K-128K tokens) and with the
structure that makes some key blocks matter more than others (attention
sinks, planted needle keys, outlier channels, RoPE-like rotation).

Every tensor is drawn from numpy's PCG64 with one child stream per
(tensor, batch, head) spawned from the workload seed, so the result does not
depend on how many threads fill it.  Values are drawn in float32 and rounded
once to the input dtype (bf16 or fp16) by torch.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    dtype: str  # "fp16" | "bf16"
    frac: float
    kind: str  # "outlier", "sinks", "rope", "heavy"
    seed: int


# The five prefill workloads (block size 64, causal).
WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 2, 1024, 64, "fp16", 0.05, "outlier", 1001),
    "llama8b_16k": Workload("llama8b_16k", 1, 32, 8, 16384, 128, "bf16", 0.05, "sinks", 1002),
    "sweep_64k": Workload("sweep_64k", 1, 32, 8, 65536, 128, "bf16", 0.05, "sinks", 1003),
    "long_128k": Workload("long_128k", 1, 32, 8, 131072, 128, "bf16", 0.05, "rope", 1004),
    "batched_32k": Workload("batched_32k", 4, 28, 4, 32768, 128, "bf16", 0.05, "heavy", 1005),
}

SWEEP_FRACS = (0.0, 0.01, 0.05, 0.2, 1.0)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal_heads(ss: np.random.SeedSequence, B: int, H: int, N: int, d: int) -> np.ndarray:
    """[B,H,N,d] float32 N(0,1), one child stream per (b, h)."""
    out = np.empty((B, H, N, d), dtype=np.float32)
    children = ss.spawn(B * H)

    def fill(i: int) -> None:
        g = np.random.Generator(np.random.PCG64(children[i]))
        out[i // H, i % H] = g.standard_normal((N, d), dtype=np.float32)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(B * H)))
    return out


def _rotate(x: np.ndarray, base: float) -> None:
    """RoPE-like rotation in place: channel pairs (c, c + d/2) of the token at
    position p are rotated by the angle p * base^(-2c/d)."""
    B, H, N, d = x.shape
    half = d // 2
    theta = base ** (-2.0 * np.arange(half, dtype=np.float64) / d)

    def rot(i: int) -> None:
        b, h = divmod(i, H)
        for p0 in range(0, N, 8192):
            p1 = min(N, p0 + 8192)
            ang = np.arange(p0, p1, dtype=np.float64)[:, None] * theta[None, :]
            cs, sn = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
            a = x[b, h, p0:p1, :half].copy()
            c = x[b, h, p0:p1, half:]
            x[b, h, p0:p1, :half] = a * cs - c * sn
            x[b, h, p0:p1, half:] = a * sn + c * cs

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(rot, range(B * H)))


def _plant_needles(g: np.random.Generator, q: np.ndarray, k: np.ndarray, counts, scale: float) -> list:
    """Copy scale * q[b, hq, t] into k[b, kvh, p] for random p < t, with hq a
    random query head of kv head kvh's group.  counts[b] needles per kv head."""
    B, Hq, N, _ = q.shape
    Hkv = k.shape[1]
    grp = Hq // Hkv
    planted = []
    for b in range(B):
        for kvh in range(Hkv):
            for _ in range(int(counts[b])):
                p = int(g.integers(0, N - 1))
                t = int(g.integers(p + 1, N))
                hq = kvh * grp + int(g.integers(0, grp))
                k[b, kvh, p] = scale * q[b, hq, t]
                planted.append((b, kvh, hq, p, t))
    return planted


def generate(name: str, N: int | None = None, B: int | None = None, seed: int | None = None) -> dict:
    """Draw (q, k, v) for a named workload.  N, B and seed may be overridden
    (smaller N keeps a workload's structure for tests the oracle can finish).

    Returns {"q","k","v": CPU torch tensors [B,H,N,d] of the workload dtype,
    "w": Workload, "needles": [(b, kv_head, q_head, key_pos, query_pos)]}."""
    w = WORKLOADS[name]
    w = dataclasses.replace(w, N=N or w.N, B=B or w.B, seed=w.seed if seed is None else seed)
    ss = np.random.SeedSequence(w.seed)
    s_q, s_k, s_v, s_struct = ss.spawn(4)
    q = _normal_heads(s_q, w.B, w.Hq, w.N, w.d)
    k = _normal_heads(s_k, w.B, w.Hkv, w.N, w.d)
    v = _normal_heads(s_v, w.B, w.Hkv, w.N, w.d)
    g = np.random.Generator(np.random.PCG64(s_struct))
    needles: list = []
    if w.kind == "outlier":
        # per-(head, channel) key offset with standard deviation 2, then 4 needles per head
        k += (2.0 * g.standard_normal((1, w.Hkv, 1, w.d))).astype(np.float32)
        needles = _plant_needles(g, q, k, [4] * w.B, 4.0)
    elif w.kind == "sinks":
        k[:, :, 0:4, :] *= 8.0
        needles = _plant_needles(g, q, k, [64] * w.B, 4.0)
    elif w.kind == "rope":
        _rotate(q, 5e5)
        _rotate(k, 5e5)
        k[:, :, 0:4, :] *= 8.0
        needles = _plant_needles(g, q, k, [256] * w.B, 4.0)
    elif w.kind == "heavy":
        for b in range(w.B):
            for h in range(w.Hkv):
                c = int(g.integers(0, w.d))
                k[b, h, :, c] = g.standard_t(3.0, size=w.N).astype(np.float32)
        counts = g.integers(16, 129, size=w.B)
        needles = _plant_needles(g, q, k, counts, 4.0)
    else:  # pragma: no cover
        raise ValueError(w.kind)
    tdt = torch.float16 if w.dtype == "fp16" else torch.bfloat16
    # values are finite and well inside the fp16 range; torch rounds to nearest-even
    out = {
        "q": torch.from_numpy(q).to(tdt),
        "k": torch.from_numpy(k).to(tdt),
        "v": torch.from_numpy(v).to(tdt),
        "w": w,
        "needles": needles,
    }
    return out


def random_qkv(B: int, Hq: int, Hkv: int, N: int, d: int, dtype: str = "fp16", seed: int = 0, scale: float = 1.0):
    """Plain N(0, scale^2) inputs for edge-case tests."""
    ss = np.random.SeedSequence(seed)
    s_q, s_k, s_v = ss.spawn(3)
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    mk = lambda s, H: torch.from_numpy(scale * _normal_heads(s, B, H, N, d)).to(tdt)
    return mk(s_q, Hq), mk(s_k, Hkv), mk(s_v, Hkv)


def bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a CPU fp16/bf16 tensor."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)
