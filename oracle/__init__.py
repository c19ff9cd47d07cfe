"""CPU oracle for the ThriftAttention prefill hot path (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers.  The product library
never imports this package and this package never imports the product.

The arithmetic lives in oracle.c (plain fp64 C, OpenMP over rows); this file
only marshals numpy arrays.  Every function follows a step of the method as
the ThriftAttention abstract states it (a heuristic marks the block pairs
that matter, FP16 for those, block-scaled 4-bit for the rest, one online
softmax over both), with the readings listed at the top of oracle.c.

Parity status per function:
  to_fp16, mx_encode, quantize  pinned (numpy float16 cast, brute-force E2M1
                                search, closed forms)
  pool, select                  pinned (numpy means, brute-force subset search,
                                list invariants, a worked example)
  normw_pool, select(score=...) pinned (exactly representable inputs against
                                numpy; brute-force scores on tiny inputs; a
                                dominant key row for max-pooled; equal-norm rows
                                reduce norm-weighted to the pooled mean)
  attn_rows                     pinned (frac=1 against textbook softmax
                                attention, frac=0 against an independent
                                numpy pure-FP4 attention on random inputs,
                                FP4-exact inputs against textbook attention,
                                closed forms, split-merge);
                                rowsum="weights": V = 1 gives O = 1 exactly,
                                frac=1 against textbook attention, split-merge,
                                closed forms; rowsum="log": the same, plus
                                log_encode against a brute-force code search
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    """Compile oracle.c into liboracle.so next to it (gcc, OpenMP)."""
    tmp = _SO + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-shared", "-fPIC", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SO)
    return _SO


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        i32, i64, f32, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_double
        L.oracle_threads.argtypes = []
        L.oracle_threads.restype = i32
        L.oracle_to_fp16.argtypes = [P, i32, P, i64]
        L.oracle_to_fp16.restype = None
        L.oracle_mx_encode.argtypes = [P, i64, P, P]
        L.oracle_mx_encode.restype = None
        L.oracle_quantize.argtypes = [i32] * 6 + [P] * 3 + [P] * 3 + [P] * 6
        L.oracle_quantize.restype = i32
        L.oracle_pool.argtypes = [P, i64, i32, i32, P]
        L.oracle_pool.restype = None
        L.oracle_list_entries.argtypes = [i32, i32, i32, i32]
        L.oracle_list_entries.restype = i64
        L.oracle_select.argtypes = [i32] * 6 + [f64] + [P] * 7
        L.oracle_select.restype = i32
        L.oracle_select_kind.argtypes = [i32] * 7 + [f64] + [P] * 7
        L.oracle_select_kind.restype = i32
        L.oracle_log_encode.argtypes = [P, i64, f64, P, P]
        L.oracle_log_encode.restype = None
        L.oracle_normw_pool.argtypes = [P, i64, i32, i32, P]
        L.oracle_normw_pool.restype = None
        L.oracle_attn_rows.argtypes = [i32] * 6 + [f32] + [P] * 9 + [P, P, P, i64, P, P, P, P, P, P, i32]
        L.oracle_attn_rows.restype = i32
        _lib = L
    return _lib


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().oracle_threads())


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


DTYPES = {"fp16": 0, "bf16": 1}


def to_fp16(x_bits: np.ndarray, in_dtype: str) -> np.ndarray:
    """fp16/bf16 bit patterns -> fp16 bit patterns, round to nearest even."""
    x = _c(x_bits, np.uint16)
    out = np.empty_like(x)
    lib().oracle_to_fp16(_p(x), DTYPES[in_dtype], _p(out), x.size)
    return out


def mx_encode(groups: np.ndarray):
    """MXFP4-encode rows of 32 float64 values -> (codes uint8 [G,32], scale bytes uint8 [G])."""
    g = _c(groups, np.float64).reshape(-1, 32)
    codes = np.empty(g.shape, dtype=np.uint8)
    scales = np.empty(g.shape[0], dtype=np.uint8)
    lib().oracle_mx_encode(_p(g), g.shape[0], _p(codes), _p(scales))
    return codes, scales


def log_encode(x: np.ndarray, M: float):
    """Exp-free encoding of rows of 32 scores (log2 units, -inf = masked)
    against the integer max M -> (codes uint8 [G,32], scale bytes uint8 [G])."""
    g = _c(x, np.float64).reshape(-1, 32)
    codes = np.empty(g.shape, dtype=np.uint8)
    scales = np.empty(g.shape[0], dtype=np.uint8)
    lib().oracle_log_encode(_p(g), g.shape[0], float(M), _p(codes), _p(scales))
    return codes, scales


def quantize(q_bits, k_bits, v_bits, in_dtype: str) -> dict:
    """FP16 copies and MXFP4 codes.  Inputs: uint16 bits [B,Hq,N,d] / [B,Hkv,N,d].
    v16 is returned token-major [B,Hkv,N,d]; v4/v4s are [B,Hkv,d,N/2] / [B,Hkv,d,N/32]."""
    q, k, v = _c(q_bits, np.uint16), _c(k_bits, np.uint16), _c(v_bits, np.uint16)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    r = {
        "q16": np.empty_like(q), "k16": np.empty_like(k), "v16": np.empty_like(v),
        "q4": np.empty((B, Hq, N, d // 2), np.uint8), "q4s": np.empty((B, Hq, N, d // 32), np.uint8),
        "k4": np.empty((B, Hkv, N, d // 2), np.uint8), "k4s": np.empty((B, Hkv, N, d // 32), np.uint8),
        "v4": np.empty((B, Hkv, d, N // 2), np.uint8), "v4s": np.empty((B, Hkv, d, N // 32), np.uint8),
    }
    rc = lib().oracle_quantize(B, Hq, Hkv, N, d, DTYPES[in_dtype], _p(q), _p(k), _p(v),
                               *[_p(r[n]) for n in ("q16", "k16", "v16", "q4", "q4s", "k4", "k4s", "v4", "v4s")])
    if rc != 0:
        raise ValueError("oracle_quantize rejected the shapes")
    return r


def pool(x16: np.ndarray) -> np.ndarray:
    x = _c(x16, np.uint16)
    B, H, N, d = x.shape
    out = np.empty((B, H, N // 64, d), np.float32)
    lib().oracle_pool(_p(x), B * H, N, d, _p(out))
    return out


def list_entries(B, Hq, N, causal) -> int:
    return int(lib().oracle_list_entries(B, Hq, N, int(causal)))


SCORES = {"pooled_mean": 0, "max_pooled": 1, "norm_weighted": 2, "block_max": 3}


def normw_pool(x16: np.ndarray) -> np.ndarray:
    """Norm-weighted means of 64-row blocks (rows weighed by their L2 norms)."""
    x = _c(x16, np.uint16)
    B, H, N, d = x.shape
    out = np.empty((B, H, N // 64, d), np.float32)
    lib().oracle_normw_pool(_p(x), B * H, N, d, _p(out))
    return out


def select(q16, k16, frac: float, causal: bool = True, score: str = "pooled_mean") -> dict:
    """Block heuristic: block means, scores and the FP16/FP4 traversal lists.
    score: "pooled_mean" (the library's default), "max_pooled",
    "norm_weighted" or "block_max" (the heuristic variants; same budget rule).
    qbar/kbar hold the pooled means (norm-weighted means for "norm_weighted")."""
    q, k = _c(q16, np.uint16), _c(k16, np.uint16)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    nb = N // 64
    E = list_entries(B, Hq, N, causal)
    idx = np.full(E, -1, np.int32)
    n16 = np.empty((B, Hq, nb), np.int32)
    qbar = np.empty((B, Hq, nb, d), np.float32)
    kbar = np.empty((B, Hkv, nb, d), np.float32)
    scores = np.full(E, np.nan, np.float64)
    rc = lib().oracle_select_kind(SCORES[score], B, Hq, Hkv, N, d, int(causal), float(frac), _p(q), _p(k),
                                  _p(idx), _p(n16), _p(qbar), _p(kbar), _p(scores))
    if rc != 0:
        raise ValueError("oracle_select rejected the arguments")
    return {"idx": idx, "n16": n16, "qbar": qbar, "kbar": kbar, "scores": scores}


def row_lists(sel: dict, B, Hq, N, causal, b, h, i):
    """(FP16 list, FP4 list) of query block i of (b, h) from a flat idx array."""
    nb = N // 64
    per = nb * (nb + 1) // 2 if causal else nb * nb
    off = (b * Hq + h) * per + (i * (i + 1) // 2 if causal else i * nb)
    nv = i + 1 if causal else nb
    row = sel["idx"][off:off + nv]
    c = int(sel["n16"][b, h, i])
    return row[:c], row[c:]


ROWSUM = {"p": 0, "weights": 1, "log": 2}


def attn_rows(qz: dict, sel: dict, rows, causal: bool = True, sm_scale: float = 0.0, blk_keep=None,
              rowsum: str = "p") -> dict:
    """Mixed-precision attention for the flat output rows ((b*Hq + h)*N + t).

    rowsum "p": the row sum adds the unquantized p; "weights": it adds the
    weights the P.V products use (fp16(p), dequantized MXFP4 P); "log": as
    "weights", with FP4 P codes from a piecewise-linear 2^y of the scores
    (no exponential on FP4 tiles).
    Returns out [R,d] (normalised), lse [R], acc [R,d] (unnormalised), l [R], m [R]."""
    q16 = qz["q16"]
    B, Hq, N, d = q16.shape
    Hkv = qz["k16"].shape[1]
    rows = _c(rows, np.int64).ravel()
    R = rows.size
    res = {"out": np.zeros((R, d)), "lse": np.zeros(R), "acc": np.zeros((R, d)), "l": np.zeros(R),
           "m": np.zeros(R)}
    keep = None if blk_keep is None else _c(blk_keep, np.uint8)
    arrs = [_c(qz[n], np.uint16 if n.endswith("16") else np.uint8)
            for n in ("q16", "k16", "v16", "q4", "q4s", "k4", "k4s", "v4", "v4s")]
    rc = lib().oracle_attn_rows(B, Hq, Hkv, N, d, int(causal), float(sm_scale), *[_p(a) for a in arrs],
                                _p(_c(sel["idx"], np.int32)), _p(_c(sel["n16"], np.int32)), _p(rows), R, _p(keep),
                                _p(res["out"]), _p(res["lse"]), _p(res["acc"]), _p(res["l"]), _p(res["m"]),
                                ROWSUM[rowsum])
    if rc != 0:
        raise ValueError("oracle_attn_rows: bad arguments or malformed lists")
    return res


def all_rows(B, Hq, N) -> np.ndarray:
    return np.arange(B * Hq * N, dtype=np.int64)
