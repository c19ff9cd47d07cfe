"""Thin ctypes binding of libthrift.so (the C ABI in include/thrift.h).

Argument marshalling only: torch provides device memory and the current
stream; every step of the path runs in the library's HIP kernels.  There is
no fallback: if the library is missing or the tensors are not on a GPU, the
call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
SO_PATH = os.path.join(HERE, "libthrift.so")

THRIFT_F16, THRIFT_BF16, THRIFT_F32 = 0, 1, 2
_DT = {torch.float16: THRIFT_F16, torch.bfloat16: THRIFT_BF16, torch.float32: THRIFT_F32}


class ThriftError(RuntimeError):
    pass


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "Hq", "Hkv", "N", "d", "block", "causal")]


_lib = None
SYMBOLS = ("thrift_quantize", "thrift_select_workspace_bytes", "thrift_list_entries", "thrift_select",
           "thrift_select_noalloc", "thrift_select_ex", "thrift_block_scores",
           "thrift_attn_fwd", "thrift_attn_fwd_wsum", "thrift_attn_fwd_ex", "thrift_attn_workspace_bytes",
           "thrift_status_str")


def lib() -> ctypes.CDLL:
    """Load libthrift.so (built in-tree by fp16_long_context_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(SO_PATH):
            raise ThriftError(f"{SO_PATH} is not built; run `python -m fp16_long_context_amd.build`")
        L = ctypes.CDLL(SO_PATH)
        P, i32, f32, f64, sz, i64 = (ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_double, ctypes.c_size_t,
                                     ctypes.c_int64)
        SP = ctypes.POINTER(Shape)
        L.thrift_quantize.argtypes = [SP, i32] + [P] * 12 + [P]
        L.thrift_quantize.restype = i32
        L.thrift_select_workspace_bytes.argtypes = [SP]
        L.thrift_select_workspace_bytes.restype = sz
        L.thrift_list_entries.argtypes = [SP]
        L.thrift_list_entries.restype = i64
        L.thrift_select.argtypes = [SP, f64, P, P, P, P, P, sz, P]
        L.thrift_select.restype = i32
        L.thrift_select_noalloc.argtypes = [SP, f64, P, P, P, P, P]
        L.thrift_select_noalloc.restype = i32
        L.thrift_select_ex.argtypes = [SP, f64, i32, P, P, P, P, P, sz, P]
        L.thrift_select_ex.restype = i32
        L.thrift_block_scores.argtypes = [SP, i32, P, P, P, P, sz, P]
        L.thrift_block_scores.restype = i32
        for fn in (L.thrift_attn_fwd, L.thrift_attn_fwd_wsum):
            fn.argtypes = [SP, f32] + [P] * 11 + [P, i32, P, P, sz, P]
            fn.restype = i32
        L.thrift_attn_fwd_ex.argtypes = [SP, f32] + [P] * 11 + [P, i32, P, P, sz, P, i32, P]
        L.thrift_attn_fwd_ex.restype = i32
        L.thrift_attn_workspace_bytes.argtypes = [SP]
        L.thrift_attn_workspace_bytes.restype = sz
        L.thrift_status_str.argtypes = [i32]
        L.thrift_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_str(rc: int) -> str:
    return lib().thrift_status_str(rc).decode()


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ThriftError(f"{what}: {status_str(rc)} ({rc})")


def make_shape(B, Hq, Hkv, N, d, causal=True, block=64) -> Shape:
    return Shape(B, Hq, Hkv, N, d, block, int(causal))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need_gpu(*ts):
    for t in ts:
        if not (t.is_cuda and t.is_contiguous()):
            raise ThriftError("tensors must be contiguous and on a GPU")
        if t.device != ts[0].device:
            raise ThriftError(f"tensors must all be on one GPU ({ts[0].device} and {t.device})")


def alloc_quantized(B, Hq, Hkv, N, d, device) -> dict:
    """Output buffers of quantize (layouts as in include/thrift.h)."""
    nb = N // 64
    u8 = dict(dtype=torch.uint8, device=device)
    return {
        "q16": torch.empty((B, Hq, N, d), dtype=torch.float16, device=device),
        "k16": torch.empty((B, Hkv, N, d), dtype=torch.float16, device=device),
        "v16": torch.empty((B, Hkv, nb, d, 64), dtype=torch.float16, device=device),
        "q4": torch.empty((B, Hq, N, d // 2), **u8), "q4s": torch.empty((B, Hq, N, d // 32), **u8),
        "k4": torch.empty((B, Hkv, N, d // 2), **u8), "k4s": torch.empty((B, Hkv, N, d // 32), **u8),
        "v4": torch.empty((B, Hkv, nb, d, 32), **u8), "v4s": torch.empty((B, Hkv, nb, d, 2), **u8),
    }


def _check_quantized(r: dict, B, Hq, Hkv, N, d) -> None:
    """Every buffer of a quantize output dict has the shape and dtype
    alloc_quantized gives it (the C ABI sees bare pointers, so this is the
    only place a wrong buffer can be caught before the kernels touch it)."""
    want = alloc_quantized(B, Hq, Hkv, N, d, "meta")
    for n, t in want.items():
        if n not in r:
            raise ThriftError(f"quantized buffer {n} missing")
        x = r[n]
        if not isinstance(x, torch.Tensor) or tuple(x.shape) != tuple(t.shape) or x.dtype != t.dtype:
            got = (tuple(x.shape), x.dtype) if isinstance(x, torch.Tensor) else type(x)
            raise ThriftError(f"quantized buffer {n} must be {tuple(t.shape)} {t.dtype}; got {got}")


def quantize(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: dict | None = None) -> dict:
    """FP16 copies and MXFP4 codes of q [B,Hq,N,d], k/v [B,Hkv,N,d] (fp16 or bf16).
    Layouts as in include/thrift.h (v16/v4/v4s are tile-major).  `out` may
    hold preallocated buffers from alloc_quantized."""
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.float16, torch.bfloat16):
        raise ThriftError("q, k, v must share dtype fp16 or bf16")
    if q.dim() != 4 or k.dim() != 4:
        raise ThriftError("q, k, v must be 4-D [B,H,N,d]")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, N, d) or tuple(v.shape) != (B, Hkv, N, d):
        raise ThriftError(f"k and v must be [B,Hkv,N,d] = [{B},Hkv,{N},{d}]; got {tuple(k.shape)}, {tuple(v.shape)}")
    dev = q.device
    r = alloc_quantized(B, Hq, Hkv, N, d, dev) if out is None else out
    _check_quantized(r, B, Hq, Hkv, N, d)
    _need_gpu(q, k, v, *r.values())
    s = make_shape(B, Hq, Hkv, N, d)
    rc = lib().thrift_quantize(ctypes.byref(s), _DT[q.dtype], _ptr(q), _ptr(k), _ptr(v),
                               *[_ptr(r[n]) for n in ("q16", "k16", "v16", "q4", "q4s", "k4", "k4s", "v4", "v4s")],
                               _stream(dev))
    _check(rc, "thrift_quantize")
    return r


def list_entries(B, Hq, N, causal=True) -> int:
    s = make_shape(B, Hq, 1, N, 64, causal)
    return int(lib().thrift_list_entries(ctypes.byref(s)))


SCORES = {"pooled_mean": 0, "max_pooled": 1, "norm_weighted": 2, "block_max": 3}


def select(q16: torch.Tensor, k16: torch.Tensor, frac: float, causal: bool = True, workspace=None, idx=None,
           n16=None, score: str = "pooled_mean"):
    """Traversal lists: idx (int32, per-row FP16 list then FP4 list) and n16 [B,Hq,nb].
    idx, n16 and the workspace may be preallocated.  score: the block score
    ("pooled_mean" = thrift_select; the others go through thrift_select_ex)."""
    if score not in SCORES:
        raise ThriftError(f"score must be one of {sorted(SCORES)}")
    if q16.dim() != 4 or k16.dim() != 4 or q16.dtype != torch.float16 or k16.dtype != torch.float16:
        raise ThriftError("q16 and k16 must be 4-D fp16 tensors")
    B, Hq, N, d = q16.shape
    Hkv = k16.shape[1]
    if tuple(k16.shape) != (B, Hkv, N, d):
        raise ThriftError(f"k16 must be [B,Hkv,N,d] = [{B},Hkv,{N},{d}]; got {tuple(k16.shape)}")
    s = make_shape(B, Hq, Hkv, N, d, causal)
    L = lib()
    ents = int(L.thrift_list_entries(ctypes.byref(s)))
    wsb = int(L.thrift_select_workspace_bytes(ctypes.byref(s)))
    if ents <= 0 or wsb <= 0:
        raise ThriftError("unsupported shape")
    if idx is None:
        idx = torch.empty(ents, dtype=torch.int32, device=q16.device)
    if n16 is None:
        n16 = torch.empty((B, Hq, N // 64), dtype=torch.int32, device=q16.device)
    if idx.numel() < ents or n16.numel() < B * Hq * (N // 64) or idx.dtype != torch.int32 or n16.dtype != torch.int32:
        raise ThriftError("idx/n16 buffers too small or not int32")
    if workspace is None:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=q16.device)
    _need_gpu(q16, k16, idx, n16, workspace)
    wsn = workspace.numel() * workspace.element_size()
    if score == "pooled_mean":
        rc = L.thrift_select(ctypes.byref(s), float(frac), _ptr(q16), _ptr(k16), _ptr(idx), _ptr(n16),
                             _ptr(workspace), wsn, _stream(q16.device))
    else:
        rc = L.thrift_select_ex(ctypes.byref(s), float(frac), SCORES[score], _ptr(q16), _ptr(k16), _ptr(idx),
                                _ptr(n16), _ptr(workspace), wsn, _stream(q16.device))
    _check(rc, "thrift_select")
    return idx, n16


def block_scores(q16: torch.Tensor, k16: torch.Tensor, score: str = "pooled_mean", causal: bool = True):
    """thrift_block_scores: the fp32 block scores sigma(i, j) the selection ranks,
    in the list layout (flat, thrift_list_entries entries)."""
    if score not in SCORES:
        raise ThriftError(f"score must be one of {sorted(SCORES)}")
    if q16.dim() != 4 or k16.dim() != 4 or q16.dtype != torch.float16 or k16.dtype != torch.float16:
        raise ThriftError("q16 and k16 must be 4-D fp16 tensors")
    B, Hq, N, d = q16.shape
    Hkv = k16.shape[1]
    if tuple(k16.shape) != (B, Hkv, N, d):
        raise ThriftError(f"k16 must be [B,Hkv,N,d] = [{B},Hkv,{N},{d}]; got {tuple(k16.shape)}")
    s = make_shape(B, Hq, Hkv, N, d, causal)
    L = lib()
    ents = int(L.thrift_list_entries(ctypes.byref(s)))
    wsb = int(L.thrift_select_workspace_bytes(ctypes.byref(s)))
    if ents <= 0 or wsb <= 0:
        raise ThriftError("unsupported shape")
    out = torch.empty(ents, dtype=torch.float32, device=q16.device)
    ws = torch.empty(wsb, dtype=torch.uint8, device=q16.device)
    _need_gpu(q16, k16, out, ws)
    rc = L.thrift_block_scores(ctypes.byref(s), SCORES[score], _ptr(q16), _ptr(k16), _ptr(out), _ptr(ws), wsb,
                               _stream(q16.device))
    _check(rc, "thrift_block_scores")
    return out


def select_noalloc(q16: torch.Tensor, k16: torch.Tensor, frac: float, causal: bool = True, idx=None, n16=None):
    """thrift_select_noalloc: the lists of select() with the pooled means in the
    library's static device array (no workspace; pass idx and n16 to allocate
    nothing here either).  Calls that overlap on one GPU race."""
    if q16.dim() != 4 or k16.dim() != 4 or q16.dtype != torch.float16 or k16.dtype != torch.float16:
        raise ThriftError("q16 and k16 must be 4-D fp16 tensors")
    B, Hq, N, d = q16.shape
    Hkv = k16.shape[1]
    if tuple(k16.shape) != (B, Hkv, N, d):
        raise ThriftError(f"k16 must be [B,Hkv,N,d] = [{B},Hkv,{N},{d}]; got {tuple(k16.shape)}")
    s = make_shape(B, Hq, Hkv, N, d, causal)
    L = lib()
    ents = int(L.thrift_list_entries(ctypes.byref(s)))
    if ents <= 0:
        raise ThriftError("unsupported shape")
    if idx is None:
        idx = torch.empty(ents, dtype=torch.int32, device=q16.device)
    if n16 is None:
        n16 = torch.empty((B, Hq, N // 64), dtype=torch.int32, device=q16.device)
    if idx.numel() < ents or n16.numel() < B * Hq * (N // 64) or idx.dtype != torch.int32 or n16.dtype != torch.int32:
        raise ThriftError("idx/n16 buffers too small or not int32")
    _need_gpu(q16, k16, idx, n16)
    rc = L.thrift_select_noalloc(ctypes.byref(s), float(frac), _ptr(q16), _ptr(k16), _ptr(idx), _ptr(n16),
                                 _stream(q16.device))
    _check(rc, "thrift_select_noalloc")
    return idx, n16


# row-sum readings of the attention call: "p" (thrift_attn_fwd), "weights"
# (thrift_attn_fwd_wsum), "log" (the weights reading with exp-free FP4 codes,
# thrift_attn_fwd_ex rowsum 2)
ROWSUM = {"p": 0, "weights": 1, "log": 2}


def attn_workspace_bytes(B, Hq, Hkv, N, d, causal=True) -> int:
    s = make_shape(B, Hq, Hkv, N, d, causal)
    return int(lib().thrift_attn_workspace_bytes(ctypes.byref(s)))


def attn_fwd(qz: dict, idx: torch.Tensor, n16: torch.Tensor, causal: bool = True, sm_scale: float = 0.0,
             out_dtype=torch.float32, want_lse: bool = False, out=None, lse=None, workspace=None,
             rowsum: str = "p", events=None):
    """Fused FP16/MXFP4 attention.  Returns (out [B,Hq,N,d], lse [B,Hq,N] or None).
    out, lse and the workspace (uint8, thrift_attn_workspace_bytes) may be preallocated.
    rowsum "p" (thrift_attn_fwd): the row sum adds the unquantized p;
    "weights" (thrift_attn_fwd_wsum): it adds the weights the P.V products use;
    "log" (thrift_attn_fwd_ex, rowsum 2): as "weights", with FP4 P codes taken
    without an exponential.
    events: optional four torch.cuda.Event(enable_timing=True), recorded on the
    current stream before, between and after the three kernels (thrift_attn_fwd_ex)."""
    if rowsum not in ROWSUM:
        raise ThriftError(f"rowsum must be one of {sorted(ROWSUM)}")
    q16 = qz["q16"]
    if q16.dim() != 4 or qz["k16"].dim() != 4:
        raise ThriftError("q16/k16 must be 4-D")
    B, Hq, N, d = q16.shape
    Hkv = qz["k16"].shape[1]
    _check_quantized(qz, B, Hq, Hkv, N, d)
    s = make_shape(B, Hq, Hkv, N, d, causal)
    L = lib()
    ents = int(L.thrift_list_entries(ctypes.byref(s)))
    wsb = int(L.thrift_attn_workspace_bytes(ctypes.byref(s)))
    if ents <= 0 or wsb <= 0:
        raise ThriftError("unsupported shape")
    if idx.dtype != torch.int32 or n16.dtype != torch.int32:
        raise ThriftError("idx and n16 must be int32")
    if idx.numel() < ents or n16.numel() < B * Hq * (N // 64):
        raise ThriftError(f"idx needs {ents} entries and n16 {B * Hq * (N // 64)}; "
                          f"got {idx.numel()} and {n16.numel()}")
    if out is None:
        out = torch.empty((B, Hq, N, d), dtype=out_dtype, device=q16.device)
    if tuple(out.shape) != (B, Hq, N, d) or out.dtype not in _DT:
        raise ThriftError("out must be [B,Hq,N,d] fp32/fp16/bf16")
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q16.device)
    if lse is not None:
        if lse.dtype != torch.float32 or lse.numel() < B * Hq * N:
            raise ThriftError(f"lse must be fp32 with at least {B * Hq * N} elements")
    if workspace is None:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=q16.device)
    _need_gpu(*qz.values(), idx, n16, out, workspace, *([lse] if lse is not None else []))
    args = [ctypes.byref(s), float(sm_scale),
            *[_ptr(qz[n]) for n in ("q16", "k16", "v16", "q4", "q4s", "k4", "k4s", "v4", "v4s")],
            _ptr(idx), _ptr(n16), _ptr(out), _DT[out.dtype], _ptr(lse), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(q16.device)]
    if events is None and rowsum != "log":
        rc = (L.thrift_attn_fwd if rowsum == "p" else L.thrift_attn_fwd_wsum)(*args)
    else:
        evs = None
        if events is not None:
            if len(events) != 4:
                raise ThriftError("events must hold four torch.cuda.Event")
            for e in events:  # make sure each event exists on the device
                e.record()
            evs = (ctypes.c_void_p * 4)(*[e.cuda_event for e in events])
        rc = L.thrift_attn_fwd_ex(*args, ROWSUM[rowsum], evs)
    _check(rc, "thrift_attn_fwd")
    return out, lse


def attention(q, k, v, frac: float = 0.05, causal: bool = True, sm_scale: float = 0.0, out_dtype=torch.float32):
    """quantize -> select -> fused attention on the current stream."""
    qz = quantize(q, k, v)
    idx, n16 = select(qz["q16"], qz["k16"], frac, causal)
    out, _ = attn_fwd(qz, idx, n16, causal, sm_scale, out_dtype)
    return out
