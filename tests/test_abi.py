"""The C ABI on the CPU: the library loads, exports every function that
include/thrift.h declares, and rejects bad arguments on the host (these calls
never reach a device: validation precedes every HIP call)."""
import ctypes
import math
import os
import re

import pytest

from fp16_long_context_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, EINVAL, EUNSUP, EWS, EHIP = 0, -1, -2, -3, -4
FAKE = ctypes.c_void_p(0x10000)  # aligned, non-null; never dereferenced on these paths


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.SO_PATH):
        from fp16_long_context_amd import build

        build.build()
    return binding.lib()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "thrift.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(thrift_\w+)\s*\(", src)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert set(names) == set(binding.SYMBOLS)
    for n in names:
        assert hasattr(L, n), n


def shape(**kw):
    base = dict(B=1, Hq=4, Hkv=2, N=1024, d=128, causal=1, block=64)
    base.update(kw)
    return binding.make_shape(base["B"], base["Hq"], base["Hkv"], base["N"], base["d"], base["causal"], base["block"])


def quant(L, s, dtype=0, ptrs=None):
    ptrs = ptrs or [FAKE] * 12
    return L.thrift_quantize(ctypes.byref(s), dtype, *ptrs, None)


def sel(L, s, frac=0.05, ptrs=None, ws=FAKE, wsb=1 << 40):
    ptrs = ptrs or [FAKE] * 4
    return L.thrift_select(ctypes.byref(s), frac, *ptrs, ws, wsb, None)


def attn(L, s, out_dtype=2, ptrs=None, lse=None, sm=0.0, ws=FAKE, wsb=1 << 40):
    """Both attention entry points validate alike; returns their common code."""
    ptrs = ptrs or [FAKE] * 12
    codes = {fn(ctypes.byref(s), sm, *ptrs[:11], ptrs[11], out_dtype, lse, ws, wsb, None)
             for fn in (L.thrift_attn_fwd, L.thrift_attn_fwd_wsum)}
    for rowsum in (0, 1):
        codes.add(L.thrift_attn_fwd_ex(ctypes.byref(s), sm, *ptrs[:11], ptrs[11], out_dtype, lse, ws, wsb, None,
                                       rowsum, None))
    assert len(codes) == 1, codes
    return codes.pop()


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), EINVAL), (dict(Hq=0), EINVAL), (dict(Hkv=-1), EINVAL), (dict(N=0), EINVAL),
    (dict(Hq=6, Hkv=4), EINVAL), (dict(causal=2), EINVAL), (dict(d=96), EUNSUP), (dict(d=256), EUNSUP),
    (dict(block=128), EUNSUP), (dict(block=0), EINVAL), (dict(N=1000), EUNSUP), (dict(N=64 * 8193), EUNSUP),
])
def test_bad_shapes(L, kw, code):
    s = shape(**kw)
    assert quant(L, s) == code
    assert sel(L, s) == code
    assert attn(L, s) == code
    assert L.thrift_select_workspace_bytes(ctypes.byref(s)) == 0
    assert L.thrift_attn_workspace_bytes(ctypes.byref(s)) == 0
    assert L.thrift_list_entries(ctypes.byref(s)) == 0


def test_null_shape(L):
    assert L.thrift_quantize(None, 0, *[FAKE] * 12, None) == EINVAL
    assert L.thrift_select(None, 0.1, *[FAKE] * 4, FAKE, 1 << 40, None) == EINVAL
    assert L.thrift_attn_fwd(None, 0.0, *[FAKE] * 12, 2, None, FAKE, 1 << 40, None) == EINVAL
    assert L.thrift_attn_fwd_wsum(None, 0.0, *[FAKE] * 12, 2, None, FAKE, 1 << 40, None) == EINVAL
    assert L.thrift_select_workspace_bytes(None) == 0 and L.thrift_list_entries(None) == 0
    assert L.thrift_attn_workspace_bytes(None) == 0


@pytest.mark.parametrize("slot", range(12))
def test_null_and_misaligned_pointers(L, slot):
    s = shape()
    for bad in (None, ctypes.c_void_p(0x10008)):
        p = [FAKE] * 12
        p[slot] = bad
        assert quant(L, s, ptrs=p) == EINVAL
        assert attn(L, s, ptrs=p) == EINVAL
        if slot < 4:
            assert sel(L, s, ptrs=p[:4]) == EINVAL
    assert attn(L, s, lse=ctypes.c_void_p(0x10004)) == EINVAL


def test_bad_values(L):
    s = shape()
    assert quant(L, s, dtype=2) == EINVAL and quant(L, s, dtype=-1) == EINVAL
    for f in (-0.01, 1.0001, math.nan, math.inf):
        assert sel(L, s, frac=f) == EINVAL
    assert attn(L, s, out_dtype=3) == EINVAL
    assert attn(L, s, sm=math.nan) == EINVAL and attn(L, s, sm=math.inf) == EINVAL


def test_attn_ex_rejects_unknown_rowsum(L):
    s = shape()
    for rowsum in (-1, 2):
        assert L.thrift_attn_fwd_ex(ctypes.byref(s), 0.0, *[FAKE] * 12, 2, None, FAKE, 1 << 40, None, rowsum,
                                    None) == EINVAL


def test_workspace(L):
    s = shape()
    need = L.thrift_select_workspace_bytes(ctypes.byref(s))
    assert need == 4 * 16 * 128 * 1 * (4 + 2)
    assert sel(L, s, ws=None) == EWS
    assert sel(L, s, wsb=need - 1) == EWS
    assert sel(L, s, ws=ctypes.c_void_p(0x10004), wsb=need) == EINVAL
    # attention: per query block of every (b, head), two waves of 64 lanes x
    # (d/2 + 2) fp32 partial state, plus one int32 redo flag
    need_a = L.thrift_attn_workspace_bytes(ctypes.byref(s))
    assert need_a == 1 * 4 * 16 * (2 * 64 * (128 // 2 + 2) + 1) * 4
    assert attn(L, s, ws=None) == EWS
    assert attn(L, s, wsb=need_a - 1) == EWS
    assert attn(L, s, ws=ctypes.c_void_p(0x10004), wsb=need_a) == EINVAL


def test_list_entries(L):
    assert L.thrift_list_entries(ctypes.byref(shape(B=2, Hq=4, N=1024))) == 2 * 4 * 16 * 17 // 2
    assert L.thrift_list_entries(ctypes.byref(shape(B=2, Hq=4, N=1024, causal=0))) == 2 * 4 * 16 * 16
    assert binding.list_entries(1, 32, 131072) == 32 * 2048 * 2049 // 2


def test_status_strings(L):
    for c in (OK, EINVAL, EUNSUP, EWS, EHIP, 7):
        assert isinstance(binding.status_str(c), str) and binding.status_str(c)
    assert binding.status_str(EWS) != binding.status_str(EINVAL)


def test_binding_refuses_cpu_tensors():
    import torch

    q = torch.zeros(1, 1, 64, 64, dtype=torch.float16)
    with pytest.raises(binding.ThriftError):
        binding.quantize(q, q, q)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    # no fallback: a missing library is an error, not a silent CPU path
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "SO_PATH", str(tmp_path / "libthrift.so"))
    with pytest.raises(binding.ThriftError):
        binding.lib()
