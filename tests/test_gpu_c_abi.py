"""The C ABI driven from a plain C++ program (tests/c_abi/c_abi_check.cpp:
the HIP runtime only, no Python binding, no torch) against the oracle on the
same inputs: lists bit-exact, attention within the parity bar."""
import os
import struct
import subprocess

import numpy as np
import pytest

import oracle
from fp16_long_context_amd import synth

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _exe():
    from tests.c_abi import build as cbuild

    if not os.path.exists(cbuild.EXE):
        cbuild.build()
    return cbuild.EXE


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal,frac", [
    (1, 4, 2, 320, 64, 1, 0.3),
    (2, 2, 1, 256, 128, 1, 0.05),
    (1, 3, 1, 192, 128, 0, 0.5),
])
def test_c_program_against_oracle(tmp_path, B, Hq, Hkv, N, d, causal, frac):
    print(f"[case] c_abi B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal} frac={frac}", flush=True)
    q, k, v = synth.random_qkv(B, Hq, Hkv, N, d, "fp16", seed=300 + N + d, scale=1.5)
    qb, kb, vb = synth.bits(q), synth.bits(k), synth.bits(v)
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(fin, "wb") as f:
        f.write(struct.pack("<6id", B, Hq, Hkv, N, d, causal, frac))
        for a in (qb, kb, vb):
            f.write(np.ascontiguousarray(a).tobytes())
    r = subprocess.run([_exe(), str(fin), str(fout)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr

    nb = N // 64
    ents = oracle.list_entries(B, Hq, N, bool(causal))
    raw = np.fromfile(fout, dtype=np.uint8)
    off = 0

    def take(dt, n):
        nonlocal off
        a = raw[off:off + n * np.dtype(dt).itemsize].view(dt)
        off += n * np.dtype(dt).itemsize
        return a

    assert take(np.int32, 1)[0] == 0
    idx, n16 = take(np.int32, ents), take(np.int32, B * Hq * nb)
    out, lse = take(np.float32, B * Hq * N * d), take(np.float32, B * Hq * N)
    assert off == raw.size

    qz = oracle.quantize(qb, kb, vb, "fp16")
    sel = oracle.select(qz["q16"], qz["k16"], frac, bool(causal))
    res = oracle.attn_rows(qz, sel, oracle.all_rows(B, Hq, N), bool(causal))
    assert np.array_equal(idx, sel["idx"]) and np.array_equal(n16, sel["n16"].ravel())
    err = np.abs(out.reshape(-1, d).astype(np.float64) - res["out"]).max() / np.abs(res["out"]).max()
    lerr = np.abs(lse.astype(np.float64) - res["lse"]).max()
    print(f"[case] c_abi: max|dO|/max|O| = {err:.3e}, max|dLSE| = {lerr:.3e}", flush=True)
    assert err <= TOL and lerr <= 1e-3
