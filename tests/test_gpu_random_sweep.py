"""GPU parity on a seeded random sweep of small problems.

Each seed draws a shape (batch, KV heads, GQA group of 1 to 5, head dim,
1 to 40 blocks, causal or not), an FP16 fraction, an input dtype and one of
four input distributions, and compares the HIP path with the CPU oracle at
the bars of the fixed cases: FP16 copies, MXFP4 codes and scales, lists and
counts bit-exact; attention within 2e-3 * max|O| and LSE within 1e-3 on a
row sample.  One distribution makes the key blocks near-duplicates of one
row, so that many block scores of a row fall within the fp32 chains' error
bound of the cut-off and the selection ranks them by their fp64 chains.
Every problem runs under the three row-sum readings; half of them also under
the three other block scores (lists and fp32 scores bit-exact, attention
over their lists within the bar).
"""
import numpy as np
import pytest
import torch

import oracle
from fp16_long_context_amd import binding, synth
from tests.test_gpu_parity import TOL, run_case, say

pytestmark = pytest.mark.gpu

FRACS = [0.0, 0.001, 0.01, 0.05, 0.1, 0.3, 0.7, 1.0]
KINDS = ["normal", "student-t(3)", "near-duplicate key blocks", "wide channel range"]


def draw(seed):
    g = np.random.default_rng(7000 + seed)
    B, Hkv, group = int(g.integers(1, 3)), int(g.integers(1, 3)), int(g.integers(1, 6))
    Hq, d, N = Hkv * group, int(g.choice([64, 128])), 64 * int(g.integers(1, 41))
    causal = bool(g.integers(0, 4) > 0)
    frac = float(g.choice(FRACS))
    dtype = torch.float16 if g.integers(0, 2) else torch.bfloat16
    kind = int(g.integers(0, len(KINDS)))
    sq, sk = (B, Hq, N, d), (B, Hkv, N, d)
    if kind == 0:
        q, k = g.standard_normal(sq), g.standard_normal(sk)
    elif kind == 1:
        q, k = np.clip(g.standard_t(3, sq), -20, 20), np.clip(g.standard_t(3, sk), -20, 20)
    elif kind == 2:
        q = g.standard_normal(sq)
        k = g.standard_normal(d) + 2.0 ** -9 * g.standard_normal(sk)
    else:
        sc = 2.0 ** g.integers(-6, 5, size=d)
        q, k = g.standard_normal(sq) * sc, g.standard_normal(sk) / sc
    v = g.standard_normal(sk)
    scale = float(g.choice([0.5, 1.0, 2.0]))
    t = lambda x: torch.from_numpy((scale * x).astype(np.float32)).to(dtype)
    rows_total = B * Hq * N
    rows = np.unique(np.concatenate([g.integers(0, rows_total, size=min(rows_total, 192)),
                                     np.arange(max(0, rows_total - 64), rows_total)]))
    label = (f"sweep seed {seed}: {KINDS[kind]}, scale {scale}")
    return t(q), t(k), t(v), frac, causal, rows, label


@pytest.mark.parametrize("rowsum", ["p", "weights", "log"])
@pytest.mark.parametrize("seed", range(24))
def test_random_problem(seed, rowsum):
    q, k, v, frac, causal, rows, label = draw(seed)
    run_case(q, k, v, frac, causal, rows=rows, label=label, rowsum=rowsum)


@pytest.mark.parametrize("score", ["max_pooled", "norm_weighted", "block_max"])
@pytest.mark.parametrize("seed", range(12))
def test_random_problem_other_scores(seed, score):
    q, k, v, frac, causal, rows, label = draw(seed)
    dt = "fp16" if q.dtype == torch.float16 else "bf16"
    B, Hq, N, d = q.shape
    say(f"[case] {label} score={score} B={B} Hq={Hq} Hkv={k.shape[1]} N={N} d={d} frac={frac} causal={causal} {dt}")
    qo = oracle.quantize(synth.bits(q), synth.bits(k), synth.bits(v), dt)
    so = oracle.select(qo["q16"], qo["k16"], frac, causal, score=score)
    dev = torch.device("cuda:0")
    qz = binding.quantize(q.to(dev), k.to(dev), v.to(dev))
    idx, n16 = binding.select(qz["q16"], qz["k16"], frac, causal, score=score)
    sc = binding.block_scores(qz["q16"], qz["k16"], score, causal)
    out, lse = binding.attn_fwd(qz, idx, n16, causal, want_lse=True)
    torch.cuda.synchronize()
    assert np.array_equal(n16.cpu().numpy(), so["n16"]), f"{label} {score}: n16 differs"
    assert np.array_equal(idx.cpu().numpy(), so["idx"]), f"{label} {score}: idx differs"
    assert np.array_equal(sc.cpu().numpy(), so["scores"].astype(np.float32)), f"{label} {score}: scores differ"
    res = oracle.attn_rows(qo, so, rows, causal)
    og = out.reshape(-1, d).cpu().numpy().astype(np.float64)[rows]
    lg = lse.reshape(-1).cpu().numpy().astype(np.float64)[rows]
    err = np.abs(og - res["out"]).max() / np.abs(res["out"]).max()
    lerr = np.abs(lg - res["lse"]).max()
    say(f"[case] {label} {score}: max|dO|/max|O| = {err:.3e}, max|dLSE| = {lerr:.3e}")
    assert err <= TOL and lerr <= 1e-3
