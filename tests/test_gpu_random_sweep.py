"""GPU parity on a seeded random sweep of small problems.

Each seed draws a shape (batch, KV heads, GQA group of 1 to 5, head dim,
1 to 40 blocks, causal or not), an FP16 fraction, an input dtype and one of
four input distributions, and compares the HIP path with the CPU oracle at
the bars of the fixed cases: FP16 copies, MXFP4 codes and scales, lists and
counts bit-exact; attention within 2e-3 * max|O| and LSE within 1e-3 on a
row sample.  One distribution makes the key blocks near-duplicates of one
row, so that many block scores of a row fall within the fp32 chains' error
bound of the cut-off and the selection ranks them by their fp64 chains.
"""
import numpy as np
import pytest
import torch

from tests.test_gpu_parity import run_case

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


@pytest.mark.parametrize("seed", range(24))
def test_random_problem(seed):
    q, k, v, frac, causal, rows, label = draw(seed)
    run_case(q, k, v, frac, causal, rows=rows, label=label)
