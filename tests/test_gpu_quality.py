"""GPU quality studies through the library: the planted-needle error of the
mixed path against the all-FP16 output at several sequence lengths.  The
outputs these errors come from are the ones the parity tests pin to the
oracle; here only the method's quality invariant is asserted."""
import math

import pytest

from fp16_long_context_amd import quality

pytestmark = pytest.mark.gpu


def test_length_sweep_mixed_beats_fp4():
    rows = quality.length_sweep([4096, 16384], "long_128k", log=lambda s: print(s, flush=True))
    assert [r["N"] for r in rows] == [4096, 16384]
    for r in rows:
        for key in ("err_mixed", "err_fp4", "needle_err_mixed", "needle_err_fp4"):
            assert math.isfinite(r[key]) and 0.0 < r[key] < 1.0, (key, r)
        assert r["mixed_below_fp4"], r
        assert r["needles"] == 2048


def test_attribution_small():
    r = quality.attribution("llama8b_16k", N=2048, log=lambda s: print(s, flush=True))
    nb = 2048 // 64
    assert r["pairs"] == 32 * nb * (nb + 1) // 2
    for key in ("spearman_score", "spearman_mass"):
        assert -1.0 <= r[key] <= 1.0
    for key in ("capture_score", "capture_mass", "capture_blockmax", "capture_select"):
        assert r[key] <= 1.0 + 1e-9
    assert 0.0 < r["concentration"] <= 1.0 + 1e-9


@pytest.mark.parametrize("workload", ["long_128k", "llama8b_16k"])
def test_heuristics_small(workload):
    rows = quality.heuristics(workload, N=2048, log=lambda s: print(s, flush=True))
    by = {r["heuristic"]: r for r in rows}
    assert list(by) == ["fp4_only", "pooled_mean", "max_pooled", "norm_weighted", "block_max"]
    assert by["fp4_only"]["fp16_tile_share"] == 0.0
    # the same budget rule at 64-row blocks gives every score the same FP16 share
    for name in ("max_pooled", "block_max", "norm_weighted"):
        assert by[name]["fp16_tile_share"] == by["pooled_mean"]["fp16_tile_share"]
        assert by[name]["select_ms"] > 0.0
    for r in rows:
        assert math.isfinite(r["err"]) and 0.0 < r["err"] < 1.0, r
        assert math.isfinite(r["needle_err"]) and 0.0 < r["needle_err"] < 1.0, r
