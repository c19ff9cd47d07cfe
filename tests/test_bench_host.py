"""Host arithmetic of bench.py (no GPU): the flop and byte counts behind its
JSON line, the VALU-issue roofline of the FP4 walk, the traffic summary's
source check, and the one-GPU guard.  Expected values are the headline
workload's figures worked out by hand (B=1, Hq=32, Hkv=8, N=131072, d=128):
140.7 TFLOP of attention, 3.649 GB moved by the quantizer, 1.611 GB by the
selection."""
import dataclasses
import hashlib
import os
import subprocess
import sys

import pytest
import torch

import bench
from fp16_long_context_amd import synth

W = synth.WORKLOADS["long_128k"]
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_attention_flops_at_128k():
    # 4 d flops (2d for Q K^T, 2d for P V) per causally valid query-key pair
    assert bench.attn_flops(W) == 4.0 * 128 * 32 * (131072 * 131073 // 2)
    assert bench.attn_flops(W) / 1e12 == pytest.approx(140.74, abs=0.01)


def test_fp16_tile_flops_count_diagonal_tiles_as_2080_pairs():
    # one head, four blocks; every row keeps its diagonal, rows 1-3 also block 0
    w = dataclasses.replace(W, B=1, Hq=1, N=256)
    n16 = torch.tensor([[[1, 2, 2, 2]]], dtype=torch.int32)
    assert bench.fp16_tile_flops(w, n16, 0.05) == 4 * 128 * (4 * 2080 + 3 * 4096)
    # a diagonal tile holds the 64 * 65 / 2 pairs on or below its diagonal
    assert 64 * 65 // 2 == 2080
    # fraction 0 keeps no FP16 tile, so no diagonal is counted
    assert bench.fp16_tile_flops(w, torch.zeros_like(n16), 0.0) == 0.0


def test_quantize_and_select_bytes_at_128k():
    assert bench.quantize_bytes(W) / 1e9 == pytest.approx(3.649, abs=1e-3)
    assert bench.select_bytes(W) / 1e9 == pytest.approx(1.611, abs=1e-3)


def test_alu_roofline_of_the_fp4_walk():
    nb = 2048
    n16 = torch.full((1, 32, nb), 5, dtype=torch.int32)  # 5 FP16 tiles in every row
    r = bench.roofline_alu(W, n16, 54.0)
    # every causally valid tile not on an FP16 list, as two 32-row waves
    assert r["block_waves"] == 2 * (32 * nb * (nb + 1) // 2 - 32 * nb * 5)
    # the walk's VALU cycles per block-wave: 736 (at the measured costs)
    assert r["valu_cycles_per_block_wave"] == pytest.approx(736.0, abs=0.1)
    assert r["mfma_cycles_per_block_wave"] == 8 * 32.0
    # 1024 SIMDs at 2.4 GHz over 736 cycles: 3.34 G block-waves per second
    assert r["peak"] == pytest.approx(3.339, abs=1e-3)
    assert r["achieved"] == pytest.approx(r["block_waves"] / 54e-3 / 1e9, rel=1e-4)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-3)
    assert r["frac"] < r["frac_valu_plus_mfma"] < 1.0


def test_traffic_is_reported_only_for_the_profiled_source(tmp_path, monkeypatch):
    src = tmp_path / "attn_fwd.hip"
    src.write_text("// kernel, version 1\n")
    summary = tmp_path / "traffic.txt"
    summary.write_text(f"source_sha256: {hashlib.sha256(src.read_bytes()).hexdigest()}\n"
                       "hbm_bytes_per_launch: 9.812423e+10\n")
    monkeypatch.setattr(bench, "ATTN_SRC", str(src))
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(summary))
    assert bench.read_traffic() == pytest.approx(9.812423e10)
    src.write_text("// kernel, version 2\n")
    assert bench.read_traffic() is None  # counters of another source are not reported
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(tmp_path / "missing.txt"))
    assert bench.read_traffic() is None


def test_cpu_model_names_the_host():
    assert bench.cpu_model().strip()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
