"""GPU parity of the heuristic variants (thrift_select_ex, thrift_block_scores)
against the oracle's variant scores: lists and counts bit-exact, the fp32
block scores equal to the oracle's fp64 scores rounded to fp32, and the
attention over each variant's lists within 2e-3 * max|O| of the oracle's."""
import numpy as np
import pytest
import torch

import oracle
from fp16_long_context_amd import binding, synth

pytestmark = pytest.mark.gpu
TOL = 2e-3
VARIANTS = ["max_pooled", "norm_weighted", "block_max"]


def say(*a):
    print(*a, flush=True)


def check(q, k, v, frac, score, causal=True, label=""):
    dt = "fp16" if q.dtype == torch.float16 else "bf16"
    B, Hq, N, d = q.shape
    say(f"[case] {label} score={score} B={B} Hq={Hq} Hkv={k.shape[1]} N={N} d={d} frac={frac} causal={causal}")
    qo = oracle.quantize(synth.bits(q), synth.bits(k), synth.bits(v), dt)
    so = oracle.select(qo["q16"], qo["k16"], frac, causal, score=score)
    dev = torch.device("cuda:0")
    qz = binding.quantize(q.to(dev), k.to(dev), v.to(dev))
    idx, n16 = binding.select(qz["q16"], qz["k16"], frac, causal, score=score)
    sc = binding.block_scores(qz["q16"], qz["k16"], score, causal)
    out, _ = binding.attn_fwd(qz, idx, n16, causal)
    torch.cuda.synchronize()
    assert np.array_equal(n16.cpu().numpy(), so["n16"]), f"{label} {score}: n16 differs"
    assert np.array_equal(idx.cpu().numpy(), so["idx"]), f"{label} {score}: idx differs"
    assert np.array_equal(sc.cpu().numpy(), so["scores"].astype(np.float32)), f"{label} {score}: scores differ"
    rows = oracle.all_rows(B, Hq, N)
    res = oracle.attn_rows(qo, so, rows, causal)
    og = out.reshape(-1, d).cpu().numpy().astype(np.float64)
    err = np.abs(og - res["out"]).max() / np.abs(res["out"]).max()
    say(f"[case] {label} {score}: max|dO|/max|O| = {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("score", VARIANTS)
def test_variants_tiny_and_rope(score):
    x = synth.generate("tiny")
    check(x["q"], x["k"], x["v"], 0.1, score, label="tiny")
    y = synth.generate("long_128k", N=1024)
    check(y["q"], y["k"], y["v"], 0.05, score, label="rope@1k")


@pytest.mark.parametrize("score", VARIANTS)
@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal,dtype,frac", [
    (1, 4, 2, 512, 64, True, "fp16", 0.3),
    (1, 3, 3, 320, 128, False, "bf16", 0.3),
    (2, 6, 2, 448, 128, True, "bf16", 0.2),
])
def test_variants_shapes(score, B, Hq, Hkv, N, d, causal, dtype, frac):
    q, k, v = synth.random_qkv(B, Hq, Hkv, N, d, dtype, seed=B * 100 + N, scale=1.5)
    check(q, k, v, frac, score, causal, label="shape")


def test_pooled_mean_scores_equal_the_oracle():
    x = synth.generate("llama8b_16k", N=2048)
    qo = oracle.quantize(synth.bits(x["q"]), synth.bits(x["k"]), synth.bits(x["v"]), "bf16")
    so = oracle.select(qo["q16"], qo["k16"], 0.05, True)
    dev = torch.device("cuda:0")
    qz = binding.quantize(*(x[n].to(dev) for n in ("q", "k", "v")))
    sc = binding.block_scores(qz["q16"], qz["k16"], "pooled_mean")
    assert np.array_equal(sc.cpu().numpy(), so["scores"].astype(np.float32))


def test_block_max_scores_past_one_launch_of_workgroups():
    # 32 heads x 1024 x 1025 / 2 valid block pairs: 16.8 M pairs, more
    # workgroups of 256 threads than one launch addresses (2^32 threads);
    # sampled scores, including the last pairs, must equal the exact ones
    B, Hq, Hkv, N, d = 1, 32, 8, 65536, 64
    q, k, v = synth.random_qkv(B, Hq, Hkv, N, d, "fp16", seed=123)
    dev = torch.device("cuda:0")
    q16, k16 = q.to(dev), k.to(dev)
    say(f"[case] block_max scores B={B} Hq={Hq} Hkv={Hkv} N={N} d={d}")
    sc = binding.block_scores(q16, k16, "block_max").cpu().numpy()
    nb = N // 64
    per = nb * (nb + 1) // 2
    qv = q.numpy().astype(np.float64)
    kv = k.numpy().astype(np.float64)
    g = np.random.default_rng(0)
    picks = [(0, 0, 0), (Hq - 1, nb - 1, nb - 1), (Hq - 1, nb - 1, 0)] + \
            [(int(h), int(i), int(g.integers(0, i + 1))) for h, i in zip(g.integers(0, Hq, 20), g.integers(0, nb, 20))]
    for h, i, j in picks:
        s = qv[0, h, 64 * i:64 * i + 64] @ kv[0, h * Hkv // Hq, 64 * j:64 * j + 64].T
        want = np.float32(s.max())  # fp16 products and these sums agree with the chain to well inside an fp32 ulp
        got = sc[h * per + i * (i + 1) // 2 + j]
        assert abs(float(got) - float(want)) <= 2e-6 * max(1.0, abs(float(want))), (h, i, j, got, want)
