"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bars: FP16 copies, MXFP4 codes and scales, traversal lists and counts are
bit-exact; attention outputs are within 2e-3 * max|O_oracle| (fp32 output,
fp32 accumulation on the GPU, fp64 in the oracle).
"""
import numpy as np
import pytest
import torch

import oracle
from fp16_long_context_amd import binding, synth

pytestmark = pytest.mark.gpu
TOL = 2e-3


def say(*a):
    print(*a, flush=True)


def gpu_layout_to_oracle(qz):
    """GPU outputs -> the oracle's layouts (token-major v16, channel-major v4/v4s)."""
    B, Hkv, nb, d, _ = qz["v16"].shape
    N = nb * 64
    o = {n: qz[n].cpu() for n in qz}
    return {
        "q16": o["q16"].view(torch.int16).numpy().view(np.uint16),
        "k16": o["k16"].view(torch.int16).numpy().view(np.uint16),
        "v16": o["v16"].permute(0, 1, 2, 4, 3).reshape(B, Hkv, N, d).contiguous().view(torch.int16).numpy().view(np.uint16),
        "q4": o["q4"].numpy(), "q4s": o["q4s"].numpy(), "k4": o["k4"].numpy(), "k4s": o["k4s"].numpy(),
        "v4": o["v4"].permute(0, 1, 3, 2, 4).reshape(B, Hkv, d, N // 2).contiguous().numpy(),
        "v4s": o["v4s"].permute(0, 1, 3, 2, 4).reshape(B, Hkv, d, N // 32).contiguous().numpy(),
    }


def run_case(q, k, v, frac, causal=True, rows=None, label="", rowsum="p"):
    """Run both sides; assert the bit-exact parts; return the attention comparison.
    rowsum selects the row-sum reading on both sides ("p" or "weights")."""
    dtype = "fp16" if q.dtype == torch.float16 else "bf16"
    B, Hq, N, d = q.shape
    say(f"[case] {label} B={B} Hq={Hq} Hkv={k.shape[1]} N={N} d={d} frac={frac} causal={causal} {dtype} rowsum={rowsum}")
    qz_o = oracle.quantize(synth.bits(q), synth.bits(k), synth.bits(v), dtype)
    sel_o = oracle.select(qz_o["q16"], qz_o["k16"], frac, causal)
    dev = torch.device("cuda:0")
    qz = binding.quantize(q.to(dev), k.to(dev), v.to(dev))
    idx, n16 = binding.select(qz["q16"], qz["k16"], frac, causal)
    out, lse = binding.attn_fwd(qz, idx, n16, causal, want_lse=True, rowsum=rowsum)
    torch.cuda.synchronize()
    g = gpu_layout_to_oracle(qz)
    for n in g:
        assert np.array_equal(g[n], qz_o[n]), f"{label}: {n} differs"
    assert np.array_equal(n16.cpu().numpy(), sel_o["n16"]), f"{label}: n16 differs"
    assert np.array_equal(idx.cpu().numpy(), sel_o["idx"]), f"{label}: idx differs"
    rows = oracle.all_rows(B, Hq, N) if rows is None else np.asarray(rows, dtype=np.int64)
    res = oracle.attn_rows(qz_o, sel_o, rows, causal, rowsum=rowsum)
    og = out.reshape(-1, d).cpu().numpy().astype(np.float64)[rows]
    lg = lse.reshape(-1).cpu().numpy().astype(np.float64)[rows]
    err = np.abs(og - res["out"]).max() / np.abs(res["out"]).max()
    lerr = np.abs(lg - res["lse"]).max()
    say(f"[case] {label}: max|dO|/max|O| = {err:.3e}, max|dLSE| = {lerr:.3e}")
    assert err <= TOL, f"{label}: output error {err:.3e} > {TOL}"
    assert lerr <= 1e-3, f"{label}: lse error {lerr:.3e}"
    return err, qz, idx, n16, out


def test_tiny_workload_all_rows():
    x = synth.generate("tiny")
    run_case(x["q"], x["k"], x["v"], 0.05, label="tiny")


@pytest.mark.parametrize("frac", [0.0, 0.01, 0.05, 0.2, 1.0])
def test_llama_shaped_frac_sweep(frac):
    x = synth.generate("llama8b_16k", N=1024)
    run_case(x["q"], x["k"], x["v"], frac, label=f"llama8b@1k frac={frac}")


def test_llama_shaped_2k_sampled():
    x = synth.generate("llama8b_16k", N=2048)
    rows = np.arange(0, 32 * 2048, 5)
    run_case(x["q"], x["k"], x["v"], 0.05, rows=rows, label="llama8b@2k")


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal,dtype,frac", [
    (2, 14, 2, 512, 128, True, "bf16", 0.05),   # GQA group of 7: three head pairs + one lone head
    (1, 10, 2, 640, 64, True, "bf16", 0.2),     # GQA group of 5, d = 64
    (1, 4, 2, 512, 64, True, "fp16", 0.3),      # group of 2, d = 64
    (1, 3, 3, 320, 128, False, "fp16", 0.3),    # non-causal, 5 blocks
    (1, 2, 1, 64, 128, True, "bf16", 0.05),     # a single block
    (1, 8, 8, 576, 64, True, "bf16", 0.5),
    (3, 6, 2, 448, 128, False, "bf16", 0.0),
    (1, 4, 1, 768, 128, True, "fp16", 1.0),
])
def test_shapes(B, Hq, Hkv, N, d, causal, dtype, frac):
    q, k, v = synth.random_qkv(B, Hq, Hkv, N, d, dtype, seed=B * 1000 + N, scale=1.5)
    run_case(q, k, v, frac, causal, label="shape")


def test_rope_and_heavy_tail_generators():
    x = synth.generate("long_128k", N=1024)
    run_case(x["q"], x["k"], x["v"], 0.05, label="rope@1k")
    y = synth.generate("batched_32k", N=512)
    run_case(y["q"], y["k"], y["v"], 0.05, label="heavy@512")


@pytest.mark.parametrize("frac", [0.1, 0.2, 0.5])
def test_select_ties_at_the_cutoff(frac):
    """Key blocks that differ only by a tiny step in one channel: their block
    scores agree in fp32 (often) and in fp64 (when the step is the same), so
    the cut-off falls among tied blocks.  The lists must still equal the
    oracle's (fp64 score descending, lower block index first)."""
    g = np.random.default_rng(5)
    B, H, N, d = 1, 2, 2048, 128
    nb = N // 64
    q = g.standard_normal((B, H, N, d))
    q[..., 0] = 2.0 ** -8  # pooled Q mean of channel 0 is exactly 2^-8
    r = g.standard_normal(d)
    r[0] = 1.0
    k = np.broadcast_to(r, (B, H, N, d)).copy()  # every key row the same
    m = g.integers(0, 4, size=(H, nb))  # block j: one row's channel 0 up by m * 2^-10
    for h in range(H):
        for j in range(nb):
            k[0, h, 64 * j, 0] += m[h, j] * 2.0 ** -10
    q16 = torch.from_numpy(q.astype(np.float16))
    k16 = torch.from_numpy(k.astype(np.float16))
    say(f"[case] select ties B={B} H={H} N={N} d={d} frac={frac}")
    sel_o = oracle.select(synth.bits(q16), synth.bits(k16), frac, True)
    dev = torch.device("cuda:0")
    idx, n16 = binding.select(q16.to(dev), k16.to(dev), frac, True)
    torch.cuda.synchronize()
    assert np.array_equal(n16.cpu().numpy(), sel_o["n16"])
    assert np.array_equal(idx.cpu().numpy(), sel_o["idx"])


@pytest.mark.parametrize("frac,steps", [(0.2, 4), (0.2, 1000), (0.05, 1000)])
def test_select_wide_band_at_the_cutoff(frac, steps):
    """256 key blocks whose pooled means differ only by multiples of 2^-16 in
    one channel: their scores differ by less than the fp32 chains' error bound,
    so most of a long row's candidates fall in the band around the cut-off
    (more than 64, the ranked-list size) and are ranked by their fp64 scores,
    with exact ties (few distinct steps) or nearly none (many).  The lists must
    equal the oracle's bit for bit."""
    g = np.random.default_rng(11)
    B, H, N, d = 1, 2, 64 * 256, 64
    nb = N // 64
    q = g.standard_normal((B, H, N, d))
    q[..., 0] = 2.0 ** -8
    r = g.standard_normal(d)
    r[0] = 1.0
    k = np.broadcast_to(r, (B, H, N, d)).copy()
    m = g.integers(0, steps, size=(H, nb))  # block j: one row's channel 0 up by m 2^-10 (fp16-exact)
    for h in range(H):
        for j in range(nb):
            k[0, h, 64 * j, 0] += m[h, j] * 2.0 ** -10
    q16 = torch.from_numpy(q.astype(np.float16))
    k16 = torch.from_numpy(k.astype(np.float16))
    say(f"[case] select wide band B={B} H={H} N={N} d={d} frac={frac} steps={steps}")
    sel_o = oracle.select(synth.bits(q16), synth.bits(k16), frac, True)
    dev = torch.device("cuda:0")
    idx, n16 = binding.select(q16.to(dev), k16.to(dev), frac, True)
    torch.cuda.synchronize()
    assert np.array_equal(n16.cpu().numpy(), sel_o["n16"])
    assert np.array_equal(idx.cpu().numpy(), sel_o["idx"])


def test_output_dtypes_and_determinism():
    x = synth.generate("llama8b_16k", N=1024)
    dev = torch.device("cuda:0")
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    qz = binding.quantize(q, k, v)
    idx, n16 = binding.select(qz["q16"], qz["k16"], 0.05)
    o32, _ = binding.attn_fwd(qz, idx, n16)
    o16, _ = binding.attn_fwd(qz, idx, n16, out_dtype=torch.float16)
    ob16, _ = binding.attn_fwd(qz, idx, n16, out_dtype=torch.bfloat16)
    assert torch.equal(o16, o32.to(torch.float16))
    assert torch.equal(ob16, o32.to(torch.bfloat16))
    # a second run on another stream gives the same bits
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        qz2 = binding.quantize(q, k, v)
        idx2, n162 = binding.select(qz2["q16"], qz2["k16"], 0.05)
        o2, _ = binding.attn_fwd(qz2, idx2, n162)
    s.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(n16, n162)
    assert torch.equal(o2, o32)


def test_preallocated_buffers_are_fully_written():
    """Every output is written completely: caller buffers filled with garbage
    and reused for two different problems give the bits of fresh buffers."""
    dev = torch.device("cuda:0")
    xs = [synth.generate("llama8b_16k", N=1024), synth.generate("long_128k", N=1024)]
    B, Hq, N, d = xs[0]["q"].shape
    Hkv = xs[0]["k"].shape[1]
    say(f"[case] preallocated buffers B={B} Hq={Hq} Hkv={Hkv} N={N} d={d}")
    qb = binding.alloc_quantized(B, Hq, Hkv, N, d, dev)
    for t in qb.values():
        t.view(torch.uint8).fill_(0x7F)
    ents = binding.list_entries(B, Hq, N)
    idx = torch.full((ents,), 12345, dtype=torch.int32, device=dev)
    n16 = torch.full((B, Hq, N // 64), 777, dtype=torch.int32, device=dev)
    sws = torch.full((1 << 22,), 0xAB, dtype=torch.uint8, device=dev)
    out = torch.full((B, Hq, N, d), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, device=dev)
    aws = torch.full((binding.attn_workspace_bytes(B, Hq, Hkv, N, d),), 0xCD, dtype=torch.uint8, device=dev)
    for x in xs:
        q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
        fq = binding.quantize(q, k, v)
        fi, fn = binding.select(fq["q16"], fq["k16"], 0.05)
        fo, fl = binding.attn_fwd(fq, fi, fn, want_lse=True)
        rq = binding.quantize(q, k, v, out=qb)
        binding.select(rq["q16"], rq["k16"], 0.05, idx=idx, n16=n16, workspace=sws)
        binding.attn_fwd(rq, idx, n16, want_lse=True, out=out, lse=lse, workspace=aws)
        torch.cuda.synchronize()
        for n in fq:
            assert torch.equal(rq[n].view(torch.uint8), fq[n].view(torch.uint8)), n
        assert torch.equal(idx, fi) and torch.equal(n16, fn)
        assert torch.equal(out, fo) and torch.equal(lse, fl)


def test_graph_capture_replays_match_eager():
    """The three calls on caller buffers can be captured in a HIP graph (they
    allocate nothing and record no memset): three replays, with eager work and
    synchronizations between them, each equal the eager run bit for bit."""
    dev = torch.device("cuda:0")
    x = synth.generate("llama8b_16k", N=1024)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    say(f"[case] graph capture B={B} Hq={Hq} Hkv={Hkv} N={N} d={d}")
    qb = binding.alloc_quantized(B, Hq, Hkv, N, d, dev)
    idx = torch.empty(binding.list_entries(B, Hq, N), dtype=torch.int32, device=dev)
    n16 = torch.empty((B, Hq, N // 64), dtype=torch.int32, device=dev)
    sws = torch.empty(1 << 22, dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    aws = torch.empty(binding.attn_workspace_bytes(B, Hq, Hkv, N, d), dtype=torch.uint8, device=dev)

    def step():
        binding.quantize(q, k, v, out=qb)
        binding.select(qb["q16"], qb["k16"], 0.05, idx=idx, n16=n16, workspace=sws)
        binding.attn_fwd(qb, idx, n16, want_lse=True, out=out, lse=lse, workspace=aws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = {n: t.clone() for n, t in qb.items()}
    ref_idx, ref_n16, ref_out, ref_lse = idx.clone(), n16.clone(), out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        for t in (idx, n16):  # eager work between replays: stale values in every output
            t.fill_(-3)
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in ref:
            assert torch.equal(qb[n].view(torch.uint8), ref[n].view(torch.uint8)), (r, n)
        assert torch.equal(idx, ref_idx) and torch.equal(n16, ref_n16), r
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), r


def sample_rows(x, B, Hq, N, n, seed, heads=(), batches=None):
    """Rows to compare at full size: n random rows, the last row of the first
    and last head of every batch, rows that look up a planted needle, and
    for each (b, h) in batches x heads one row of every query block, at a
    position that moves through the block and alternates between its two
    32-row halves (the two waves of the FP4 workgroup)."""
    g = np.random.default_rng(seed)
    rows = list(g.integers(0, B * Hq * N, n))
    rows += [(b * Hq + h) * N + N - 1 for b in range(B) for h in (0, Hq - 1)]  # longest rows
    for (b, kvh, hq, p, t) in x["needles"][:8]:  # rows that look up a planted needle
        rows.append((b * Hq + hq) * N + t)
    nb = N // 64
    for b in (range(B) if batches is None else batches):
        for h in heads:
            i = np.arange(nb)
            t = 64 * i + 32 * (i % 2) + (i * 7 + h * 13 + b * 5) % 32
            rows += list((b * Hq + h) * N + t)
    return np.array(sorted(set(int(r) for r in rows)), dtype=np.int64)


# per workload: query heads with one row of every query block (heads 0 and 1
# share a two-head FP4 workgroup; the last head is in the last KV group)
FULL_SIZE_HEADS = {"llama8b_16k": tuple(range(32)), "batched_32k": (0, 1, 27), "long_128k": (0, 1, 31)}


@pytest.mark.parametrize("name", ["llama8b_16k", "batched_32k", "long_128k"])
def test_full_size_workloads_sampled(name):
    # full sizes, the launch configuration the benchmark times; attention
    # checked on several thousand rows (every list and code is checked in full)
    x = synth.generate(name)
    w = x["w"]
    rows = sample_rows(x, w.B, w.Hq, w.N, 40, 7, heads=FULL_SIZE_HEADS[name])
    say(f"[case] {name}: {len(rows)} rows compared")
    run_case(x["q"], x["k"], x["v"], w.frac, rows=rows, label=name)


def test_frac_sweep_64k_sampled():
    """The 64K configuration's FP16 fractions on the same tensors: codes once,
    then at every fraction the lists bit-exact and attention on sampled rows
    within the bar (the fraction moves work between the two kernels)."""
    x = synth.generate("sweep_64k")
    w = x["w"]
    say(f"[case] sweep_64k B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} fracs 0..1")
    qz_o = oracle.quantize(synth.bits(x["q"]), synth.bits(x["k"]), synth.bits(x["v"]), "bf16")
    dev = torch.device("cuda:0")
    qz = binding.quantize(x["q"].to(dev), x["k"].to(dev), x["v"].to(dev))
    g = gpu_layout_to_oracle(qz)
    for n in g:
        assert np.array_equal(g[n], qz_o[n]), f"sweep_64k: {n} differs"
    del g
    rows = sample_rows(x, w.B, w.Hq, w.N, 24, 11, heads=(0, w.Hq - 1))
    say(f"[case] sweep_64k: {len(rows)} rows compared at every fraction")
    for frac in (0.0, 0.01, 0.05, 0.2, 1.0):
        sel_o = oracle.select(qz_o["q16"], qz_o["k16"], frac, True)
        idx, n16 = binding.select(qz["q16"], qz["k16"], frac, True)
        out, lse = binding.attn_fwd(qz, idx, n16, True, want_lse=True)
        torch.cuda.synchronize()
        assert np.array_equal(n16.cpu().numpy(), sel_o["n16"]), f"frac {frac}: n16 differs"
        assert np.array_equal(idx.cpu().numpy(), sel_o["idx"]), f"frac {frac}: idx differs"
        res = oracle.attn_rows(qz_o, sel_o, rows, True)
        og = out.reshape(-1, w.d).cpu().numpy().astype(np.float64)[rows]
        lg = lse.reshape(-1).cpu().numpy().astype(np.float64)[rows]
        err = np.abs(og - res["out"]).max() / np.abs(res["out"]).max()
        lerr = np.abs(lg - res["lse"]).max()
        say(f"[case] sweep_64k frac {frac}: max|dO|/max|O| = {err:.3e}, max|dLSE| = {lerr:.3e}")
        assert err <= TOL and lerr <= 1e-3, (frac, err, lerr)
        del idx, n16, out, lse


def test_attention_composer_and_sm_scale():
    """binding.attention (quantize -> select -> attention in one call) with a
    non-default softmax scale: equal to the three calls made one by one, and
    within the bar of the oracle at the same scale."""
    q, k, v = synth.random_qkv(1, 4, 2, 384, 64, "bf16", seed=17, scale=1.5)
    dev = torch.device("cuda:0")
    sm = 0.2
    say("[case] attention() B=1 Hq=4 Hkv=2 N=384 d=64 bf16 frac=0.1 sm_scale=0.2")
    out = binding.attention(q.to(dev), k.to(dev), v.to(dev), frac=0.1, sm_scale=sm)
    qz = binding.quantize(q.to(dev), k.to(dev), v.to(dev))
    idx, n16 = binding.select(qz["q16"], qz["k16"], 0.1, True)
    out2, _ = binding.attn_fwd(qz, idx, n16, True, sm)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    qz_o = oracle.quantize(synth.bits(q), synth.bits(k), synth.bits(v), "bf16")
    sel_o = oracle.select(qz_o["q16"], qz_o["k16"], 0.1, True)
    res = oracle.attn_rows(qz_o, sel_o, oracle.all_rows(1, 4, 384), True, sm_scale=sm)
    og = out.reshape(-1, 64).cpu().numpy().astype(np.float64)
    err = np.abs(og - res["out"]).max() / np.abs(res["out"]).max()
    say(f"[case] attention(): max|dO|/max|O| = {err:.3e}")
    assert err <= TOL


def test_non_finite_inputs_stay_in_bounds():
    """Inputs outside the contract (inf and NaN) give undefined lists and
    outputs, but every write stays inside its buffer: the slack after idx
    keeps its fill, every list entry is a block of its row or the fill, and
    the attention call completes."""
    g = np.random.default_rng(3)
    B, Hq, Hkv, N, d = 1, 2, 1, 1024, 64
    q, k, v = g.standard_normal((B, Hq, N, d)), g.standard_normal((B, Hkv, N, d)), g.standard_normal((B, Hkv, N, d))
    q[0, 0, 5, 3] = np.nan
    q[0, 1, 900, 2] = np.inf
    k[0, 0, 70, 1] = np.inf
    k[0, 0, 200, 0] = -np.inf
    v[0, 0, 300, 7] = np.nan
    dev = torch.device("cuda:0")
    t = lambda x: torch.from_numpy(x.astype(np.float16)).to(dev)
    say(f"[case] non-finite inputs B={B} Hq={Hq} Hkv={Hkv} N={N} d={d}")
    qz = binding.quantize(t(q), t(k), t(v))
    nb = N // 64
    ents = B * Hq * nb * (nb + 1) // 2
    fill = -7
    idx = torch.full((ents + 4096,), fill, dtype=torch.int32, device=dev)
    n16 = torch.full((B, Hq, nb), fill, dtype=torch.int32, device=dev)
    row_of = np.tile(np.repeat(np.arange(nb), np.arange(1, nb + 1)), B * Hq)  # query block of each entry
    for frac in (0.05, 0.3, 1.0):
        idx.fill_(fill)
        binding.select(qz["q16"], qz["k16"], frac, True, idx=idx, n16=n16)
        out, lse = binding.attn_fwd(qz, idx, n16, True, want_lse=True)
        torch.cuda.synchronize()
        i = idx.cpu().numpy()
        assert np.all(i[ents:] == fill), f"frac {frac}: a list write left the array"
        e = i[:ents]
        assert np.all((e == fill) | ((e >= 0) & (e <= row_of))), f"frac {frac}: an entry outside its row"
        c = n16.cpu().numpy().reshape(B * Hq, nb)
        assert np.all((c >= 1) & (c <= np.arange(1, nb + 1))), f"frac {frac}: a count outside its row"
        assert out.shape == (B, Hq, N, d) and lse.shape == (B, Hq, N)


def test_maximum_blocks():
    # N = 64 * 8192, the largest supported block count
    q, k, v = synth.random_qkv(1, 2, 1, 64 * 8192, 64, "fp16", seed=77)
    rows = np.array([0, 63, 64, 100000, 524287, 524288 + 524287, 524288 + 4097])
    run_case(q, k, v, 0.05, rows=rows, label="max-blocks")


def test_redo_walk_on_overflow():
    """A key far above every FP16 block of its rows sits in an FP4 block: the
    fixed-max FP4 walk flags the work item (p would be ~2^190) and the redo
    kernel recomputes it with the rescaling walk; the result must still
    match the oracle."""
    q, k, v = synth.random_qkv(1, 4, 1, 512, 128, "fp16", seed=77)
    # key 200 (block 3, on no FP16 list at frac=0) aligned with query 450 of
    # head 0 (block 7): score ~ 12 |q|^2 ~ 1500, x ~ 190 log2 units
    k[0, 0, 200] = (12.0 * q[0, 0, 450].float()).to(q.dtype)
    run_case(q, k, v, 0.0, label="redo walk")


@pytest.mark.parametrize("rowsum", ["p", "weights"])
def test_redo_walk_odd_group(rowsum):
    """A GQA group of 3: heads 0-1 run in two-head FP4 workgroups and head 2
    in the one-head launch, whose redo flags sit after the pairs'.  Overflow
    keys planted for head 2 and for head 0 (different query blocks) must be
    recomputed by the redo kernel of their own launch."""
    q, k, v = synth.random_qkv(1, 3, 1, 512, 128, "fp16", seed=91)
    k[0, 0, 200] = (12.0 * q[0, 2, 450].float()).to(q.dtype)  # head 2 (lone head), query block 7
    k[0, 0, 70] = (12.0 * q[0, 0, 330].float()).to(q.dtype)   # head 0 (pair), query block 5
    run_case(q, k, v, 0.0, label="redo walk, group of 3", rowsum=rowsum)


@pytest.mark.parametrize("delta", [0, 5, 15])
def test_single_fp16_block_lists(delta):
    """Lists that are not the selection's (one FP16 block per row block, at
    a fixed diagonal offset, nothing forced), as the error-attribution study
    feeds them: the attention must still match the oracle on the same lists."""
    from fp16_long_context_amd.quality import offset_lists

    x = synth.generate("llama8b_16k", N=1024)
    q, k, v = x["q"], x["k"], x["v"]
    B, Hq, N, d = q.shape
    nb = N // 64
    say(f"[case] single FP16 block at offset {delta}, llama8b@1k")
    # the oracle's lists, written out row by row
    idx_o, n16_o = [], np.zeros((B, Hq, nb), dtype=np.int32)
    for b in range(B):
        for h in range(Hq):
            for i in range(nb):
                j16 = i - delta
                idx_o += ([j16] if j16 >= 0 else []) + [j for j in range(i + 1) if j != j16]
                n16_o[b, h, i] = 1 if j16 >= 0 else 0
    idx_o = np.asarray(idx_o, dtype=np.int32)
    dev = torch.device("cuda:0")
    qz = binding.quantize(q.to(dev), k.to(dev), v.to(dev))
    idx, n16 = offset_lists(B, Hq, nb, delta, dev)
    assert np.array_equal(idx.cpu().numpy(), idx_o) and np.array_equal(n16.cpu().numpy(), n16_o)
    out, _ = binding.attn_fwd(qz, idx, n16, True)
    qz_o = oracle.quantize(synth.bits(q), synth.bits(k), synth.bits(v), "bf16")
    rows = oracle.all_rows(B, Hq, N)
    res = oracle.attn_rows(qz_o, {"idx": idx_o, "n16": n16_o}, rows, True)
    og = out.reshape(-1, d).cpu().numpy().astype(np.float64)[rows]
    err = np.abs(og - res["out"]).max() / np.abs(res["out"]).max()
    say(f"[case] offset {delta}: max|dO|/max|O| = {err:.3e}")
    assert err <= TOL


# ------------------------------------------- row sum over the quantized weights


def test_wsum_tiny_and_generators():
    x = synth.generate("tiny")
    run_case(x["q"], x["k"], x["v"], 0.05, label="tiny", rowsum="weights")
    y = synth.generate("long_128k", N=1024)
    run_case(y["q"], y["k"], y["v"], 0.05, label="rope@1k", rowsum="weights")


@pytest.mark.parametrize("frac", [0.0, 0.05, 1.0])
def test_wsum_llama_shaped(frac):
    x = synth.generate("llama8b_16k", N=1024)
    run_case(x["q"], x["k"], x["v"], frac, label=f"llama8b@1k frac={frac}", rowsum="weights")


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal,dtype,frac", [
    (2, 14, 2, 512, 128, True, "bf16", 0.05),
    (1, 4, 2, 512, 64, True, "fp16", 0.3),
    (1, 3, 3, 320, 128, False, "fp16", 0.3),
    (1, 2, 1, 64, 128, True, "bf16", 0.05),
])
def test_wsum_shapes(B, Hq, Hkv, N, d, causal, dtype, frac):
    q, k, v = synth.random_qkv(B, Hq, Hkv, N, d, dtype, seed=B * 1000 + N, scale=1.5)
    run_case(q, k, v, frac, causal, label="shape", rowsum="weights")


def test_wsum_constant_values_give_one():
    # V = 1: the weights row sum makes every output exactly a sum of weights
    # over itself; the GPU's fp32 sums of the same weights differ only in order
    q, k, _ = synth.random_qkv(1, 8, 2, 2048, 128, "bf16", seed=53, scale=1.5)
    v = torch.ones((1, 2, 2048, 128), dtype=torch.bfloat16)
    dev = torch.device("cuda:0")
    qz = binding.quantize(q.to(dev), k.to(dev), v.to(dev))
    for frac in (0.0, 0.05, 1.0):
        idx, n16 = binding.select(qz["q16"], qz["k16"], frac)
        out, _ = binding.attn_fwd(qz, idx, n16, rowsum="weights")
        err = (out - 1.0).abs().max().item()
        say(f"[case] V=1 frac={frac}: max|O - 1| = {err:.3e}")
        assert err < 1e-5


def test_wsum_redo_walk_on_overflow():
    q, k, v = synth.random_qkv(1, 4, 1, 512, 128, "fp16", seed=77)
    k[0, 0, 200] = (12.0 * q[0, 0, 450].float()).to(q.dtype)
    run_case(q, k, v, 0.0, label="redo walk", rowsum="weights")


def test_wsum_full_size_sampled():
    x = synth.generate("llama8b_16k")
    w = x["w"]
    rows = sample_rows(x, w.B, w.Hq, w.N, 40, 7)
    run_case(x["q"], x["k"], x["v"], w.frac, rows=rows, label="llama8b_16k", rowsum="weights")


def test_timing_hook_events_and_same_output():
    # thrift_attn_fwd_ex with four events: the same output bits as
    # thrift_attn_fwd, and the events bracket the three kernels in order
    x = synth.generate("llama8b_16k", N=2048)
    dev = torch.device("cuda:0")
    qz = binding.quantize(*(x[n].to(dev) for n in ("q", "k", "v")))
    idx, n16 = binding.select(qz["q16"], qz["k16"], 0.05)
    plain, _ = binding.attn_fwd(qz, idx, n16)
    for rowsum in ("p", "weights"):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        hooked, _ = binding.attn_fwd(qz, idx, n16, rowsum=rowsum, events=ev)
        ref, _ = binding.attn_fwd(qz, idx, n16, rowsum=rowsum)
        torch.cuda.synchronize()
        assert torch.equal(hooked, ref)
        if rowsum == "p":
            assert torch.equal(hooked, plain)
        t = [ev[0].elapsed_time(ev[i]) for i in (1, 2, 3)]
        say(f"[case] timing hook {rowsum}: kernel ends at {t} ms")
        assert 0.0 <= t[0] <= t[1] <= t[2]


# --------------------------- exp-free FP4 P under the weights reading (rowsum "log")


def test_log_tiny_and_generators():
    x = synth.generate("tiny")
    run_case(x["q"], x["k"], x["v"], 0.05, label="tiny", rowsum="log")
    y = synth.generate("long_128k", N=1024)
    run_case(y["q"], y["k"], y["v"], 0.05, label="rope@1k", rowsum="log")


@pytest.mark.parametrize("frac", [0.0, 0.05, 1.0])
def test_log_llama_shaped(frac):
    x = synth.generate("llama8b_16k", N=1024)
    run_case(x["q"], x["k"], x["v"], frac, label=f"llama8b@1k frac={frac}", rowsum="log")


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal,dtype,frac", [
    (2, 14, 2, 512, 128, True, "bf16", 0.05),
    (1, 4, 2, 512, 64, True, "fp16", 0.3),
    (1, 3, 3, 320, 128, False, "fp16", 0.3),
    (1, 2, 1, 64, 128, True, "bf16", 0.05),
])
def test_log_shapes(B, Hq, Hkv, N, d, causal, dtype, frac):
    q, k, v = synth.random_qkv(B, Hq, Hkv, N, d, dtype, seed=B * 1000 + N, scale=1.5)
    run_case(q, k, v, frac, causal, label="shape", rowsum="log")


def test_log_constant_values_give_one():
    q, k, _ = synth.random_qkv(1, 8, 2, 2048, 128, "bf16", seed=59, scale=1.5)
    v = torch.ones((1, 2, 2048, 128), dtype=torch.bfloat16)
    dev = torch.device("cuda:0")
    qz = binding.quantize(q.to(dev), k.to(dev), v.to(dev))
    for frac in (0.0, 0.05, 1.0):
        idx, n16 = binding.select(qz["q16"], qz["k16"], frac)
        out, _ = binding.attn_fwd(qz, idx, n16, rowsum="log")
        err = (out - 1.0).abs().max().item()
        say(f"[case] log V=1 frac={frac}: max|O - 1| = {err:.3e}")
        assert err < 1e-5


@pytest.mark.parametrize("Hq", [4, 3])
def test_log_redo_walk_on_overflow(Hq):
    # a planted key far above every FP16 block of its rows: the fixed-max
    # walk flags the item and the redo walk (exp-free codes too) recomputes it
    q, k, v = synth.random_qkv(1, Hq, 1, 512, 128, "fp16", seed=77)
    k[0, 0, 200] = (12.0 * q[0, Hq - 1, 450].float()).to(q.dtype)
    run_case(q, k, v, 0.0, label=f"redo walk Hq={Hq}", rowsum="log")


def test_log_full_size_sampled():
    x = synth.generate("llama8b_16k")
    w = x["w"]
    rows = sample_rows(x, w.B, w.Hq, w.N, 40, 7)
    run_case(x["q"], x["k"], x["v"], w.frac, rows=rows, label="llama8b_16k", rowsum="log")
