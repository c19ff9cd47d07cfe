"""Quality studies of the mixed FP16/FP4 attention on seeded synthetic inputs.

The method's claim ("ThriftAttention: Selective Mixed Precision for
Long-Context FP4 Attention", abstract) is that a small FP16 share of the
block pairs recovers most of the quality lost by going from FP16 to FP4,
and that this pays off more as sequences get longer.  The pages measure this on
benchmarks with trained models; here the planted-needle workloads stand in:

* errors(): err(f) = ||O_f - O_1||_F / ||O_1||_F against the all-FP16 output
  (frac = 1), over all rows and over the rows whose query looks up a planted
  needle, for the mixed fraction and for pure FP4 (frac = 0);
* length_sweep(): the same at several sequence lengths of one generator;
* attribution(): the gain of computing single blocks in FP16, against the
  selection heuristic's block score and the exact attention mass;
* heuristics(): the output error when the FP16 blocks are picked by the
  other block scores the library offers (thrift_select_ex: max-pooled,
  norm-weighted, exact block max) under the same budget rule, and what each
  selection costs.

Everything runs through the library (quantize, select, attention); nothing
here is an oracle.

    python -m fp16_long_context_amd.quality --sweep 4096,16384,65536,131072
    python -m fp16_long_context_amd.quality --attribution --workload llama8b_16k --N 4096
    python -m fp16_long_context_amd.quality --heuristics --workload long_128k --N 16384
"""
from __future__ import annotations

import argparse
import json
import math
import sys
import time


def errors(binding, torch, qz: dict, w, needles, frac: float, rowsum: str = "p") -> dict:
    """err(frac) and err(0) against frac = 1, all rows and needle rows (the
    frac = 1 reference is always the plain FP16 attention, rowsum "p")."""
    outs = {}
    for f in (1.0, frac, 0.0):
        idx, n16 = binding.select(qz["q16"], qz["k16"], f, True)
        outs[f], _ = binding.attn_fwd(qz, idx, n16, True, rowsum="p" if f == 1.0 else rowsum)
        del idx, n16
    ref = outs[1.0]
    dev = ref.device
    rows = torch.tensor([(b * w.Hq + hq) * w.N + t for (b, kvh, hq, p, t) in needles], device=dev)
    res = {}
    for f, name in ((frac, "mixed"), (0.0, "fp4")):
        d_all = torch.linalg.vector_norm((outs[f] - ref).reshape(-1)).item() / torch.linalg.vector_norm(ref).item()
        r2 = ref.reshape(-1, w.d)[rows]
        d_ndl = (torch.linalg.vector_norm(outs[f].reshape(-1, w.d)[rows] - r2) / torch.linalg.vector_norm(r2)).item()
        res[f"err_{name}"] = d_all
        res[f"needle_err_{name}"] = d_ndl
    del outs
    res["frac"] = frac
    res["mixed_below_fp4"] = bool(res["err_mixed"] < res["err_fp4"] and res["needle_err_mixed"] < res["needle_err_fp4"])
    res["gap_recovered"] = 1.0 - res["err_mixed"] / res["err_fp4"]
    res["needle_gap_recovered"] = 1.0 - res["needle_err_mixed"] / res["needle_err_fp4"]
    return {k: (round(v, 6) if isinstance(v, float) else v) for k, v in res.items()}


def length_sweep(Ns, workload: str = "long_128k", frac: float | None = None, log=None) -> list:
    """errors() of one generator at each sequence length in Ns (same seed,
    so shorter runs are not prefixes of longer ones: every N is drawn anew)."""
    import torch

    from . import binding, synth

    dev = torch.device("cuda:0")
    out = []
    for N in Ns:
        t0 = time.perf_counter()
        x = synth.generate(workload, N=N)
        w = x["w"]
        f = w.frac if frac is None else frac
        q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
        del x["q"], x["k"], x["v"]
        qz = binding.quantize(q, k, v)
        del q, k, v
        r = errors(binding, torch, qz, w, x["needles"], f)
        del qz
        torch.cuda.synchronize()
        r.update({"workload": workload, "N": N, "needles": len(x["needles"]), "seconds": round(time.perf_counter() - t0, 2)})
        if log:
            log(json.dumps(r))
        out.append(r)
        torch.cuda.empty_cache()
    return out


def offset_lists(B: int, Hq: int, nb: int, delta: int, device):
    """Causal traversal lists in which row block i has exactly one FP16 block,
    i - delta (none when i < delta), and every other valid block in FP4.
    Returns (idx int32 [B*Hq*nb(nb+1)/2], n16 int32 [B,Hq,nb]) in the
    library's list layout (per row: the FP16 list, then the FP4 list, each
    ascending)."""
    import torch

    i = torch.repeat_interleave(torch.arange(nb, device=device), torch.arange(1, nb + 1, device=device))
    pos = torch.arange(nb * (nb + 1) // 2, device=device) - i * (i + 1) // 2
    j16 = i - delta
    has = j16 >= 0
    rest = torch.where(pos - 1 < j16, pos - 1, pos)  # FP4 entry pos-1 skips block j16
    val = torch.where(has, torch.where(pos == 0, j16, rest), pos)
    idx = val.to(torch.int32).repeat(B * Hq)
    n16 = (torch.arange(nb, device=device) >= delta).to(torch.int32).expand(B, Hq, nb).contiguous()
    return idx, n16


def _ranks(x):
    """Ranks 0..n-1 of a 1-D tensor (ties broken by position)."""
    import torch

    r = torch.empty_like(x, dtype=torch.float64)
    r[torch.argsort(x)] = torch.arange(x.numel(), device=x.device, dtype=torch.float64)
    return r


def _spearman(a, b) -> float:
    import torch

    ra, rb = _ranks(a), _ranks(b)
    ra -= ra.mean()
    rb -= rb.mean()
    return float((ra * rb).sum() / torch.sqrt((ra * ra).sum() * (rb * rb).sum()))


def attribution(workload: str = "llama8b_16k", N: int | None = None, frac: float = 0.05, log=None) -> dict:
    """Block-level error attribution (the pages' core observation: the output
    error of FP4 concentrates in a few important blocks).

    For every causal block pair (i, j) of every head, gain(i, j) is the drop
    of the squared output error of row block i against the all-FP16 output
    when only block j of that row block is computed in FP16 and every other
    block in FP4.  One attention run per diagonal offset delta = i - j gives
    the gains of all pairs on that offset at once.  The gains are compared
    with the selection heuristic's score (dot product of the pooled block
    means) and with the exact FP16 attention mass of the block:

    * spearman_*: rank correlation with the gain over all causal pairs;
    * capture_*: the gain of the top ceil(frac * (i+1)) blocks of each row
      block ranked by that quantity (score: pooled-mean dot product;
      blockmax: the block's largest exact score; mass), over the gain of the
      top blocks ranked by the gain itself (1 = the best single-block picks);
      capture_select takes the library's FP16 lists at frac instead (first
      and diagonal blocks forced);
    * concentration: the gain of those best picks over the total gain.
    """
    import torch

    from . import binding, synth

    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    x = synth.generate(workload, N=N)
    w = x["w"]
    B, Hq, Hkv, Nn, d = w.B, w.Hq, w.Hkv, w.N, w.d
    nb = Nn // 64
    grp = Hq // Hkv
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    qz = binding.quantize(q, k, v)
    del q, k, v
    ws = torch.empty(binding.attn_workspace_bytes(B, Hq, Hkv, Nn, d), dtype=torch.uint8, device=dev)
    outs = {}
    for f in (1.0, 0.0):
        idx, n16 = binding.select(qz["q16"], qz["k16"], f, True)
        outs[f], _ = binding.attn_fwd(qz, idx, n16, True, workspace=ws)
    o16 = outs[1.0]

    def block_err(o):  # [B,Hq,nb] squared error of each row block
        return ((o - o16) ** 2).view(B, Hq, nb, 64 * d).sum(-1, dtype=torch.float64)

    base = block_err(outs[0.0])
    gain = torch.full((B, Hq, nb, nb), float("nan"), dtype=torch.float64, device=dev)
    buf = torch.empty_like(o16)
    ar = torch.arange(nb, device=dev)
    for delta in range(nb):
        idx, n16 = offset_lists(B, Hq, nb, delta, dev)
        binding.attn_fwd(qz, idx, n16, True, out=buf, workspace=ws)
        rows = ar[delta:]
        gain[:, :, rows, rows - delta] = (base - block_err(buf))[:, :, rows]
    # the heuristic's block score and the block's largest exact score, as the
    # library computes them (thrift_block_scores), on a [B,Hq,nb,nb] grid
    score = scores_grid(binding.block_scores(qz["q16"], qz["k16"], "pooled_mean"), B, Hq, nb)
    bmax = scores_grid(binding.block_scores(qz["q16"], qz["k16"], "block_max"), B, Hq, nb)
    # exact attention mass of each block under FP16 attention
    mass = torch.zeros((B, Hq, nb, nb), dtype=torch.float64, device=dev)
    sm = 1.0 / math.sqrt(d)
    kf = qz["k16"].float()
    for b in range(B):
        for h in range(Hq):
            kh = kf[b, h // grp]
            for r0 in range(0, Nn, 2048):
                r1 = min(Nn, r0 + 2048)
                s_ = torch.matmul(qz["q16"][b, h, r0:r1].float(), kh[:r1].t().contiguous()) * sm
                t = torch.arange(r0, r1, device=dev)[:, None]
                s_.masked_fill_(torch.arange(r1, device=dev)[None, :] > t, float("-inf"))
                p_ = torch.softmax(s_, dim=-1)
                pad = (-r1) % 64
                if pad:
                    p_ = torch.nn.functional.pad(p_, (0, pad))
                m_ = p_.view((r1 - r0) // 64, 64, -1, 64).sum((1, 3), dtype=torch.float64)
                mass[b, h, r0 // 64:r1 // 64, : m_.shape[1]] = m_
    valid = ~torch.isnan(gain)
    g_all, s_all, m_all = gain[valid], score[valid], mass[valid]
    res = {
        "workload": workload, "N": Nn, "pairs": int(valid.sum()), "frac": frac,
        "spearman_score": round(_spearman(g_all, s_all), 4),
        "spearman_mass": round(_spearman(g_all, m_all), 4),
    }
    # per row block: top ceil(frac*(i+1)) picks by each ranking
    kk = torch.ceil(frac * (ar + 1).double()).long()  # [nb]
    neg = float("-inf")

    def picked_gain(key):
        kmask = torch.where(valid, key, torch.full_like(key, neg))
        order = torch.argsort(kmask, dim=-1, descending=True)
        g_sorted = torch.gather(torch.nan_to_num(gain, nan=0.0), -1, order)
        take = ar[None, None, None, :] < kk[None, None, :, None]
        return (g_sorted * take).sum()

    best = picked_gain(torch.nan_to_num(gain, nan=neg))
    total = torch.nan_to_num(gain, nan=0.0).sum()
    res["capture_score"] = round(float(picked_gain(score) / best), 4)
    res["capture_blockmax"] = round(float(picked_gain(bmax) / best), 4)
    res["capture_mass"] = round(float(picked_gain(mass) / best), 4)
    # the library's own selection at frac (first and diagonal blocks forced,
    # then the best pooled scores): gain of the FP16 lists it returns
    idx, n16 = binding.select(qz["q16"], qz["k16"], frac, True)
    T = nb * (nb + 1) // 2
    rb = torch.repeat_interleave(ar, ar + 1)  # row block of each list position
    pos = torch.arange(T, device=dev) - rb * (rb + 1) // 2
    in16 = pos[None, None, :] < n16.long()[:, :, rb]  # [B,Hq,T] FP16-list positions
    j = idx.long().view(B, Hq, T)
    g_sel = torch.gather(torch.nan_to_num(gain, nan=0.0).view(B, Hq, nb * nb), -1, rb[None, None, :] * nb + j)
    res["capture_select"] = round(float((g_sel * in16).sum() / best), 4)
    res["concentration"] = round(float(best / total), 4)
    res["seconds"] = round(time.perf_counter() - t0, 2)
    if log:
        log(json.dumps(res))
    return res


def scores_grid(flat, B: int, Hq: int, nb: int):
    """Causal block scores in the list layout (row i of each head at
    i(i+1)/2, entry j) -> a [B,Hq,nb,nb] fp64 grid, -inf above the diagonal."""
    import torch

    dev = flat.device
    ar = torch.arange(nb, device=dev)
    rb = torch.repeat_interleave(ar, ar + 1)
    pos = torch.arange(nb * (nb + 1) // 2, device=dev) - rb * (rb + 1) // 2
    g = torch.full((B, Hq, nb * nb), float("-inf"), dtype=torch.float64, device=dev)
    g[:, :, rb * nb + pos] = flat.view(B, Hq, -1).double()
    return g.view(B, Hq, nb, nb)


def heuristics(workload: str = "long_128k", N: int | None = None, frac: float = 0.05, log=None) -> list:
    """Output error of the mixed path when the FP16 blocks come from the
    library's other block scores (thrift_select_ex), each under the same
    budget rule (first and diagonal blocks forced):

    * pooled_mean: the selector's own score (thrift_select);
    * max_pooled: max over the key rows r of block j of (q-block mean . k_r),
      so a single strong key is not averaged away;
    * norm_weighted: block means weighted by each row's L2 norm;
    * block_max: the block's largest exact score (needs the full QK^T; a
      comparator, not a cheap heuristic).

    Each entry: err and needle-row err against the all-FP16 output, the
    share of causal tiles computed in FP16, and the selection's time.
    """
    import torch

    from . import binding, synth

    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    x = synth.generate(workload, N=N)
    w = x["w"]
    B, Hq, Hkv, Nn, d = w.B, w.Hq, w.Hkv, w.N, w.d
    nb = Nn // 64
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    qz = binding.quantize(q, k, v)
    del q, k, v
    ws = torch.empty(binding.attn_workspace_bytes(B, Hq, Hkv, Nn, d), dtype=torch.uint8, device=dev)
    rows = torch.tensor([(b * Hq + hq) * Nn + t for (b, kvh, hq, p, t) in x["needles"]], device=dev)
    idx, n16 = binding.select(qz["q16"], qz["k16"], 1.0, True)
    ref, _ = binding.attn_fwd(qz, idx, n16, True, workspace=ws)
    r2 = ref.reshape(-1, d)[rows]
    ref_norm, r2_norm = torch.linalg.vector_norm(ref).item(), torch.linalg.vector_norm(r2).item()
    tiles = B * Hq * nb * (nb + 1) // 2
    out = []

    def run(name, idx, n16, **extra):
        o, _ = binding.attn_fwd(qz, idx, n16, True, workspace=ws)
        r = {"heuristic": name, "workload": workload, "N": Nn, "frac": frac,
             "err": round(torch.linalg.vector_norm(o - ref).item() / ref_norm, 6),
             "needle_err": round(torch.linalg.vector_norm(o.reshape(-1, d)[rows] - r2).item() / r2_norm, 6),
             "fp16_tile_share": round(float(n16.sum()) / tiles, 5), **extra}
        if log:
            log(json.dumps(r))
        out.append(r)

    idx0, n160 = binding.select(qz["q16"], qz["k16"], 0.0, True)
    run("fp4_only", idx0, n160)
    del idx0, n160
    # each block score through the library's selection (thrift_select for the
    # pooled mean, thrift_select_ex for the others), timed alone
    sws = torch.empty(binding.lib().thrift_select_workspace_bytes(binding.make_shape(B, Hq, Hkv, Nn, d)),
                      dtype=torch.uint8, device=dev)
    for name in ("pooled_mean", "max_pooled", "norm_weighted", "block_max"):
        idx, n16 = binding.select(qz["q16"], qz["k16"], frac, True, workspace=sws, score=name)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        binding.select(qz["q16"], qz["k16"], frac, True, workspace=sws, idx=idx, n16=n16, score=name)
        e1.record()
        torch.cuda.synchronize()
        run(name, idx, n16, select_ms=round(e0.elapsed_time(e1), 4))
        del idx, n16
    for r in out:
        r["seconds"] = round(time.perf_counter() - t0, 2)
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--sweep", default="4096,8192,16384,32768,65536,131072",
                    help="comma-separated sequence lengths (multiples of 64)")
    ap.add_argument("--workload", default="long_128k")
    ap.add_argument("--frac", type=float, default=None)
    ap.add_argument("--attribution", action="store_true",
                    help="block-level error attribution instead of the length sweep")
    ap.add_argument("--heuristics", action="store_true",
                    help="output error under other block scores and at block size 128")
    ap.add_argument("--N", type=int, default=None, help="sequence length of the attribution or heuristics run")
    args = ap.parse_args(argv)
    Ns = [int(s) for s in args.sweep.split(",") if s]
    if any(n <= 0 or n % 64 for n in Ns) or (args.N is not None and (args.N <= 0 or args.N % 64)):
        print("sequence lengths must be positive multiples of 64", file=sys.stderr)
        return 2
    log = lambda s: print(s, flush=True)  # noqa: E731
    if args.attribution:
        attribution(args.workload, args.N, 0.05 if args.frac is None else args.frac, log=log)
    elif args.heuristics:
        heuristics(args.workload, args.N, 0.05 if args.frac is None else args.frac, log=log)
    else:
        length_sweep(Ns, args.workload, args.frac, log=log)
    return 0


if __name__ == "__main__":
    sys.exit(main())
