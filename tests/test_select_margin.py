"""The error bound behind the selection's fp32 scoring (no GPU).

The library ranks block pairs by sequential fp32 fma chains over the
channels and settles every block within M = 2 d 2^-24 |q| max_j |k_j| of the
cut-off by its fp64 chain.  That is exact only if every fp32 chain lies within
M of the fp64 chain.  These tests emulate both chains (an fma rounds the exact
a*b + s once: a*b of two fp32 values is exact in fp64, so the fp64 sum rounded
to fp32 is the fma up to a double rounding of at most 2^-53 relative) and check
the bound on random, cancelling and wide-range means, with the norms rounded
up as the library computes them."""
import numpy as np
import pytest


def fp32_chain(q, k):
    """Sequential fp32 fma chains of every (row of q, row of k), channel order."""
    s = np.zeros((q.shape[0], k.shape[0]), np.float32)
    for c in range(q.shape[1]):
        s = (np.outer(q[:, c].astype(np.float64), k[:, c].astype(np.float64)) + s.astype(np.float64)).astype(np.float32)
    return s.astype(np.float64)


def fp64_chain(q, k):
    s = np.zeros((q.shape[0], k.shape[0]))
    for c in range(q.shape[1]):
        s = np.outer(q[:, c].astype(np.float64), k[:, c].astype(np.float64)) + s
    return s


def norms_up(x):
    """fp64 norm of each fp32 row, rounded up to fp32."""
    n = np.sqrt((x.astype(np.float64) ** 2).sum(1))
    f = n.astype(np.float32)
    return np.where(f.astype(np.float64) < n, np.nextafter(f, np.float32(np.inf)), f).astype(np.float64)


def margin(q, k):
    d = q.shape[1]
    kmax = norms_up(k)[1:].max()  # block 0 is never a candidate
    return 2.0 * d * 2.0 ** -24 * norms_up(q)[:, None] * kmax


def cases(d, seed):
    g = np.random.default_rng(seed)
    n = 96
    yield "normal", g.standard_normal((n, d)), g.standard_normal((n, d))
    # heavy cancellation: large terms of both signs that nearly cancel
    base = g.standard_normal(d) * 1e3
    q = np.tile(base, (n, 1)) * np.where(np.arange(d) % 2, 1.0, -1.0) + g.standard_normal((n, d)) * 1e-3
    yield "cancelling", q, np.tile(np.abs(base), (n, 1)) + g.standard_normal((n, d)) * 1e-3
    # wide dynamic range across channels and blocks
    scale = 2.0 ** g.integers(-30, 20, size=(1, d))
    yield "wide range", g.standard_normal((n, d)) * scale, g.standard_normal((n, d)) / scale
    # nearly parallel rows (scores close together, the selection's hard case)
    r = g.standard_normal(d)
    yield "near-parallel", np.tile(r, (n, 1)) + g.standard_normal((n, d)) * 1e-6, \
        np.tile(r, (n, 1)) + g.standard_normal((n, d)) * 1e-6


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("seed", [1, 2])
def test_fp32_chains_lie_within_the_margin(d, seed):
    for name, q, k in cases(d, seed):
        q32, k32 = q.astype(np.float32), k.astype(np.float32)
        s32, s64 = fp32_chain(q32, k32), fp64_chain(q32, k32)
        err = np.abs(s32 - s64)
        m = margin(q32, k32)
        # block 0 is excluded from the max norm and never ranked: check j >= 1
        assert np.all(err[:, 1:] <= m[:, :]), (name, float((err[:, 1:] / m).max()))
        # and the bound is not vacuous: the chains do differ
        assert err.max() > 0, name


def test_margin_has_room_for_the_worst_chain():
    # the worst case of a sequential chain, d terms of one sign and growing
    # partial sums, stays below half the margin (the factor 2 is slack)
    d = 128
    q = np.full((2, d), 1.0 + 2.0 ** -12, np.float32)
    k = np.full((2, d), 1.0 - 2.0 ** -13, np.float32)
    err = np.abs(fp32_chain(q, k) - fp64_chain(q, k))
    assert np.all(err <= 0.5 * margin(q, k))
