"""Host-side checks of the quality-study entry point (no GPU)."""
from fp16_long_context_amd import quality


def test_rejects_lengths_not_multiple_of_block():
    assert quality.main(["--sweep", "4096,100"]) == 2
    assert quality.main(["--sweep", "0"]) == 2


def test_offset_lists_layout():
    # row block i: FP16 list [i - delta] (none when i < delta), then the other
    # valid blocks ascending; n16 counts the FP16 entry
    for nb in (1, 2, 5, 9):
        for delta in range(nb + 1):
            idx, n16 = quality.offset_lists(2, 3, nb, delta, "cpu")
            want = []
            for i in range(nb):
                j16 = i - delta
                want += ([j16] if j16 >= 0 else []) + [j for j in range(i + 1) if j != j16]
            assert idx.tolist() == want * 6
            assert n16.shape == (2, 3, nb)
            assert n16[1, 2].tolist() == [1 if i >= delta else 0 for i in range(nb)]


def _select_brute(score, frac, causal):
    """The budget rule written out per row block (plain Python)."""
    import math

    nb = len(score)
    ppm = int(math.floor(frac * 1e6 + 0.5))
    out = []
    for i in range(nb):
        valid = list(range(i + 1)) if causal else list(range(nb))
        if ppm == 0:
            out.append(set())
            continue
        forced = {0, i}
        k = min(len(valid), max(len(forced), -(-ppm * len(valid) // 1000000)))
        rest = sorted((j for j in valid if j not in forced), key=lambda j: (-score[i][j], j))
        out.append(forced | set(rest[: k - len(forced)]))
    return out


def test_select_mask_matches_budget_rule():
    import numpy as np
    import torch

    g = np.random.default_rng(7)
    for nb in (1, 2, 3, 8, 13):
        for frac in (0.0, 0.05, 0.3, 0.5, 1.0):
            for causal in (True, False):
                for ties in (False, True):
                    sc = g.integers(-2, 3, (nb, nb)).astype(float) if ties else g.standard_normal((nb, nb))
                    m = quality.select_mask(torch.tensor(sc)[None, None], frac, causal)[0, 0]
                    want = _select_brute(sc.tolist(), frac, causal)
                    got = [set(np.nonzero(m[i].numpy())[0].tolist()) for i in range(nb)]
                    assert got == want, (nb, frac, causal, ties)


def test_lists_from_mask_layout():
    import numpy as np
    import torch

    g = np.random.default_rng(3)
    for nb in (1, 4, 7):
        for causal in (True, False):
            m = torch.tensor(g.random((2, 3, nb, nb)) < 0.3)
            idx, n16 = quality.lists_from_mask(m, causal)
            want, wn = [], []
            for b in range(2):
                for h in range(3):
                    for i in range(nb):
                        valid = range(i + 1) if causal else range(nb)
                        f16 = [j for j in valid if m[b, h, i, j]]
                        want += f16 + [j for j in valid if not m[b, h, i, j]]
                        wn.append(len(f16))
            assert idx.tolist() == want
            assert n16.reshape(-1).tolist() == wn


def test_pooling_and_sequential_scores():
    import numpy as np
    import torch

    g = np.random.default_rng(5)
    x = torch.tensor(g.standard_normal((1, 2, 256, 16)), dtype=torch.float16)
    m = quality.pooled_means(x)  # [1, 2, 4, 16]
    xd = x.double().numpy().reshape(1, 2, 4, 64, 16)
    assert np.array_equal(m.numpy(), (xd.sum(3) / 64).astype(np.float32))
    m2 = quality.pooled_means(x, 128)
    assert np.array_equal(m2.numpy(), (xd.reshape(1, 2, 2, 128, 16).sum(3) / 128).astype(np.float32))
    s = quality.sequential_scores(m, m)
    for i in range(4):
        for j in range(4):
            acc = 0.0
            for c in range(16):
                acc = acc + float(m[0, 1, i, c]) * float(m[0, 1, j, c])
            assert s[0, 1, i, j].item() == acc
    e = quality.expand_mask(torch.tensor([[True, False], [False, True]]), 2)
    assert e.tolist() == [[1, 1, 0, 0], [1, 1, 0, 0], [0, 0, 1, 1], [0, 0, 1, 1]]
