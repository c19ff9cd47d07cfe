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


def test_scores_grid_layout():
    # list-layout scores (row i at i(i+1)/2, entry j) land at [b, h, i, j];
    # above the diagonal stays -inf
    import torch

    B, Hq, nb = 2, 3, 5
    T = nb * (nb + 1) // 2
    flat = torch.arange(B * Hq * T, dtype=torch.float32)
    g = quality.scores_grid(flat, B, Hq, nb)
    for b in range(B):
        for h in range(Hq):
            for i in range(nb):
                for j in range(nb):
                    want = float((b * Hq + h) * T + i * (i + 1) // 2 + j) if j <= i else float("-inf")
                    assert g[b, h, i, j].item() == want
