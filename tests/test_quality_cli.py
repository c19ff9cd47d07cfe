"""Host-side checks of the quality-study entry point (no GPU)."""
from fp16_long_context_amd import quality


def test_rejects_lengths_not_multiple_of_block():
    assert quality.main(["--sweep", "4096,100"]) == 2
    assert quality.main(["--sweep", "0"]) == 2
