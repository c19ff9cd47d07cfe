"""The seeded generators: deterministic, shaped like the workloads, with the
planted structure (needles, sinks) present."""
import hashlib

import numpy as np
import torch

from fp16_long_context_amd import synth


def digest(t):
    return hashlib.sha256(synth.bits(t).tobytes()).hexdigest()


def test_deterministic_and_thread_independent(monkeypatch):
    a = synth.generate("tiny")
    monkeypatch.setattr(synth, "_threads", lambda: 1)
    b = synth.generate("tiny")
    for n in ("q", "k", "v"):
        assert digest(a[n]) == digest(b[n])
    c = synth.generate("tiny", seed=5)
    assert digest(a["q"]) != digest(c["q"])


def test_shapes_dtypes_and_needles():
    x = synth.generate("tiny")
    w = x["w"]
    assert x["q"].shape == (1, 2, 1024, 64) and x["q"].dtype == torch.float16
    assert len(x["needles"]) == 4 * 2
    for (b, kvh, hq, p, t) in x["needles"]:
        assert p < t
        assert torch.equal(x["k"][b, kvh, p], (4 * x["q"][b, hq, t].float()).to(torch.float16))
    y = synth.generate("llama8b_16k", N=2048)
    assert y["q"].shape == (1, 32, 2048, 128) and y["k"].shape == (1, 8, 2048, 128)
    assert y["q"].dtype == torch.bfloat16
    # sinks: keys 0-3 boosted x8
    assert y["k"][:, :, :4].float().abs().mean() > 5 * y["k"][:, :, 4:].float().abs().mean()
    assert len(y["needles"]) == 8 * 64
    z = synth.generate("batched_32k", N=1024, B=2)
    counts = np.bincount([n[0] for n in z["needles"]], minlength=2) // 4
    assert all(16 <= c <= 128 for c in counts)
    r = synth.generate("long_128k", N=512)
    assert r["q"].shape == (1, 32, 512, 128) and torch.isfinite(r["q"].float()).all()
