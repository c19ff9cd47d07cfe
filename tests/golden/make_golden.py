"""Write oracle_tiny.json: the oracle's results on one tiny seeded case.

A regression fixture of the oracle, not a pin: the ThriftAttention pages
print no worked example, table or value of the method's output, so nothing
here comes from them.  It records what the oracle (as pinned by
tests/test_oracle_pins.py) computes, so that any later change of its
arithmetic shows up in tests/test_golden.py and has to be justified.

Calls only oracle/ and the seeded input generator.  Run from the repository
root:  python tests/golden/make_golden.py
"""
from __future__ import annotations

import hashlib
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
FIXTURE = os.path.join(HERE, "oracle_tiny.json")
CASE = {"B": 1, "Hq": 2, "Hkv": 1, "N": 192, "d": 64, "dtype": "fp16", "seed": 4242, "scale": 1.5,
        "frac": 0.3, "causal": True}
ROW_STEP = 29      # sampled output rows: every 29th flat row
OUT_ROWS = 4       # full output vectors stored for the first few sampled rows


def compute() -> dict:
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import oracle
    from fp16_long_context_amd import synth

    c = CASE
    q, k, v = synth.random_qkv(c["B"], c["Hq"], c["Hkv"], c["N"], c["d"], c["dtype"], seed=c["seed"],
                               scale=c["scale"])
    qz = oracle.quantize(synth.bits(q), synth.bits(k), synth.bits(v), c["dtype"])
    sel = oracle.select(qz["q16"], qz["k16"], c["frac"], c["causal"])
    rows = np.arange(0, c["B"] * c["Hq"] * c["N"], ROW_STEP, dtype=np.int64)
    res = {"case": c, "row_step": ROW_STEP,
           "sha256": {n: hashlib.sha256(np.ascontiguousarray(qz[n]).tobytes()).hexdigest() for n in sorted(qz)},
           "idx": sel["idx"].tolist(), "n16": sel["n16"].ravel().tolist(), "rows": rows.tolist()}
    for rs in ("p", "weights"):
        r = oracle.attn_rows(qz, sel, rows, c["causal"], rowsum=rs)
        res[f"lse_{rs}"] = r["lse"].tolist()
        res[f"l_{rs}"] = r["l"].tolist()
        res[f"m_{rs}"] = r["m"].tolist()
        res[f"out_{rs}"] = r["out"][:OUT_ROWS].tolist()
    return res


if __name__ == "__main__":
    with open(FIXTURE, "w") as f:
        json.dump(compute(), f, indent=0)
        f.write("\n")
    print(f"wrote {FIXTURE} ({os.path.getsize(FIXTURE)} bytes)")
