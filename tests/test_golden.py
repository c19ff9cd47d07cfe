"""The oracle against its regression record (tests/golden/oracle_tiny.json,
written by tests/golden/make_golden.py from the oracle alone)."""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))
import make_golden  # noqa: E402


def test_oracle_matches_its_record():
    with open(make_golden.FIXTURE) as f:
        want = json.load(f)
    got = make_golden.compute()
    assert got["case"] == want["case"] and got["rows"] == want["rows"]
    assert got["sha256"] == want["sha256"]        # FP16 copies and MXFP4 codes, bit for bit
    assert got["idx"] == want["idx"] and got["n16"] == want["n16"]
    for key in ("lse_p", "l_p", "m_p", "out_p", "lse_weights", "l_weights", "m_weights", "out_weights"):
        a, b = np.asarray(got[key]), np.asarray(want[key])
        assert a.shape == b.shape, key
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14, err_msg=key)
