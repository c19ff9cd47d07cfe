"""The oracle's pins are sharp: each planted mistake below, applied to a
scratch copy of oracle/oracle.c, must make tests/test_oracle_pins.py fail,
and an edit that changes nothing (the control) must leave it passing.

CPU only.  Every mistake runs the pins in a subprocess on its own copy (the
oracle package builds its library next to its source), stopping at the first
failing pin; the copies run side by side, a few at a time, and each test
then reads its mistake's outcome.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (what the mistake is, exact text in oracle.c, replacement)
MISTAKES = [
    ("row sum dropped", "l += p[key];", "l += 0.0;"),
    ("wrong V scale group", "v4s[(kvh * d + ch) * (N / 32) + k0 / 32]", "v4s[(kvh * d + ch) * (N / 32) + (k0 / 32) ^ 1]"),
    ("diagonal block not forced", "in16[i] = 1;", "in16[i] = 0;"),
    ("real-valued running max", "M = ceil(xmax);", "M = xmax;"),
    ("E2M1 tie rounded away from even", "if (y <= 0.25) return 0;", "if (y < 0.25) return 0;"),
    ("nibble order swapped", "(uint8_t)(c[2 * i] | (c[2 * i + 1] << 4))", "(uint8_t)(c[2 * i + 1] | (c[2 * i] << 4))"),
    ("scale exponent off by one", "e = (e2 - 1) - 2;", "e = (e2 - 1) - 3;"),
    ("FP16 P not rounded", "double p16 = half_bits_to_double(double_to_half_bits(p[key]));", "double p16 = p[key];"),
    ("causal mask off by one", "if (causal && key > t) continue;", "if (causal && key > t + 1) continue;"),
    ("K scale dropped", "s += e8m0_value(qrow4s[m]) * e8m0_value(k4s[krow * (d / 32) + m]) * gs;",
     "s += e8m0_value(qrow4s[m]) * gs;"),
    ("wrong GQA map", "int64_t g = h * Hkv / Hq;", "int64_t g = h % Hkv;"),
    ("budget rounded down", "long long want = (ppm * nv + 999999) / 1000000;", "long long want = (ppm * nv) / 1000000;"),
    ("ranking ascending", "if (a->s > b->s) return -1;", "if (a->s < b->s) return -1;"),
    ("weights reading: FP16 term unrounded", "if (rowsum >= 1) l += p16;", "if (rowsum >= 1) l += p[key];"),
    ("weights reading: FP4 group scale dropped", "l += e8m0_value(ps) * gw;", "l += gw;"),
    ("max-pooled score misses the last key row",
     "for (int r = 0; r < 64; r++) {\n    double s = 0.0;\n    for (int c = 0; c < d; c++) s += (double)q[c]",
     "for (int r = 0; r < 63; r++) {\n    double s = 0.0;\n    for (int c = 0; c < d; c++) s += (double)q[c]"),
    ("norm weights squared", "w[r] = sqrt(ss);", "w[r] = ss;"),
    ("norm-weighted mean divided by the row count", "(float)(acc / wsum)", "(float)(acc / 64.0)"),
    ("block max misses the last query row", "for (int a = 0; a < 64; a++)", "for (int a = 0; a < 63; a++)"),
    ("exp-free codes: stand-in without the leading 1", "z = ldexp(1.0 + (y - f), (int)f);", "z = ldexp(y - f, (int)f);"),
    ("exp-free codes: group exponent off by one", "(int)floor(xmax - M) - 2;", "(int)floor(xmax - M) - 1;"),
    ("exp-free reading falls back to exact codes", "if (rowsum == 2) {", "if (rowsum == 3) {"),
    ("pooled mean over 63 rows", "out[(bh * nb + i) * d + c] = (float)(s / 64.0);",
     "out[(bh * nb + i) * d + c] = (float)(s / 63.0);"),
    ("LSE left in log2 units", "(M + log2(l)) * 0.69314718055994530942", "(M + log2(l))"),
    ("score scale without log2(e)", "(double)sm * 1.4426950408889634074", "(double)sm"),
]
CONTROL = ("control: no change in meaning", "l += p[key];", "l += 1.0 * p[key];")


def _run_pins(tmp_path, old, new, threads):
    work = tmp_path / "copy"
    work.mkdir()
    shutil.copytree(os.path.join(ROOT, "oracle"), work / "oracle",
                    ignore=shutil.ignore_patterns("*.so", "*.so.tmp", "__pycache__"))
    shutil.copytree(os.path.join(ROOT, "fp16_long_context_amd"), work / "fp16_long_context_amd",
                    ignore=shutil.ignore_patterns("*.so", "csrc", "__pycache__"))
    (work / "tests").mkdir()
    for f in ("__init__.py", "conftest.py", "textbook.py", "test_oracle_pins.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), work / "tests" / f)
    src_path = work / "oracle" / "oracle.c"
    src = src_path.read_text()
    assert src.count(old) >= 1, f"text not found in oracle.c: {old}"
    src_path.write_text(src.replace(old, new))
    env = dict(os.environ, OMP_NUM_THREADS=str(threads))
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=work, capture_output=True, text=True, timeout=900, env=env)
    return r.returncode, (r.stdout + r.stderr)[-800:]


@pytest.fixture(scope="module")
def outcomes(tmp_path_factory):
    """(return code, output tail) of the pins on every mistake and the
    control, keyed by description."""
    cases = list(MISTAKES) + [CONTROL]
    workers = max(1, min(len(cases), (os.cpu_count() or 2) // 2))
    threads = max(1, (os.cpu_count() or 2) // workers)
    dirs = [tmp_path_factory.mktemp(f"mistake{i}") for i in range(len(cases))]
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        runs = ex.map(lambda a: (a[1][0], _run_pins(a[0], a[1][1], a[1][2], threads)), zip(dirs, cases))
        return dict(runs)


@pytest.mark.slow
@pytest.mark.parametrize("what", [m[0] for m in MISTAKES])
def test_pins_catch_planted_mistake(outcomes, what):
    rc, tail = outcomes[what]
    assert rc == 1, f"{what}: the pins did not fail (rc {rc})\n{tail}"


@pytest.mark.slow
def test_control_edit_passes(outcomes):
    rc, tail = outcomes[CONTROL[0]]
    assert rc == 0, f"control edit broke the pins (rc {rc})\n{tail}"
