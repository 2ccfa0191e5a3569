"""The oracle's pins catch plausible mistakes: each case plants one mistake in a temporary copy
of the oracle (a textual substitution in oracle/bsfa_oracle.py, on the CPU) and runs the pins
(tests/test_oracle_pins.py) against it in a fresh interpreter; at least one pin must fail.

The planted mistakes are the slips a reader of the pages could make: ">" for ">=" at the
threshold, a dropped softmax scale, an off-by-one diagonal region, the rescale factor inverted,
the relative statistic taken over the wrong extreme, the k-th highest off by one, the wrong
threshold column past the calibrated length, the wrong KV head, the wrong mean in calibration;
for mean correction a dropped log|B| shift, a summed mean, a dropped scale, the block max for the
mean key; for the FP8 gate a signed amax, round-half-up, a wrong minimum exponent, a wrong
largest value and a dropped row scale.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle", "bsfa_oracle.py")

MUTATIONS = [
    ("'>' instead of '>=' at the threshold", "keep = st >= thr", "keep = st > thr"),
    ("softmax scale dropped", "s = (q @ K[b, c0:c1, g, :].T) * sc\n",
     "s = (q @ K[b, c0:c1, g, :].T) * 1.0\n"),
    ("diagonal region one block late", "n_off = (prefix + i * block_q) // block_k",
     "n_off = (prefix + i * block_q) // block_k + 1"),
    ("rescale factor inverted", "alpha = np.exp(m - m_new)", "alpha = np.exp(m_new - m)"),
    ("relative statistic over the wrong extreme", "st = float((rmax - m).max())",
     "st = float((rmax - m).min())"),
    ("k-th highest off by one", "[::-1][k - 1])", "[::-1][k])"),
    ("first column past the calibrated length",
     "return float(table[budget_slice, h, min(i, t_len - 1)])",
     "return float(table[budget_slice, h, min(i, t_len - 1) if i < t_len else 0])"),
    ("wrong KV head", "absorb(s, V[b, c0:c1, g, :])", "absorb(s, V[b, c0:c1, h % V.shape[2], :])"),
    ("wrong mean over calibration samples", "return (acc / count).astype(np.float32)",
     "return (acc / max(1, count - 1)).astype(np.float32)"),
    ("mean correction without the log|B| shift", "* sc + dtype(math.log(c1 - c0))", "* sc"),
    ("mean correction with a summed value", "vbar = V[b, c0:c1, g, :].mean(axis=0)",
     "vbar = V[b, c0:c1, g, :].sum(axis=0)"),
    ("mean correction without the scale", "sbar = (q @ kbar) * sc + dtype(",
     "sbar = (q @ kbar) + dtype("),
    ("mean correction with the block max key", "kbar = K[b, c0:c1, g, :].mean(axis=0)",
     "kbar = K[b, c0:c1, g, :].max(axis=0)"),
    ("FP8 row scale from a signed amax", "amax = np.abs(Q).max(axis=-1)", "amax = Q.max(axis=-1)"),
    ("FP8 rounding half up", "q = np.minimum(np.round(a / step) * step, E4M3_MAX)",
     "q = np.minimum(np.floor(a / step + 0.5) * step, E4M3_MAX)"),
    ("FP8 minimum exponent -7", "step = np.exp2(np.maximum(e, -6.0) - 3.0)",
     "step = np.exp2(np.maximum(e, -7.0) - 3.0)"),
    ("FP8 largest value 447", "E4M3_MAX = 448.0", "E4M3_MAX = 447.0"),
    ("FP8 row scale dropped",
     "Q8f = (q8.astype(np.float64) * q8s[..., None]).astype(dtype)",
     "Q8f = q8.astype(dtype)"),
]


def _run_pins(tmp_path, old, new):
    src = open(ORACLE).read()
    assert src.count(old) >= 1, f"mutation target not found: {old!r}"
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle",
                    ignore=shutil.ignore_patterns("__pycache__"))
    (tmp_path / "oracle" / "bsfa_oracle.py").write_text(src.replace(old, new))
    tdir = tmp_path / "tests"
    tdir.mkdir()
    for f in ("test_oracle_pins.py", "pins_util.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), tdir / f)
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), tdir / "golden")
    # the mutated oracle first on the path; the rest of the repository after it
    (tdir / "conftest.py").write_text(
        "import sys\n"
        f"sys.path.insert(0, {str(tmp_path)!r})\n"
        f"sys.path.insert(1, {ROOT!r})\n"
        "import pytest, os\n"
        "@pytest.fixture(scope='session')\n"
        "def golden_dir():\n"
        f"    return {str(tdir / 'golden')!r}\n")
    env = dict(os.environ, PYTHONPATH=str(tmp_path), PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        str(tdir / "test_oracle_pins.py")], cwd=str(tmp_path), env=env,
                       capture_output=True, text=True, timeout=600)
    return r


def test_unmutated_copy_passes_the_pins(tmp_path):
    # the harness itself: the copy without a planted mistake passes
    r = _run_pins(tmp_path, "keep = st >= thr", "keep = st >= thr")
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("what,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(what, old, new, tmp_path):
    r = _run_pins(tmp_path, old, new)
    # 1: tests ran and at least one failed (not a collection or import error)
    assert r.returncode == 1, f"no pin caught: {what}\n{r.stdout[-2000:]}"
