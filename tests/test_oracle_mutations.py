"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a copy of the oracle -- a dropped
score scale, an off-by-one band edge, a dropped D term, a perturbed or
transposed gradient product, a shifted key range, a wrong sign, narrower
bands first, a wrong FULL test -- and runs the oracle's own pin tests
(tests/test_oracle_*.py with their golden fixtures) against that copy in a
separate pytest process.  The pins must fail for every mutant, and pass for
the unmutated copy: a pin set that a planted mistake survives would not
distinguish a wrong oracle from a right one.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, file under oracle/, exact text, replacement)
MUTANTS = [
    ("dropped score scale", "attention.py",
     "s = np.where(mask, (qb @ kb.T) * sc, -np.inf)", "s = np.where(mask, (qb @ kb.T), -np.inf)"),
    ("dropped scale in the dense form", "attention.py",
     "s = (q @ k.T) * sc", "s = (q @ k.T)"),
    ("band upper edge off by one", "attention.py",
     "m = (dist >= max(lo, 0)) & (dist <= hi)", "m = (dist >= max(lo, 0)) & (dist < hi)"),
    ("band lower edge off by one", "attention.py",
     "m = (dist >= max(lo, 0)) & (dist <= hi)", "m = (dist > max(lo, 0)) & (dist <= hi)"),
    ("dropped D term", "attention.py",
     "ds = p * (dp - dcoef[:, None])\n                dq[b, h, i0:i1]", "ds = p * dp\n                dq[b, h, i0:i1]"),
    ("perturbed dK", "attention.py",
     "dk[b, h, jidx] += sc * (ds.T @ qb)", "dk[b, h, jidx] += 1.001 * sc * (ds.T @ qb)"),
    ("transposed operand in dQ", "attention.py",
     "dq[b, h, i0:i1] = sc * (ds @ kb)", "dq[b, h, i0:i1] = sc * (ds @ vb)"),
    ("shifted key range", "attention.py",
     "return max(0, i0 - hi), (i1 - 1) - lo\n", "return max(0, i0 - hi), (i1 - 1) - lo - 1\n"),
    ("LSE sign", "attention.py",
     "out = p @ vb\n    lse = np.where(nonempty, shift + np.log(safe), -np.inf)",
     "out = p @ vb\n    lse = np.where(nonempty, shift - np.log(safe), -np.inf)"),
    ("narrower bands first", "band.py",
     "width = base + (1 if h < extra else 0)", "width = base + (1 if h >= H - extra else 0)"),
    ("FULL test too strict", "tiles.py",
     "full = any(a <= d0 and d1 <= b for a, b in ranges)", "full = any(a <= d0 and d1 < b for a, b in ranges)"),
    ("window off by one", "attention.py",
     "m = m | ((dist >= 0) & (dist <= local_window - 1))", "m = m | ((dist >= 0) & (dist <= local_window))"),
]


def _tree(dst, mutant):
    """The oracle package (with one mutation applied) and its pin tests."""
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(dst, "oracle"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    tdir = os.path.join(dst, "tests")
    os.makedirs(tdir)
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(tdir, "golden"))
    for f in sorted(os.listdir(os.path.join(ROOT, "tests"))):
        if f.startswith("test_oracle_") and f.endswith(".py") and f != os.path.basename(__file__):
            shutil.copy(os.path.join(ROOT, "tests", f), tdir)
    with open(os.path.join(tdir, "conftest.py"), "w") as fh:
        fh.write("import os, sys\nsys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))\n")
    with open(os.path.join(dst, "pytest.ini"), "w") as fh:
        fh.write("[pytest]\ntestpaths = tests\n")
    if mutant is not None:
        _, fname, old, new = mutant
        path = os.path.join(dst, "oracle", fname)
        src = open(path).read()
        assert src.count(old) == 1, f"mutation site not unique in {fname}: {old!r}"
        with open(path, "w") as fh:
            fh.write(src.replace(old, new))


def _run_pins(dst):
    env = dict(os.environ, OMP_NUM_THREADS="2", OPENBLAS_NUM_THREADS="2", MKL_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-c",
                        os.path.join(dst, "pytest.ini"), "--rootdir", dst],
                       cwd=dst, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


def test_every_planted_mistake_fails_a_pin(tmp_path):
    dirs = []
    for i, m in enumerate([None] + MUTANTS):
        d = str(tmp_path / f"m{i}")
        os.makedirs(d)
        _tree(d, m)
        dirs.append(d)
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(_run_pins, dirs))
    rc0, out0 = results[0]
    assert rc0 == 0, f"the unmutated oracle must pass its pins:\n{out0}"
    survived = [MUTANTS[i][0] for i, (rc, _) in enumerate(results[1:]) if rc == 0]
    assert not survived, f"mutants not caught by any pin: {survived}"
    for (name, *_), (rc, out) in zip(MUTANTS, results[1:]):
        assert rc == 1, f"{name}: pytest exit {rc} (not a test failure):\n{out}"
