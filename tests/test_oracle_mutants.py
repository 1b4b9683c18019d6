"""The oracle's pins must catch plausible mistakes in it.

Each case plants one mistake in a copy of the oracle's C source (a dropped
term, a flipped sign, a wrong index, the running state used where the pages
take the chunk-start state, ...), builds the copy, and runs the pin suite
(tests/test_oracle_pins.py, or tests/test_oracle_glue.py for the layer glue's
oracle) against it in a separate process: the suite must fail.  The real
oracle is never modified.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (what the mistake is, exact text in osr_oracle.c, replacement)
MUTANTS = [
    ("update adds the write instead of subtracting it",
     "S[(size_t)i * d + j] = Ghat[i] * S[(size_t)i * d + j] - khat[i] * h[j];",
     "S[(size_t)i * d + j] = Ghat[i] * S[(size_t)i * d + j] + khat[i] * h[j];"),
    ("update norm adds the projection term (the appendix's printed sign)",
     "double dsq = wi * wi * (hsq - dot * dot);",
     "double dsq = wi * wi * (hsq + dot * dot);"),
    ("beta without the forget gate",
     "const double beta = 1.0 / sqrt(mu * mu + dsq);",
     "const double beta = 1.0 / sqrt(1.0 + dsq);"),
    ("gate without the projection coefficient",
     "? mu * beta : mu * beta + htil[i] * khat[i];",
     "? mu * beta : mu * beta;"),
    ("first linearisation: projection term on the running slot",
     "+ htil[i] * khat[i] * Z[(size_t)i * d + j]",
     "+ htil[i] * khat[i] * S[(size_t)i * d + j]"),
    ("first linearisation: projection term dropped",
     "+ htil[i] * khat[i] * Z[(size_t)i * d + j]",
     "+ 0.0 * Z[(size_t)i * d + j]"),
    ("decoding error from the running state instead of the chunk-start state",
     "acc += kt[i] * Z[(size_t)i * d + j];",
     "acc += kt[i] * S[(size_t)i * d + j];"),
    ("projection coefficient from the running state",
     "dot += Z[(size_t)i * d + j] * h[j];",
     "dot += S[(size_t)i * d + j] * h[j];"),
    ("decoding error with v added",
     "h[j] = p->mode == ORACLE_MODE_ENC ? vt[j] : acc - vt[j];",
     "h[j] = p->mode == ORACLE_MODE_ENC ? vt[j] : acc + vt[j];"),
    ("read-out from the chunk-start state",
     "acc += qt[i] * S[(size_t)i * d + j];",
     "acc += qt[i] * Z[(size_t)i * d + j];"),
    ("per-slot gamma read as per-token",
     "const double g = p->gamma_per_slot ? gt[i] : gt[0];",
     "const double g = gt[0];"),
    ("encoding layer: h = -v",
     "h[j] = p->mode == ORACLE_MODE_ENC ? vt[j] : acc - vt[j];",
     "h[j] = p->mode == ORACLE_MODE_ENC ? -vt[j] : acc - vt[j];"),
    ("encoding layer: error with its sign reversed",
     "const double ci = p->mode == ORACLE_MODE_ENC ? dot - kt[i] : kt[i];",
     "const double ci = p->mode == ORACLE_MODE_ENC ? kt[i] - dot : kt[i];"),
    ("encoding layer written with k instead of its error",
     "const double ci = p->mode == ORACLE_MODE_ENC ? dot - kt[i] : kt[i];",
     "const double ci = kt[i];"),
    ("slots not projected at chunk starts",
     "        int rc = project_slots(S, m, d);\n        if (rc != ORACLE_OK) return rc;\n        memcpy(Z, S,",
     "        int rc = ORACLE_OK;\n        if (t0 == 0) rc = project_slots(S, m, d);\n        if (rc != ORACLE_OK) return rc;\n        memcpy(Z, S,"),
]


def _copy_tree(dst):
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(dst, "oracle"),
                    ignore=shutil.ignore_patterns("*.so", "*.tmp", "__pycache__"))
    pkg = os.path.join(dst, "compressed_memory_linear_amd")
    os.makedirs(pkg)
    shutil.copy(os.path.join(ROOT, "compressed_memory_linear_amd", "synth.py"), pkg)
    with open(os.path.join(pkg, "__init__.py"), "w") as f:
        f.write("")
    tdir = os.path.join(dst, "tests")
    os.makedirs(tdir)
    for name in ("test_oracle_pins.py", "test_oracle_glue.py", "conftest.py"):
        shutil.copy(os.path.join(ROOT, "tests", name), tdir)
    shutil.copy(os.path.join(ROOT, "pytest.ini"), dst)


def _run_pins(dst, suite="test_oracle_pins.py"):
    env = dict(os.environ, PYTHONPATH=dst, OMP_NUM_THREADS="1")
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           os.path.join("tests", suite)],
                          cwd=dst, env=env, capture_output=True, text=True, timeout=600)


def test_unmodified_copy_passes(tmp_path):
    """Control: the copied tree with the oracle as it is passes every pin."""
    dst = str(tmp_path)
    _copy_tree(dst)
    r = _run_pins(dst)
    assert r.returncode == 0 and " passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]


@pytest.mark.parametrize("what,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, what, old, new):
    dst = str(tmp_path)
    _copy_tree(dst)
    src = os.path.join(dst, "oracle", "osr_oracle.c")
    with open(src) as f:
        text = f.read()
    assert text.count(old) == 1, f"mutation site not found once: {what}"
    with open(src, "w") as f:
        f.write(text.replace(old, new))
    r = _run_pins(dst)
    # a pin assertion must fail (not a build or collection error)
    assert " failed" in r.stdout and r.returncode == 1, f"no pin caught: {what}\n{r.stdout[-2000:]}"


# Mistakes in the layer glue's oracle (osr_glue.c), caught by tests/test_oracle_glue.py.
GLUE_MUTANTS = [
    ("convolution taps reversed",
     "acc += w[(size_t)n * GLUE_W + j] * xv;",
     "acc += w[(size_t)n * GLUE_W + (GLUE_W - 1 - j)] * xv;"),
    ("convolution bias dropped",
     "double acc = b ? b[n] : 0.0;",
     "double acc = 0.0;"),
    ("handed-on history one row early",
     "const int s = T - P + r;",
     "const int s = T - P + r - 1;"),
    ("sigmoid of the negated logit",
     "out[i] = 1.0 / (1.0 + exp(-logit[i]));",
     "out[i] = 1.0 / (1.0 + exp(logit[i]));"),
    ("GeLU with Phi(-x)",
     "out[i] = y[i] * (x * (0.5 * erfc(-x / sqrt(2.0))));",
     "out[i] = y[i] * (x * (0.5 * erfc(x / sqrt(2.0))));"),
    ("GeLU without its factor x",
     "out[i] = y[i] * (x * (0.5 * erfc(-x / sqrt(2.0))));",
     "out[i] = y[i] * (0.5 * erfc(-x / sqrt(2.0)));"),
]


def test_unmodified_copy_passes_glue_pins(tmp_path):
    dst = str(tmp_path)
    _copy_tree(dst)
    r = _run_pins(dst, "test_oracle_glue.py")
    assert r.returncode == 0 and " passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]


@pytest.mark.parametrize("what,old,new", GLUE_MUTANTS, ids=[m[0] for m in GLUE_MUTANTS])
def test_glue_pins_catch_planted_mistake(tmp_path, what, old, new):
    dst = str(tmp_path)
    _copy_tree(dst)
    src = os.path.join(dst, "oracle", "osr_glue.c")
    with open(src) as f:
        text = f.read()
    assert text.count(old) == 1, f"mutation site not found once: {what}"
    with open(src, "w") as f:
        f.write(text.replace(old, new))
    r = _run_pins(dst, "test_oracle_glue.py")
    assert " failed" in r.stdout and r.returncode == 1, f"no pin caught: {what}\n{r.stdout[-2000:]}"
