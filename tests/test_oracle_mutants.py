"""The pins must catch plausible mistakes.  Each case plants one mistake in a
copy of the oracle's source (on the CPU, in a temporary directory; the
oracle itself is untouched), builds it, runs the pin tests that cover that
step against the mutant (LH_ORACLE_LIB), and requires at least one failure.
"""
import os
import subprocess
import sys
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "lh_oracle.c")

PINS = "tests/test_oracle_pins.py"
RULES = "tests/test_oracle_rules.py"
RAGGED = "tests/test_oracle_ragged.py"
DIAG = "tests/test_oracle_diag.py"
GPTQ = "tests/test_oracle_gptq.py"

# (name, exact source text, replacement, pin files expected to catch it)
MUTANTS = [
    ("E2M1 ties to the odd code", "d < bd || (d == bd && (c % 2) == 0)", "d < bd || (d == bd && (c % 2) == 1)", [PINS]),
    ("no saturation above 6", "if (!(x <= 6.0f))\n        return 7;", "if (!(x <= 6.0f))\n        return 0;", [PINS]),
    ("amax divisor 448 instead of 6*448", "float Sg = g / 2688.0f; /* one", "float Sg = g / 448.0f; /* one", [PINS]),
    ("subnormal E4M3 values off by 2", "return ldexp((double)m, -9);", "return ldexp((double)m, -10);", [PINS]),
    ("reciprocal multiply in the cast", "float x = a / s; /* IEEE fp32 division */",
     "float x = a * (1.0f / s); /* IEEE fp32 division */", [PINS]),
    ("residual with the wrong sign", "dw[i] = (double)oracle_quantize(w[i], s[k], 0) - (double)w[i];",
     "dw[i] = (double)oracle_quantize(w[i], s[k], 0) + (double)w[i];", [PINS]),
    ("off-diagonal Hessian terms dropped", "e += dw[i] * (double)H[i * 16 + j] * dw[j];",
     "e += (i == j) ? dw[i] * (double)H[i * 16 + j] * dw[j] : 0.0;", [PINS]),
    ("ties to the highest index", "if (E[k] < E[kb])", "if (E[k] <= E[kb])", [PINS]),
    ("Hessian not normalised", "double v = alpha * acc;", "double v = acc;", [PINS]),
    ("running mean without the old weight", "v = ((double)nold * old + acc) / (double)(nold + ng);",
     "v = (old + acc) / (double)(nold + ng);", [RAGGED]),
    ("histogram bins off by one", "const float y = x * bins_per_unit;", "const float y = x * bins_per_unit + 1.0f;",
     [DIAG]),
    ("GPTQ without dampening", "Hp[i * n + i] += damp * mean;", "Hp[i * n + i] += 0.0 * damp * mean;", [GPTQ]),
]


@pytest.mark.parametrize("name,old,new,files", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, old, new, files):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation target not found once in the oracle: %r" % old
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "mutant.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        lib = os.path.join(d, "libmutant.so")
        subprocess.run(["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared",
                        "-fPIC", "-o", lib, path, "-lm"], check=True)
        env = dict(os.environ, LH_ORACLE_LIB=lib, OMP_NUM_THREADS="4")
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider"]
                           + files, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, "mutant '%s' passed the pins:\n%s" % (name, r.stdout[-2000:])
