"""Mutation check of the oracle's pins, CPU only.

Each case plants one plausible mistake in a copy of oracle/oracle.c (a wrong
tie rule, a dropped term, a swapped operand, a wrong index, a lost scale...),
builds it, and runs the oracle's pin tests against that build in a
subprocess (oracle honours MOELORA_ORACLE_LIB for exactly this).  The pins
must fail for every planted mistake; the unmodified oracle passes the same
tests in the regular suite.  The mistakes are planted in the oracle only, on
the CPU: nothing here touches the HIP library or a GPU.
"""
import os
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
SRC = ROOT / "oracle" / "oracle.c"
PINS = ["tests/test_oracle_route.py", "tests/test_oracle_align.py", "tests/test_oracle_forward.py",
        "tests/test_oracle_mxfp8.py"]

# (name, text in oracle.c, replacement, occurrence to replace (0-based))
MUTATIONS = [
    ("tie_rule_higher_index_wins", "if (best < 0 || l[e] > l[best])", "if (best < 0 || l[e] >= l[best])", 0),
    ("renorm_drops_first_term", "for (int64_t j = 0; j < K; ++j)\n            s += ex[j];",
     "for (int64_t j = 1; j < K; ++j)\n            s += ex[j];", 0),
    ("shared_weight_one", "w[K + q] = 1.0f / rsf;", "w[K + q] = 1.0f;", 0),
    ("missing_rsf", "o[hh] *= (double)rsf;", "o[hh] *= 1.0;", 0),
    ("silu_sign", "return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));", 0),
    ("gate_up_swapped", "hv[i] = silu(g[i]) * g[I + i];", "hv[i] = silu(g[I + i]) * g[i];", 0),
    ("down_lora_dropped", "y[n] += acc;", "y[n] += 0.0 * acc;", 0),
    ("adapter_index_dropped", "int64_t ae = a * Ep + e;", "int64_t ae = e;", 0),
    ("w2_reduction_index_reversed", "acc += ld(w2, base + i, dtype) * hv[i];",
     "acc += ld(w2, base + (I - 1 - i), dtype) * hv[i];", 0),
    ("align_scatter_unstable", "for (int64_t f = 0; f < P; ++f) {", "for (int64_t f = P - 1; f >= 0; --f) {", 1),
    ("bias_sign_flipped", "double k = score[e] + (bias ? (double)bias[e] : 0.0);",
     "double k = score[e] - (bias ? (double)bias[e] : 0.0);", 0),
    ("bias_reaches_the_weights", "w[j] = (float)(renorm ? score[ids[j]] / s : score[ids[j]]);",
     "w[j] = (float)(renorm ? (score[ids[j]] + (bias ? (double)bias[ids[j]] : 0.0)) / s : score[ids[j]]);", 0),
    ("e4m3_exponent_bias", "v = ldexp(8.0 + (double)man, ex - 10);", "v = ldexp(8.0 + (double)man, ex - 9);", 0),
]


def _replace_nth(text: str, old: str, new: str, n: int) -> str:
    at = -1
    for _ in range(n + 1):
        at = text.index(old, at + 1)
    return text[:at] + new + text[at + len(old):]


@pytest.mark.parametrize("name,old,new,nth", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(name, old, new, nth, tmp_path):
    src = SRC.read_text()
    assert src.count(old) > nth, f"mutation site of {name} not found"
    bad = tmp_path / "oracle_mutant.c"
    bad.write_text(_replace_nth(src, old, new, nth))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", str(bad), "-o", str(lib), "-lm"],
                   check=True)
    env = dict(os.environ, MOELORA_ORACLE_LIB=str(lib), OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, f"{name}: pins did not fail (rc {r.returncode})\n{r.stdout[-2000:]}"
