"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of the oracle's C source -- a dropped
term, a wrong sign, a wrong or transposed operand, a wrong index, a wrong
constant -- builds it in a temporary directory and runs the pin suite against
that build in a child process.  The pin suite must fail for every one.  The
mistakes live only in the temporary copies.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "vjsd_oracle.c")

# (name, text in the oracle source, planted replacement, occurrence to replace)
MUTANTS = [
    ("logprob_sign", "return (v - m) - lnZ;", "return (v - m) + lnZ;", 0),
    ("merge_no_rescale", "Z += Zk[k] * exp(mk[k] - m);", "Z += Zk[k];", 0),
    ("merge_wrong_max", "if (mk[k] > m)\n            m = mk[k];", "if (mk[k] < m)\n            m = mk[k];", 0),
    ("jsd_dropped_term", "*loss = beta * KT + (1.0 - beta) * KS;", "*loss = beta * KT;", 0),
    ("jsd_weights_swapped", "*loss = beta * KT + (1.0 - beta) * KS;",
     "*loss = (1.0 - beta) * KT + beta * KS;", 0),
    ("mixture_transposed", "logaddexp(lnb + lpt, ln1mb + lps)", "logaddexp(lnb + lps, ln1mb + lpt)", 0),
    ("mixture_transposed_bwd", "logaddexp(lnb + lpt, ln1mb + lps)",
     "logaddexp(lnb + lps, ln1mb + lpt)", 1),
    ("grad_s_wrong_K", "(lps - lM - KS)", "(lps - lM - KT)", 0),
    ("grad_t_wrong_weight", "g * beta * pt * (lpt - lM - KT)", "g * (1.0 - beta) * pt * (lpt - lM - KT)", 0),
    ("fwdkl_grad_sign", "dsj = g * (ps - pt);", "dsj = g * (pt - ps);", 0),
    ("fwdkl_grad_dropped_K", "g * pt * (lpt - lps - KT)", "g * pt * (lpt - lps)", 0),
    ("revkl_swapped", "pKS += exp(lps) * (lps - lpt);", "pKS += exp(lpt) * (lpt - lps);", 0),
    ("inf_flag_lost", "infinite = 1;", "infinite = 0;", 0),
    ("undefined_row_grad", "if (gs) gs[j] = 0.0;", "if (gs) gs[j] = 1.0;", 0),
    ("entropy_grad_sign", "gx[j] = -g * exp(lp) * (lp + H);", "gx[j] = -g * exp(lp) * (lp - H);", 0),
    ("entropy_value_sign", "part -= exp(lp) * lp;", "part += exp(lp) * lp;", 0),
    ("logprobs_wrong_index", "gx[id] += g[k];", "gx[id] += g[0];", 0),
    ("logprobs_ignore_value", "out[k] = 0.0;\n            continue;", "out[k] = -1.0;\n            continue;", 0),
    ("half_exponent_bias", "v = ldexp((double)(f | 0x400), e - 25);", "v = ldexp((double)(f | 0x400), e - 24);", 0),
    ("bf16_shift", "uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;", 0),
]


def _plant(text, old, new, occ):
    start = -1
    for _ in range(occ + 1):
        start = text.find(old, start + 1)
        if start < 0:
            raise AssertionError(f"mutation anchor not found: {old!r}")
    return text[:start] + new + text[start + len(old):]


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new, occ):
    src = open(SRC).read()
    mutated = _plant(src, old, new, occ)
    assert mutated != src
    csrc = tmp_path / "mutant.c"
    csrc.write_text(mutated)
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-std=gnu11", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(lib),
                    str(csrc), "-lm"], check=True)
    env = dict(os.environ, VJSD_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"planted mistake {name} passed every pin:\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout or "error" in r.stdout.lower()
