"""Plant plausible mistakes in copies of the C oracle and check the pins catch each.

Every mutant is the oracle source with one edit (a wrong constant, sign,
index, comparison or dropped term), compiled on the CPU into a temporary
library; the oracle pin tests and worked examples are then run against it in
a subprocess and must fail. The real oracle is never modified.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "rowstats_oracle.c")
sys.path.insert(0, ROOT)
from oracle.build import CFLAGS  # noqa: E402

MUTANTS = [
    ("philox_multiplier", "0xD2511F53u;", "0xD2511F57u;"),
    ("philox_key_bump_first_round", "if (round > 0) {", "if (round >= 0) {"),
    ("philox_hi_lo_swapped", "uint32_t n1 = (uint32_t)p1;", "uint32_t n1 = (uint32_t)(p1 >> 32);"),
    ("counter_uses_column", "uint64_t q = (uint64_t)col >> 2;", "uint64_t q = (uint64_t)col;"),
    ("uniform_without_half", "((double)w + 0.5)", "((double)w + 0.0)"),
    ("gumbel_sign", "*g_out = -log(-log(u));", "*g_out = log(-log(u));"),
    ("clamp_constant", "const float lo = 1e-10f;", "const float lo = 1e-9f;"),
    ("greedy_rule", "return !(t > 0.0f);", "return !(t >= 0.0f);"),
    ("argmax_last_index", "    if (s[c] > m) {\n      m = s[c];\n      am = c;",
     "    if (s[c] >= m) {\n      m = s[c];\n      am = c;"),
    ("entropy_sign", "res->entropy = logS - sum_pd;", "res->entropy = logS + sum_pd;"),
    ("entropy_mask_dropped", "    if (p > 0.0) {\n      sum_pd", "    if (1) {\n      sum_pd"),
    ("bf16_truncates", "double r = nearbyint(v / quantum);", "double r = floor(v / quantum);"),
    ("fp16_min_exponent", "round_to_format(p, 10, -14);", "round_to_format(p, 10, -15);"),
    ("topk_tie_order", "return (x->c < y->c) ? -1 : (x->c > y->c);", "return (x->c > y->c) ? -1 : (x->c < y->c);"),
    ("topk_logprob_drops_logS", "out_vals[i * K + k] = (float)(((double)e[k].s - (double)m) - logS);",
     "out_vals[i * K + k] = (float)(((double)e[k].s - (double)m));"),
    ("temperature_slot", "float t = temps[row / canvas_len];", "float t = temps[row % canvas_len];"),
    ("probs_unnormalised", "double p = exp(d) / S;", "double p = exp(d);"),
    ("sample_without_noise", "double z = (double)s[c] + g;", "double z = (double)s[c] + 0.0 * g;"),
    ("noise_row_word_swap", "(uint32_t)(uint64_t)row,\n", "(uint32_t)((uint64_t)row >> 32),\n"),
]


def _run_mutant(name, old, new, workdir):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation {name} does not match exactly once"
    msrc = os.path.join(workdir, f"{name}.c")
    lib = os.path.join(workdir, f"{name}.so")
    with open(msrc, "w") as f:
        f.write(src.replace(old, new))
    subprocess.run(["gcc", *CFLAGS, "-w", "-o", lib, msrc, "-lm"], check=True)
    env = dict(os.environ, ROWSTATS_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_golden.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode


def test_every_planted_mistake_is_caught():
    workdir = tempfile.mkdtemp(prefix="oracle_mutants")
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(lambda m: _run_mutant(*m, workdir), MUTANTS))
    survivors = [name for name, rc in results if rc == 0]
    assert not survivors, f"mutants not caught by the pins: {survivors}"
