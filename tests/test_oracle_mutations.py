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


# The numpy oracle of the stash, mutated the same way and run against its pins.
STASH_SRC = os.path.join(ROOT, "oracle", "stash.py")
STASH_MUTANTS = [
    ("stash_ties_to_higher_id", "order = np.lexsort((np.arange(V), -s64))",
     "order = np.lexsort((-np.arange(V), -s64))"),
    ("stash_rank_strict", "rank = int(np.count_nonzero(s64 >= s64[top]))",
     "rank = int(np.count_nonzero(s64 > s64[top]))"),
    ("stash_valid_not_cut", "n = min(max(int(valid[j]), 0), canvas_len)", "n = max(int(valid[j]), 0)"),
    ("stash_row_from_slot", "row = int(src[j]) * canvas_len + p", "row = int(slots[j]) * canvas_len + p"),
    ("stash_pad_id_one", "out_ids = np.zeros(width, np.int32)", "out_ids = np.ones(width, np.int32)"),
    ("stash_no_temperature", "s = (logits[row].astype(np.float32) / tc).astype(np.float32)",
     "s = logits[row].astype(np.float32)"),
    ("stash_logprob_drops_logS", "return np.float32((s64[c] - m) - logS)", "return np.float32(s64[c] - m)"),
    ("stash_ids_not_cut_at_width", "cnt = min(int(num_token_ids[j]), width - 1, token_ids.shape[1])",
     "cnt = min(int(num_token_ids[j]), token_ids.shape[1])"),
    ("stash_zero_ids_means_ids", "if token_ids is not None and int(num_token_ids[j]) > 0:",
     "if token_ids is not None and int(num_token_ids[j]) >= 0:"),
    ("stash_keep_ignored", "        if not keep[j]:\n            continue", "        if False:\n            continue"),
    ("stash_clamp_constant", "T_MIN = np.float32(1e-10)", "T_MIN = np.float32(1e-9)"),
    ("stash_logits_mode_logprob", "        if logits_mode:\n            return np.float32(s[c])",
     "        if logits_mode:\n            return np.float32((s64[c] - m) - logS)"),
]


def _run_stash_mutant(name, old, new, workdir):
    src = open(STASH_SRC).read()
    assert src.count(old) == 1, f"mutation {name} does not match exactly once"
    path = os.path.join(workdir, f"{name}.py")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    env = dict(os.environ, ROWSTATS_STASH_ORACLE=path)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_stash.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode


def test_stash_pins_reject_every_mutant():
    with tempfile.TemporaryDirectory() as d:
        # control: an unchanged copy loaded the same way passes the pins
        assert _run_stash_mutant("control", "T_MIN = np.float32(1e-10)", "T_MIN = np.float32(1e-10)", d)[1] == 0
        with ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda m: _run_stash_mutant(*m, d), STASH_MUTANTS))
    survivors = [name for name, rc in results if rc == 0]
    assert not survivors, f"stash mutants not caught by any pin: {survivors}"
