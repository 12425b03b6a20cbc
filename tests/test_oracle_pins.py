"""Pins of the CPU oracle against sources other than itself.

Each test ties one part of the oracle to something fixed outside its code:
an independent Philox implementation (PyTorch's header-only engine), numpy's
IEEE fp32 division and argmax, closed-form entropies and probabilities,
scipy's softmax/entropy, PyTorch's and numpy's float rounding, a brute-force
sort, the Gumbel distribution function and sample frequencies.

Semantics: the vLLM API page "diffusion_gemma_sampler" (sample_row_stats and
its docstring, sample_row_stats_reference, the _lp_topk_kernel docstring and
the stash_converged_logprobs docstring).
"""
import math
import os
import subprocess
import tempfile

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

import oracle

RNG = np.random.default_rng(12345)


# --------------------------------------------------------------------------
# Philox4x32-10: bit-exact against PyTorch's at::philox_engine
# --------------------------------------------------------------------------
@pytest.fixture(scope="module")
def torch_philox():
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    src = os.path.join(os.path.dirname(__file__), "torch_philox_kat.cpp")
    d = tempfile.mkdtemp(prefix="kat")
    exe = os.path.join(d, "kat")
    subprocess.run(["g++", "-O1", "-std=c++17", f"-I{inc}", "-o", exe, src], check=True)

    def run(triples):
        txt = "\n".join(f"{s} {r} {o}" for s, r, o in triples) + "\n"
        out = subprocess.run([exe], input=txt, capture_output=True, text=True, check=True).stdout
        return [tuple(int(v) for v in line.split()) for line in out.strip().splitlines()]
    return run


def test_philox_block_matches_torch_engine(torch_philox):
    triples = [(0, 0, 0), (1234, 0, 0), (1234, 5, 7), (2**64 - 1, 2**64 - 1, 2**64 - 1),
               (2**32, 2**32 + 3, 2**32 + 9), (0xDEADBEEFCAFEBABE, 77, 65535)]
    for _ in range(300):
        triples.append((int(RNG.integers(0, 2**63)) * 2 + int(RNG.integers(0, 2)),
                        int(RNG.integers(0, 2**40)), int(RNG.integers(0, 2**36))))
    ref = torch_philox(triples)
    for (seed, sub, off), words in zip(triples, ref):
        ctr = [off & 0xFFFFFFFF, off >> 32, sub & 0xFFFFFFFF, sub >> 32]
        key = [seed & 0xFFFFFFFF, seed >> 32]
        got = oracle.philox4x32_10(ctr, key)
        assert tuple(int(v) for v in got) == words, (seed, sub, off)


def test_noise_word_layout_matches_engine(torch_philox):
    # column c of row r draws word c & 3 of the block at offset c >> 2 of
    # subsequence r: the engine's four successive outputs of that block
    seed = 1234
    cases = [(r, c) for r in (0, 1, 63, 4095, 2**33 + 5) for c in (0, 1, 2, 3, 4, 5, 262143, 131077)]
    ref = torch_philox([(seed, r, c >> 2) for r, c in cases])
    for (r, c), words in zip(cases, ref):
        assert oracle.noise_word(seed, r, c) == words[c & 3]


# --------------------------------------------------------------------------
# Uniform and Gumbel maps: range ends and the Gumbel distribution function
# --------------------------------------------------------------------------
def test_uniform_range_and_gumbel_extremes():
    u0, g0 = oracle.uniform_gumbel(0)
    u1, g1 = oracle.uniform_gumbel(2**32 - 1)
    assert u0 == 2.0 ** -33
    assert u1 == 1.0 - 2.0 ** -33
    # the extremes of a standard Gumbel quantile at these u
    assert g0 == pytest.approx(-math.log(33 * math.log(2.0)), rel=1e-12)
    assert 22.87 < g1 < 22.88
    assert -3.131 < g0 < -3.129


def test_gumbel_is_the_quantile_of_the_gumbel_cdf():
    # F(g) = exp(-exp(-g)) is the standard Gumbel CDF; g(w) must be its
    # quantile at u(w) for every word
    for w in list(range(0, 2**32, 2**26)) + [1, 2**31, 2**32 - 2]:
        u, g = oracle.uniform_gumbel(w)
        assert math.exp(-math.exp(-g)) == pytest.approx(u, rel=1e-12, abs=1e-300)
    gs = [oracle.uniform_gumbel(w)[1] for w in range(0, 2**32, 2**20)]
    assert all(a < b for a, b in zip(gs, gs[1:]))  # strictly increasing


# --------------------------------------------------------------------------
# Temperature scaling: bit-exact IEEE fp32 division (numpy) with the clamp
# --------------------------------------------------------------------------
def _special_values(n):
    x = RNG.standard_normal(n).astype(np.float32) * 5
    x[:16] = np.array([0.0, -0.0, np.inf * -1, 1e-45, -1e-45, 1.17549435e-38, 3e38, -3e38,
                       1.0, -1.0, 2.0 ** -130, 7.0, 1e-40, 0.1, 16777217.0, 5e-39],
                      dtype=np.float32)
    sub = (RNG.integers(1, 2**23, size=n // 4) * 2.0 ** -149).astype(np.float32)
    x[16:16 + sub.size] = sub
    return x


@pytest.mark.parametrize("t", [0.0, -1.0, 1e-10, 1e-11, 0.1, 0.7, 1.0, 1.3, 1.5, 0.33333334])
def test_scale_is_ieee_fp32_division(t):
    x = _special_values(4096)
    tc = np.float32(max(np.float32(t), np.float32(1e-10)))
    with np.errstate(all="ignore"):
        ref = x / tc
    got = oracle.scale_row(x, t)
    assert np.array_equal(got.view(np.uint32), ref.astype(np.float32).view(np.uint32))


def test_scale_random_temperatures():
    x = _special_values(2048)
    for t in RNG.uniform(0.05, 1.6, size=40).astype(np.float32):
        with np.errstate(all="ignore"):
            ref = x / t
        assert np.array_equal(oracle.scale_row(x, float(t)).view(np.uint32), ref.view(np.uint32))


# --------------------------------------------------------------------------
# argmax / ties / +-0: numpy's first-maximum argmax on the scaled row
# --------------------------------------------------------------------------
def test_argmax_lowest_index_and_signed_zero():
    rows, vocab = 400, 37
    x = RNG.integers(-3, 3, size=(rows, vocab)).astype(np.float32)
    x[0] = 0.0
    x[0, ::2] = -0.0           # all +-0: the first column wins
    x[1] = -np.inf
    x[1, 5] = 0.0
    x[1, 9] = -0.0             # max +-0 at 5 and 9: 5 wins
    temps = np.array([1.0, 0.7, 0.0], np.float32)
    canvas = 1
    rid = np.arange(rows)
    tv = np.resize(temps, rows).astype(np.float32)
    out = oracle.rowstats(x, rid, tv, canvas, seed=9)
    for i in range(rows):
        s = oracle.scale_row(x[i], tv[i])
        assert out["argmax"][i] == int(np.argmax(s)), i
    assert out["argmax"][0] == 0 and out["argmax"][1] == 5


# --------------------------------------------------------------------------
# Entropy and probs: closed forms
# --------------------------------------------------------------------------
@pytest.mark.parametrize("vocab", [1, 2, 3, 64, 1000, 32768])
def test_uniform_row(vocab):
    x = np.full((1, vocab), 1.25, np.float32)
    out = oracle.rowstats(x, [0], [1.0], 1, seed=1, probs_dtype=oracle.PROBS_BF16)
    assert out["entropy"][0] == pytest.approx(math.log(vocab), abs=1e-12)
    assert out["argmax"][0] == 0
    ref = torch.tensor([1.0 / vocab], dtype=torch.float32).to(torch.bfloat16).view(torch.int16)
    assert int(out["probs"][0, 0]) == int(ref.item()) & 0xFFFF
    assert np.all(out["probs"][0] == out["probs"][0, 0])


@pytest.mark.parametrize("vocab,k,a,b,t", [(10, 3, 2.0, -1.0, 1.0), (1000, 1, 4.0, 0.0, 0.5),
                                           (4096, 17, -3.0, -3.5, 1.0), (5, 4, 1.0, 0.0, 2.0)])
def test_two_level_row_closed_form(vocab, k, a, b, t):
    # k columns at a and vocab-k at b: p_a = e^(a/t) / (k e^(a/t) + (V-k) e^(b/t))
    x = np.full((1, vocab), b, np.float32)
    pos = RNG.choice(vocab, size=k, replace=False)
    x[0, pos] = a
    out = oracle.rowstats(x, [0], [t], 1, seed=3, probs_dtype=oracle.PROBS_FP16)
    sa, sb = a / t, b / t
    zmax = max(sa, sb)
    za, zb = math.exp(sa - zmax), math.exp(sb - zmax)
    Z = k * za + (vocab - k) * zb
    pa, pb = za / Z, zb / Z
    H = -(k * pa * math.log(pa) + ((vocab - k) * pb * math.log(pb) if vocab > k else 0.0))
    assert out["entropy"][0] == pytest.approx(H, rel=1e-12, abs=1e-14)
    assert out["entropy_plogp"][0] == pytest.approx(H, rel=1e-12, abs=1e-14)
    ha = np.float16(pa).view(np.uint16)
    assert int(out["probs"][0, pos[0]]) == int(ha)
    assert out["argmax"][0] == (min(pos) if a > b else min(set(range(vocab)) - set(pos.tolist())))


def test_dominant_token_entropy_zero():
    vocab = 4096
    x = np.zeros((1, vocab), np.float32)
    x[0, 1234] = 200.0
    out = oracle.rowstats(x, [0], [1.0], 1, seed=5, probs_dtype=oracle.PROBS_BF16)
    assert out["entropy"][0] < 1e-70
    assert out["argmax"][0] == 1234 and out["sample"][0] == 1234
    assert out["probs"][0, 1234] == 0x3F80  # bf16 1.0
    assert np.count_nonzero(out["probs"][0]) == 1


def test_greedy_rows():
    # T = 0 (and negative T): sample == argmax, entropy is log(#ties of max)
    rows, vocab = 60, 50
    x = RNG.integers(-4, 4, size=(rows, vocab)).astype(np.float32)
    temps = np.array([0.0, -2.0, 0.0], np.float32)
    out = oracle.rowstats(x, np.arange(rows), temps, 20, seed=11, probs_dtype=oracle.PROBS_BF16)
    for i in range(rows):
        assert out["sample"][i] == out["argmax"][i]
        nt = int(np.sum(x[i] == x[i].max()))
        assert out["entropy"][i] == pytest.approx(math.log(nt), abs=1e-12)
        assert np.isinf(out["gap"][i])
        # one-hot (or 1/k over k tied maxima) in bf16
        ref = torch.tensor([1.0 / nt], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).item() & 0xFFFF
        assert set(out["probs"][i][x[i] == x[i].max()].tolist()) == {ref}
        assert np.all(out["probs"][i][x[i] != x[i].max()] == 0)


def test_neg_inf_columns_drop_out():
    vocab = 300
    base = RNG.standard_normal(vocab).astype(np.float32)
    keep = RNG.random(vocab) < 0.6
    x = base.copy()
    x[~keep] = -np.inf
    a = oracle.rowstats(x[None], [0], [0.8], 1, seed=2, probs_dtype=oracle.PROBS_BF16)
    b = oracle.rowstats(np.ascontiguousarray(base[keep][None]), [0], [0.8], 1, seed=2,
                        probs_dtype=oracle.PROBS_BF16)
    assert a["entropy"][0] == pytest.approx(b["entropy"][0], rel=1e-13)
    assert np.all(a["probs"][0][~keep] == 0)
    assert np.array_equal(a["probs"][0][keep], b["probs"][0])
    assert np.isfinite(a["entropy"][0])


def test_entropy_matches_scipy_and_both_forms():
    rows, vocab = 50, 3000
    x = (RNG.standard_normal((rows, vocab)) * 2.5).astype(np.float32)
    temps = RNG.uniform(0.1, 1.5, size=rows).astype(np.float32)
    out = oracle.rowstats(x, np.arange(rows), temps, 1, seed=4)
    for i in range(rows):
        s = oracle.scale_row(x[i], temps[i]).astype(np.float64)
        p = scipy.special.softmax(s)
        h = scipy.stats.entropy(p)
        assert out["entropy"][i] == pytest.approx(h, abs=1e-10)
        assert out["entropy_plogp"][i] == pytest.approx(out["entropy"][i], abs=1e-12)


def test_probs_are_rounded_softmax():
    rows, vocab = 8, 5000
    x = (RNG.standard_normal((rows, vocab)) * 3).astype(np.float32)
    temps = np.full(rows, 0.9, np.float32)
    out_b = oracle.rowstats(x, np.arange(rows), temps, 1, seed=4, probs_dtype=oracle.PROBS_BF16)
    out_h = oracle.rowstats(x, np.arange(rows), temps, 1, seed=4, probs_dtype=oracle.PROBS_FP16)
    for i in range(rows):
        s = oracle.scale_row(x[i], temps[i]).astype(np.float64)
        p = scipy.special.softmax(s)
        # fp16: numpy rounds float64 -> float16 directly to nearest-even
        assert np.array_equal(out_h["probs"][i], p.astype(np.float16).view(np.uint16))
        # bf16: decoded values within half a bf16 ulp of the exact probability
        dec = (out_b["probs"][i].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        ulp = np.maximum(np.exp2(np.floor(np.log2(np.maximum(p, 2.0 ** -126))) - 7), 2.0 ** -133)
        assert np.all(np.abs(dec - p) <= ulp / 2 + 1e-300)


def test_bf16_rounding_matches_torch():
    v = np.concatenate([RNG.random(20000).astype(np.float32),
                        (RNG.integers(1, 2**23, 5000) * 2.0 ** -149).astype(np.float32),
                        np.float32(2.0) ** -RNG.integers(1, 140, 2000).astype(np.float32),
                        np.array([1.0, 0.0, 1 + 2**-8, 1 + 3 * 2**-8, 2**-133, 2**-134, 3 * 2**-134],
                                 np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_bits(float(a)) for a in v], np.uint16)
    assert np.array_equal(got, ref)


def test_fp16_rounding_matches_numpy():
    v = np.concatenate([RNG.random(20000), RNG.random(5000) * 2.0 ** -14,
                        RNG.random(2000) * 2.0 ** -24,
                        np.array([1.0, 0.0, 1 + 2**-11, 1 + 2**-11 + 2**-40, 2**-25, 3 * 2**-25,
                                  2**-14 - 2**-26])])
    ref = v.astype(np.float16).view(np.uint16)
    got = np.array([oracle.fp16_bits(float(a)) for a in v], np.uint16)
    assert np.array_equal(got, ref)


# --------------------------------------------------------------------------
# Gumbel-max sample: frequencies follow the softmax (chi-square)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("t", [1.0, 0.5])
def test_sample_frequencies_follow_softmax(t):
    vocab, rows = 6, 120000
    logits = np.array([1.0, 0.0, -1.0, 2.0, 0.5, 2.0], np.float32)
    x = np.tile(logits, (rows, 1))
    out = oracle.rowstats(x, np.arange(rows), np.array([t], np.float32), rows, seed=2024)
    counts = np.bincount(out["sample"], minlength=vocab)
    p = scipy.special.softmax(logits.astype(np.float64) / t)
    chi2, pval = scipy.stats.chisquare(counts, p * rows)
    assert pval > 1e-4, (counts, p * rows, pval)
    # the two equal logits (columns 3 and 5) are sampled equally often
    assert abs(counts[3] - counts[5]) < 5 * math.sqrt(counts[3] + counts[5])


def test_sample_depends_on_seed_and_row_only():
    x = (RNG.standard_normal((64, 257))).astype(np.float32)
    rows = np.arange(64)
    a = oracle.rowstats(x, rows, [1.0], 64, seed=77)
    b = oracle.rowstats(x[[2, 0]].copy(), [2, 0], [1.0], 64, seed=77)
    assert a["sample"][2] == b["sample"][0] and a["sample"][0] == b["sample"][1]
    # another seed is another noise stream: the words differ and, over 64 rows
    # of 257 near-uniform columns, so do some samples
    c = oracle.rowstats(x, rows, [1.0], 64, seed=78)
    assert oracle.noise_word(77, 5, 9) != oracle.noise_word(78, 5, 9)
    assert np.count_nonzero(a["sample"] != c["sample"]) >= 32
    # and another row of the same values draws other noise
    d = oracle.rowstats(np.repeat(x[:1], 64, axis=0), rows, [1.0], 64, seed=77)
    assert len(set(d["sample"].tolist())) >= 16
    assert np.all(a["gap"] >= 0)


def test_sample_is_argmax_of_perturbed_scores():
    # brute force on tiny V: recompute z = s + g from the noise words
    x = (RNG.standard_normal((30, 9)) * 2).astype(np.float32)
    seed = 99
    out = oracle.rowstats(x, np.arange(30), [0.75], 30, seed=seed)
    for r in range(30):
        s = oracle.scale_row(x[r], 0.75).astype(np.float64)
        g = np.array([oracle.uniform_gumbel(oracle.noise_word(seed, r, c))[1] for c in range(9)])
        z = s + g
        assert out["sample"][r] == int(np.argmax(z))
        zs = np.sort(z)
        assert out["gap"][r] == pytest.approx(zs[-1] - zs[-2], abs=1e-15)


# --------------------------------------------------------------------------
# Top-K logprobs: brute-force sort, closed forms, kept/non-kept rows
# --------------------------------------------------------------------------
def test_topk_matches_bruteforce_sort():
    rows, vocab, canvas, K = 24, 40, 4, 7
    x = RNG.integers(-5, 5, size=(rows, vocab)).astype(np.float32)
    x[0] = -0.0
    x[0, 1::3] = 0.0
    temps = np.array([1.0, 0.0, 0.5, 2.0, 1.0, 0.3], np.float32)
    keep = np.array([1, 1, 0, 1, 1, 1], np.uint8)
    vals = np.full((rows, K), 7.0, np.float32)
    idx = np.full((rows, K), -7, np.int64)
    oracle.topk_logprobs(x, np.arange(rows), temps, canvas, keep, K, vals, idx)
    for r in range(rows):
        slot = r // canvas
        if not keep[slot]:
            assert np.all(vals[r] == 7.0) and np.all(idx[r] == -7)
            continue
        s = oracle.scale_row(x[r], temps[slot])
        order = np.lexsort((np.arange(vocab), -s.astype(np.float64)))
        assert np.array_equal(idx[r], order[:K]), r
        # reference in the row-centred frame: (s - m) - logsumexp(s - m)
        sd = s.astype(np.float64) - float(s.max())
        ref = (sd[order[:K]] - scipy.special.logsumexp(sd)).astype(np.float32)
        assert np.allclose(vals[r], ref, rtol=1e-6, atol=1e-6)
        if temps[slot] <= 0:
            # greedy rows: the tied maxima share the mass exactly, -log(#ties)
            nt = int(np.sum(s == s.max()))
            assert vals[r][0] == np.float32(-math.log(nt))


def test_topk_full_row_logprobs_normalise():
    vocab = 50
    x = (RNG.standard_normal((3, vocab)) * 3).astype(np.float32)
    vals, idx = oracle.topk_logprobs(x, [0, 1, 2], [1.3], 3, [1], vocab)
    for r in range(3):
        assert sorted(idx[r].tolist()) == list(range(vocab))
        assert np.exp(vals[r].astype(np.float64)).sum() == pytest.approx(1.0, abs=1e-5)
        assert np.all(np.diff(vals[r]) <= 0)


def test_topk_two_level_closed_form():
    vocab, k = 100, 3
    x = np.zeros((1, vocab), np.float32)
    x[0, [70, 5, 33]] = 2.0
    vals, idx = oracle.topk_logprobs(x, [0], [1.0], 1, [1], 5)
    Z = k * math.exp(2.0) + (vocab - k)
    assert idx[0].tolist() == [5, 33, 70, 0, 1]
    assert vals[0, 0] == pytest.approx(2.0 - math.log(Z), abs=1e-6)
    assert vals[0, 3] == pytest.approx(-math.log(Z), abs=1e-6)


def test_block_max_threshold_lemma():
    # the maxima of K different blocks are K different elements, none below
    # the K-th largest block maximum t, so every top-K element is >= t; checked on data
    # with many duplicates and on every block width
    for trial in range(200):
        vocab = int(RNG.integers(1, 300))
        K = int(RNG.integers(1, vocab + 1))
        width = int(RNG.integers(1, 40))
        x = RNG.integers(-4, 4, size=vocab).astype(np.float32)
        nb = (vocab + width - 1) // width
        bmax = np.array([x[b * width:(b + 1) * width].max() for b in range(nb)])
        order = np.lexsort((np.arange(vocab), -x.astype(np.float64)))
        top = x[order[:K]]
        if K <= nb:
            t = np.sort(bmax)[::-1][K - 1]
            assert np.all(top >= t)
