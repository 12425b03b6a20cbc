"""Parity of the HIP path (called through the C ABI) with the CPU oracle.

Small cases compare every row element by element; the full-size workloads
compare seeded samples of rows (always including the rows with planted
structure) and check properties that hold on every row. Bars: argmax and
top-K indices bit-exact; sample exact outside the 1e-6 near-tie band;
entropy within 1e-4; probs within 1 ulp; logprobs within 1e-5 relative.
"""
import numpy as np
import pytest
import torch

import synthetic as syn
import row_softmax_statistics_amd as rs
from parity import (check_properties, compare_rowstats, compare_topk, gpu_rowstats,
                    probs_bits)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def sample_rows(rows, n, seed, extra=()):
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(rows, size=min(n, rows), replace=False).tolist())
    pick |= {int(r) for r in extra}
    return sorted(pick)


def done():
    rs.check_device()
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------
# row statistics
# --------------------------------------------------------------------------
def test_c1_all_rows():
    w = syn.c1(DEV)
    out = gpu_rowstats(w)
    print("C1 near-tie rows:", compare_rowstats(w, out, range(w.rows), "C1"))
    check_properties(w, out)
    done()


SMALL_V = [1, 2, 3, 4, 5, 63, 64, 65, 255, 4095, 4096, 4097, 16383, 16384, 16385, 32769, 65537]


@pytest.mark.parametrize("probs_dtype", [None, torch.bfloat16, torch.float16],
                         ids=["none", "bf16", "fp16"])
@pytest.mark.parametrize("pad", [0, 3, 8], ids=["contig", "pad3", "pad8"])
@pytest.mark.parametrize("vocab", SMALL_V)
def test_small_shapes(vocab, pad, probs_dtype):
    w = syn.random_case(DEV, rows=5, vocab=vocab, canvas_len=2, seed=vocab + pad,
                        ld=vocab + pad, probs_dtype=probs_dtype)
    out = gpu_rowstats(w)
    compare_rowstats(w, out, range(w.rows), f"V={vocab} pad={pad}")
    done()


@pytest.mark.parametrize("canvas", [1, 7, 13, 39, 40, 41, 1000003, 2**31 + 5])
def test_temperature_slots(canvas):
    # row r takes temps[r // canvas]; the kernel divides by a multiplier
    w = syn.random_case(DEV, rows=40, vocab=300, canvas_len=canvas, seed=canvas % 997,
                        t_choices=(0.0, 0.3, 0.7, 1.0, 1.9))
    out = gpu_rowstats(w)
    compare_rowstats(w, out, range(w.rows), f"canvas={canvas}")
    done()


@pytest.mark.parametrize("probs_dtype", [None, torch.bfloat16], ids=["none", "bf16"])
def test_many_rows_per_group(probs_dtype):
    # more rows than the statically assigned first rows of every group, so
    # most rows are handed out through the groups' rings
    w = syn.random_case(DEV, rows=333, vocab=200003, canvas_len=10, seed=17,
                        t_choices=(0.0, 0.6, 1.0), probs_dtype=probs_dtype)
    out = gpu_rowstats(w)
    compare_rowstats(w, out, range(w.rows), "rows=333")
    done()


@pytest.mark.parametrize("probs_dtype", [None, torch.float16], ids=["none", "fp16"])
def test_one_wave_groups(probs_dtype):
    # vocab <= 2048: a group is one wave, which claims, posts and reads its
    # own rows; many more rows than groups
    w = syn.random_case(DEV, rows=20000, vocab=37, canvas_len=7, seed=29,
                        t_choices=(0.0, 0.6, 1.0, 1.4), probs_dtype=probs_dtype)
    out = gpu_rowstats(w)
    rows = sample_rows(w.rows, 3000, 6, extra=[0, 1, w.rows - 2, w.rows - 1])
    compare_rowstats(w, out, rows, "one-wave groups")
    check_properties(w, out)
    done()


def test_alternating_entry_points():
    # row-stats and top-K calls share the row-claim counters; each call must
    # find its counter at zero whatever the previous call was
    w = syn.random_case(DEV, rows=600, vocab=200003, canvas_len=6, seed=31,
                        t_choices=(0.0, 0.5, 1.0), probs_dtype=torch.bfloat16)
    w.keep_mask = (torch.arange(w.temps.numel(), device=DEV) % 4 != 2).to(torch.uint8)
    w.K = 11
    for it in range(3):
        out = gpu_rowstats(w)
        compare_rowstats(w, out, sample_rows(w.rows, 60, it), f"alternating rowstats {it}")
        vals, idx = _run_topk(w)
        _check_untouched(w, vals, idx)
        compare_topk(w, vals, idx, sample_rows(w.rows, 60, 10 + it), f"alternating topk {it}")
    done()


@pytest.mark.parametrize("vocab", [37, 20000, 49153])
def test_quantised_ties(vocab):
    # logits on a 0.5 grid: exact duplicates everywhere, including the max
    w = syn.random_case(DEV, rows=40, vocab=vocab, canvas_len=3, seed=7, ties=True,
                        t_choices=(0.0, 0.5, 1.0, 0.7))
    out = gpu_rowstats(w)
    compare_rowstats(w, out, range(w.rows), f"ties V={vocab}")
    done()


def test_duplicate_max_across_slices():
    vocab = 3 * 16384 + 5
    w = syn.random_case(DEV, rows=6, vocab=vocab, canvas_len=1, seed=11,
                        t_choices=(1.0,), probs_dtype=torch.bfloat16)
    cols = [[16383, 16384], [16384, 32768], [5, 49152 + 4], [32767, 0], [49155, 49156], [1, 2]]
    for r, cs in enumerate(cols):
        w.logits[r, cs] = 30.0
    w.temps.fill_(0.0)
    out = gpu_rowstats(w)
    compare_rowstats(w, out, range(w.rows), "dup max")
    assert out[0].tolist() == [16383, 16384, 5, 0, 49155, 1]
    done()


def test_zero_rows():
    x = torch.empty(0, 100, device=DEV)
    a, s, e, p = rs.sample_row_stats(x, torch.ones(1, device=DEV), 4, 1, torch.bfloat16)
    assert a.numel() == 0 and p.shape == (0, 100)


def test_repeat_runs_are_bit_identical():
    w = syn.random_case(DEV, rows=64, vocab=100000, canvas_len=8, seed=5,
                        t_choices=(0.0, 0.8, 1.2))
    a = gpu_rowstats(w)
    b = gpu_rowstats(w)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y)
    done()


def test_sample_frequencies_follow_softmax():
    import scipy.special
    import scipy.stats
    vocab, rows = 6, 200000
    logits = torch.tensor([1.0, 0.0, -1.0, 2.0, 0.5, 2.0], device=DEV)
    x = logits.repeat(rows, 1)
    _, smp, _, _ = rs.sample_row_stats(x, torch.tensor([1.0], device=DEV), rows, 31337)
    counts = np.bincount(smp.cpu().numpy(), minlength=vocab)
    p = scipy.special.softmax(logits.cpu().double().numpy())
    _, pval = scipy.stats.chisquare(counts, p * rows)
    assert pval > 1e-4, (counts, p * rows)
    done()


def test_c2_full_size():
    w = syn.c2(DEV)
    out = gpu_rowstats(w)
    check_properties(w, out)
    rows = sample_rows(w.rows, 40, 2, extra=w.special_rows["peaked"][:8].tolist())
    print("C2 near-tie rows:", compare_rowstats(w, out, rows, "C2"))
    del out, w
    done()


def test_c3_full_size_with_adversarial_rows():
    w = syn.c3(DEV)
    out = gpu_rowstats(w)
    check_properties(w, out)
    adv = torch.cat(list(w.special_rows.values())).tolist()
    rows = sample_rows(w.rows, 40, 3, extra=adv)
    print("C3 near-tie rows:", compare_rowstats(w, out, rows, "C3"))
    del out, w
    done()


def test_c5_full_size_padded_stride():
    w = syn.c5(DEV)
    assert w.logits.stride(0) == w.vocab + 128
    out = gpu_rowstats(w)
    check_properties(w, out)
    rows = sample_rows(w.rows, 40, 5, extra=w.special_rows["zipf"][:8].tolist())
    print("C5 near-tie rows:", compare_rowstats(w, out, rows, "C5"))
    del out, w
    done()


# --------------------------------------------------------------------------
# top-K logprobs
# --------------------------------------------------------------------------
def _topk_case(rows, vocab, canvas, K, seed, ties=False, ld=None):
    w = syn.random_case(DEV, rows=rows, vocab=vocab, canvas_len=canvas, seed=seed, ties=ties,
                        ld=ld, t_choices=(0.0, 1.0, 0.5), probs_dtype=None)
    slots = w.temps.numel()
    w.keep_mask = (torch.arange(slots, device=DEV) % 3 != 1).to(torch.uint8)
    w.K = K
    return w


def _run_topk(w):
    vals = torch.full((w.rows, w.K), 7.0, device=DEV)
    idx = torch.full((w.rows, w.K), -7, dtype=torch.int64, device=DEV)
    rs.topk_logprobs(w.logits, w.temps, w.canvas_len, w.keep_mask, w.K, vals, idx)
    return vals, idx


def _check_untouched(w, vals, idx):
    slot = torch.arange(w.rows, device=DEV) // w.canvas_len
    dropped = w.keep_mask[slot] == 0
    assert torch.all(vals[dropped] == 7.0) and torch.all(idx[dropped] == -7)


@pytest.mark.parametrize("vocab,K", [(1, 1), (2, 2), (5, 3), (20, 20), (64, 20), (100, 64),
                                     (4097, 20), (16385, 5), (40000, 20), (40000, 64),
                                     (70001, 1)])
@pytest.mark.parametrize("ties", [False, True], ids=["plain", "ties"])
def test_topk_small(vocab, K, ties):
    w = _topk_case(rows=9, vocab=vocab, canvas=3, K=K, seed=vocab + K, ties=ties,
                   ld=vocab + (3 if vocab % 2 else 0))
    vals, idx = _run_topk(w)
    _check_untouched(w, vals, idx)
    compare_topk(w, vals, idx, range(w.rows), f"topk V={vocab} K={K}")
    done()


def test_topk_adversarial_rows():
    vocab, K = 40000, 20
    w = _topk_case(rows=6, vocab=vocab, canvas=1, K=K, seed=3)
    w.keep_mask = torch.ones(6, dtype=torch.uint8, device=DEV)
    w.logits[0] = 1.5                       # every lane max ties: overflow path
    w.logits[1, 100:39000] = float("-inf")   # -inf spans
    w.logits[2] = -0.0
    w.logits[2, ::3] = 0.0                   # signed zeros tie
    w.logits[3, 5000:5300] = 9.0             # 300 duplicates of the max
    w.logits[4] = torch.linspace(-1, 1, vocab, device=DEV)
    vals, idx = _run_topk(w)
    compare_topk(w, vals, idx, range(w.rows), "topk adversarial")
    done()


def _magnitude_rows(rows, vocab, seed):
    """Rows whose values span the fp32 range: ordinary, tiny (below 2^-100),
    subnormal, zero, huge and -inf, so that chunks fall on both sides of the
    fp32 scaling's range check."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn(rows, vocab, generator=g) * 2.0
    kinds = torch.arange(rows) % 6
    x[kinds == 1] *= 1e-32                           # tiny
    x[kinds == 2] *= 1e-39                           # subnormal
    x[kinds == 3, ::7] = 0.0                         # zeros
    x[kinds == 4] *= 1e22                            # huge (x / T stays finite)
    x[kinds == 5, 100:2000] = float("-inf")          # a -inf span
    return x


@pytest.mark.parametrize("temp", [0.0, 1e-3, 0.37, 1.0, 3.7, 1000.0])
def test_scaling_ranges(temp):
    # s = fl32(x / max(T, 1e-10)) must be the IEEE quotient on every path
    rows, vocab = 12, 6000
    x = _magnitude_rows(rows, vocab, seed=int(temp * 1000) % 9973)
    w = syn.Workload(f"mag{temp}", x.to(DEV), torch.full((rows,), temp, device=DEV), 1, 4242,
                     torch.bfloat16)
    out = gpu_rowstats(w)
    compare_rowstats(w, out, range(rows), f"magnitudes T={temp}")
    w.keep_mask = torch.ones(rows, dtype=torch.uint8, device=DEV)
    w.K = 9
    vals, idx = _run_topk(w)
    compare_topk(w, vals, idx, range(rows), f"topk magnitudes T={temp}")
    done()


def test_topk_many_rows_per_group():
    # kept rows handed out through the groups' rings (see test_many_rows_per_group)
    w = _topk_case(rows=500, vocab=200003, canvas=5, K=17, seed=23)
    vals, idx = _run_topk(w)
    _check_untouched(w, vals, idx)
    compare_topk(w, vals, idx, range(w.rows), "topk rows=500")
    done()


def test_topk_one_wave_groups():
    w = _topk_case(rows=20000, vocab=300, canvas=5, K=5, seed=37)
    vals, idx = _run_topk(w)
    _check_untouched(w, vals, idx)
    compare_topk(w, vals, idx, sample_rows(w.rows, 3000, 7, extra=[w.rows - 1]), "topk one-wave")
    done()


def test_c4_topk_full_size():
    w = syn.c4(DEV)
    vals, idx = _run_topk(w)
    _check_untouched(w, vals, idx)
    kept_rows = [r for r in range(w.rows) if int(w.keep_mask[r // w.canvas_len])]
    rows = sample_rows(w.rows, 24, 4, extra=w.special_rows["kth_tie"][:8].tolist()
                       + kept_rows[:2] + kept_rows[-2:])
    compare_topk(w, vals, idx, rows, "C4")
    del vals, idx, w
    done()
