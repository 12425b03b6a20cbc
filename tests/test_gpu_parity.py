"""Parity of the HIP path (called through the C ABI) with the CPU oracle.

Every case compares every row element by element with the oracle, the
full-size workloads included (in blocks of rows, in the launch
configuration the benchmark times), and checks properties that hold on
every row. Bars: argmax and top-K indices bit-exact; sample exact outside
the 1e-6 near-tie band (inside it, the GPU's column must score within the
band of the best); entropy within 1e-4; probs within 1 ulp; logprobs within
1e-5 relative.
"""
import numpy as np
import pytest
import torch

import synthetic as syn
import row_softmax_statistics_amd as rs
from parity import (check_properties, compare_all_rows, compare_rowstats, compare_topk,
                    gpu_rowstats, probs_bits, record)

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
    compare_all_rows(w, out, "C1")
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
    compare_all_rows(w, out, "one-wave groups", block=5000)
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
        compare_rowstats(w, out, range(w.rows), f"alternating rowstats {it}")
        vals, idx = _run_topk(w)
        _check_untouched(w, vals, idx)
        compare_topk(w, vals, idx, range(w.rows), f"alternating topk {it}")
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


def _same(a, b):
    for x, y in zip(a, b):
        if x is None:
            assert y is None
            continue
        if x.dtype in (torch.bfloat16, torch.float16):
            x, y = x.view(torch.int16), y.view(torch.int16)
        assert torch.equal(x, y)


def test_repeat_runs_are_bit_identical():
    w = syn.random_case(DEV, rows=64, vocab=100000, canvas_len=8, seed=5,
                        t_choices=(0.0, 0.8, 1.2))
    _same(gpu_rowstats(w), gpu_rowstats(w))
    done()


@pytest.mark.parametrize("name", ["C2", "C3"])
def test_full_size_repeat_runs_are_bit_identical(name):
    # at full size every group reduces many rows, most of them dealt out
    # through the rings at run time: the outputs must not depend on which
    # group took which row, nor on the order in which chunks were merged
    w = syn.WORKLOADS[name](DEV)
    a = gpu_rowstats(w)
    b = gpu_rowstats(w)
    _same(a, b)
    del a, b, w
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
    compare_all_rows(w, out, "C2")
    del out, w
    done()


def test_c3_full_size_with_adversarial_rows():
    w = syn.c3(DEV)
    out = gpu_rowstats(w)
    check_properties(w, out)
    compare_all_rows(w, out, "C3")
    del out, w
    done()


def test_c5_full_size_padded_stride():
    w = syn.c5(DEV)
    assert w.logits.stride(0) == w.vocab + 128
    out = gpu_rowstats(w)
    check_properties(w, out)
    compare_all_rows(w, out, "C5")
    del out, w
    done()


@pytest.mark.parametrize("temp", [1.0, 0.5, 0.07])
def test_probs_of_chunks_far_below_the_row_max(temp):
    # each 2048-column chunk sits d below the row maximum; a chunk 65 to 92
    # below still holds nonzero bf16 probabilities (normal down to e^-87.3,
    # subnormal to e^-92), which must survive the scaling from the chunk's
    # own maximum to the row's
    drops = [20, 40, 60, 66, 72, 78, 81, 84, 86, 87.5, 89, 90.5, 92, 95, 100, 130]
    rows, vocab = 6, 2048 * len(drops)
    g = torch.Generator().manual_seed(int(temp * 100))
    x = torch.randn(rows, vocab, generator=g) * (0.4 * temp)
    for c, d in enumerate(drops):
        x[:, 2048 * c:2048 * (c + 1)] -= d * temp
    x[:, 5] = 0.0                                   # the row maximum: S is about 1
    x[1] = x[1].roll(4096, dims=0)
    x[2, ::3] = float("-inf")
    w = syn.Workload(f"far chunks T={temp}", x.to(DEV), torch.full((rows,), temp, device=DEV), 1,
                     99, torch.bfloat16)
    out = gpu_rowstats(w)
    compare_rowstats(w, out, range(rows), f"far chunks T={temp}")
    p = out[3].float()
    assert float(p[0, 2048 * 9:2048 * 10].max()) >= 2.0 ** -126     # 87.5 below: normal
    sub = float(p[0, 2048 * 11:2048 * 12].max())                   # 90.5 below: subnormal
    assert 0.0 < sub < 2.0 ** -126
    done()


def _coop_case(vocab, probs_dtype):
    x = torch.zeros(1, vocab, device=DEV)
    return x, torch.ones(1, device=DEV)


@pytest.mark.parametrize("probs_dtype,vocab", [(torch.bfloat16, 2049 * 2048),
                                               (None, 4097 * 2048)], ids=["bf16", "none"])
def test_vocab_beyond_co_residency_is_rejected(probs_dtype, vocab):
    # a row's chunks must all be resident at once (2048 waves with probs,
    # 4096 without on one MI355X): the planner refuses before any launch
    x, t = _coop_case(vocab, probs_dtype)
    out = (torch.full((1,), -5, dtype=torch.int64, device=DEV),
           torch.full((1,), -5, dtype=torch.int64, device=DEV),
           torch.full((1,), -5.0, device=DEV),
           torch.empty(1, vocab, dtype=probs_dtype, device=DEV) if probs_dtype else None)
    with pytest.raises(rs.RowStatsError) as e:
        rs.sample_row_stats(x, t, 1, 0, probs_dtype, out=out)
    assert e.value.code == -6
    assert int(out[0][0]) == -5 and int(out[1][0]) == -5
    if probs_dtype is None:
        # top-K keeps 4096 chunks resident as well (4 waves per SIMD)
        with pytest.raises(rs.RowStatsError) as e:
            rs.topk_logprobs(x, t, 1, torch.ones(1, dtype=torch.uint8, device=DEV), 3)
        assert e.value.code == -6
    # the largest vocab that fits still runs
    ok = 2048 * (2048 if probs_dtype else 4096)
    w = syn.random_case(DEV, rows=2, vocab=ok, canvas_len=1, seed=8, t_choices=(0.0, 1.0),
                        probs_dtype=probs_dtype)
    compare_rowstats(w, gpu_rowstats(w), range(2), "largest resident vocab")
    done()


def _midpoint_quotients(temp: float, count: int):
    """Logits x whose quotient x / temp is a midpoint of the fp32 subnormal
    grid and whose fl32(x * fl64(1 / temp)) rounds the other way (found by
    brute force over every subnormal x, on the host)."""
    xs = np.arange(1, 1 << 23, dtype=np.uint32).view(np.float32)
    fast = (xs.astype(np.float64) * (1.0 / np.float64(temp))).astype(np.float32)
    ieee = xs / np.float32(temp)
    bad = xs[fast != ieee]
    assert bad.size > 0, temp
    return bad[np.linspace(0, bad.size - 1, count).astype(np.int64)]


@pytest.mark.parametrize("temp", [98.0, 150.0, 364.0, 936.0])
def test_subnormal_midpoint_quotients(temp):
    # x / T lands exactly between two subnormal fp32 values; IEEE division
    # breaks the tie to even. Each row pairs such an x (column 2k) with the
    # x' whose quotient is the even neighbour (column 2k + 1): the two tie
    # only if x / T was rounded to even, which decides the argmax and top-K.
    xs = _midpoint_quotients(temp, 24)
    ieee = xs / np.float32(temp)
    partner = (ieee.astype(np.float64) * temp).astype(np.float32)   # exact: a multiple of T
    assert np.all(partner / np.float32(temp) == ieee)
    rows, vocab = 24, 64
    x = np.full((rows, vocab), -1.0, np.float32)
    for r in range(rows):
        x[r, 2 * (r % 8)] = xs[r]
        x[r, 2 * (r % 8) + 1] = partner[r]
        if r >= 12:   # another midpoint value elsewhere, larger or smaller
            x[r, 40 + r % 7] = xs[(r + 5) % rows]
    w = syn.Workload(f"midpoints T={temp}", torch.from_numpy(x).to(DEV),
                     torch.full((rows,), temp, device=DEV), 1, 77, torch.bfloat16)
    out = gpu_rowstats(w)
    compare_rowstats(w, out, range(rows), f"midpoints T={temp}")
    # in the rows holding only the pair, the two tie at the maximum
    assert out[0].cpu().tolist()[:12] == [2 * (r % 8) for r in range(12)]
    w.keep_mask = torch.ones(rows, dtype=torch.uint8, device=DEV)
    w.K = 3
    vals, idx = _run_topk(w)
    compare_topk(w, vals, idx, range(rows), f"topk midpoints T={temp}")
    # the stash: one request per row; logits mode writes the scaled values
    # themselves, and the rank counts the ties at the maximum
    import test_gpu_stash as ts
    ar = torch.arange(rows, dtype=torch.int32)
    for mode in (False, True):
        sw = syn.StashWorkload(f"midpoint stash T={temp}", w.logits, 1, ar.to(DEV), ar.to(DEV),
                               torch.ones(rows, dtype=torch.uint8, device=DEV),
                               torch.ones(rows, dtype=torch.int32, device=DEV), w.temps, 3,
                               torch.zeros(rows, dtype=torch.int32, device=DEV), None, rows, 1, 4,
                               mode)
        ts.compare(ts.run_gpu(sw), ts.run_oracle(sw), mode, f"stash midpoints T={temp} {mode}")
    done()


def test_calls_on_two_streams_are_ordered():
    # the three entry points share one scratch buffer and its row-claim
    # counters; a call queued on another stream than the previous call waits
    # for it on the device, so interleaved streams give the one-stream results
    w = syn.random_case(DEV, rows=300, vocab=120001, canvas_len=5, seed=41,
                        t_choices=(0.0, 0.6, 1.0), probs_dtype=torch.bfloat16)
    w.keep_mask = (torch.arange(w.temps.numel(), device=DEV) % 3 != 0).to(torch.uint8)
    w.K = 7
    ref = gpu_rowstats(w)
    ref_v, ref_i = _run_topk(w)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for it in range(3):
        with torch.cuda.stream(s1 if it % 2 == 0 else s2):
            o = gpu_rowstats(w)
        with torch.cuda.stream(s2 if it % 2 == 0 else s1):
            v = torch.full((w.rows, w.K), 7.0, device=DEV)
            i = torch.full((w.rows, w.K), -7, dtype=torch.int64, device=DEV)
            rs.topk_logprobs(w.logits, w.temps, w.canvas_len, w.keep_mask, w.K, v, i)
        outs.append((o, v, i))
    torch.cuda.synchronize()
    for o, v, i in outs:
        _same(ref, o)
        assert torch.equal(v, ref_v) and torch.equal(i, ref_i)
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
                                     (70001, 1),
                                     # two values per lane in the chunk threshold
                                     (40000, 33), (40000, 48), (4097, 63), (70001, 40)])
@pytest.mark.parametrize("ties", [False, True], ids=["plain", "ties"])
def test_topk_small(vocab, K, ties):
    w = _topk_case(rows=9, vocab=vocab, canvas=3, K=K, seed=vocab + K, ties=ties,
                   ld=vocab + (3 if vocab % 2 else 0))
    vals, idx = _run_topk(w)
    _check_untouched(w, vals, idx)
    compare_topk(w, vals, idx, range(w.rows), f"topk V={vocab} K={K}")
    done()


@pytest.mark.parametrize("K", [20, 50])
def test_topk_adversarial_rows(K):
    vocab = 40000
    w = _topk_case(rows=6, vocab=vocab, canvas=1, K=K, seed=3)
    w.keep_mask = torch.ones(6, dtype=torch.uint8, device=DEV)
    w.logits[0] = 1.5                       # every lane max ties: overflow path
    w.logits[1, 100:39000] = float("-inf")   # -inf spans
    w.logits[2] = -0.0
    w.logits[2, ::3] = 0.0                   # signed zeros tie
    w.logits[3, 5000:5300] = 9.0             # 300 duplicates of the max
    w.logits[4] = torch.linspace(-1, 1, vocab, device=DEV)
    vals, idx = _run_topk(w)
    compare_topk(w, vals, idx, range(w.rows), f"topk adversarial K={K}")
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
    for K in (9, 45):
        w.K = K
        vals, idx = _run_topk(w)
        compare_topk(w, vals, idx, range(rows), f"topk magnitudes T={temp} K={K}")
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
    compare_topk(w, vals, idx, range(w.rows), "topk one-wave")
    done()


@pytest.mark.parametrize("K", [20, 64])
def test_c4_topk_full_size(K):
    # K = 64 takes the two-values-per-lane chunk threshold
    w = syn.c4(DEV, K=K)
    vals, idx = _run_topk(w)
    _check_untouched(w, vals, idx)
    kept_rows = [r for r in range(w.rows) if int(w.keep_mask[r // w.canvas_len])]
    for b in range(0, len(kept_rows), 256):
        compare_topk(w, vals, idx, kept_rows[b:b + 256], f"C4 K={K} kept rows {b}+")
    record("C4" if K == 20 else f"C4 K={K}", rows=w.rows, kept_rows=len(kept_rows),
           compared="all kept rows")
    del vals, idx, w
    done()
