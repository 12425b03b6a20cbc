"""Parity of top-K logprobs for K above 64 (the workgroup-per-row kernel)
with the oracle's full sort, through the C ABI: indices exact, logprobs
within 1e-5 relative, rows of slots that are not kept untouched.

Covers K = vocab (the whole row in key order), batches of 4096 keys (one,
two and three), ties at the batch boundaries, quantised values, -inf spans,
signed zeros, all-equal rows, the scalar-load path (odd strides) and a row
length of 262144.
"""
import pytest
import torch

import synthetic as syn
import row_softmax_statistics_amd as rs
from parity import compare_topk

pytestmark = pytest.mark.gpu
DEV = "cuda"


def done():
    rs.check_device()
    torch.cuda.empty_cache()


def case(rows, vocab, canvas, K, seed, ties=False, ld=None, temps=(0.0, 1.0, 0.5)):
    w = syn.random_case(DEV, rows=rows, vocab=vocab, canvas_len=canvas, seed=seed, ties=ties,
                        ld=ld, t_choices=temps, probs_dtype=None)
    w.keep_mask = (torch.arange(w.temps.numel(), device=DEV) % 3 != 1).to(torch.uint8)
    w.K = K
    return w


def run(w):
    vals = torch.full((w.rows, w.K), 7.0, device=DEV)
    idx = torch.full((w.rows, w.K), -7, dtype=torch.int64, device=DEV)
    rs.topk_logprobs(w.logits, w.temps, w.canvas_len, w.keep_mask, w.K, vals, idx)
    return vals, idx


def check_untouched(w, vals, idx):
    slot = torch.arange(w.rows, device=DEV) // w.canvas_len
    dropped = w.keep_mask[slot] == 0
    assert torch.all(vals[dropped] == 7.0) and torch.all(idx[dropped] == -7)


@pytest.mark.parametrize("vocab,K", [(65, 65), (100, 65), (100, 100), (4097, 300), (5000, 4096),
                                     (5000, 4097), (20000, 9000), (70001, 128)])
@pytest.mark.parametrize("ties", [False, True], ids=["plain", "ties"])
def test_large_k(vocab, K, ties):
    print(f"case topk-wide V={vocab} K={K} ties={ties}", flush=True)
    w = case(rows=7, vocab=vocab, canvas=2, K=K, seed=vocab + K, ties=ties,
             ld=vocab + (3 if vocab % 2 else 0))
    vals, idx = run(w)
    check_untouched(w, vals, idx)
    compare_topk(w, vals, idx, range(w.rows), f"topk-wide V={vocab} K={K}")
    done()


def test_adversarial_rows():
    vocab, K = 12000, 5000
    w = case(rows=6, vocab=vocab, canvas=1, K=K, seed=5)
    w.keep_mask = torch.ones(6, dtype=torch.uint8, device=DEV)
    w.logits[0] = 1.5                        # all equal: the lowest K columns
    w.logits[1, 100:11000] = float("-inf")   # -inf keys inside the top-K
    w.logits[2] = -0.0
    w.logits[2, ::3] = 0.0                   # signed zeros tie
    w.logits[3, 5000:9500] = 9.0             # 4500 duplicates of the max across a batch edge
    w.logits[4] = torch.linspace(-1, 1, vocab, device=DEV)
    vals, idx = run(w)
    compare_topk(w, vals, idx, range(w.rows), "topk-wide adversarial")
    done()


@pytest.mark.parametrize("temp", [0.0, 1e-3, 0.37, 3.7, 1000.0])
def test_temperatures(temp):
    w = case(rows=4, vocab=3000, canvas=1, K=700, seed=11, temps=(temp,))
    w.keep_mask = torch.ones(4, dtype=torch.uint8, device=DEV)
    vals, idx = run(w)
    compare_topk(w, vals, idx, range(w.rows), f"topk-wide T={temp}")
    done()


def test_full_length_rows():
    # rows of 262144 columns, K = 1000
    w = case(rows=12, vocab=262144, canvas=4, K=1000, seed=13)
    vals, idx = run(w)
    check_untouched(w, vals, idx)
    compare_topk(w, vals, idx, range(w.rows), "topk-wide V=262144 K=1000")
    done()


def test_repeat_calls_are_bit_identical():
    w = case(rows=9, vocab=30000, canvas=3, K=2000, seed=17, ties=True)
    a, b = run(w), run(w)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    done()


def test_calls_on_two_streams_are_ordered():
    # the workgroup-per-row path shares the scratch head and the kept-row
    # lists with the other entry points: calls alternating between two
    # streams (row statistics, a one-pass top-K and a stash in between)
    # give the results of one stream
    w = case(rows=12, vocab=20000, canvas=3, K=700, seed=19, ties=True)
    ref = run(w)
    sw = syn.stash_case(DEV, m=5, canvas_len=3, vocab=5000, K=90, seed=20)
    ids = torch.full((sw.n_slots, sw.positions, sw.width), -7, dtype=torch.int32, device=DEV)
    lp = torch.full((sw.n_slots, sw.positions, sw.width), 7.0, device=DEV)
    rk = torch.full((sw.n_slots, sw.positions), -7, dtype=torch.int32, device=DEV)

    def stash():
        rs.stash_converged_logprobs(sw.logits, sw.canvas_len, sw.src, sw.slots, sw.keep,
                                    sw.valid, sw.temps, sw.K, sw.num_ids, sw.ids, ids, lp, rk,
                                    sw.logits_mode)
        return ids.clone(), lp.clone(), rk.clone()

    ref_stash = stash()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for it in range(3):
        a, b = (s1, s2) if it % 2 == 0 else (s2, s1)
        with torch.cuda.stream(a):
            rs.sample_row_stats(w.logits, w.temps, w.canvas_len, 5, torch.bfloat16)
            got = run(w)
        with torch.cuda.stream(b):
            rs.topk_logprobs(w.logits, w.temps, w.canvas_len, w.keep_mask, 20)
            got_stash = stash()
        outs.append((got, got_stash))
    torch.cuda.synchronize()
    for got, got_stash in outs:
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
        for x, y in zip(got_stash, ref_stash):
            assert torch.equal(x, y)
    done()
