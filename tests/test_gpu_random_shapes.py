"""Parity with the oracle on seeded random shapes: row statistics (with bf16,
fp16 or no probs) and top-K logprobs (K on both sides of 64) over random
row counts, vocabularies from 1 to 300000, row strides, canvas lengths,
value spreads, quantised ties and temperature mixes, and stash calls with
random request sets; every row and stash position is compared. The shapes
come from fixed seeds, so the cases are the same on every run.
"""
import numpy as np
import pytest
import torch

import synthetic as syn
import row_softmax_statistics_amd as rs
from parity import compare_rowstats, compare_topk, record

pytestmark = pytest.mark.gpu
DEV = "cuda"
N_CASES = 16


def shape(i):
    """Case i: rows, vocab, row stride, canvas, spread, ties, temperatures."""
    r = np.random.default_rng(9000 + i)
    vocab = int(np.exp(r.uniform(0.0, np.log(300000.0))))
    rows = int(r.integers(1, max(2, min(300, 20_000_000 // vocab)) + 1))
    ld = vocab + int(r.choice([0, 0, 1, 3, 128]))
    canvas = int(r.integers(1, 8))
    std = float(r.choice([0.5, 2.0, 8.0]))
    ties = bool(r.integers(0, 2))
    temps = tuple(float(t) for t in r.choice([0.0, 0.3, 0.7, 1.0, 1.5, 2.5, 40.0],
                                             size=int(r.integers(1, 4)), replace=False))
    K = int(r.integers(1, min(vocab, 200) + 1))
    return rows, vocab, ld, canvas, std, ties, temps, K


@pytest.mark.parametrize("i", range(N_CASES))
def test_rowstats_random_shape(i):
    rows, vocab, ld, canvas, std, ties, temps, _ = shape(i)
    dtype = (torch.bfloat16, torch.float16, None)[i % 3]
    label = f"random {i}: {rows}x{vocab} ld={ld} canvas={canvas} std={std} ties={ties} T={temps}"
    print("case", label, flush=True)
    w = syn.random_case(DEV, rows=rows, vocab=vocab, canvas_len=canvas, seed=300 + i, std=std,
                        ld=ld, t_choices=temps, probs_dtype=dtype, ties=ties)
    near, differs = compare_rowstats(w, rs.sample_row_stats(w.logits, w.temps, w.canvas_len,
                                                            w.seed, dtype), range(rows), label)
    record(f"random shape {i}", rows=rows, vocab=vocab, compared="all", near_tie_rows=near,
           near_tie_sample_differs=differs)
    rs.check_device()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("i", range(N_CASES))
def test_topk_random_shape(i):
    rows, vocab, ld, canvas, std, ties, temps, K = shape(i)
    label = f"random topk {i}: {rows}x{vocab} ld={ld} canvas={canvas} K={K}"
    print("case", label, flush=True)
    w = syn.random_case(DEV, rows=rows, vocab=vocab, canvas_len=canvas, seed=400 + i, std=std,
                        ld=ld, t_choices=temps, probs_dtype=None, ties=ties)
    slots = w.temps.numel()
    w.keep_mask = (torch.arange(slots, device=DEV) % 4 != 2).to(torch.uint8)
    w.K = K
    vals = torch.full((rows, K), 7.0, device=DEV)
    idx = torch.full((rows, K), -7, dtype=torch.int64, device=DEV)
    rs.topk_logprobs(w.logits, w.temps, w.canvas_len, w.keep_mask, K, vals, idx)
    dropped = w.keep_mask[torch.arange(rows, device=DEV) // canvas] == 0
    assert torch.all(vals[dropped] == 7.0) and torch.all(idx[dropped] == -7)
    compare_topk(w, vals, idx, range(rows), label)
    rs.check_device()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("i", range(8))
def test_stash_random_shape(i):
    import test_gpu_stash as ts
    r = np.random.default_rng(9500 + i)
    vocab = int(np.exp(r.uniform(0.0, np.log(150000.0))))
    K = int(r.integers(0, min(vocab, 200) + 1))
    m = int(r.integers(1, 40))
    canvas = int(r.integers(1, 7))
    with_ids, logits_mode, ties = (bool(r.integers(0, 2)) for _ in range(3))
    label = (f"random stash {i}: m={m} canvas={canvas} V={vocab} K={K} ids={with_ids} "
             f"logits={logits_mode} ties={ties}")
    print("case", label, flush=True)
    w = syn.stash_case(DEV, m=m, canvas_len=canvas, vocab=vocab, K=K, seed=500 + i,
                       ld=vocab + int(r.choice([0, 1, 5])), with_ids=with_ids, ties=ties,
                       logits_mode=logits_mode)
    ts.check(w, label)
