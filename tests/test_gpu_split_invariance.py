"""Results do not depend on how the work is split: the rows are dealt to row
groups dynamically (and, in the product, to 128-row tiles), so a prefix of
the rows run on its own is split differently from the same rows inside the
full batch, yet every output of those rows must be bit-identical. This
catches races and order dependences in the combine steps that a comparison
of one split with the oracle's tolerances could miss.
"""
import pytest
import torch

import synthetic as syn
import row_softmax_statistics_amd as rs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def done():
    rs.check_device()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("probs_dtype", [None, torch.bfloat16], ids=["none", "bf16"])
def test_rowstats_prefix_rows_are_bit_identical(probs_dtype):
    # 49 chunks per row: about 40 row groups, each dealt about 50 rows of the
    # full batch, one row or none of the shortest prefix
    w = syn.random_case(DEV, rows=2000, vocab=100000, canvas_len=40, seed=31,
                        t_choices=(0.0, 0.6, 1.0, 1.3), probs_dtype=probs_dtype)
    full = rs.sample_row_stats(w.logits, w.temps, w.canvas_len, w.seed, probs_dtype)
    for r in (1, 37, 700):
        part = rs.sample_row_stats(w.logits[:r], w.temps, w.canvas_len, w.seed, probs_dtype)
        for name, a, b in zip(("argmax", "sample", "entropy", "probs"), full, part):
            if a is None:
                continue
            assert torch.equal(a[:r], b), f"{name} of the first {r} rows differs"
    done()


def test_topk_prefix_rows_are_bit_identical():
    w = syn.random_case(DEV, rows=1500, vocab=70000, canvas_len=30, seed=32,
                        t_choices=(0.0, 1.0), probs_dtype=None)
    keep = (torch.arange(w.temps.numel(), device=DEV) % 3 != 1).to(torch.uint8)
    fv, fi = rs.topk_logprobs(w.logits, w.temps, w.canvas_len, keep, 17)
    for r in (5, 400):
        pv, pi = rs.topk_logprobs(w.logits[:r], w.temps, w.canvas_len, keep, 17)
        kept = keep[torch.arange(r, device=DEV) // w.canvas_len] != 0
        assert torch.equal(fv[:r][kept], pv[kept]) and torch.equal(fi[:r][kept], pi[kept])
    done()


def test_selfcond_prefix_rows_are_bit_identical():
    w = syn.random_case(DEV, rows=300, vocab=40000, canvas_len=10, seed=33,
                        t_choices=(0.0, 0.7, 1.0), probs_dtype=None)
    embed = syn.embedding(w.vocab, 768, seed=34, device=DEV)
    full = rs.selfcond_embed(w.logits, w.temps, w.canvas_len, w.seed, embed)
    for r in (1, 129):
        part = rs.selfcond_embed(w.logits[:r], w.temps, w.canvas_len, w.seed, embed)
        for name, a, b in zip(("argmax", "sample", "entropy", "product"), full, part):
            assert torch.equal(a[:r], b), f"{name} of the first {r} rows differs"
    done()
