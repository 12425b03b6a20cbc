"""Parity of rowstats_selfcond (the softmax in the model dtype, bf16 or fp16,
times the embedding table, on the matrix cores) with the oracle, through the
C ABI.

The statistics must equal rowstats_run's; the product must lie within the
bound derived in tests/parity.py (one bf16 unit on probabilities within
2^-14 of a rounding boundary, plus the fp32 summation bound); closed forms
(uniform rows: the column mean of E; greedy rows: the argmax's embedding)
must hold bit for bit.
"""
import numpy as np
import pytest
import torch

import synthetic as syn
import row_softmax_statistics_amd as rs
from parity import compare_selfcond, record

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run(w, embed):
    return rs.selfcond_embed(w.logits, w.temps, w.canvas_len, w.seed, embed)


def done():
    rs.check_device()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("rows,vocab,d,pad", [
    (1, 1, 256, 0), (5, 31, 256, 3), (7, 100, 512, 0), (9, 2048, 256, 0), (33, 2049, 256, 1),
    (300, 4097, 256, 0), (257, 20000, 512, 4), (40, 70001, 768, 0), (3, 262144, 256, 0)])
def test_small_shapes(rows, vocab, d, pad):
    w = syn.random_case(DEV, rows=rows, vocab=vocab, canvas_len=3, seed=vocab + d,
                        ld=vocab + pad, t_choices=(0.0, 0.6, 1.0, 98.0))
    embed = syn.embedding(vocab, d, seed=vocab, device=DEV)
    out = run(w, embed)
    worst = compare_selfcond(w, embed, out, range(rows), f"selfcond {rows}x{vocab} d={d}")
    record(f"selfcond {rows}x{vocab} d={d}", worst_error_over_bound=round(worst, 4))
    done()


@pytest.mark.parametrize("rows,vocab,d,pad", [
    (5, 31, 256, 3), (33, 2049, 256, 1), (257, 20000, 512, 4), (40, 70001, 768, 0),
    (3, 262144, 256, 0)])
def test_small_shapes_fp16(rows, vocab, d, pad):
    # the fp16 model dtype: probabilities and table in IEEE half, fp16 matrix cores
    w = syn.random_case(DEV, rows=rows, vocab=vocab, canvas_len=3, seed=vocab + d + 7,
                        ld=vocab + pad, t_choices=(0.0, 0.6, 1.0, 98.0))
    embed = syn.embedding(vocab, d, seed=vocab + 1, device=DEV, dtype=torch.float16)
    out = run(w, embed)
    worst = compare_selfcond(w, embed, out, range(rows), f"selfcond fp16 {rows}x{vocab} d={d}")
    record(f"selfcond fp16 {rows}x{vocab} d={d}", worst_error_over_bound=round(worst, 4))
    done()


def test_fp16_closed_forms():
    # uniform rows: p = 2^-12 exactly, small-integer E: the column mean bit for
    # bit; greedy rows: the argmax's embedding bit for bit
    vocab, d = 4096, 512
    x = torch.full((3, vocab), 0.5, device=DEV)
    embed = syn.embedding(vocab, d, seed=19, device=DEV, ints=True, dtype=torch.float16)
    _, _, _, out = rs.selfcond_embed(x, torch.tensor([1.0, 0.4, 7.0], device=DEV), 1, 5, embed)
    assert torch.equal(out, embed.float().mean(dim=0).expand(3, d))
    w = syn.random_case(DEV, rows=20, vocab=30000, canvas_len=5, seed=18, t_choices=(0.0,))
    e2 = syn.embedding(w.vocab, 768, seed=20, device=DEV, dtype=torch.float16)
    a, _, _, out2 = run(w, e2)
    assert torch.equal(out2, e2[a].float())
    done()


def test_statistics_equal_rowstats_run():
    w = syn.random_case(DEV, rows=70, vocab=30001, canvas_len=7, seed=3,
                        t_choices=(0.0, 0.5, 1.0))
    embed = syn.embedding(w.vocab, 256, seed=4, device=DEV)
    a = run(w, embed)
    b = rs.sample_row_stats(w.logits, w.temps, w.canvas_len, w.seed, None)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)
    done()


def test_uniform_rows_give_the_column_mean_exactly():
    # p = 2^-12 exactly; E holds small integers, so every fp32 partial sum is
    # exact and the product is the column mean bit for bit
    vocab, d = 4096, 512
    x = torch.full((6, vocab), -0.375, device=DEV)
    temps = torch.tensor([1.0, 0.3, 2.5, 0.0, 98.0, 1e-3], device=DEV)
    embed = syn.embedding(vocab, d, seed=9, device=DEV, ints=True)
    _, _, _, out = rs.selfcond_embed(x, temps, 1, 5, embed)
    mean = embed.float().mean(dim=0)
    assert torch.equal(out, mean.expand(6, d))
    done()


def test_greedy_rows_give_the_argmax_embedding_exactly():
    w = syn.random_case(DEV, rows=50, vocab=50000, canvas_len=10, seed=12, t_choices=(0.0,))
    embed = syn.embedding(w.vocab, 768, seed=13, device=DEV)
    a, _, _, out = run(w, embed)
    assert torch.equal(out, embed[a].float())
    done()


def test_repeat_calls_are_bit_identical():
    w = syn.random_case(DEV, rows=300, vocab=65536, canvas_len=30, seed=14,
                        t_choices=(0.0, 0.7, 1.0))
    embed = syn.embedding(w.vocab, 512, seed=15, device=DEV)
    a, b = run(w, embed), run(w, embed)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    done()


def test_c2_full_size_d2560():
    # the C2 logits (4096 x 262144) and a 262144 x 2560 table (the width of a
    # Gemma-3-4B-sized embedding): sampled rows against the oracle, every
    # greedy row (unique maximum) against its argmax's embedding
    w = syn.c2(DEV)
    embed = syn.embedding(w.vocab, 2560, seed=21, device=DEV)
    out = run(w, embed)
    # three seeded rows of every slot (16 slots of 256 rows: every temperature
    # and every pair of 128-row tiles of the product) and two peaked rows,
    # against the oracle
    rng = np.random.default_rng(22)
    rows = sorted(set((256 * np.repeat(np.arange(16), 3) + rng.integers(0, 256, 48)).tolist())
                  | set(w.special_rows["peaked"][:2].tolist()))
    worst = compare_selfcond(w, embed, out, rows, "selfcond C2 d=2560")
    greedy = (w.temps[torch.arange(w.rows, device=DEV) // w.canvas_len] == 0)
    g = torch.nonzero(greedy).flatten()
    assert torch.equal(out[3][g], embed[out[0][g]].float())
    record("selfcond C2 d=2560", rows_compared=len(rows), greedy_rows_exact=int(g.numel()),
           worst_error_over_bound=round(worst, 4))
    del out, embed
    # the fp16 model dtype at the same size: one seeded row per slot
    embed = syn.embedding(w.vocab, 2560, seed=23, device=DEV, dtype=torch.float16)
    out = run(w, embed)
    rows16 = (256 * np.arange(16) + rng.integers(0, 256, 16)).tolist()
    worst = compare_selfcond(w, embed, out, rows16, "selfcond fp16 C2 d=2560")
    assert torch.equal(out[3][g], embed[out[0][g]].float())
    record("selfcond fp16 C2 d=2560", rows_compared=len(rows16), greedy_rows_exact=int(g.numel()),
           worst_error_over_bound=round(worst, 4))
    del out, embed, w
    done()
