"""Parity of the self-conditioning product of given probabilities
(rowstats_pack_embed + rowstats_selfcond_product) with the oracle, through the
C ABI.

Given probabilities (seeded, log-normal, bf16 or fp16) times a packed table
must lie within the fp32 summation bound of oracle.probs_product; the path
rowstats_run (probs) -> product must match oracle.selfcond within the bound
of the fused product (one unit on probabilities near a rounding boundary);
closed forms hold bit for bit; the packed table is the layout the header
documents.
"""
import numpy as np
import pytest
import torch

import synthetic as syn
import row_softmax_statistics_amd as rs
from parity import (compare_product, compare_rowstats, compare_selfcond, product_k_range,
                    record)

pytestmark = pytest.mark.gpu
DEV = "cuda"
NAMES = {torch.bfloat16: "bf16", torch.float16: "fp16"}


def done():
    rs.check_device()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("rows,vocab,d,ld", [
    (1, 1, 256, None), (5, 31, 256, 33), (7, 100, 512, None), (33, 2049, 256, None),
    (65, 5000, 256, 5003), (129, 4097, 768, 4104), (300, 20000, 512, None),
    (40, 70001, 768, None), (3, 262144, 256, None), (17, 3000, 4096, None),
    (9, 5000, 1280, 5008)])
def test_given_probabilities(rows, vocab, d, ld, dtype):
    # odd strides and odd vocab take the element-load path, the others the
    # 16-byte path; 64-row steps leave ragged ends in most ranges
    label = f"product {NAMES[dtype]} {rows}x{vocab} d={d} ld={ld or vocab}"
    print("case", label, flush=True)
    q = syn.probabilities(rows, vocab, seed=rows + vocab, device=DEV, dtype=dtype, ld=ld)
    e = syn.embedding(vocab, d, seed=vocab + d, device=DEV, dtype=dtype)
    out = rs.selfcond_product(q, rs.pack_embed(e))
    worst = compare_product(q, e, out, np.arange(rows), label)
    record(label, worst_error_over_bound=round(worst, 4))
    done()


def test_packed_table_is_the_documented_layout():
    # element (b, j, h, l, i) of the packed table is
    # E[32 b + 16 h + 8 (l // 32) + i][32 j + l % 32], zero past the last row
    vocab, d = 300, 512
    e = syn.embedding(vocab, d, seed=3, device=DEV)
    packed = rs.pack_embed(e)
    assert packed.data.numel() == 384 * d * 2
    got = packed.data.view(torch.int16).view(-1, d // 32, 2, 64, 8)
    nb = got.shape[0]
    b = torch.arange(nb, device=DEV).view(-1, 1, 1, 1, 1)
    j = torch.arange(d // 32, device=DEV).view(1, -1, 1, 1, 1)
    h = torch.arange(2, device=DEV).view(1, 1, -1, 1, 1)
    lane = torch.arange(64, device=DEV).view(1, 1, 1, -1, 1)
    i = torch.arange(8, device=DEV).view(1, 1, 1, 1, -1)
    padded = torch.zeros(nb * 32, d, dtype=torch.int16, device=DEV)
    padded[:vocab] = e.view(torch.int16)
    want = padded[32 * b + 16 * h + 8 * (lane // 32) + i, 32 * j + lane % 32]
    assert torch.equal(got, want)
    done()


def test_one_hot_rows_give_embedding_rows_exactly():
    rows, vocab, d = 200, 30000, 768
    g = torch.Generator(device=DEV).manual_seed(5)
    cols = torch.randint(0, vocab, (rows,), generator=g, device=DEV)
    q = torch.zeros(rows, vocab, dtype=torch.bfloat16, device=DEV)
    q[torch.arange(rows, device=DEV), cols] = 1.0
    e = syn.embedding(vocab, d, seed=6, device=DEV)
    out = rs.selfcond_product(q, rs.pack_embed(e))
    assert torch.equal(out, e[cols].float())
    done()


def test_uniform_rows_give_the_column_mean_exactly():
    # q = 2^-12 and small-integer E: every fp32 partial sum is exact
    vocab, d = 4096, 512
    for dtype in (torch.bfloat16, torch.float16):
        q = torch.full((9, vocab), 2.0 ** -12, dtype=dtype, device=DEV)
        e = syn.embedding(vocab, d, seed=9, device=DEV, ints=True, dtype=dtype)
        out = rs.selfcond_product(q, rs.pack_embed(e))
        assert torch.equal(out, e.float().mean(dim=0).expand(9, d))
    done()


def test_subnormal_probabilities():
    # rows made only of bf16 values below 2^-126 (and zeros): their products
    # with E are fp32 subnormals, which the bound requires to be kept
    rows, vocab, d = 16, 8192, 256
    g = torch.Generator(device=DEV).manual_seed(8)
    k = torch.randint(0, 9, (rows, vocab), generator=g, device=DEV)
    q = torch.where(k == 0, torch.zeros(rows, vocab, device=DEV),
                    torch.ldexp(torch.ones(rows, vocab, device=DEV), -126 - k)).to(torch.bfloat16)
    assert torch.all(q.float() < 2.0 ** -126)
    e = syn.embedding(vocab, d, seed=10, device=DEV)
    out = rs.selfcond_product(q, rs.pack_embed(e))
    worst = compare_product(q, e, out, np.arange(rows), "product bf16 subnormal rows")
    record("product bf16 subnormal rows", worst_error_over_bound=round(worst, 4))
    done()


def test_repeat_calls_and_row_prefixes_are_bit_identical():
    q = syn.probabilities(300, 65536, seed=11, device=DEV)
    packed = rs.pack_embed(syn.embedding(65536, 512, seed=12, device=DEV))
    a = rs.selfcond_product(q, packed)
    assert torch.equal(a, rs.selfcond_product(q, packed))
    for r in (1, 129):
        assert torch.equal(a[:r], rs.selfcond_product(q[:r], packed))
    done()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("rows,vocab,d,pad", [
    (5, 31, 256, 3), (33, 2049, 256, 1), (257, 20000, 512, 4), (40, 70001, 768, 0)])
def test_from_logits_through_rowstats_probs(rows, vocab, d, pad, dtype):
    # rowstats_run writes the probabilities, the product reads them: the same
    # self-conditioning input as rowstats_selfcond, within its bound
    label = f"probs->product {NAMES[dtype]} {rows}x{vocab} d={d}"
    print("case", label, flush=True)
    w = syn.random_case(DEV, rows=rows, vocab=vocab, canvas_len=3, seed=vocab + d + 3,
                        ld=vocab + pad, t_choices=(0.0, 0.6, 1.0, 98.0), probs_dtype=dtype)
    stats = rs.sample_row_stats(w.logits, w.temps, w.canvas_len, w.seed, dtype)
    compare_rowstats(w, stats, range(rows), label)
    e = syn.embedding(vocab, d, seed=vocab + 2, device=DEV, dtype=dtype)
    out = rs.selfcond_product(stats[3], rs.pack_embed(e))
    worst = compare_selfcond(w, e, (*stats[:3], out), range(rows), label,
                             k_range=product_k_range(vocab))
    record(label, worst_error_over_bound=round(worst, 4))
    done()


def test_c2_full_size_d2560():
    # the C2 logits (4096 x 262144) with bf16 probs and a 262144 x 2560 table:
    # sampled rows against the oracle, every greedy row against its argmax's
    # embedding
    w = syn.c2(DEV)
    argmax, sample, entropy, probs = rs.sample_row_stats(w.logits, w.temps, w.canvas_len,
                                                         w.seed, torch.bfloat16)
    embed = syn.embedding(w.vocab, 2560, seed=21, device=DEV)
    out = rs.selfcond_product(probs, rs.pack_embed(embed))
    del probs
    rng = np.random.default_rng(24)
    rows = sorted(set((256 * np.repeat(np.arange(16), 3) + rng.integers(0, 256, 48)).tolist())
                  | set(w.special_rows["peaked"][:2].tolist()))
    worst = compare_selfcond(w, embed, (argmax, sample, entropy, out), rows,
                             "probs->product C2 d=2560", k_range=product_k_range(w.vocab))
    greedy = (w.temps[torch.arange(w.rows, device=DEV) // w.canvas_len] == 0)
    g = torch.nonzero(greedy).flatten()
    assert torch.equal(out[g], embed[argmax[g]].float())
    record("probs->product C2 d=2560", rows_compared=len(rows), greedy_rows_exact=int(g.numel()),
           worst_error_over_bound=round(worst, 4))
    done()


def test_calls_on_two_streams_are_ordered():
    # both products use the library's one partial-product buffer; calls that
    # alternate between two streams (a larger one in between) give the
    # results of one stream
    w = syn.random_case(DEV, rows=300, vocab=50000, canvas_len=5, seed=42,
                        t_choices=(0.0, 0.7, 1.0), probs_dtype=torch.bfloat16)
    e = syn.embedding(w.vocab, 512, seed=43, device=DEV)
    packed = rs.pack_embed(e)
    probs = rs.sample_row_stats(w.logits, w.temps, w.canvas_len, w.seed, torch.bfloat16)[3]
    big = syn.probabilities(700, w.vocab, seed=44, device=DEV)
    ref_sc = rs.selfcond_embed(w.logits, w.temps, w.canvas_len, w.seed, e)
    ref_p = rs.selfcond_product(probs, packed)
    ref_big = rs.selfcond_product(big, packed)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for it in range(3):
        a, b = (s1, s2) if it % 2 == 0 else (s2, s1)
        with torch.cuda.stream(a):
            sc = rs.selfcond_embed(w.logits, w.temps, w.canvas_len, w.seed, e)
        with torch.cuda.stream(b):
            p = rs.selfcond_product(probs, packed)
        with torch.cuda.stream(a):
            g = rs.selfcond_product(big, packed)
        outs.append((sc, p, g))
    torch.cuda.synchronize()
    for sc, p, g in outs:
        for x, y in zip(sc, ref_sc):
            assert torch.equal(x, y)
        assert torch.equal(p, ref_p) and torch.equal(g, ref_big)
    done()
