"""Pins of the oracle's self-conditioning input (oracle.selfcond): the bf16
softmax of each row times the embedding table, against closed forms and a
brute-force sum (diffusion_gemma_sampler page, module docstring: the softmax
in the model dtype feeds the self-conditioning matmul)."""
import numpy as np
import pytest
import torch

import oracle


def bf16_bits(a) -> np.ndarray:
    """bf16 bit patterns of float values, rounded to nearest-even by torch."""
    return torch.as_tensor(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def small_int_embed(vocab, d, seed):
    rng = np.random.default_rng(seed)
    e = rng.integers(-4, 5, size=(vocab, d)).astype(np.float32)
    return e, bf16_bits(e)


def test_uniform_rows_give_the_column_mean():
    # equal logits: p = 1 / V = 2^-12 exactly in bf16, so out is the mean of E
    vocab, d = 4096, 24
    e, eb = small_int_embed(vocab, d, 1)
    x = np.full((3, vocab), 0.75, np.float32)
    out = oracle.selfcond(x, [0, 1, 2], [1.0, 0.3, 0.0], 1, eb)
    assert np.array_equal(out, np.repeat(e.astype(np.float64).mean(axis=0)[None], 3, axis=0))


def test_greedy_row_gives_the_argmax_embedding():
    # T = 0 divides by 1e-10: every other column's probability is exp(-1e9) = 0
    vocab, d = 5000, 16
    e, eb = small_int_embed(vocab, d, 2)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, vocab)).astype(np.float32)
    out = oracle.selfcond(x, np.arange(4), [0.0], 4, eb)
    for r in range(4):
        assert np.array_equal(out[r], e[int(np.argmax(x[r]))].astype(np.float64))


@pytest.mark.parametrize("k", [2, 3, 7])
def test_greedy_ties_share_the_mass(k):
    vocab, d = 300, 8
    e, eb = small_int_embed(vocab, d, 4)
    x = np.zeros((1, vocab), np.float32)
    cols = np.arange(5, 5 + 11 * k, 11)
    x[0, cols] = 2.0
    out = oracle.selfcond(x, [0], [0.0], 1, eb)
    share = oracle.bf16_to_f64(bf16_bits([1.0 / k]))[0]   # bf16(1/k)
    assert np.array_equal(out[0], share * e[cols].astype(np.float64).sum(axis=0))


def test_two_level_rows_closed_form():
    # k columns at a, the rest at b: two probabilities, each rounded to bf16
    vocab, d, k, a, b, T = 1000, 12, 13, 1.5, -0.25, 0.8
    e, eb = small_int_embed(vocab, d, 5)
    rng = np.random.default_rng(6)
    hi = rng.choice(vocab, size=k, replace=False)
    x = np.full((1, vocab), b, np.float32)
    x[0, hi] = a
    sa, sb = np.float32(a) / np.float32(T), np.float32(b) / np.float32(T)
    pa = 1.0 / (k + (vocab - k) * np.exp(float(sb) - float(sa)))
    pb = pa * np.exp(float(sb) - float(sa))
    qa, qb = oracle.bf16_to_f64(bf16_bits([pa, pb]))
    lo = np.setdiff1d(np.arange(vocab), hi)
    want = qa * e[hi].astype(np.float64).sum(axis=0) + qb * e[lo].astype(np.float64).sum(axis=0)
    out = oracle.selfcond(x, [0], [T], 1, eb)
    np.testing.assert_allclose(out[0], want, rtol=1e-14, atol=1e-14)


def test_brute_force_small():
    # explicit sums over the vocab, term by term, from the oracle's bf16 probs
    rng = np.random.default_rng(7)
    vocab, d, rows = 9, 5, 6
    x = (rng.standard_normal((rows, vocab)) * 2).astype(np.float32)
    e = rng.standard_normal((vocab, d)).astype(np.float32)
    eb = bf16_bits(e)
    ev = oracle.bf16_to_f64(eb)
    temps = [0.7, 0.0, 1.3]
    out = oracle.selfcond(x, np.arange(rows), temps, 2, eb, block=4)
    probs = oracle.rowstats(x, np.arange(rows), temps, 2, 0, oracle.PROBS_BF16)["probs"]
    for r in range(rows):
        p = oracle.bf16_to_f64(probs[r])
        for j in range(d):
            acc = 0.0
            for c in range(vocab):
                acc += p[c] * ev[c, j]
            assert abs(out[r, j] - acc) <= 1e-15 * (1 + abs(acc))


def test_vocab_permutation_and_linearity():
    rng = np.random.default_rng(8)
    vocab, d = 700, 16
    x = (rng.standard_normal((3, vocab)) * 2).astype(np.float32)
    e1 = bf16_bits(rng.integers(-3, 4, size=(vocab, d)))
    e2 = bf16_bits(rng.integers(-3, 4, size=(vocab, d)))
    e12 = bf16_bits(oracle.bf16_to_f64(e1) + oracle.bf16_to_f64(e2))   # small ints: exact
    a = oracle.selfcond(x, [0, 1, 2], [0.9], 3, e1)
    b = oracle.selfcond(x, [0, 1, 2], [0.9], 3, e2)
    np.testing.assert_allclose(oracle.selfcond(x, [0, 1, 2], [0.9], 3, e12), a + b,
                               rtol=1e-13, atol=1e-15)
    perm = rng.permutation(vocab)
    np.testing.assert_allclose(oracle.selfcond(x[:, perm].copy(), [0, 1, 2], [0.9], 3, e1[perm]),
                               a, rtol=1e-13, atol=1e-15)


# --- fp16 model dtype (the same product with probabilities and E in IEEE half)
def fp16_bits(a) -> np.ndarray:
    """IEEE half bit patterns of float values, rounded to nearest-even by numpy."""
    return np.asarray(a, np.float32).astype(np.float16).view(np.uint16)


def test_fp16_uniform_rows_give_the_column_mean():
    # p = 2^-12 is exact in fp16 too
    vocab, d = 4096, 16
    rng = np.random.default_rng(11)
    e = rng.integers(-4, 5, size=(vocab, d)).astype(np.float32)
    out = oracle.selfcond(np.full((2, vocab), -3.0, np.float32), [0, 1], [0.7, 1.0], 1,
                          fp16_bits(e), dtype=oracle.PROBS_FP16)
    assert np.array_equal(out, np.repeat(e.astype(np.float64).mean(axis=0)[None], 2, axis=0))


def test_fp16_greedy_ties_share_the_mass():
    # 1/3 rounded to fp16 (11 significant bits) differs from its bf16 rounding
    vocab, d, k = 200, 6, 3
    rng = np.random.default_rng(12)
    e = rng.integers(-4, 5, size=(vocab, d)).astype(np.float32)
    x = np.zeros((1, vocab), np.float32)
    cols = np.array([3, 90, 150])
    x[0, cols] = 1.0
    out = oracle.selfcond(x, [0], [0.0], 1, fp16_bits(e), dtype=oracle.PROBS_FP16)
    share = float(np.float16(1.0 / k))
    assert share != oracle.bf16_to_f64(bf16_bits([1.0 / k]))[0]
    assert np.array_equal(out[0], share * e[cols].astype(np.float64).sum(axis=0))


def test_fp16_brute_force_small_and_subnormal_probabilities():
    # one dominant column drives the others' probabilities into the fp16
    # subnormal range (below 2^-14), where they keep a few bits or flush to 0
    rng = np.random.default_rng(13)
    vocab, d, rows = 40, 5, 4
    x = (rng.standard_normal((rows, vocab)) * 0.5).astype(np.float32)
    x[:, 7] += 12.0
    e = rng.standard_normal((vocab, d)).astype(np.float32)
    eb = fp16_bits(e)
    ev = eb.view(np.float16).astype(np.float64)
    out = oracle.selfcond(x, np.arange(rows), [1.0, 0.9], 2, eb, block=16, dtype=oracle.PROBS_FP16)
    probs = oracle.rowstats(x, np.arange(rows), [1.0, 0.9], 2, 0, oracle.PROBS_FP16)["probs"]
    p = probs.view(np.float16).astype(np.float64)
    assert np.any((p > 0) & (p < 2.0 ** -14)), "the case must reach fp16 subnormals"
    for r in range(rows):
        for j in range(d):
            acc = 0.0
            for c in range(vocab):
                acc += p[r, c] * ev[c, j]
            assert abs(out[r, j] - acc) <= 1e-15 * (1 + abs(acc))


def test_dtype_is_checked():
    with pytest.raises(ValueError):
        oracle.selfcond(np.zeros((1, 4), np.float32), [0], [1.0], 1, np.zeros((4, 2), np.uint16),
                        dtype=oracle.PROBS_NONE)


# --- the product of given probabilities (oracle.probs_product)
def test_product_one_hot_rows_pick_embedding_rows():
    # q[i] = 1 at column c_i: out[i] = E[c_i] exactly, whatever E holds
    rng = np.random.default_rng(21)
    vocab, d, rows = 300, 40, 7
    e = rng.standard_normal((vocab, d)).astype(np.float32)
    eb = bf16_bits(e)
    cols = rng.integers(0, vocab, size=rows)
    q = np.zeros((rows, vocab), np.float32)
    q[np.arange(rows), cols] = 1.0
    out = oracle.probs_product(bf16_bits(q), eb, block=64)
    assert np.array_equal(out, oracle.bf16_to_f64(eb)[cols])


def test_product_brute_force_non_square_signed_and_subnormal():
    # explicit sums with rows != vocab != d (a transposed operand fails),
    # signed values (a dropped sign fails) and bf16 subnormals in both operands
    rng = np.random.default_rng(22)
    rows, vocab, d = 3, 11, 5
    q = rng.standard_normal((rows, vocab)).astype(np.float32)
    q[0, 2] = 3.0e-39
    e = rng.standard_normal((vocab, d)).astype(np.float32)
    e[4, 1] = -5.0e-39
    qb, eb = bf16_bits(q), bf16_bits(e)
    qv, ev = oracle.bf16_to_f64(qb), oracle.bf16_to_f64(eb)
    assert qv[0, 2] != 0.0 and abs(qv[0, 2]) < 2.0 ** -126
    out = oracle.probs_product(qb, eb, block=4)
    for r in range(rows):
        for j in range(d):
            acc = 0.0
            for c in range(vocab):
                acc += qv[r, c] * ev[c, j]
            assert abs(out[r, j] - acc) <= 1e-15 * (1 + abs(acc))


def test_product_fp16_closed_form():
    # fp16 q = 1/4 on four columns of small integers: the exact column means
    vocab, d = 64, 6
    rng = np.random.default_rng(23)
    e = rng.integers(-8, 9, size=(vocab, d)).astype(np.float32)
    q = np.zeros((2, vocab), np.float32)
    q[0, [1, 9, 17, 60]] = 0.25
    q[1, [0, 63, 5, 6]] = 0.25
    out = oracle.probs_product(fp16_bits(q), fp16_bits(e), block=16, dtype=oracle.PROBS_FP16)
    want = np.stack([e[[1, 9, 17, 60]].mean(axis=0), e[[0, 63, 5, 6]].mean(axis=0)])
    assert np.array_equal(out, want.astype(np.float64))


def test_selfcond_is_the_product_of_the_oracle_probabilities():
    rng = np.random.default_rng(24)
    vocab, d = 500, 8
    x = (rng.standard_normal((4, vocab)) * 2).astype(np.float32)
    eb = bf16_bits(rng.standard_normal((vocab, d)))
    probs = oracle.rowstats(x, np.arange(4), [0.8, 0.0], 2, 0, oracle.PROBS_BF16)["probs"]
    assert np.array_equal(oracle.selfcond(x, np.arange(4), [0.8, 0.0], 2, eb),
                          oracle.probs_product(probs, eb))
