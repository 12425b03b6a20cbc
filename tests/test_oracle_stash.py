"""Pins of the stash oracle (CPU only).

The layout rules come from the stash_converged_logprobs docstring on the
vLLM API page "diffusion_gemma_sampler": for a kept request j, position p
below valid[j] reads row src[j] * canvas_len + p, scaled by 1 / temps[j],
and writes out_*[slots[j], p]; column 0 of a stash row is the argmax, the
next ones the request's listed token ids or else its num_topk largest
(equal values by lower id), the rest token 0 at -inf. The values are pinned to the separately
pinned C oracle of the top-K entry point, to closed forms and to
invariants of log-softmax.
"""
import importlib.util
import math
import os

import numpy as np
import pytest

import oracle
from oracle import stash

# ROWSTATS_STASH_ORACLE lets the mutation test load a deliberately broken
# copy of the stash oracle and check that these pins reject it
if os.environ.get("ROWSTATS_STASH_ORACLE"):
    _spec = importlib.util.spec_from_file_location("stash_mutant",
                                                   os.environ["ROWSTATS_STASH_ORACLE"])
    stash = importlib.util.module_from_spec(_spec)
    _spec.loader.exec_module(stash)

pytestmark = pytest.mark.filterwarnings("ignore:divide by zero")

NEG = -np.inf


def _run(logits, canvas_len, src, slots, keep, valid, temps, K, nids, ids, n_slots, width,
         logits_mode=False, positions=None):
    positions = positions or canvas_len
    out_ids = np.full((n_slots, positions, width), -7, np.int32)
    out_lp = np.full((n_slots, positions, width), 99.0, np.float32)
    out_rk = np.full((n_slots, positions), -7, np.int32)
    stash.stash_converged_logprobs(logits, canvas_len, np.asarray(src), np.asarray(slots),
                                   np.asarray(keep), np.asarray(valid),
                                   np.asarray(temps, np.float32), K, nids, ids, out_ids, out_lp,
                                   out_rk, logits_mode)
    return out_ids, out_lp, out_rk


def _worked_example():
    # 12 logits rows of vocab 6 (4 canvases of 3 positions)
    x = np.zeros((12, 6), np.float32)
    x[6] = [0, 3, 1, 3, NEG, 2]
    x[7] = [5, 5, 5, 5, 5, 5]
    x[3] = [1, 2, 0, 0, -1, 0]
    x[4] = [NEG, NEG, 7, NEG, NEG, NEG]
    x[5] = [0.5] * 6
    src = [2, 0, 1]
    slots = [1, 0, 2]
    keep = [1, 0, 1]
    valid = [2, 3, 5]
    temps = [1.0, 1.0, 0.5]
    nids = np.array([0, 2, 2], np.int32)
    ids = np.array([[9, 9], [1, 1], [4, 0]], np.int32)
    return x, src, slots, keep, valid, temps, nids, ids


def test_worked_example_layout():
    """Which cells are written, and with which ids and ranks, worked out by
    hand from the docstring's rules."""
    x, src, slots, keep, valid, temps, nids, ids = _worked_example()
    oi, ov, rk = _run(x, 3, src, slots, keep, valid, temps, 3, nids, ids, n_slots=3, width=5)
    # slot 0 belongs to a request that is not kept: untouched
    assert np.all(oi[0] == -7) and np.all(ov[0] == 99.0) and np.all(rk[0] == -7)
    # request 0 -> slot 1, positions 0 and 1 (valid = 2); position 2 untouched
    assert oi[1, 0].tolist() == [1, 1, 3, 5, 0]  # argmax (tie 1/3 -> 1), top-3, pad
    assert oi[1, 1].tolist() == [0, 0, 1, 2, 0]
    assert rk[1, 0] == 2 and rk[1, 1] == 6
    assert np.all(oi[1, 2] == -7) and rk[1, 2] == -7
    assert ov[1, 0, 4] == NEG and ov[1, 1, 4] == NEG
    # request 2 -> slot 2, positions 0..2 (valid 5 cut to the canvas), ids [4, 0]
    assert oi[2, 0].tolist() == [1, 4, 0, 0, 0]
    assert oi[2, 1].tolist() == [2, 4, 0, 0, 0]
    assert oi[2, 2].tolist() == [0, 4, 0, 0, 0]
    assert rk[2].tolist() == [1, 1, 6]
    assert np.all(ov[2, :, 3:] == NEG)


def test_worked_example_values():
    x, src, slots, keep, valid, temps, nids, ids = _worked_example()
    oi, ov, rk = _run(x, 3, src, slots, keep, valid, temps, 3, nids, ids, n_slots=3, width=5)
    # uniform rows: every logprob is -ln 6
    assert np.allclose(ov[1, 1, :4], -math.log(6), rtol=0, atol=1e-6)
    assert np.allclose(ov[2, 2, :3], -math.log(6), rtol=0, atol=1e-6)
    # one finite column: logprob 0 there, -inf elsewhere
    assert ov[2, 1].tolist() == [0.0, NEG, NEG, NEG, NEG]
    # row 6 (T = 1): the softmax of [0, 3, 1, 3, -inf, 2]
    z = 1 + 2 * math.exp(3) + math.exp(1) + math.exp(2)
    want = [3 - math.log(z), 3 - math.log(z), 3 - math.log(z), 2 - math.log(z)]
    assert np.allclose(ov[1, 0, :4], want, rtol=0, atol=2e-6)
    # row 3 at T = 0.5: s = [2, 4, 0, 0, -2, 0]; ids 4 and 0
    z = math.exp(2) + math.exp(4) + 3 + math.exp(-2)
    assert np.allclose(ov[2, 0, :3], [4 - math.log(z), -2 - math.log(z), 2 - math.log(z)],
                       rtol=0, atol=2e-6)


def test_logits_mode_writes_scaled_logits():
    x, src, slots, keep, valid, temps, nids, ids = _worked_example()
    oi, ov, rk = _run(x, 3, src, slots, keep, valid, temps, 3, nids, ids, n_slots=3, width=5,
                      logits_mode=True)
    assert ov[1, 0].tolist() == [3.0, 3.0, 3.0, 2.0, NEG]
    assert ov[2, 0].tolist() == [4.0, -2.0, 2.0, NEG, NEG]  # s = x / 0.5
    assert ov[2, 1].tolist() == [14.0, NEG, NEG, NEG, NEG]


def test_topk_matches_c_oracle():
    """Columns 1..K of a top-K stash row equal the separately pinned C
    oracle of the top-K entry point on the same rows (identity layout)."""
    rng = np.random.default_rng(5)
    m, W, V, K = 4, 3, 1000, 9
    x = (rng.standard_normal((m * W, V)) * 2).astype(np.float32)
    x[4, 10:20] = x[4].max()  # ties at the maximum
    temps = np.array([1.0, 0.7, 0.0, 1.3], np.float32)
    keep = np.array([1, 1, 1, 0], np.uint8)
    oi, ov, rk = _run(x, W, np.arange(m), np.arange(m), keep, [W] * m, temps, K, None, None,
                      n_slots=m, width=K + 3)
    ref_v, ref_i = oracle.topk_logprobs(x, np.arange(m * W), temps, W, keep, K)
    for r in range(m * W):
        j, p = divmod(r, W)
        if not keep[j]:
            assert np.all(oi[j, p] == -7)
            continue
        assert oi[j, p, 1:K + 1].tolist() == ref_i[r].tolist()
        assert oi[j, p, 0] == ref_i[r, 0]
        np.testing.assert_allclose(ov[j, p, 1:K + 1], ref_v[r], rtol=1e-6, atol=1e-6)
        assert np.all(oi[j, p, K + 1:] == 0) and np.all(ov[j, p, K + 1:] == NEG)


def test_ranks_count_ties_at_the_maximum():
    rng = np.random.default_rng(8)
    V = 257
    x = rng.standard_normal((5, V)).astype(np.float32)
    for r, n in enumerate([1, 2, 3, 40, V]):
        top = np.float32(x.max() + 1)
        cols = rng.choice(V, n, replace=False)
        x[r, cols] = top
    oi, ov, rk = _run(x, 5, [0], [0], [1], [5], [1.0], 2, None, None, n_slots=1, width=3)
    assert rk[0].tolist() == [1, 2, 3, 40, V]
    for r in range(5):
        cols = np.flatnonzero(x[r] == x[r].max())
        assert oi[0, r, 0] == cols.min()
    # -0 and +0 tie at the maximum: the lower column is the argmax
    z = -np.abs(x[:1]) - 1
    z[0, 7], z[0, 3] = 0.0, -0.0
    oi, ov, rk = _run(z, 1, [0], [0], [1], [1], [1.0], 2, None, None, n_slots=1, width=3)
    assert oi[0, 0].tolist() == [3, 3, 7] and rk[0, 0] == 2


def test_ids_cover_the_whole_distribution():
    """With every column listed as a token id, the listed probabilities sum
    to one."""
    rng = np.random.default_rng(2)
    V = 300
    x = (rng.standard_normal((2, V)) * 3).astype(np.float32)
    ids = np.arange(V, dtype=np.int32)[None, :]
    oi, ov, rk = _run(x, 2, [0], [0], [1], [2], [0.8], 0, np.array([V], np.int32), ids,
                      n_slots=1, width=V + 1)
    for p in range(2):
        assert oi[0, p, 1:].tolist() == list(range(V))
        assert abs(math.fsum(np.exp(ov[0, p, 1:].astype(np.float64))) - 1.0) < 1e-5


def test_shift_invariance():
    """Adding a constant to a row leaves its logprobs unchanged (integer
    logits and shift keep every fp32 value exact)."""
    rng = np.random.default_rng(4)
    x = rng.integers(-20, 20, (3, 128)).astype(np.float32)
    y = x + np.float32(64)
    a = _run(x, 3, [0], [0], [1], [3], [1.0], 5, None, None, n_slots=1, width=8)
    b = _run(y, 3, [0], [0], [1], [3], [1.0], 5, None, None, n_slots=1, width=8)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[2], b[2])
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-6)
    c = _run(x, 3, [0], [0], [1], [3], [1.0], 5, None, None, n_slots=1, width=8,
             logits_mode=True)
    d = _run(y, 3, [0], [0], [1], [3], [1.0], 5, None, None, n_slots=1, width=8,
             logits_mode=True)
    fin = np.isfinite(c[1])
    assert np.array_equal(d[1][fin] - c[1][fin], np.full(fin.sum(), 64, np.float32))


def test_id_count_limits_and_bad_ids():
    x = np.arange(10, dtype=np.float32)[None, :].repeat(2, 0)
    ids = np.array([[3, 12, -1, 5, 6, 7]], np.int32)
    oi, ov, rk = _run(x, 2, [0], [0], [1], [1], [1.0], 1, np.array([6], np.int32), ids,
                      n_slots=1, width=4)
    # width 4 leaves room for 3 ids; ids outside [0, vocab) get -inf
    assert oi[0, 0].tolist() == [9, 3, 12, -1]
    assert ov[0, 0, 1] < 0 and ov[0, 0, 2] == NEG and ov[0, 0, 3] == NEG
    # num_token_ids 0 means top-K even when ids are given
    oi, ov, rk = _run(x, 2, [0], [0], [1], [1], [1.0], 2, np.array([0], np.int32), ids,
                      n_slots=1, width=4)
    assert oi[0, 0].tolist() == [9, 9, 8, 0]


def test_num_topk_equal_to_the_vocabulary():
    """With num_topk = V the row lists every column once, in descending value
    with equal values by lower id (a brute-force sort on quantised values),
    and the probabilities of the list sum to one."""
    rng = np.random.default_rng(5)
    V = 257
    x = (np.round(rng.standard_normal((3, V)) * 2.0) / 2.0).astype(np.float32)
    oi, ov, rk = _run(x, 3, [0], [0], [1], [3], [1.0], V, np.zeros(1, np.int32), None,
                      n_slots=1, width=V + 1)
    for p in range(3):
        want = sorted(range(V), key=lambda c: (-float(x[p, c]), c))
        assert oi[0, p, 1:].tolist() == want
        assert oi[0, p, 0] == want[0]
        assert rk[0, p] == int(np.count_nonzero(x[p] == x[p].max()))
        assert abs(math.fsum(np.exp(ov[0, p, 1:].astype(np.float64))) - 1.0) < 1e-5
