"""GPU parity of the converged-logprob stash with the stash oracle.

Ids and ranks must match exactly. Logprobs follow the top-K bar
(|gpu - oracle| <= 1e-5 max(1, |oracle|)); in logits mode the values are the
scaled logits, which both sides round once from x / T, so they must be
equal. Cells that the call must not write keep their sentinel.
"""
import numpy as np
import pytest
import torch

import synthetic as syn
import row_softmax_statistics_amd as rs
from oracle import stash as ostash
from parity import LOGPROB_TOL, host_rows, record

pytestmark = pytest.mark.gpu
DEV = "cuda"
SENT_ID, SENT_VAL = -7, 1e30


def run_gpu(w):
    out_ids = torch.full((w.n_slots, w.positions, w.width), SENT_ID, dtype=torch.int32, device=DEV)
    out_lp = torch.full((w.n_slots, w.positions, w.width), SENT_VAL, dtype=torch.float32,
                        device=DEV)
    out_rk = torch.full((w.n_slots, w.positions), SENT_ID, dtype=torch.int32, device=DEV)
    rs.stash_converged_logprobs(w.logits, w.canvas_len, w.src, w.slots, w.keep, w.valid, w.temps,
                                w.K, w.num_ids, w.ids, out_ids, out_lp, out_rk, w.logits_mode)
    return out_ids.cpu().numpy(), out_lp.cpu().numpy(), out_rk.cpu().numpy()


def run_oracle(w, x=None):
    x = w.logits.cpu().numpy() if x is None else x
    out_ids = np.full((w.n_slots, w.positions, w.width), SENT_ID, np.int32)
    out_lp = np.full((w.n_slots, w.positions, w.width), SENT_VAL, np.float32)
    out_rk = np.full((w.n_slots, w.positions), SENT_ID, np.int32)
    ids = w.ids.cpu().numpy() if w.ids is not None else None
    ostash.stash_converged_logprobs(x, w.canvas_len, w.src.cpu().numpy(), w.slots.cpu().numpy(),
                                    w.keep.cpu().numpy(), w.valid.cpu().numpy(),
                                    w.temps.cpu().numpy(), w.K, w.num_ids.cpu().numpy(), ids,
                                    out_ids, out_lp, out_rk, w.logits_mode)
    return out_ids, out_lp, out_rk


def compare(g, o, logits_mode, label):
    gi, gl, gr = g
    oi, ol, orr = o
    bad = np.argwhere(gi != oi)
    assert bad.size == 0, f"{label}: ids differ at {bad[:5].tolist()}: gpu {gi[tuple(bad[0])]} oracle {oi[tuple(bad[0])]}"
    bad = np.argwhere(gr != orr)
    assert bad.size == 0, f"{label}: ranks differ at {bad[:5].tolist()}: gpu {gr[tuple(bad[0])]} oracle {orr[tuple(bad[0])]}"
    fin = np.isfinite(ol) & (ol != SENT_VAL)
    assert np.array_equal(gl[~fin], ol[~fin]), f"{label}: non-finite or unwritten cells differ"
    if logits_mode:
        assert np.array_equal(gl[fin], ol[fin]), f"{label}: scaled logits differ"
    else:
        ref = ol[fin].astype(np.float64)
        err = np.abs(gl[fin].astype(np.float64) - ref)
        tol = LOGPROB_TOL * np.maximum(1.0, np.abs(ref))
        assert np.all(err <= tol), f"{label}: logprobs off by {err.max():.3g}"


def check(w, label):
    g = run_gpu(w)
    rs.check_device()
    compare(g, run_oracle(w), w.logits_mode, label)
    torch.cuda.empty_cache()


CASES = [  # vocab, K, with_ids, logits_mode, ld pad
    (1, 0, False, False, 0), (1, 1, True, True, 0), (2, 2, True, False, 1),
    (7, 0, True, False, 0), (7, 5, False, True, 3), (1000, 0, False, False, 0),
    (1000, 5, True, False, 0), (1000, 20, True, True, 0), (4096, 64, True, False, 0),
    (5001, 1, True, False, 3), (5001, 20, False, True, 0), (70001, 20, True, False, 0),
    (70001, 0, True, True, 5), (40000, 64, False, False, 0),
]


@pytest.mark.parametrize("vocab,K,with_ids,logits_mode,pad", CASES)
def test_stash_small(vocab, K, with_ids, logits_mode, pad):
    w = syn.stash_case(DEV, m=6, canvas_len=4, vocab=vocab, K=K, seed=vocab + 7 * K,
                       ld=vocab + pad, with_ids=with_ids, logits_mode=logits_mode)
    check(w, f"stash V={vocab} K={K} ids={with_ids} logits={logits_mode}")


LARGE_K = [  # vocab, K, with_ids, logits_mode, ld pad: num_topk above 64
    (65, 65, False, False, 0), (100, 65, True, False, 0), (300, 300, False, True, 1),
    (4097, 300, True, False, 3), (5000, 4096, False, False, 0), (5000, 4097, True, True, 0),
    (20000, 9000, False, False, 0), (70001, 128, True, False, 5),
]


@pytest.mark.parametrize("vocab,K,with_ids,logits_mode,pad", LARGE_K)
def test_stash_large_k(vocab, K, with_ids, logits_mode, pad):
    # the workgroup-per-row kernel writes these stash rows
    w = syn.stash_case(DEV, m=5, canvas_len=3, vocab=vocab, K=K, seed=vocab + K,
                       ld=vocab + pad, with_ids=with_ids, logits_mode=logits_mode)
    check(w, f"stash V={vocab} K={K} ids={with_ids} logits={logits_mode}")


@pytest.mark.parametrize("K", [0, 2, 20, 200])
def test_stash_ties(K):
    # quantised values: exact duplicates of the maximum are common
    w = syn.stash_case(DEV, m=8, canvas_len=5, vocab=3000, K=K, seed=50 + K, ties=True, std=1.0)
    check(w, f"stash ties K={K}")


@pytest.mark.parametrize("K", [0, 3, 64, 100, 8999])
def test_stash_equal_rows_and_spans(K):
    """All-equal rows (every key ties at the maximum: the rank counts the
    whole row), rows with long -inf spans, and a row that is -inf but one
    column."""
    w = syn.stash_case(DEV, m=4, canvas_len=3, vocab=9000, K=K, seed=60 + K, with_ids=True)
    w.keep.fill_(1)
    w.valid.fill_(3)
    rows = (w.src.long() * 3).tolist()
    w.logits[rows[0]] = 1.25
    w.logits[rows[0] + 1] = -3.0
    w.logits[rows[1], 100:8000] = float("-inf")
    w.logits[rows[2]] = float("-inf")
    w.logits[rows[2], 4321] = 0.5
    check(w, f"stash equal rows K={K}")


def test_stash_many_requests():
    w = syn.stash_case(DEV, m=300, canvas_len=7, vocab=2500, K=10, seed=71)
    check(w, "stash m=300")


def test_stash_more_requests_than_lds_offsets():
    # above 4096 requests the pre-pass lists rows thread by thread
    w = syn.stash_case(DEV, m=5000, canvas_len=2, vocab=300, K=4, seed=72)
    check(w, "stash m=5000")


def test_stash_wider_positions():
    # the stash holds more positions than a canvas: the extra ones stay untouched
    w = syn.stash_case(DEV, m=5, canvas_len=3, vocab=900, K=2, seed=73)
    w.positions = 7
    check(w, "stash positions=7")


@pytest.mark.parametrize("K", [3, 80])
def test_stash_bad_indices_are_skipped_and_flagged(K):
    w = syn.stash_case(DEV, m=5, canvas_len=4, vocab=700, K=K, seed=80, with_ids=True)
    w.keep.fill_(1)
    w.valid.fill_(4)
    w.num_ids.zero_()
    canvases = w.logits.shape[0] // w.canvas_len
    w.src[1] = canvases          # rows past the logits: request skipped
    w.slots[2] = w.n_slots       # slot past the stash: request skipped
    w.num_ids[3] = 3
    w.ids[3, :3] = torch.tensor([5, w.vocab, -2], dtype=torch.int32, device=DEV)
    g = run_gpu(w)
    with pytest.raises(rs.RowStatsError) as e:
        rs.check_device()
    assert e.value.code == -7
    rs.check_device()  # the flag is cleared
    # the oracle has no notion of a skipped request: compare with requests
    # 1 and 2 dropped, and with the bad ids written as given at -inf
    w.keep[1] = 0
    w.keep[2] = 0
    o = run_oracle(w)
    compare(g, o, False, "stash bad indices")
    slot3 = int(w.slots[3])
    assert g[0][slot3, 0, 1:4].tolist() == [5, w.vocab, -2]
    assert np.all(g[1][slot3, :, 2:4] == -np.inf)


def test_stash_between_other_calls():
    """The stash shares scratch with the other entry points: alternate them."""
    w = syn.stash_case(DEV, m=6, canvas_len=4, vocab=5000, K=7, seed=90)
    tk = syn.random_case(DEV, rows=12, vocab=3000, canvas_len=4, seed=91, probs_dtype=None)
    keep = torch.ones(tk.temps.numel(), dtype=torch.uint8, device=DEV)
    o = run_oracle(w)
    for it in range(3):
        rs.topk_logprobs(tk.logits, tk.temps, tk.canvas_len, keep, 5)
        rs.sample_row_stats(tk.logits, tk.temps, tk.canvas_len, 3, torch.bfloat16)
        compare(run_gpu(w), o, False, f"stash alternating {it}")
    rs.check_device()


def _oracle_positions(w, picks, x):
    """The oracle's stash rows for the kept positions `picks` = [(j, p)],
    each as a one-position request over its logits row x[i]; rows are split
    over threads (the oracle's sorts release the interpreter lock)."""
    from concurrent.futures import ThreadPoolExecutor

    temps = w.temps.cpu()
    num_ids = w.num_ids.cpu()
    ids = w.ids.cpu() if w.ids is not None else None

    def part(lo, hi):
        js = [j for j, _ in picks[lo:hi]]
        n = hi - lo
        one = syn.StashWorkload(
            "S4 rows", None, 1, torch.arange(n, dtype=torch.int32),
            torch.arange(n, dtype=torch.int32), torch.ones(n, dtype=torch.uint8),
            torch.ones(n, dtype=torch.int32), temps[js], w.K, num_ids[js],
            ids[js] if ids is not None else None, n, 1, w.width)
        return run_oracle(one, x[lo:hi])

    step = max(1, (len(picks) + 15) // 16)
    bounds = [(lo, min(len(picks), lo + step)) for lo in range(0, len(picks), step)]
    with ThreadPoolExecutor(len(bounds)) as ex:
        parts = list(ex.map(lambda b: part(*b), bounds))
    return tuple(np.concatenate([q[k] for q in parts]) for k in range(3))


def _compare_positions(w, g, blk, label):
    src = w.src.cpu().numpy()
    slots = w.slots.cpu().numpy()
    rows = [int(src[j]) * w.canvas_len + p for j, p in blk]
    o = _oracle_positions(w, blk, host_rows(w.logits, rows))
    gsel = (np.stack([g[0][slots[j], p] for j, p in blk])[:, None],
            np.stack([g[1][slots[j], p] for j, p in blk])[:, None],
            np.array([g[2][slots[j], p] for j, p in blk])[:, None])
    compare(gsel, o, False, label)


def test_stash_c4_full_size():
    """The S4 stash (C4's 4096 x 262144 logits): every kept position checked
    against the oracle, 256 positions at a time."""
    w = syn.stash_c4(DEV)
    g = run_gpu(w)
    rs.check_device()
    keep = w.keep.cpu().numpy()
    valid = w.valid.cpu().numpy()
    src = w.src.cpu().numpy()
    slots = w.slots.cpu().numpy()
    picks = [(int(j), p) for j in np.flatnonzero(keep)
             for p in range(min(int(valid[j]), w.canvas_len))]
    for b in range(0, len(picks), 256):
        _compare_positions(w, g, picks[b:b + 256], f"S4 positions {b}+")
    record("S4", kept_positions=len(picks), compared="all kept positions")
    # positions past valid and slots of dropped requests keep their sentinel
    for j in range(w.m):
        n = min(int(valid[j]), w.canvas_len) if keep[j] else 0
        assert np.all(g[2][slots[j], n:] == SENT_ID)
    used = set(slots[keep != 0].tolist())
    for sl in range(w.n_slots):
        if sl not in used:
            assert np.all(g[0][sl] == SENT_ID)
    torch.cuda.empty_cache()


def test_stash_c4_full_size_num_topk_1000():
    """The S4 stash with num_topk = 1000 (the workgroup-per-row kernel):
    64 sampled kept positions against the oracle, the others' sentinels."""
    w = syn.stash_c4(DEV, K=1000)
    g = run_gpu(w)
    rs.check_device()
    keep = w.keep.cpu().numpy()
    valid = w.valid.cpu().numpy()
    slots = w.slots.cpu().numpy()
    picks = [(int(j), p) for j in np.flatnonzero(keep)
             for p in range(min(int(valid[j]), w.canvas_len))]
    rng = np.random.default_rng(31)
    blk = [picks[i] for i in sorted(rng.choice(len(picks), 64, replace=False))]
    _compare_positions(w, g, blk, "S4 num_topk=1000")
    record("S4 num_topk=1000", kept_positions=len(picks), compared=len(blk))
    for j in range(w.m):
        n = min(int(valid[j]), w.canvas_len) if keep[j] else 0
        assert np.all(g[2][slots[j], :n] >= 1)
        assert np.all(g[2][slots[j], n:] == SENT_ID)
    torch.cuda.empty_cache()
