"""rowstats_run_noalloc (the entry point that allocates nothing) against
rowstats_run, through the C ABI.

Both run the same kernels, so the outputs must be bit-identical; the first
call is also compared with the oracle on a sample of rows. Two calls in a
row on the fixed scratch array, the second smaller than the first (the
array keeps the first call's contents), then a call that needs more than
the array holds, which must be refused before anything is queued. And a
call captured into a graph, replayed three times on new logits with eager
calls in between: every replay must give rowstats_run's bits.
"""
import ctypes

import numpy as np
import pytest
import torch

import synthetic as syn
import row_softmax_statistics_amd as rs
from parity import compare_rowstats

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _outputs(w):
    dev = w.logits.device
    return (torch.full((w.rows,), -3, dtype=torch.int64, device=dev),
            torch.full((w.rows,), -3, dtype=torch.int64, device=dev),
            torch.full((w.rows,), -3.0, dtype=torch.float32, device=dev),
            torch.empty(w.rows, w.vocab, dtype=w.probs_dtype, device=dev)
            if w.probs_dtype is not None else None)


def _bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t


def _check_same(w, label, oracle_rows):
    ref = rs.sample_row_stats(w.logits, w.temps, w.canvas_len, w.seed, w.probs_dtype)
    out = rs.sample_row_stats_noalloc(w.logits, w.temps, w.canvas_len, w.seed, w.probs_dtype,
                                      _outputs(w))
    rs.check_device()
    for a, b in zip(ref, out):
        if a is None:
            assert b is None
        else:
            assert torch.equal(_bits(a), _bits(b)), label
    compare_rowstats(w, out, oracle_rows, label)


def test_noalloc_matches_rowstats_run_twice():
    # first call: the C2 workload (4096 x 262144, bf16 probs: 32 MiB of the array)
    w = syn.c2(DEV)
    _check_same(w, "noalloc C2", list(range(0, w.rows, 97)) + [w.rows - 1])
    del w
    torch.cuda.empty_cache()
    # second call, smaller, other shape and dtype, on the array the first left
    w = syn.random_case(DEV, rows=300, vocab=100003, canvas_len=7, seed=13,
                        t_choices=(0.0, 0.6, 1.0), probs_dtype=torch.float16, ld=100007)
    _check_same(w, "noalloc small", range(w.rows))
    torch.cuda.empty_cache()


def test_noalloc_refuses_more_than_the_array():
    # 9000 rows of 262144 columns need 9000 * 128 * 64 B of summaries > 64 MiB;
    # the pointers are never dereferenced: the call is refused while planning
    fake = ctypes.c_void_p(0x1000)
    null = ctypes.c_void_p(0)
    torch.cuda.init()
    rc = rs.lib().rowstats_run_noalloc(fake, 262144, 9000, 262144, fake, 1, 0, 0, fake, fake,
                                       fake, null, null)
    assert rc == -8, (rc, rs.last_error())
    assert "scratch" in rs.last_error()


@pytest.mark.parametrize("rows,vocab", [(64, 30000), (600, 262144)])
def test_noalloc_graph_replays_match_eager(rows, vocab):
    w = syn.random_case(DEV, rows=rows, vocab=vocab, canvas_len=4, seed=77,
                        t_choices=(0.0, 0.7, 1.0), probs_dtype=torch.bfloat16)
    x = w.logits.clone()  # the captured call reads this buffer on every replay
    outs = _outputs(w)
    rs.sample_row_stats_noalloc(x, w.temps, w.canvas_len, w.seed, w.probs_dtype, outs)
    rs.check_device()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rs.sample_row_stats_noalloc(x, w.temps, w.canvas_len, w.seed, w.probs_dtype, outs)
    for it in range(3):
        x.copy_(syn.random_case(DEV, rows=rows, vocab=vocab, canvas_len=4, seed=100 + it).logits)
        ref = rs.sample_row_stats(x, w.temps, w.canvas_len, w.seed, w.probs_dtype)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        rs.check_device()
        for a, b in zip(ref, outs):
            assert torch.equal(_bits(a), _bits(b)), f"replay {it}"
    del g
    torch.cuda.empty_cache()
