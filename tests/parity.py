"""Shared helpers of the GPU parity tests: run the HIP path and the oracle on
the same rows and compare them to the bar each output has.

Tolerances (derived in the design notes from the arithmetic of both sides):
  argmax, top-K indices        bit-exact
  sample                       exact, except rows whose oracle top-two
                               perturbed scores are within 1e-6 (counted)
  entropy                      |gpu - oracle| <= 1e-4
  probs (bf16 / fp16)          at most 1 unit in the last place
  top-K logprobs               |gpu - oracle| <= 1e-5 * max(1, |oracle|)
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import row_softmax_statistics_amd as rs

ENTROPY_TOL = 1e-4
GAP_BAND = 1e-6
LOGPROB_TOL = 1e-5
PROBS_CODE = {None: oracle.PROBS_NONE, torch.bfloat16: oracle.PROBS_BF16,
              torch.float16: oracle.PROBS_FP16}


def host_rows(logits: torch.Tensor, rows) -> np.ndarray:
    idx = torch.as_tensor(rows, dtype=torch.int64, device=logits.device)
    return logits.index_select(0, idx).float().cpu().numpy()


def gpu_rowstats(w):
    return rs.sample_row_stats(w.logits, w.temps, w.canvas_len, w.seed, w.probs_dtype)


def probs_bits(p: torch.Tensor) -> np.ndarray:
    return p.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def compare_rowstats(w, out, rows, label=""):
    """Compares the GPU outputs `out` on `rows` with the oracle; returns the
    number of near-tie sample rows that were excused."""
    argmax, sample, entropy, probs = out
    rows = np.asarray(rows, dtype=np.int64)
    x = host_rows(w.logits, rows)
    ref = oracle.rowstats(x, rows, w.temps.cpu().numpy(), w.canvas_len, w.seed,
                          PROBS_CODE[w.probs_dtype])
    ridx = torch.as_tensor(rows, device=argmax.device)
    g_arg = argmax[ridx].cpu().numpy()
    g_smp = sample[ridx].cpu().numpy()
    g_ent = entropy[ridx].cpu().numpy().astype(np.float64)
    bad = np.nonzero(g_arg != ref["argmax"])[0]
    assert bad.size == 0, f"{label} argmax differs on rows {rows[bad][:10]}: gpu {g_arg[bad][:10]} oracle {ref['argmax'][bad][:10]}"
    near = ref["gap"] < GAP_BAND
    smp_bad = np.nonzero((g_smp != ref["sample"]) & ~near)[0]
    assert smp_bad.size == 0, f"{label} sample differs on rows {rows[smp_bad][:10]}: gpu {g_smp[smp_bad][:10]} oracle {ref['sample'][smp_bad][:10]} gap {ref['gap'][smp_bad][:10]}"
    err = np.abs(g_ent - ref["entropy"])
    assert np.all(err <= ENTROPY_TOL), f"{label} entropy off by {err.max():.3g} on row {rows[np.argmax(err)]}"
    if w.probs_dtype is not None:
        gp = probs_bits(probs.index_select(0, ridx))
        d = np.abs(gp.astype(np.int64) - ref["probs"].astype(np.int64))
        worst = int(d.max()) if d.size else 0
        if worst > 1:
            r, c = np.unravel_index(np.argmax(d), d.shape)
            raise AssertionError(f"{label} probs differ by {worst} ulp at row {rows[r]} col {c}: "
                                 f"gpu {gp[r, c]:#06x} oracle {ref['probs'][r, c]:#06x}")
    return int(near.sum())


def compare_topk(w, vals, idx, rows, label=""):
    rows = np.asarray(rows, dtype=np.int64)
    x = host_rows(w.logits, rows)
    ref_v, ref_i = oracle.topk_logprobs(x, rows, w.temps.cpu().numpy(), w.canvas_len,
                                        w.keep_mask.cpu().numpy(), w.K)
    keep = w.keep_mask.cpu().numpy()[rows // w.canvas_len] != 0
    ridx = torch.as_tensor(rows, device=vals.device)
    gv = vals[ridx].cpu().numpy()
    gi = idx[ridx].cpu().numpy()
    for n, r in enumerate(rows):
        if not keep[n]:
            continue
        assert np.array_equal(gi[n], ref_i[n]), f"{label} top-K indices differ on row {r}: gpu {gi[n]} oracle {ref_i[n]}"
        tol = LOGPROB_TOL * np.maximum(1.0, np.abs(ref_v[n].astype(np.float64)))
        err = np.abs(gv[n].astype(np.float64) - ref_v[n].astype(np.float64))
        assert np.all(err <= tol), f"{label} logprobs off by {err.max():.3g} on row {r}"


def check_properties(w, out):
    """Checks on every row that hold at any size: the argmax attains the
    row max of the scaled logits at its lowest column, greedy rows sample
    their argmax, and rounded probs sum to 1 within their rounding."""
    argmax, sample, entropy, probs = out
    rows = w.rows
    slot = torch.arange(rows, device=w.logits.device) // w.canvas_len
    T = w.temps[slot]
    Tc = torch.clamp(T, min=1e-10).unsqueeze(1)
    greedy = ~(T > 0)
    assert torch.equal(sample[greedy], argmax[greedy])
    assert torch.all(torch.isfinite(entropy))
    assert int(argmax.min()) >= 0 and int(argmax.max()) < w.vocab
    assert int(sample.min()) >= 0 and int(sample.max()) < w.vocab
    for r0 in range(0, rows, 128):
        r1 = min(rows, r0 + 128)
        # fp32 quotient via an fp64 division (correctly rounded in both steps)
        s = (w.logits[r0:r1].double() / Tc[r0:r1].double()).float()
        m = s.max(dim=1, keepdim=True).values
        first = torch.argmax((s == m).to(torch.int8), dim=1)
        assert torch.equal(first, argmax[r0:r1]), f"argmax property fails in rows {r0}..{r1}"
        if probs is not None and probs.dtype == torch.bfloat16:
            tot = probs[r0:r1].double().sum(dim=1)
            assert float((tot - 1.0).abs().max()) < 2.0 ** -7, f"probs do not sum to 1 in rows {r0}..{r1}"
