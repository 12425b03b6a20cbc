"""Shared helpers of the GPU parity tests: run the HIP path and the oracle on
the same rows and compare them to the bar each output has.

Tolerances (derived in the design notes from the arithmetic of both sides):
  argmax, top-K indices        bit-exact
  sample                       exact, except rows whose oracle top-two
                               perturbed scores are within 1e-6; there the
                               GPU's column must itself score within 1e-6 of
                               the best (its exact score is recomputed from
                               the oracle's scale, noise word and Gumbel map),
                               and such rows are counted and recorded
  entropy                      |gpu - oracle| <= 1e-4
  probs (bf16 / fp16)          at most 1 unit in the last place
  top-K logprobs               |gpu - oracle| <= 1e-5 * max(1, |oracle|)

Near-tie counts go to stdout and, when ROWSTATS_PARITY_LOG names a file, to
that file as one JSON line per compared case.
"""
from __future__ import annotations

import json
import os

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


def record(case: str, **fields):
    """Prints a parity record and appends it to $ROWSTATS_PARITY_LOG."""
    line = {"case": case, **fields}
    print("parity:", json.dumps(line), flush=True)
    path = os.environ.get("ROWSTATS_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(line) + "\n")


def exact_score(x_row: np.ndarray, row: int, col: int, temp: float, seed: int) -> float:
    """The oracle's perturbed score z = s + g of one column, from its parts."""
    s = float(oracle.scale_row(x_row[col:col + 1], temp)[0])
    return s + oracle.uniform_gumbel(oracle.noise_word(seed, row, col))[1]


def compare_rowstats(w, out, rows, label=""):
    """Compares the GPU outputs `out` on `rows` with the oracle; returns
    (near-tie rows, near-tie rows whose sample differs from the oracle's)."""
    argmax, sample, entropy, probs = out
    rows = np.asarray(rows, dtype=np.int64)
    x = host_rows(w.logits, rows)
    temps = w.temps.cpu().numpy()
    ref = oracle.rowstats(x, rows, temps, w.canvas_len, w.seed, PROBS_CODE[w.probs_dtype])
    ridx = torch.as_tensor(rows, device=argmax.device)
    g_arg = argmax[ridx].cpu().numpy()
    g_smp = sample[ridx].cpu().numpy()
    g_ent = entropy[ridx].cpu().numpy().astype(np.float64)
    bad = np.nonzero(g_arg != ref["argmax"])[0]
    assert bad.size == 0, f"{label} argmax differs on rows {rows[bad][:10]}: gpu {g_arg[bad][:10]} oracle {ref['argmax'][bad][:10]}"
    near = ref["gap"] < GAP_BAND
    smp_bad = np.nonzero((g_smp != ref["sample"]) & ~near)[0]
    assert smp_bad.size == 0, f"{label} sample differs on rows {rows[smp_bad][:10]}: gpu {g_smp[smp_bad][:10]} oracle {ref['sample'][smp_bad][:10]} gap {ref['gap'][smp_bad][:10]}"
    excused = np.nonzero((g_smp != ref["sample"]) & near)[0]
    for i in excused:
        # several columns are within the band of the best: the GPU's must be one
        r = int(rows[i])
        t = float(temps[r // w.canvas_len])
        z_best = exact_score(x[i], r, int(ref["sample"][i]), t, w.seed)
        z_gpu = exact_score(x[i], r, int(g_smp[i]), t, w.seed)
        assert 0.0 <= z_best - z_gpu <= GAP_BAND, (
            f"{label} row {r}: the GPU's sample {g_smp[i]} scores {z_gpu!r}, "
            f"more than {GAP_BAND} below the best {z_best!r} (column {ref['sample'][i]})")
    err = np.abs(g_ent - ref["entropy"])
    assert np.all(err <= ENTROPY_TOL), f"{label} entropy off by {err.max():.3g} on row {rows[np.argmax(err)]}"
    if w.probs_dtype is not None:
        gp = probs_bits(probs.index_select(0, ridx))
        ne = np.nonzero(gp != ref["probs"])
        if ne[0].size:
            d = np.abs(gp[ne].astype(np.int32) - ref["probs"][ne].astype(np.int32))
            worst = int(d.max())
            if worst > 1:
                k = int(np.argmax(d))
                r, c = ne[0][k], ne[1][k]
                raise AssertionError(f"{label} probs differ by {worst} ulp at row {rows[r]} col {c}: "
                                     f"gpu {gp[r, c]:#06x} oracle {ref['probs'][r, c]:#06x}")
    return int(near.sum()), int(excused.size)


def compare_all_rows(w, out, label, block=256):
    """compare_rowstats over every row of the workload, `block` rows at a
    time (host memory stays bounded); records the near-tie counts."""
    near = excused = 0
    for r0 in range(0, w.rows, block):
        n, e = compare_rowstats(w, out, range(r0, min(w.rows, r0 + block)), f"{label} rows {r0}+")
        near += n
        excused += e
    record(label, rows=w.rows, compared="all", near_tie_rows=near,
           near_tie_sample_differs=excused)
    return near


def compare_topk(w, vals, idx, rows, label=""):
    rows = np.asarray(rows, dtype=np.int64)
    x = host_rows(w.logits, rows)
    ref_v, ref_i = oracle.topk_logprobs(x, rows, w.temps.cpu().numpy(), w.canvas_len,
                                        w.keep_mask.cpu().numpy(), w.K)
    keep = w.keep_mask.cpu().numpy()[rows // w.canvas_len] != 0
    ridx = torch.as_tensor(rows, device=vals.device)
    gv = vals[ridx].cpu().numpy()
    gi = idx[ridx].cpu().numpy()
    bad = np.nonzero(np.any(gi != ref_i, axis=1) & keep)[0]
    assert bad.size == 0, f"{label} top-K indices differ on row {rows[bad[0]]}: gpu {gi[bad[0]]} oracle {ref_i[bad[0]]}"
    kv = gv[keep].astype(np.float64)
    rv = ref_v[keep].astype(np.float64)
    # equal values (a -inf logit's logprob is -inf on both sides) are exact
    with np.errstate(invalid="ignore"):
        err = np.where(kv == rv, 0.0, np.abs(kv - rv))
    tol = LOGPROB_TOL * np.maximum(1.0, np.abs(rv))
    assert np.all(err <= tol), f"{label} logprobs off by {err.max():.3g}"


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


# Self-conditioning product (rowstats_selfcond). The kernel forms each
# probability in fp32 from s - m, a fused multiply-add, exp2 and 1 / S; its
# relative error stays below about 2^-15.8 (s - m down to -92, where bf16
# ends), so its value in the model dtype (bf16 or fp16) can differ from the
# oracle's only where the exact probability lies within SELFCOND_EPS of a
# rounding boundary, and then by one unit. The fp32 sums of each of the 8
# vocab ranges, then of the ranges, add at most (K_range + 9) 2^-24 sum |p E|
# (every product of two bf16 or two fp16 values is exact in fp32).
SELFCOND_EPS = 2.0 ** -14
SELFCOND_SPLITS = 8
PRODUCT_STEP = 64


def selfcond_k_range(vocab: int) -> int:
    per = -(-vocab // SELFCOND_SPLITS)
    return -(-per // 32) * 32


def bf16_ulp(q: np.ndarray) -> np.ndarray:
    """Unit in the last place of bf16 values q >= 0 (2^-133 below 2^-126)."""
    e = np.floor(np.log2(np.maximum(q, 2.0 ** -126)))
    return np.where(q >= 2.0 ** -126, 2.0 ** (e - 7), 2.0 ** -133)


def fp16_ulp(q: np.ndarray) -> np.ndarray:
    """Unit in the last place of fp16 values q >= 0 (2^-24 below 2^-14)."""
    e = np.floor(np.log2(np.maximum(q, 2.0 ** -14)))
    return np.where(q >= 2.0 ** -14, 2.0 ** (e - 10), 2.0 ** -24)


def product_k_range(vocab: int) -> int:
    """Vocab rows of one split range of the product of given probabilities
    (64-row steps)."""
    per = -(-vocab // SELFCOND_SPLITS)
    return -(-per // PRODUCT_STEP) * PRODUCT_STEP


def selfcond_bound(x: np.ndarray, rows, temps, canvas_len: int, embed_bits: np.ndarray,
                   f16: bool = False, k_range: int | None = None):
    """Per-element bound of |gpu - oracle| for the rows' products (see above);
    f16: the model dtype is fp16 (else bf16); k_range: the vocab rows of one
    split range (default: the fused product's)."""
    if k_range is None:
        k_range = selfcond_k_range(x.shape[1])
    rows = np.asarray(rows, dtype=np.int64)
    code = oracle.PROBS_FP16 if f16 else oracle.PROBS_BF16
    to_f64 = oracle.fp16_to_f64 if f16 else oracle.bf16_to_f64
    ref = oracle.rowstats(x, rows, temps, canvas_len, 0, code)
    q = to_f64(ref["probs"])
    ulp = fp16_ulp(q) if f16 else bf16_ulp(q)
    w = np.empty_like(q)
    for i, r in enumerate(rows):
        s = oracle.scale_row(x[i], float(np.asarray(temps)[r // canvas_len])).astype(np.float64)
        e = np.exp(s - s.max())
        p = e / e.sum()
        near = np.minimum(np.abs(p - (q[i] + ulp[i] / 2)),
                          np.minimum(np.abs(p - (q[i] - ulp[i] / 2)), np.abs(p - (q[i] - ulp[i] / 4))))
        amb = near <= SELFCOND_EPS * p + 2.0 ** -149
        w[i] = amb * ulp[i] + (k_range + 9) * 2.0 ** -24 * (q[i] + ulp[i])
    bound = np.zeros((len(rows), embed_bits.shape[1]))
    for c0 in range(0, embed_bits.shape[0], 16384):
        bound += w[:, c0:c0 + 16384] @ np.abs(to_f64(embed_bits[c0:c0 + 16384]))
    return bound + 2.0 ** -140


def compare_selfcond(w, embed: torch.Tensor, out, rows, label="", k_range: int | None = None):
    """Statistics as compare_rowstats (no probs) and the product within
    selfcond_bound of the oracle's; returns the worst error / bound."""
    import dataclasses
    argmax, sample, entropy, res = out
    compare_rowstats(dataclasses.replace(w, probs_dtype=None), (argmax, sample, entropy, None),
                     rows, label)
    rows = np.asarray(rows, dtype=np.int64)
    x = host_rows(w.logits, rows)
    eb = embed.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    temps = w.temps.cpu().numpy()
    f16 = embed.dtype == torch.float16
    ref = oracle.selfcond(x, rows, temps, w.canvas_len, eb,
                          dtype=oracle.PROBS_FP16 if f16 else oracle.PROBS_BF16)
    got = res[torch.as_tensor(rows, device=res.device)].double().cpu().numpy()
    bound = selfcond_bound(x, rows, temps, w.canvas_len, eb, f16, k_range)
    err = np.abs(got - ref)
    ratio = err / bound
    k = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert np.all(err <= bound), (f"{label} product off by {err[k]:.3g} (bound {bound[k]:.3g}) "
                                  f"at row {rows[k[0]]} column {k[1]}: gpu {got[k]!r} oracle {ref[k]!r}")
    return float(ratio.max())


def compare_product(probs: torch.Tensor, embed: torch.Tensor, out: torch.Tensor, rows,
                    label=""):
    """The product of given probabilities against oracle.probs_product: every
    product of two bf16 (fp16) values is exact in fp32, and each output is a
    chain of at most k_range + 9 fp32 additions (one split range, then the 8
    partials), so |gpu - oracle| <= (k_range + 9) 2^-24 sum_c |q_c| |e_cj|.
    Returns the worst error / bound."""
    rows = np.asarray(rows, dtype=np.int64)
    idx = torch.as_tensor(rows, device=probs.device)
    f16 = probs.dtype == torch.float16
    code = oracle.PROBS_FP16 if f16 else oracle.PROBS_BF16
    to_f64 = oracle.fp16_to_f64 if f16 else oracle.bf16_to_f64
    qb = probs_bits(probs.index_select(0, idx))
    eb = embed.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle.probs_product(qb, eb, dtype=code)
    w = (product_k_range(probs.shape[1]) + 9) * 2.0 ** -24 * np.abs(to_f64(qb))
    bound = np.zeros_like(ref)
    for c0 in range(0, eb.shape[0], 16384):
        bound += w[:, c0:c0 + 16384] @ np.abs(to_f64(eb[c0:c0 + 16384]))
    bound += 2.0 ** -140
    got = out.index_select(0, idx).double().cpu().numpy()
    err = np.abs(got - ref)
    ratio = err / bound
    k = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert np.all(err <= bound), (f"{label} product off by {err[k]:.3g} (bound {bound[k]:.3g}) "
                                  f"at row {rows[k[0]]} column {k[1]}: gpu {got[k]!r} oracle {ref[k]!r}")
    return float(ratio.max())
