"""CPU oracle of the converged-logprob stash.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline may import this module; the product path never does.

Follows the vLLM API page "diffusion_gemma_sampler", the docstring and the
launcher of ``stash_converged_logprobs``:

* the rows of request ``j`` are ``src[j] * canvas_len + p``, one per position
  ``p`` below ``valid[j]`` (and below ``canvas_len``: the launch grid has one
  program per canvas position), each scaled by ``1 / temps[j]``;
* a request is read only when ``keep[j]`` is set; position ``p`` of it is
  written to ``out_*[slots[j], p]``;
* within a stash row, column 0 is the argmax; the next columns hold the
  request's token ids when it lists some, otherwise its ``num_topk``
  largest (equal values by lower id); the cells left are token 0 at -inf;
  the launcher checks ``num_topk + 1 <= width``.

Readings where the page shows no body (each is listed in the design notes):

* the temperature is clamped at 1e-10 as in ``sample_row_stats`` (so T <= 0
  divides by 1e-10, as the top-K entry point does);
* the value written is the logprob ``s - log Z`` in fp32, or with
  ``logits_mode`` the scaled logit ``s`` itself;
* ``out_ranks[slots[j], p]`` is the rank of the argmax in the vLLM sense:
  the number of columns whose value is at least the argmax's (so the number
  of columns tied at the maximum);
* a request "has" token ids when ids are given and ``num_token_ids[j] > 0``;
  it then lists ``min(num_token_ids[j], width - 1, ids_stride)`` ids; an id
  outside ``[0, vocab)`` is written as given with value -inf;
* ids, slots and ranks are int32.

Plain numpy, one row at a time: fp32 division for the scaled logits (as the
page's ``logits.float() / temp``), then float64 for log Z and the logprobs.
"""
from __future__ import annotations

import numpy as np

T_MIN = np.float32(1e-10)


def clamp_temp(t: float) -> np.float32:
    t = np.float32(t)
    return t if t > T_MIN else T_MIN


def stash_row_layout(s: np.ndarray, K: int, ids, width: int, logits_mode: bool):
    """One stash row from the fp32 scaled logits s of a row.

    Returns (ids int32 [width], values fp32 [width], rank int). ``ids`` is
    None for a top-K row, else the request's list of token ids (already cut
    to at most width - 1 entries).
    """
    V = s.shape[0]
    s64 = s.astype(np.float64)
    m = s64.max()
    S = np.exp(s64 - m).sum()
    logS = np.log(S)

    def value(c):
        if logits_mode:
            return np.float32(s[c])
        return np.float32((s64[c] - m) - logS)

    # value descending, then column ascending (-0 and +0 compare equal)
    order = np.lexsort((np.arange(V), -s64))
    top = int(order[0])
    out_ids = np.zeros(width, np.int32)
    out_val = np.full(width, -np.inf, np.float32)
    out_ids[0] = top
    out_val[0] = value(top)
    if ids is None:
        for k in range(K):
            c = int(order[k])
            out_ids[1 + k] = c
            out_val[1 + k] = value(c)
    else:
        for i, c in enumerate(ids):
            c = int(c)
            out_ids[1 + i] = c
            out_val[1 + i] = value(c) if 0 <= c < V else np.float32(-np.inf)
    rank = int(np.count_nonzero(s64 >= s64[top]))
    return out_ids, out_val, rank


def stash_converged_logprobs(logits: np.ndarray, canvas_len: int, src, slots, keep, valid,
                             temps, num_topk: int, num_token_ids, token_ids,
                             out_ids: np.ndarray, out_logprobs: np.ndarray,
                             out_ranks: np.ndarray, logits_mode: bool) -> None:
    """Writes the stash rows of the kept requests into the given arrays.

    logits: [rows, vocab] fp32 (any row stride). out_ids / out_logprobs:
    [n_slots, positions, width]; out_ranks: [n_slots, positions]. Cells of
    requests not kept, and positions at or past valid[j], are left as they
    are. token_ids is None or [m, ids_stride] int32.
    """
    m = len(slots)
    width = out_logprobs.shape[-1]
    assert num_topk + 1 <= width
    for j in range(m):
        if not keep[j]:
            continue
        n = min(max(int(valid[j]), 0), canvas_len)
        tc = clamp_temp(temps[j])
        ids = None
        if token_ids is not None and int(num_token_ids[j]) > 0:
            cnt = min(int(num_token_ids[j]), width - 1, token_ids.shape[1])
            ids = [int(c) for c in token_ids[j, :cnt]]
        for p in range(n):
            row = int(src[j]) * canvas_len + p
            s = (logits[row].astype(np.float32) / tc).astype(np.float32)
            oi, ov, rank = stash_row_layout(s, num_topk, ids, width, logits_mode)
            out_ids[slots[j], p] = oi
            out_logprobs[slots[j], p] = ov
            out_ranks[slots[j], p] = rank
