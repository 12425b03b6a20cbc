"""CPU oracle for the row-statistics sampler and the top-K logprobs.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline may import this package; the product path (the HIP library and its
Python binding) never does, and shares no code with it.

Semantics follow the vLLM API page "diffusion_gemma_sampler" (module
docstring; ``sample_row_stats`` and ``sample_row_stats_reference``;
``stash_converged_logprobs`` and the ``_lp_topk_kernel`` docstring). The
arithmetic lives in ``rowstats_oracle.c`` (plain C, fp32 divide then double
reductions); this module marshals numpy arrays through ctypes, and
``selfcond`` multiplies the oracle's bf16 probabilities by an embedding table
with a float64 matrix product (``probs_product``, which also serves given
probabilities).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

PROBS_NONE, PROBS_BF16, PROBS_FP16 = 0, 1, 2

_i64p = ctypes.POINTER(ctypes.c_int64)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_u8p = ctypes.POINTER(ctypes.c_uint8)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # ROWSTATS_ORACLE_LIB lets the mutation test load a deliberately broken
    # copy of the oracle and check that the pins reject it
    path = os.environ.get("ROWSTATS_ORACLE_LIB") or _build.ensure_built()
    lib = ctypes.CDLL(path)
    lib.oracle_philox4x32_10.argtypes = [_u32p, _u32p, _u32p]
    lib.oracle_philox4x32_10.restype = None
    lib.oracle_uniform_gumbel.argtypes = [ctypes.c_uint32, _f64p, _f64p]
    lib.oracle_uniform_gumbel.restype = None
    lib.oracle_noise_word.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64]
    lib.oracle_noise_word.restype = ctypes.c_uint32
    lib.oracle_scale_row.argtypes = [_f32p, ctypes.c_int64, ctypes.c_float, _f32p]
    lib.oracle_scale_row.restype = None
    lib.oracle_bf16_bits.argtypes = [ctypes.c_double]
    lib.oracle_bf16_bits.restype = ctypes.c_uint16
    lib.oracle_fp16_bits.argtypes = [ctypes.c_double]
    lib.oracle_fp16_bits.restype = ctypes.c_uint16
    lib.oracle_rowstats.argtypes = [
        _f32p, ctypes.c_int64, ctypes.c_int64, _i64p, ctypes.c_int64, _f32p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_uint64, ctypes.c_int,
        _i64p, _i64p, _f64p, _f64p, _f64p, _u16p]
    lib.oracle_rowstats.restype = ctypes.c_int
    lib.oracle_topk_logprobs.argtypes = [
        _f32p, ctypes.c_int64, ctypes.c_int64, _i64p, ctypes.c_int64, _f32p,
        ctypes.c_int64, ctypes.c_int64, _u8p, ctypes.c_int32, _f32p, _i64p]
    lib.oracle_topk_logprobs.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray, typ):
    return a.ctypes.data_as(typ)


def num_threads() -> int:
    """OpenMP threads the oracle runs its row loop on."""
    return int(_load().oracle_num_threads())


def philox4x32_10(ctr, key) -> np.ndarray:
    """One Philox4x32-10 block: counter of 4 words, key of 2 words -> 4 words."""
    lib = _load()
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib.oracle_philox4x32_10(_ptr(c, _u32p), _ptr(k, _u32p), _ptr(out, _u32p))
    return out


def noise_word(seed: int, row: int, col: int) -> int:
    """The 32-bit Philox word that the noise of (seed, row, col) comes from."""
    return int(_load().oracle_noise_word(seed, row, col))


def uniform_gumbel(w: int) -> tuple[float, float]:
    """(u, g) for one 32-bit word: u = (w + 0.5) 2^-32, g = -log(-log u)."""
    u = ctypes.c_double()
    g = ctypes.c_double()
    _load().oracle_uniform_gumbel(w, ctypes.byref(u), ctypes.byref(g))
    return u.value, g.value


def scale_row(x: np.ndarray, t: float) -> np.ndarray:
    """x / clamp(t, 1e-10) as one fp32 division per element."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty_like(x)
    _load().oracle_scale_row(_ptr(x, _f32p), x.size, t, _ptr(out, _f32p))
    return out


def bf16_bits(p: float) -> int:
    return int(_load().oracle_bf16_bits(p))


def fp16_bits(p: float) -> int:
    return int(_load().oracle_fp16_bits(p))


def _rows_view(logits: np.ndarray):
    if logits.dtype != np.float32 or logits.ndim != 2:
        raise ValueError("logits must be a 2-D float32 array")
    if logits.strides[1] != 4:
        raise ValueError("logits must have unit column stride")
    # a single row may carry any stride on its (unused) row axis
    ld = logits.strides[0] // 4 if logits.shape[0] > 1 else logits.shape[1]
    if ld < logits.shape[1] or logits.strides[0] % 4:
        raise ValueError("logits rows must not overlap")
    return logits, ld


def rowstats(logits: np.ndarray, row_ids, temps, canvas_len: int, seed: int,
             probs_dtype: int = PROBS_NONE) -> dict:
    """Row statistics of the given rows.

    ``logits[i]`` holds global row ``row_ids[i]`` (its temperature slot is
    ``row_ids[i] // canvas_len`` and its noise stream is that row index).
    Returns a dict with ``argmax``, ``sample`` (int64), ``entropy`` and
    ``entropy_plogp`` (float64), ``gap`` (top-two perturbed-score gap,
    +inf on greedy rows) and ``probs`` (uint16 bf16/fp16 bit patterns, or
    None).
    """
    lib = _load()
    x, ld = _rows_view(logits)
    n, vocab = x.shape
    rid = np.ascontiguousarray(row_ids, dtype=np.int64)
    if rid.shape != (n,):
        raise ValueError("row_ids must have one entry per logits row")
    tp = np.ascontiguousarray(temps, dtype=np.float32)
    out = {
        "argmax": np.zeros(n, np.int64),
        "sample": np.zeros(n, np.int64),
        "entropy": np.zeros(n, np.float64),
        "entropy_plogp": np.zeros(n, np.float64),
        "gap": np.zeros(n, np.float64),
    }
    probs = np.zeros((n, vocab), np.uint16) if probs_dtype else None
    xbase = x.ctypes.data_as(_f32p)
    rc = lib.oracle_rowstats(
        xbase, ld, n, _ptr(rid, _i64p), vocab, _ptr(tp, _f32p), tp.size,
        canvas_len, ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF), probs_dtype,
        _ptr(out["argmax"], _i64p), _ptr(out["sample"], _i64p),
        _ptr(out["entropy"], _f64p), _ptr(out["entropy_plogp"], _f64p),
        _ptr(out["gap"], _f64p),
        _ptr(probs, _u16p) if probs is not None else None)
    if rc != 0:
        raise RuntimeError(f"oracle_rowstats failed with code {rc}")
    out["probs"] = probs
    return out


def topk_logprobs(logits: np.ndarray, row_ids, temps, canvas_len: int,
                  keep_mask, K: int, out_vals: np.ndarray | None = None,
                  out_idx: np.ndarray | None = None):
    """Top-K logprobs of the kept rows (full sort by value desc, index asc).

    Rows whose slot is not kept are left as they are in ``out_vals`` /
    ``out_idx`` (zeros when those are not given).
    """
    lib = _load()
    x, ld = _rows_view(logits)
    n, vocab = x.shape
    rid = np.ascontiguousarray(row_ids, dtype=np.int64)
    tp = np.ascontiguousarray(temps, dtype=np.float32)
    km = np.ascontiguousarray(keep_mask, dtype=np.uint8)
    if out_vals is None:
        out_vals = np.zeros((n, K), np.float32)
    if out_idx is None:
        out_idx = np.zeros((n, K), np.int64)
    assert out_vals.flags.c_contiguous and out_idx.flags.c_contiguous
    rc = lib.oracle_topk_logprobs(
        x.ctypes.data_as(_f32p), ld, n, _ptr(rid, _i64p), vocab, _ptr(tp, _f32p),
        tp.size, canvas_len, _ptr(km, _u8p), K, _ptr(out_vals, _f32p),
        _ptr(out_idx, _i64p))
    if rc != 0:
        raise RuntimeError(f"oracle_topk_logprobs failed with code {rc}")
    return out_vals, out_idx


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(
        np.float64)


def fp16_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE half bit patterns (uint16) -> float64 values (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def selfcond(logits: np.ndarray, row_ids, temps, canvas_len: int, embed_bits: np.ndarray,
             block: int = 16384, dtype: int = PROBS_BF16) -> np.ndarray:
    """Self-conditioning input of the given rows (diffusion_gemma_sampler page,
    module docstring: the softmax in the model dtype feeds the self-conditioning
    matmul): out[i, :] = sum_c q_i[c] * E[c, :], where q_i are this oracle's
    probabilities of row ``row_ids[i]`` rounded once to the model dtype
    (``rowstats`` with PROBS_BF16 or PROBS_FP16, ``dtype``) and
    ``embed_bits`` is E as bit patterns of the same dtype [vocab, d]. Products
    and sums in float64, the vocab taken ``block`` columns at a time (a
    float64 matrix product per block).
    """
    if dtype not in (PROBS_BF16, PROBS_FP16):
        raise ValueError("dtype must be PROBS_BF16 or PROBS_FP16")
    ref = rowstats(logits, row_ids, temps, canvas_len, 0, dtype)
    return probs_product(ref["probs"], embed_bits, block, dtype)


def probs_product(probs_bits: np.ndarray, embed_bits: np.ndarray, block: int = 16384,
                  dtype: int = PROBS_BF16) -> np.ndarray:
    """The self-conditioning matmul of given probabilities (diffusion_gemma_sampler
    page, module docstring: the model-dtype softmax times the embedding
    table): out[i, :] = sum_c q[i, c] * E[c, :] with ``probs_bits`` q
    [rows, vocab] and ``embed_bits`` E [vocab, d], both bit patterns of the
    model dtype (bf16 for PROBS_BF16, fp16 for PROBS_FP16). Products and sums
    in float64, ``block`` vocabulary rows at a time (a float64 matrix product
    per block)."""
    if dtype not in (PROBS_BF16, PROBS_FP16):
        raise ValueError("dtype must be PROBS_BF16 or PROBS_FP16")
    to_f64 = bf16_to_f64 if dtype == PROBS_BF16 else fp16_to_f64
    p = to_f64(np.asarray(probs_bits))
    vocab, d = embed_bits.shape
    if vocab != p.shape[1]:
        raise ValueError("embed must have one row per probability column")
    out = np.zeros((p.shape[0], d), np.float64)
    for c0 in range(0, vocab, block):
        out += p[:, c0:c0 + block] @ to_f64(embed_bits[c0:c0 + block])
    return out
