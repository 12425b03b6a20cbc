"""Python binding of librowstats (HIP, gfx950): one-pass row statistics and
top-K logprobs for the DiffusionGemma denoise sampler (vLLM API page
"diffusion_gemma_sampler": ``sample_row_stats`` and
``stash_converged_logprobs``).

This module only marshals torch tensors (device memory) and torch's current
HIP stream into the C ABI declared in ``include/rowstats.h``; every step of
the computation runs in the library's kernels. There is no fallback: if the
library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import atexit
import ctypes
import dataclasses
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librowstats.so")

ROWSTATS_OK = 0
STATUS_NAMES = {
    -1: "ROWSTATS_ERR_NULL", -2: "ROWSTATS_ERR_SHAPE", -3: "ROWSTATS_ERR_K",
    -4: "ROWSTATS_ERR_DTYPE", -5: "ROWSTATS_ERR_HIP", -6: "ROWSTATS_ERR_COOP",
    -7: "ROWSTATS_ERR_DEVICE", -8: "ROWSTATS_ERR_SCRATCH",
}
PROBS_CODES = {None: 0, torch.bfloat16: 1, torch.float16: 2}

# Entry points declared in include/rowstats.h, with their ctypes signatures.
_SIGNATURES = {
    "rowstats_run": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "rowstats_run_noalloc": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "rowstats_selfcond": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "rowstats_packed_embed_bytes": (ctypes.c_int64, [ctypes.c_int64, ctypes.c_int64]),
    "rowstats_pack_embed": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
        ctypes.c_void_p]),
    "rowstats_selfcond_product": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]),
    "topk_logprobs": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p]),
    "stash_converged_logprobs": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]),
    "rowstats_last_error": (ctypes.c_char_p, []),
    "rowstats_check_device": (ctypes.c_int, [ctypes.c_void_p]),
    "rowstats_release": (ctypes.c_int, []),
}

_lib = None


class RowStatsError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what} failed: {STATUS_NAMES.get(code, code)}: {last_error()}")


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python row_softmax_statistics_amd/build.py`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
        atexit.register(_release_at_exit)
    return _lib


def _release_at_exit():
    """Frees the library's scratch before the interpreter (and the HIP
    runtime under it) shuts down, once queued work has finished."""
    if _lib is None or not torch.cuda.is_initialized():
        return
    try:
        torch.cuda.synchronize()
        _lib.rowstats_release()
    except Exception:
        pass


def last_error() -> str:
    msg = lib().rowstats_last_error()
    return msg.decode() if msg else ""


def _check(code: int, what: str):
    if code != ROWSTATS_OK:
        raise RowStatsError(code, what)


def _stream_ptr(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def _check_logits(logits: torch.Tensor):
    if logits.dim() != 2 or logits.dtype != torch.float32:
        raise ValueError("logits must be a 2-D float32 tensor")
    if not logits.is_cuda:
        raise ValueError("logits must be on the GPU")
    if logits.shape[0] > 0 and logits.shape[1] > 0 and logits.stride(1) != 1:
        raise ValueError("logits must have unit column stride")


def _check_out(t: torch.Tensor, name: str, shape, dtype, device):
    if (not isinstance(t, torch.Tensor) or t.dtype != dtype or t.device != device
            or tuple(t.shape) != tuple(shape) or not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} "
                         f"on {device}")


def _check_temps(temps: torch.Tensor, rows: int, canvas_len: int, device):
    if temps.dtype != torch.float32 or temps.device != device or not temps.is_contiguous():
        raise ValueError("temps must be a contiguous float32 tensor on the logits' device")
    if canvas_len < 1:
        raise ValueError("canvas_len must be >= 1")
    if rows > 0 and temps.numel() < (rows + canvas_len - 1) // canvas_len:
        raise ValueError("temps needs ceil(rows / canvas_len) entries")


def _rowstats_call(entry: str, logits, temps, canvas_len, seed, probs_dtype, out):
    _check_logits(logits)
    if probs_dtype not in PROBS_CODES:
        raise ValueError("probs_dtype must be None, torch.bfloat16 or torch.float16")
    rows, vocab = logits.shape
    dev = logits.device
    _check_temps(temps, rows, canvas_len, dev)
    if out is None:
        argmax = torch.empty(rows, dtype=torch.int64, device=dev)
        sample = torch.empty(rows, dtype=torch.int64, device=dev)
        entropy = torch.empty(rows, dtype=torch.float32, device=dev)
        probs = (torch.empty(rows, vocab, dtype=probs_dtype, device=dev)
                 if probs_dtype is not None else None)
    else:
        argmax, sample, entropy, probs = out
        _check_out(argmax, "argmax", (rows,), torch.int64, dev)
        _check_out(sample, "sample", (rows,), torch.int64, dev)
        _check_out(entropy, "entropy", (rows,), torch.float32, dev)
        if probs_dtype is not None:
            _check_out(probs, "probs", (rows, vocab), probs_dtype, dev)
        elif probs is not None:
            raise ValueError("probs must be None when probs_dtype is None")
    rc = getattr(lib(), entry)(
        _ptr(logits), logits.stride(0) if rows > 1 else vocab, rows, vocab, _ptr(temps),
        canvas_len, ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF), PROBS_CODES[probs_dtype],
        _ptr(argmax), _ptr(sample), _ptr(entropy), _ptr(probs), _stream_ptr(dev))
    _check(rc, entry)
    return argmax, sample, entropy, probs


def sample_row_stats(logits: torch.Tensor, temps: torch.Tensor, canvas_len: int, seed: int,
                     probs_dtype: torch.dtype | None = None, *, out=None):
    """Per row of temperature-scaled logits: the argmax, one Gumbel-max draw,
    the softmax entropy and, if ``probs_dtype`` is given, the softmax.

    Row ``i`` of ``logits`` ([rows, vocab] fp32, unit column stride, any row
    stride) uses temperature ``temps[i // canvas_len]``; a temperature <= 0 is
    greedy. Returns ``(argmax int64, sample int64, entropy fp32,
    probs [rows, vocab] in probs_dtype or None)``. ``out`` may pass
    preallocated ``(argmax, sample, entropy, probs)`` tensors.
    """
    return _rowstats_call("rowstats_run", logits, temps, canvas_len, seed, probs_dtype, out)


def sample_row_stats_noalloc(logits: torch.Tensor, temps: torch.Tensor, canvas_len: int,
                             seed: int, probs_dtype: torch.dtype | None, out):
    """``sample_row_stats`` through the allocation-free entry point: the
    caller passes every output in ``out``; the library uses its fixed
    per-GPU scratch array (see rowstats_run_noalloc in include/rowstats.h)."""
    if out is None:
        raise ValueError("the allocation-free call needs preallocated outputs")
    return _rowstats_call("rowstats_run_noalloc", logits, temps, canvas_len, seed, probs_dtype,
                          out)


def selfcond_embed(logits: torch.Tensor, temps: torch.Tensor, canvas_len: int, seed: int,
                   embed: torch.Tensor, *, out=None):
    """The row statistics (as ``sample_row_stats`` without probs) and the
    self-conditioning input: each row's softmax in the model dtype times
    ``embed`` ([vocab, d] in bfloat16 or float16, which sets that dtype; d a
    multiple of 256), accumulated in fp32, computed without writing the
    probabilities.

    Returns ``(argmax int64, sample int64, entropy fp32, out fp32 [rows, d])``.
    ``out`` may pass preallocated ``(argmax, sample, entropy, out)``.
    """
    _check_logits(logits)
    rows, vocab = logits.shape
    dev = logits.device
    _check_temps(temps, rows, canvas_len, dev)
    if (embed.dtype not in (torch.bfloat16, torch.float16) or embed.device != dev
            or embed.dim() != 2 or embed.shape[0] != vocab or not embed.is_contiguous()):
        raise ValueError("embed must be a contiguous bfloat16 or float16 [vocab, d] tensor on "
                         "the logits' device")
    d = embed.shape[1]
    if out is None:
        out = (torch.empty(rows, dtype=torch.int64, device=dev),
               torch.empty(rows, dtype=torch.int64, device=dev),
               torch.empty(rows, dtype=torch.float32, device=dev),
               torch.empty(rows, d, dtype=torch.float32, device=dev))
    argmax, sample, entropy, res = out
    _check_out(argmax, "argmax", (rows,), torch.int64, dev)
    _check_out(sample, "sample", (rows,), torch.int64, dev)
    _check_out(entropy, "entropy", (rows,), torch.float32, dev)
    _check_out(res, "out", (rows, d), torch.float32, dev)
    rc = lib().rowstats_selfcond(
        _ptr(logits), logits.stride(0) if rows > 1 else vocab, rows, vocab, _ptr(temps),
        canvas_len, ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF), PROBS_CODES[embed.dtype],
        _ptr(embed), d, _ptr(argmax), _ptr(sample), _ptr(entropy), _ptr(res), _stream_ptr(dev))
    _check(rc, "rowstats_selfcond")
    return argmax, sample, entropy, res


@dataclasses.dataclass(frozen=True)
class PackedEmbed:
    """An embedding table in the matrix-core order of
    ``rowstats_pack_embed`` (``data``: uint8 device bytes)."""
    data: torch.Tensor
    vocab: int
    d: int
    dtype: torch.dtype


def pack_embed(embed: torch.Tensor) -> PackedEmbed:
    """Packs ``embed`` ([vocab, d] bfloat16 or float16, d a multiple of 256)
    for ``selfcond_product``; done once per table."""
    if (embed.dtype not in (torch.bfloat16, torch.float16) or not embed.is_cuda
            or embed.dim() != 2 or not embed.is_contiguous()):
        raise ValueError("embed must be a contiguous bfloat16 or float16 [vocab, d] GPU tensor")
    vocab, d = embed.shape
    nbytes = lib().rowstats_packed_embed_bytes(vocab, d)
    _check(int(nbytes) if nbytes < 0 else ROWSTATS_OK, "rowstats_packed_embed_bytes")
    data = torch.empty(nbytes, dtype=torch.uint8, device=embed.device)
    rc = lib().rowstats_pack_embed(_ptr(embed), vocab, d, PROBS_CODES[embed.dtype], _ptr(data),
                                   _stream_ptr(embed.device))
    _check(rc, "rowstats_pack_embed")
    return PackedEmbed(data, vocab, d, embed.dtype)


def selfcond_product(probs: torch.Tensor, packed: PackedEmbed, *, out=None) -> torch.Tensor:
    """The self-conditioning input from given probabilities: ``probs``
    ([rows, vocab] in the packed table's dtype, unit column stride) times the
    packed embedding table, accumulated in fp32. Returns ``out`` fp32
    [rows, d] (``out`` may pass it preallocated)."""
    if (probs.dim() != 2 or probs.dtype != packed.dtype or probs.device != packed.data.device
            or probs.shape[1] != packed.vocab):
        raise ValueError("probs must be a 2-D tensor of the packed table's dtype, device and "
                         "vocab")
    rows, vocab = probs.shape
    if rows > 0 and probs.stride(1) != 1:
        raise ValueError("probs must have unit column stride")
    dev = probs.device
    if out is None:
        out = torch.empty(rows, packed.d, dtype=torch.float32, device=dev)
    _check_out(out, "out", (rows, packed.d), torch.float32, dev)
    rc = lib().rowstats_selfcond_product(
        _ptr(probs), probs.stride(0) if rows > 1 else vocab, rows, vocab,
        PROBS_CODES[probs.dtype], _ptr(packed.data), packed.d, _ptr(out), _stream_ptr(dev))
    _check(rc, "rowstats_selfcond_product")
    return out


def topk_logprobs(logits: torch.Tensor, temps: torch.Tensor, canvas_len: int,
                  keep_mask: torch.Tensor, K: int, out_vals: torch.Tensor | None = None,
                  out_idx: torch.Tensor | None = None):
    """For the rows of kept slots: the K largest scaled logits as logprobs, in
    descending order with equal values ordered by column.

    Rows of slots with ``keep_mask[slot] == 0`` are not written. Returns
    ``(out_vals fp32 [rows, K], out_idx int64 [rows, K])``.
    """
    _check_logits(logits)
    rows, vocab = logits.shape
    dev = logits.device
    _check_temps(temps, rows, canvas_len, dev)
    slots = (rows + canvas_len - 1) // canvas_len
    if (keep_mask.dtype not in (torch.uint8, torch.bool) or keep_mask.device != dev
            or keep_mask.dim() != 1 or keep_mask.numel() < slots):
        raise ValueError("keep_mask must be a 1-D uint8/bool tensor of ceil(rows / canvas_len) "
                         "entries on the logits' device")
    keep_mask = keep_mask.contiguous()
    if out_vals is None:
        out_vals = torch.empty(rows, K, dtype=torch.float32, device=dev)
    if out_idx is None:
        out_idx = torch.empty(rows, K, dtype=torch.int64, device=dev)
    _check_out(out_vals, "out_vals", (rows, K), torch.float32, dev)
    _check_out(out_idx, "out_idx", (rows, K), torch.int64, dev)
    rc = lib().topk_logprobs(
        _ptr(logits), logits.stride(0) if rows > 1 else vocab, rows, vocab, _ptr(temps),
        canvas_len, _ptr(keep_mask), int(K), _ptr(out_vals), _ptr(out_idx), _stream_ptr(dev))
    _check(rc, "topk_logprobs")
    return out_vals, out_idx


def _gpu_vec(t: torch.Tensor, dtype, name: str, m: int):
    if t.dtype != dtype or not t.is_cuda or t.dim() != 1 or t.numel() < m:
        raise ValueError(f"{name} must be a 1-D {dtype} GPU tensor of at least {m} entries")
    return t.contiguous()


def stash_converged_logprobs(logits: torch.Tensor, canvas_len: int, src: torch.Tensor,
                             slots: torch.Tensor, keep: torch.Tensor, valid: torch.Tensor,
                             temps: torch.Tensor, num_topk: int,
                             num_token_ids: torch.Tensor | None,
                             token_ids: torch.Tensor | None, out_ids: torch.Tensor,
                             out_logprobs: torch.Tensor, out_ranks: torch.Tensor,
                             logits_mode: bool) -> None:
    """Fills the stash rows of the kept requests (argument order of the
    page's launcher).

    The rows of request ``j`` are ``src[j] * canvas_len + p`` for positions
    ``p < valid[j]``, scaled by ``1 / temps[j]``. For a kept request (``keep[j]``)
    position ``p`` fills ``out_*[slots[j], p]`` with the argmax first, then
    either the request's own token ids (when ``num_token_ids[j] > 0``) or its
    ``num_topk`` largest columns, and token 0 at -inf in the remaining cells. ``src``, ``slots``, ``valid``, ``num_token_ids``,
    ``token_ids``, ``out_ids`` and ``out_ranks`` are int32; ``out_ids`` and
    ``out_logprobs`` are ``[slots, positions, width]``, ``out_ranks``
    ``[slots, positions]``, all contiguous.
    """
    _check_logits(logits)
    m = int(slots.numel())
    src = _gpu_vec(src, torch.int32, "src", m)
    slots = _gpu_vec(slots, torch.int32, "slots", m)
    valid = _gpu_vec(valid, torch.int32, "valid", m)
    temps = _gpu_vec(temps, torch.float32, "temps", m)
    if keep.dtype not in (torch.uint8, torch.bool) or not keep.is_cuda or keep.numel() < m:
        raise ValueError("keep must be a uint8/bool GPU tensor of m entries")
    keep = keep.contiguous()
    ids_stride = 0
    if token_ids is not None:
        num_token_ids = _gpu_vec(num_token_ids, torch.int32, "num_token_ids", m)
        if token_ids.dtype != torch.int32 or not token_ids.is_cuda or token_ids.dim() != 2:
            raise ValueError("token_ids must be a 2-D int32 GPU tensor")
        if token_ids.shape[0] < m or token_ids.shape[1] < 1:
            raise ValueError("token_ids needs a row of at least one id per request")
        if token_ids.stride(1) != 1:
            token_ids = token_ids.contiguous()
        ids_stride = token_ids.stride(0) if token_ids.shape[0] > 1 else token_ids.shape[1]
    if out_logprobs.dim() != 3 or out_ids.shape != out_logprobs.shape:
        raise ValueError("out_ids and out_logprobs must be [slots, positions, width]")
    if out_ranks.shape != out_logprobs.shape[:2]:
        raise ValueError("out_ranks must be [slots, positions]")
    if (out_ids.dtype != torch.int32 or out_logprobs.dtype != torch.float32
            or out_ranks.dtype != torch.int32):
        raise ValueError("out_ids / out_ranks must be int32 and out_logprobs float32")
    if not (out_ids.is_contiguous() and out_logprobs.is_contiguous()
            and out_ranks.is_contiguous()):
        raise ValueError("stash outputs must be contiguous")
    rows, vocab = logits.shape
    n_slots, positions, width = out_logprobs.shape
    dev = logits.device
    rc = lib().stash_converged_logprobs(
        _ptr(logits), logits.stride(0) if rows > 1 else vocab, rows, vocab, canvas_len, m,
        _ptr(src), _ptr(slots), _ptr(keep), _ptr(valid), _ptr(temps), int(num_topk),
        _ptr(num_token_ids if token_ids is not None else None), _ptr(token_ids), ids_stride,
        n_slots, positions, width, _ptr(out_ids), _ptr(out_logprobs), _ptr(out_ranks),
        1 if logits_mode else 0, _stream_ptr(dev))
    _check(rc, "stash_converged_logprobs")


def check_device(stream=None):
    """Synchronise and raise if a kernel flagged a failure (see rowstats.h)."""
    s = ctypes.c_void_p(stream.cuda_stream if stream is not None
                        else torch.cuda.current_stream().cuda_stream)
    _check(lib().rowstats_check_device(s), "rowstats_check_device")


def release():
    _check(lib().rowstats_release(), "rowstats_release")
