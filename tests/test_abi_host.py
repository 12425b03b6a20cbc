"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every entry point include/rowstats.h declares,
and reject bad arguments with the documented status codes before it makes
any HIP call (so these run without a device). Contracts: include/rowstats.h.
"""
import ctypes
import os
import re

import pytest

import row_softmax_statistics_amd as rs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rowstats.h")


@pytest.fixture(scope="module", autouse=True)
def built_library():
    """The library under test: built in-tree first if a fresh checkout has
    none (hipcc cross-compiles for gfx950 without a GPU); skipped when it
    cannot be built here."""
    if not os.path.exists(rs.LIB_PATH):
        from row_softmax_statistics_amd import build
        try:
            build.build()
        except Exception as e:  # no hipcc in this environment
            pytest.skip(f"librowstats.so is not built and cannot be built here: {e}")
    return rs.lib()

OK, ERR_NULL, ERR_SHAPE, ERR_K, ERR_DTYPE = 0, -1, -2, -3, -4
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation
NULL = ctypes.c_void_p(0)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(["rowstats_run", "rowstats_run_noalloc",
                                           "rowstats_selfcond", "rowstats_packed_embed_bytes",
                                           "rowstats_pack_embed", "rowstats_selfcond_product",
                                           "topk_logprobs", "stash_converged_logprobs",
                                           "rowstats_last_error", "rowstats_check_device",
                                           "rowstats_release"])


def test_library_exports_every_declared_symbol():
    lib = rs.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    # the binding covers exactly the declared entry points
    assert sorted(rs._SIGNATURES) == declared_functions()


def run(logits=FAKE, stride=8, rows=4, vocab=8, temps=FAKE, canvas=2, seed=1, dtype=0,
        argmax=FAKE, sample=FAKE, entropy=FAKE, probs=NULL, entry="rowstats_run"):
    return getattr(rs.lib(), entry)(logits, stride, rows, vocab, temps, canvas, seed, dtype,
                                    argmax, sample, entropy, probs, NULL)


def topk(logits=FAKE, stride=8, rows=4, vocab=8, temps=FAKE, canvas=2, keep=FAKE, K=2,
         vals=FAKE, idx=FAKE):
    return rs.lib().topk_logprobs(logits, stride, rows, vocab, temps, canvas, keep, K, vals, idx,
                                  NULL)


@pytest.mark.parametrize("kwargs,code", [
    (dict(dtype=3), ERR_DTYPE),
    (dict(dtype=-1), ERR_DTYPE),
    (dict(rows=-1), ERR_SHAPE),
    (dict(rows=2**31), ERR_SHAPE),
    (dict(vocab=0), ERR_SHAPE),
    (dict(vocab=2**31), ERR_SHAPE),
    (dict(stride=7), ERR_SHAPE),
    (dict(canvas=0), ERR_SHAPE),
    (dict(logits=NULL), ERR_NULL),
    (dict(temps=NULL), ERR_NULL),
    (dict(argmax=NULL), ERR_NULL),
    (dict(sample=NULL), ERR_NULL),
    (dict(entropy=NULL), ERR_NULL),
    (dict(dtype=1, probs=NULL), ERR_NULL),
    (dict(dtype=2, probs=NULL), ERR_NULL),
])
@pytest.mark.parametrize("entry", ["rowstats_run", "rowstats_run_noalloc"])
def test_rowstats_run_rejects(kwargs, code, entry):
    assert run(entry=entry, **kwargs) == code
    assert rs.last_error() != ""


@pytest.mark.parametrize("entry", ["rowstats_run", "rowstats_run_noalloc"])
def test_rowstats_run_zero_rows_is_a_no_op(entry):
    # nothing is dereferenced and no HIP call is made
    assert run(rows=0, logits=NULL, temps=NULL, argmax=NULL, sample=NULL, entropy=NULL,
               entry=entry) == OK


@pytest.mark.parametrize("kwargs,code", [
    (dict(K=0), ERR_K),
    (dict(K=9), ERR_K),
    (dict(K=101, vocab=100, stride=100), ERR_K),
    (dict(rows=-2), ERR_SHAPE),
    (dict(rows=2**31), ERR_SHAPE),
    (dict(vocab=0), ERR_SHAPE),
    (dict(stride=3), ERR_SHAPE),
    (dict(canvas=0), ERR_SHAPE),
    (dict(keep=NULL), ERR_NULL),
    (dict(vals=NULL), ERR_NULL),
    (dict(idx=NULL), ERR_NULL),
    (dict(logits=NULL), ERR_NULL),
])
def test_topk_rejects(kwargs, code):
    assert topk(**kwargs) == code
    assert rs.last_error() != ""


def selfcond(logits=FAKE, stride=8, rows=4, vocab=8, temps=FAKE, canvas=2, seed=1, dtype=1,
             embed=FAKE, d=256, argmax=FAKE, sample=FAKE, entropy=FAKE, out=FAKE):
    return rs.lib().rowstats_selfcond(logits, stride, rows, vocab, temps, canvas, seed, dtype,
                                      embed, d, argmax, sample, entropy, out, NULL)


@pytest.mark.parametrize("kwargs,code", [
    (dict(rows=-1), ERR_SHAPE),
    (dict(vocab=0), ERR_SHAPE),
    (dict(stride=7), ERR_SHAPE),
    (dict(canvas=0), ERR_SHAPE),
    (dict(dtype=0), ERR_DTYPE),
    (dict(dtype=3), ERR_DTYPE),
    (dict(d=0), ERR_SHAPE),
    (dict(d=128), ERR_SHAPE),
    (dict(d=300), ERR_SHAPE),
    (dict(d=2 ** 21), ERR_SHAPE),
    (dict(embed=ctypes.c_void_p(0x1008)), ERR_SHAPE),   # not 16-byte aligned
    (dict(out=ctypes.c_void_p(0x1004)), ERR_SHAPE),
    (dict(logits=NULL), ERR_NULL),
    (dict(temps=NULL), ERR_NULL),
    (dict(embed=NULL), ERR_NULL),
    (dict(out=NULL), ERR_NULL),
    (dict(argmax=NULL), ERR_NULL),
])
def test_selfcond_rejects(kwargs, code):
    assert selfcond(**kwargs) == code
    assert rs.last_error() != ""


def test_selfcond_zero_rows_is_a_no_op():
    assert selfcond(rows=0, logits=NULL, temps=NULL, embed=NULL, out=NULL, argmax=NULL,
                    sample=NULL, entropy=NULL) == OK


def test_packed_embed_bytes():
    lib = rs.lib()
    # vocab rows padded to a multiple of 128, 2 bytes per element
    assert lib.rowstats_packed_embed_bytes(262144, 2560) == 262144 * 2560 * 2
    assert lib.rowstats_packed_embed_bytes(1, 256) == 128 * 256 * 2
    assert lib.rowstats_packed_embed_bytes(129, 512) == 256 * 512 * 2
    for vocab, d in ((0, 256), (2 ** 31, 256), (100, 0), (100, 128), (100, 300), (100, 2 ** 21)):
        assert lib.rowstats_packed_embed_bytes(vocab, d) == ERR_SHAPE
        assert rs.last_error() != ""


def pack(embed=FAKE, vocab=100, d=256, dtype=1, packed=FAKE):
    return rs.lib().rowstats_pack_embed(embed, vocab, d, dtype, packed, NULL)


@pytest.mark.parametrize("kwargs,code", [
    (dict(vocab=0), ERR_SHAPE),
    (dict(d=200), ERR_SHAPE),
    (dict(dtype=0), ERR_DTYPE),
    (dict(dtype=3), ERR_DTYPE),
    (dict(embed=NULL), ERR_NULL),
    (dict(packed=NULL), ERR_NULL),
    (dict(embed=ctypes.c_void_p(0x1001)), ERR_SHAPE),   # odd address
    (dict(packed=ctypes.c_void_p(0x1008)), ERR_SHAPE),  # not 16-byte aligned
])
def test_pack_embed_rejects(kwargs, code):
    assert pack(**kwargs) == code
    assert rs.last_error() != ""


def product(probs=FAKE, stride=8, rows=4, vocab=8, dtype=1, packed=FAKE, d=256, out=FAKE):
    return rs.lib().rowstats_selfcond_product(probs, stride, rows, vocab, dtype, packed, d, out,
                                              NULL)


@pytest.mark.parametrize("kwargs,code", [
    (dict(rows=-1), ERR_SHAPE),
    (dict(rows=2 ** 31), ERR_SHAPE),
    (dict(vocab=0), ERR_SHAPE),
    (dict(stride=7), ERR_SHAPE),
    (dict(d=128), ERR_SHAPE),
    (dict(d=2 ** 21), ERR_SHAPE),
    (dict(dtype=0), ERR_DTYPE),
    (dict(dtype=3), ERR_DTYPE),
    (dict(probs=NULL), ERR_NULL),
    (dict(packed=NULL), ERR_NULL),
    (dict(out=NULL), ERR_NULL),
    (dict(probs=ctypes.c_void_p(0x1001)), ERR_SHAPE),
    (dict(packed=ctypes.c_void_p(0x1004)), ERR_SHAPE),
    (dict(out=ctypes.c_void_p(0x1008)), ERR_SHAPE),
])
def test_selfcond_product_rejects(kwargs, code):
    assert product(**kwargs) == code
    assert rs.last_error() != ""


def test_selfcond_product_zero_rows_is_a_no_op():
    assert product(rows=0, probs=NULL, packed=NULL, out=NULL) == OK


def test_topk_zero_rows_is_a_no_op():
    assert topk(rows=0, logits=NULL, keep=NULL, vals=NULL, idx=NULL) == OK


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(2, 8)
    with pytest.raises(ValueError):
        rs.sample_row_stats(x, torch.ones(1), 2, 0)
    with pytest.raises(ValueError):
        rs.topk_logprobs(x, torch.ones(1), 2, torch.ones(1, dtype=torch.uint8), 2)
    with pytest.raises(ValueError):
        rs.sample_row_stats_noalloc(x, torch.ones(1), 2, 0, None, None)


def stash(logits=FAKE, stride=8, lrows=8, vocab=8, canvas=2, m=3, src=FAKE, slots=FAKE,
          keep=FAKE, valid=FAKE, temps=FAKE, K=2, nids=FAKE, ids=NULL, ids_stride=0,
          n_slots=4, positions=2, width=3, out_ids=FAKE, out_lp=FAKE, out_rk=FAKE, mode=0):
    return rs.lib().stash_converged_logprobs(
        logits, stride, lrows, vocab, canvas, m, src, slots, keep, valid, temps, K, nids, ids,
        ids_stride, n_slots, positions, width, out_ids, out_lp, out_rk, mode, NULL)


@pytest.mark.parametrize("kwargs,code", [
    (dict(m=-1), ERR_SHAPE),
    (dict(lrows=0), ERR_SHAPE),
    (dict(vocab=0), ERR_SHAPE),
    (dict(stride=7), ERR_SHAPE),
    (dict(canvas=0), ERR_SHAPE),
    (dict(m=2**30, canvas=4, positions=4), ERR_SHAPE),
    (dict(K=-1), ERR_K),
    (dict(K=9), ERR_K),
    (dict(K=101, vocab=100, stride=100, width=110), ERR_K),
    (dict(width=2), ERR_SHAPE),        # num_topk + 1 <= width
    (dict(K=65, vocab=100, stride=100, width=65), ERR_SHAPE),
    (dict(n_slots=0), ERR_SHAPE),
    (dict(positions=1), ERR_SHAPE),    # positions >= canvas_len
    (dict(logits=NULL), ERR_NULL),
    (dict(temps=NULL), ERR_NULL),
    (dict(src=NULL), ERR_NULL),
    (dict(slots=NULL), ERR_NULL),
    (dict(keep=NULL), ERR_NULL),
    (dict(valid=NULL), ERR_NULL),
    (dict(out_ids=NULL), ERR_NULL),
    (dict(out_lp=NULL), ERR_NULL),
    (dict(out_rk=NULL), ERR_NULL),
    (dict(ids=FAKE, nids=NULL, ids_stride=2), ERR_NULL),
    (dict(ids=FAKE, ids_stride=0), ERR_SHAPE),
])
def test_stash_rejects(kwargs, code):
    assert stash(**kwargs) == code
    assert rs.last_error() != ""


def test_stash_zero_requests_is_a_no_op():
    assert stash(m=0, logits=NULL, src=NULL, slots=NULL, keep=NULL, valid=NULL, temps=NULL,
                 out_ids=NULL, out_lp=NULL, out_rk=NULL) == OK
