"""The kernels' temperature scale against IEEE fp32 division, on the host.

The kernels compute s = x / Tc (Tc = max(T, 1e-10f), one IEEE fp32 division
by the page's reading) as fl32(fl64(x) * fl64(1 / Tc)) and, on rows with
Tc >= 2, recompute results at or below 2^-126 in magnitude with the
double-double form fl32(fma(x, r_hi, fl64(x r_lo))) (the proof is written
beside the device code). These tests evaluate the same formulas in IEEE
fp64/fp32 arithmetic on the host (numpy, and tests/scale_check.c where a
fused multiply-add is needed) and compare them with fp32 division over every
input whose quotient can be subnormal, for temperatures on both sides of 2,
and over random inputs of every magnitude.
"""
import ctypes
import os
import subprocess
import tempfile

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker():
    out = os.path.join(tempfile.mkdtemp(prefix="scale_check"), "libscale_check.so")
    subprocess.run(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                    "-shared", "-o", out, os.path.join(HERE, "scale_check.c"), "-lm"], check=True)
    lib = ctypes.CDLL(out)
    lib.scale_mismatches.argtypes = [ctypes.c_float, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int]
    lib.scale_mismatches.restype = ctypes.c_long
    return lib

TINY = np.float32(2.0 ** -126)


def fast(x, t):
    return (x.astype(np.float64) * (1.0 / np.float64(t))).astype(np.float32)


FAST, DOUBLE_DOUBLE, KERNEL = 0, 1, 2


# Both formulas and the division are odd functions of x (rounding to nearest
# is symmetric), so positive inputs cover both signs.
def positive_floats(lo_bits, hi_bits, step=1 << 21):
    """Every positive fp32 with bit pattern in [lo_bits, hi_bits), in chunks."""
    for b in range(lo_bits, hi_bits, step):
        yield np.arange(b, min(hi_bits, b + step), dtype=np.uint32).view(np.float32)


def bits_of(v: float) -> int:
    return int(np.array([v], np.float32).view(np.uint32)[0])


# subnormals and the first normal binade: every x whose quotient is
# subnormal when Tc < 2
SMALL_BITS = (1, 0x01000000)


@pytest.mark.parametrize("t", [1e-10, 1e-3, 0.1, 0.37, 0.7, 1.0, 1.3, 1.5, 1.9999999])
def test_fast_form_is_ieee_below_two(t):
    tc = max(np.float32(t), np.float32(1e-10))
    for xs in positive_floats(*SMALL_BITS):
        assert np.array_equal(fast(xs, tc), xs / tc), t


@pytest.mark.parametrize("t", [2.0, 6.0, 98.0, 150.0, 364.0])
def test_kernel_form_is_ieee_from_two(checker, t):
    # every x whose quotient can be subnormal (x < 2^-126 t), and a margin
    hi = bits_of(2.0 ** -126 * t * 2)
    assert checker.scale_mismatches(t, 1, hi, KERNEL) == 0
    assert checker.scale_mismatches(t, 1, hi, DOUBLE_DOUBLE) == 0


@pytest.mark.parametrize("t", [1e-10, 0.37, 1.5, 936.0, 3.3e4, 1.7e9])
def test_double_double_form_is_ieee(checker, t):
    # the double-double form alone is exact too, at any temperature
    # (subnormal and first-binade inputs)
    assert checker.scale_mismatches(t, *SMALL_BITS, DOUBLE_DOUBLE) == 0


def test_fast_form_misses_midpoints_at_98(checker):
    # 147 2^-149 / 98 = 3 2^-150: ties to the even 2^-148, but fl64(1 / 98)
    # is below 1/98, so the product falls just under the midpoint
    x = np.array([147 * 2.0 ** -149], np.float32)
    t = np.float32(98.0)
    assert (x / t)[0] == np.float32(2.0 ** -148)
    assert fast(x, t)[0] == np.float32(2.0 ** -149)
    # and it is not a rare case at this temperature
    assert checker.scale_mismatches(98.0, 1, 1 << 23, FAST) == 19950


def test_every_magnitude_random():
    # normal results: the fast form is exact at any temperature
    rng = np.random.default_rng(5)
    bits = rng.integers(1, 0x7F7FFFFF, size=4_000_000, dtype=np.uint32)
    x = bits.view(np.float32) * np.where(rng.random(bits.size) < 0.5, -1, 1).astype(np.float32)
    for t in [1e-10, 0.013, 0.5, 0.7, 1.0, 1.5, 2.5, 98.0, 3.3e4, 1.7e9]:
        t32 = np.float32(t)
        with np.errstate(over="ignore", under="ignore"):
            ref = x / t32
            got = fast(x, t32)
        ok = np.isfinite(ref) & (np.abs(ref) > TINY)   # overflow is outside the contract
        assert np.array_equal(got[ok], ref[ok]), t
