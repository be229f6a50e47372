"""Comparison rules between the HIP path and the oracle.

Codes (E4M3 x / h, bf16 h): >= 99.9% equal by value (+0 == -0) and never
more than one code step apart on the monotone code rank.  x codes and x
scales are decided in fp32 on both sides from identical inputs, so they must
be bit-exact.  h scales: relative difference <= SH_RTOL (the kernel's fp32 h
at the row maximum against the exact one: fp32 sums of exact products, then
about eight roundings of 2^-24 in the scale products, the SiLU's exponential
and reciprocal and the product with U; measured at most 3.3e-7 over the
parity cases).  y: normwise relative error <= 2e-3 and max abs error
<= 1e-2 * max|y_ref|.
"""

import numpy as np

from oracle.formats import bf16_to_f64

Y_NORM_TOL = 2e-3
Y_MAX_TOL = 1e-2
CODE_EQ_MIN = 0.999
SH_RTOL = 2e-6


def e4m3_rank(c):
    c = np.asarray(c, dtype=np.int32)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def bf16_rank(b):
    b = np.asarray(b, dtype=np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def check_codes(got, ref, rank, what, near_zero_ok=None):
    """>= 99.9% equal, and at most one step apart except where near_zero_ok
    (a boolean mask) marks a difference that is tiny on the row's scale.
    The entries so excused are counted among the unequal ones (so they too
    stay within the 0.1% budget) and their number is printed."""
    rg, rr = rank(got), rank(ref)
    eq = np.mean(rg == rr) if rg.size else 1.0
    far = np.abs(rg - rr) > 1
    excused = 0
    if near_zero_ok is not None:
        excused = int(np.sum(far & near_zero_ok))
        far &= ~near_zero_ok
    print("%s: %.5f%% equal, %d more than one step apart but excused as near zero (of %d)"
          % (what, 100 * eq, excused, rg.size))
    assert eq >= CODE_EQ_MIN, "%s: only %.5f%% of codes equal" % (what, 100 * eq)
    assert excused <= (1 - CODE_EQ_MIN) * rg.size, "%s: %d near-zero exceptions" % (what, excused)
    if np.any(far):
        i = tuple(np.argwhere(far)[0])
        raise AssertionError("%s: %d codes more than one step apart, e.g. at %s: got %#x ref %#x"
                             % (what, int(far.sum()), i, int(got[i]), int(ref[i])))
    return eq


def bf16_near_zero(got, ref):
    """bf16 has no per-row scale: for |h| near zero (cancellation in the
    sums) fp32 accumulation error spans several ulps.  A difference counts as
    near zero when it is below 2^-16 of the row's largest |h|."""
    g, r = bf16_to_f64(got), bf16_to_f64(ref)
    rowmax = np.max(np.abs(r), axis=-1, keepdims=True)
    return np.abs(g - r) <= rowmax * 2.0 ** -16


def check_y(y_bits, y_ref_bits, what="y", strict=True):
    """Normwise and max-abs errors of y against y_ref (asserted unless
    strict is False, which only measures them)."""
    y = bf16_to_f64(y_bits)
    yr = bf16_to_f64(y_ref_bits)
    nref = np.linalg.norm(yr)
    err = np.linalg.norm(y - yr)
    rel = err / nref if nref > 0 else err
    mx = np.max(np.abs(y - yr)) if y.size else 0.0
    mref = np.max(np.abs(yr)) if yr.size else 0.0
    if strict:
        assert rel <= Y_NORM_TOL, "%s: normwise relative error %.3e" % (what, rel)
        assert mx <= Y_MAX_TOL * mref, "%s: max abs error %.3e vs %.3e" % (what, mx, mref)
    return rel, mx / mref if mref > 0 else 0.0
