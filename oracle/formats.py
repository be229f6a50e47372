"""Number formats used by the block: OCP FP8 E4M3, OCP FP4 E2M1 and bfloat16.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The post ("OCRia 推理栈：单卡 B200 提速近 10 倍", section "Reducing the data
moved: workload-aware quantization") only names the precisions it mixes
(BF16, FP8, NVFP4).  The bit-level definitions here are the public ones:

* E4M3 (OCP 8-bit Floating Point Specification, the "FN" variant): sign bit,
  4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
  subnormals m/8 * 2^-6; S.1111.111 is NaN; no infinities; largest finite
  value 448.
* E2M1 (OCP Microscaling Formats v1.0, FP4 element type): sign bit, 2 exponent
  bits with bias 1, 1 mantissa bit; magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}.
* bfloat16: the upper 16 bits of an IEEE binary32.

Encoding is "nearest representable value, ties to the even code, saturating
at the largest finite magnitude, sign taken from the input's sign bit" --
the plainest reading of round-to-nearest-even for a saturating conversion.
The encoders are table searches over the decoded code values, not bit
tricks, so they can be checked against the closed-form tables by eye.
"""

import numpy as np

# ----------------------------------------------------------------------------
# decode tables (closed form, one entry per code)
# ----------------------------------------------------------------------------


def e4m3_value(code):
    """Value of one E4M3 code (OCP FP8 E4M3FN), from its fields."""
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = (m / 8.0) * 2.0 ** -6          # subnormal
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


def e2m1_value(code):
    """Value of one E2M1 code (OCP MX FP4), from its fields."""
    s = (code >> 3) & 1
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        mag = m * 0.5                          # subnormal: 0 or 0.5
    else:
        mag = (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return -mag if s else mag


E4M3 = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)

E4M3_MAX = 448.0
E2M1_MAX = 6.0

# non-negative magnitudes in code order; codes 0..126 (E4M3) and 0..7 (E2M1)
# are increasing in value, so the code of a magnitude is its table index.
_E4M3_POS = E4M3[0:127].copy()
_E2M1_POS = E2M1[0:8].copy()


def _encode_nearest(v, table, sign_code):
    """Nearest table entry to |v| (ties -> even code), sign from v's sign bit.

    `table` holds the non-negative values of codes 0..n-1 in increasing
    order.  Magnitudes above the last entry saturate to it.  For both formats
    the neighbours of a magnitude lie within a factor of two of each other,
    so the two distances below are exact in fp64 and a tie is detected
    exactly.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    n = len(table)
    hi = np.searchsorted(table, a, side="left")        # table[hi-1] < a <= table[hi]
    hi_c = np.clip(hi, 1, n - 1)
    lo_c = hi_c - 1
    d_lo = a - table[lo_c]
    d_hi = table[hi_c] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi_c % 2 == 0))
    mag = np.where(pick_hi, hi_c, lo_c)
    mag = np.where(hi == 0, 0, mag)                    # a == 0
    mag = np.where(hi >= n, n - 1, mag)                # saturate
    code = mag.astype(np.uint8) | np.where(np.signbit(v), sign_code, 0).astype(np.uint8)
    return code.astype(np.uint8)


def enc_e4m3(v):
    """Round values to E4M3 codes (nearest, ties to even, saturate at 448)."""
    return _encode_nearest(v, _E4M3_POS, 0x80)


def enc_e2m1(v):
    """Round values to E2M1 codes (nearest, ties to even, saturate at 6)."""
    return _encode_nearest(v, _E2M1_POS, 0x8)


def dec_e4m3(codes):
    return E4M3[np.asarray(codes, dtype=np.uint8)]


def dec_e2m1(codes):
    return E2M1[np.asarray(codes, dtype=np.uint8) & 0xF]


# ----------------------------------------------------------------------------
# bfloat16
# ----------------------------------------------------------------------------


def bf16_to_f64(bits):
    """bfloat16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def rne_bf16(v):
    """Round float64 values directly to bfloat16 (8 significant bits, ties to
    even, no intermediate binary32 rounding); returns uint16 bit patterns.

    The value is split as m * 2^e with 0.5 <= |m| < 1, the quantum of the
    bfloat16 grid at that binade is 2^(e-8) (2^-133 below the normal range),
    and np.rint rounds the exact multiple count half-to-even.
    """
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    exp_q = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(v, -exp_q)), exp_q)  # exact: power-of-two scaling
    with np.errstate(over="ignore"):
        r32 = r.astype(np.float32)                      # exact (<= 8 significant bits)
    return (r32.view(np.uint32) >> 16).astype(np.uint16)
