"""Pins for the oracle's number formats (CPU only).

Each check ties the oracle to something other than itself: the closed-form
field definitions, hand-derived rounding tables (tests/golden), exhaustive
nearest-value search with exact rational arithmetic, and torch's own FP8 /
bfloat16 conversions (a separate implementation of the same public formats).
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import parse_num, read_golden
from oracle import formats as F


# ---------------------------------------------------------------- E4M3 table

def test_e4m3_spot_values():
    assert F.E4M3[0x7E] == 448.0
    assert F.E4M3[0xFE] == -448.0
    assert F.E4M3[0x38] == 1.0
    assert F.E4M3[0x08] == 2.0 ** -6       # smallest normal
    assert F.E4M3[0x01] == 2.0 ** -9       # smallest subnormal
    assert F.E4M3[0x07] == 7 * 2.0 ** -9   # largest subnormal
    assert F.E4M3[0x00] == 0.0 and not np.signbit(F.E4M3[0x00])
    assert F.E4M3[0x80] == 0.0 and np.signbit(F.E4M3[0x80])
    assert np.isnan(F.E4M3[0x7F]) and np.isnan(F.E4M3[0xFF])
    assert np.sum(np.isnan(F.E4M3)) == 2


def test_e4m3_table_matches_torch_decode():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ref) & np.isnan(F.E4M3)
    assert np.all(both_nan | (ref == F.E4M3))
    assert np.array_equal(np.signbit(ref[~both_nan]), np.signbit(F.E4M3[~both_nan]))


def test_e4m3_monotone_positive_codes():
    pos = F.E4M3[:127]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(F.E4M3[128:255], -pos)


def test_e4m3_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(F.enc_e4m3(F.E4M3[codes]), codes)


def test_e4m3_golden_ties():
    for val, code, why in read_golden("e4m3_rne_cases.txt"):
        got = int(F.enc_e4m3(np.array([parse_num(val)]))[0])
        assert got == int(code, 16), (val, code, why, hex(got))


def _brute_nearest(v, table_codes, table):
    """Exhaustive nearest value with exact rationals; ties -> even code;
    the sign follows v (so a zero result keeps v's sign)."""
    a = Fraction(abs(v))
    best = None
    for c in table_codes:
        d = abs(Fraction(float(table[c])) - a)
        key = (d, c % 2, c)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_e4m3_encoder_vs_exhaustive_search():
    rng = np.random.default_rng(1)
    pos_codes = list(range(127))
    vals = list(rng.standard_normal(400) * 50.0)
    vals += list(rng.uniform(-2 ** -5, 2 ** -5, 200))            # subnormal region
    mids = (F.E4M3[:126] + F.E4M3[1:127]) / 2                      # every exact midpoint
    vals += list(mids) + list(-mids)
    vals += [500.0, -470.0, 448.0001, 447.99]
    vals = np.array(vals)
    got = F.enc_e4m3(vals)
    for v, g in zip(vals, got):
        mag = min(_brute_nearest(v, pos_codes, F.E4M3), 126) if abs(v) <= 448 else 126
        exp = mag | (0x80 if np.signbit(v) else 0)
        assert g == exp, (v, hex(g), hex(exp))


def test_e4m3_encoder_matches_torch_below_464():
    # torch's float32 -> float8_e4m3fn cast is round-to-nearest-even but not
    # saturating (500 -> NaN), so it is a cross-check only for |v| < 464.
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 100,
                        rng.uniform(-460, 460, 20000).astype(np.float32),
                        rng.uniform(-0.02, 0.02, 20000).astype(np.float32)])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.enc_e4m3(v.astype(np.float64)), ref)


# ---------------------------------------------------------------- E2M1 table

def test_e2m1_values_and_roundtrip():
    assert list(F.E2M1[:8]) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert np.array_equal(F.E2M1[8:], -F.E2M1[:8])
    assert np.signbit(F.E2M1[8])
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(F.enc_e2m1(F.E2M1[codes]), codes)


def test_e2m1_golden_ties():
    for val, code, why in read_golden("e2m1_rne_cases.txt"):
        got = int(F.enc_e2m1(np.array([parse_num(val)]))[0])
        assert got == int(code, 16), (val, code, why, got)


def test_e2m1_encoder_vs_exhaustive_search():
    rng = np.random.default_rng(3)
    vals = np.concatenate([rng.uniform(-7, 7, 2000), (F.E2M1[:7] + F.E2M1[1:8]) / 2])
    got = F.enc_e2m1(vals)
    for v, g in zip(vals, got):
        mag = _brute_nearest(v, list(range(8)), F.E2M1) if abs(v) <= 6 else 7
        assert g == (mag | (0x8 if np.signbit(v) else 0)), (v, g)


# ---------------------------------------------------------------- bfloat16

def test_bf16_golden_direct_rounding():
    for val, bits, why in read_golden("bf16_rne_cases.txt"):
        got = int(F.rne_bf16(np.array([parse_num(val)]))[0])
        assert got == int(bits, 16), (val, bits, why, hex(got))


def test_bf16_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(4)
    v = np.concatenate([rng.standard_normal(50000).astype(np.float32) * 3,
                        (rng.standard_normal(5000) * 1e-39).astype(np.float32),   # fp32 subnormals
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -0.0, 0.0], np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.rne_bf16(v.astype(np.float64)), ref)


def test_bf16_exact_rational_rounding():
    # direct fp64 rounding against exact rational rounding on random fp64 inputs
    rng = np.random.default_rng(5)
    v = rng.standard_normal(3000) * np.exp2(rng.integers(-20, 20, 3000))
    got = F.rne_bf16(v)
    back = F.bf16_to_f64(got)
    for x, b in zip(v, back):
        e = np.frexp(x)[1]
        q = Fraction(2) ** (int(e) - 8)
        r = Fraction(float(x)) / q
        n = int(r)                      # truncation toward zero
        frac = abs(r - n)
        if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and n % 2 == 1):
            n += 1 if r > 0 else -1
        assert Fraction(float(b)) == n * q, (x, b)


def test_bf16_decode():
    bits = np.array([0x3F80, 0xBF80, 0x7F7F, 0x0001, 0x8000], dtype=np.uint16)
    exp = [1.0, -1.0, float.fromhex("0x1.fep127"), 2.0 ** -133, -0.0]
    got = F.bf16_to_f64(bits)
    assert list(got) == exp and np.signbit(got[-1])
