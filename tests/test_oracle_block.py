"""Pins for the oracle's block forward and weight packing (CPU only).

The block has no worked example in the pages, so the oracle is pinned by
(1) lossless special cases: inputs and weights chosen on the quantization
grids (x rows = E4M3 values * 2^k with a +-448 in each row, weight rows likewise,
NVFP4 weights = E2M1 * E4M3 block scale * 2^-12) make every quantization step
exact, so G, U and the down projection must equal the textbook SiLU-gated MLP
computed here with numpy matmuls, torch's SiLU and torch's FP8 / bf16 casts;
(2) invariants of the definition (scale rule, zero rows, power-of-two row
scaling, row independence); (3) the error bound of round-to-nearest.
"""

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import mlp as O
from quantized_memory_bound_amd import inputs as I


# ------------------------------------------------------------------ helpers

def _grid_rows(rng, n, k, exps):
    """n x k values E4M3 * 2^e_row, each row holding one +-448 (so the row's
    scale is exactly 2^e_row and its codes are the chosen codes)."""
    codes = rng.integers(0, 0x7F, size=(n, k)).astype(np.uint8)      # 0..126, no NaN
    codes |= (rng.integers(0, 2, size=(n, k)) * 0x80).astype(np.uint8)
    pos = rng.integers(0, k, size=n)
    codes[np.arange(n), pos] = np.where(rng.integers(0, 2, n) > 0, 0x7E, 0xFE)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    e = rng.choice(exps, size=n)
    return codes, e, vals * np.exp2(e)[:, None]


def _bf16_bits_exact(v):
    t = torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16)
    assert np.array_equal(t.to(torch.float64).numpy(), np.asarray(v, np.float64))
    return t.view(torch.int16).numpy().view(np.uint16)


def _torch_e4m3_codes(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_e4m3_values(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _agree_up_to_binary32_ties(got, ref, exact):
    """got: values the oracle decided from the exact values `exact`; ref: a
    library's decision on their float32 rounding.  They may differ only
    where that rounding moved a value onto or across a midpoint, so a
    differing entry of got must be at least as near to the exact value."""
    diff = got != ref
    assert np.all(np.abs(got[diff] - exact[diff]) <= np.abs(ref[diff] - exact[diff]))
    assert np.mean(diff) <= 1e-3


def _silu_torch(g):
    return torch.nn.functional.silu(torch.from_numpy(g)).numpy()


def _lossless_setup(seed, M=5, H=64, Iw=48):
    rng = np.random.default_rng(seed)
    xc, xe, x = _grid_rows(rng, M, H, np.arange(-6, 1))
    gc, ge, wg = _grid_rows(rng, Iw, H, np.arange(-16, -10))
    uc, ue, wu = _grid_rows(rng, Iw, H, np.arange(-16, -10))
    x_bits = _bf16_bits_exact(x)
    return rng, dict(x=x, x_bits=x_bits, xc=xc, xe=xe, wg=wg.astype(np.float32), gc=gc, ge=ge,
                     wu=wu.astype(np.float32), uc=uc, ue=ue)


# ------------------------------------------------------------------ lossless special cases

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_lossless_fp8_block_equals_textbook_mlp(seed):
    rng, d = _lossless_setup(seed)
    H = d["x"].shape[1]
    dc, de, wd = _grid_rows(rng, H, d["wg"].shape[0], np.arange(-16, -10))
    packed = O.pack_block(d["wg"], d["wu"], wd.astype(np.float32), O.PREC_FP8)
    # packing recovers the chosen codes and the power-of-two scales exactly
    assert np.array_equal(packed["gate"][0], d["gc"]) and np.array_equal(packed["gate"][1], np.exp2(d["ge"]))
    assert np.array_equal(packed["up"][0], d["uc"]) and np.array_equal(packed["up"][1], np.exp2(d["ue"]))
    assert np.array_equal(packed["down"][0], dc) and np.array_equal(packed["down"][1], np.exp2(de))

    out = O.forward(d["x_bits"], packed)
    assert np.array_equal(out["xq"], d["xc"]) and np.array_equal(out["sx"], np.exp2(d["xe"]))
    # gate/up: textbook x W^T (every step exact on these grids)
    G = d["x"] @ d["wg"].astype(np.float64).T
    U = d["x"] @ d["wu"].astype(np.float64).T
    h = _silu_torch(G) * U
    np.testing.assert_allclose(out["h"], h, rtol=1e-13, atol=0)
    # requant of the exact h: scale = fl32(amax/448); codes by torch's own E4M3
    # cast, which rounds through float32 and may differ only where that
    # rounding decides a near-tie (there the oracle's code must be the nearer)
    sh = (np.max(np.abs(h), axis=1) / 448.0).astype(np.float32)
    assert np.array_equal(out["sh"], sh)
    q = h / sh[:, None].astype(np.float64)
    _agree_up_to_binary32_ties(F.dec_e4m3(out["hq"]), _torch_e4m3_values(_torch_e4m3_codes(q)), q)
    # down: textbook (dequantized h) W_d^T, W_d exact on its grid
    Y = (_torch_e4m3_values(out["hq"]) * sh[:, None].astype(np.float64)) @ wd.T
    np.testing.assert_allclose(out["Y"], Y, rtol=1e-13, atol=1e-300)
    yb = torch.from_numpy(Y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.mean(out["y"] != yb) <= 1e-3      # torch rounds fp64 -> bf16 via fp32 (rare double rounding)


@pytest.mark.parametrize("seed", [3, 4])
def test_lossless_bf16_down_equals_textbook(seed):
    rng, d = _lossless_setup(seed)
    H, Iw = d["x"].shape[1], d["wg"].shape[0]
    wd = torch.from_numpy(rng.standard_normal((H, Iw)).astype(np.float32) * 0.05).to(torch.bfloat16)
    wd = wd.to(torch.float32).numpy()                       # exactly bf16-valued
    out = O.block_reference(d["x_bits"], d["wg"], d["wu"], wd, O.PREC_FP8_DOWN_BF16)
    G = d["x"] @ d["wg"].astype(np.float64).T
    U = d["x"] @ d["wu"].astype(np.float64).T
    h = _silu_torch(G) * U
    np.testing.assert_allclose(out["h"], h, rtol=1e-13)
    # bf16(h) rounded once from the exact h; torch rounds through float32
    hb_t = torch.from_numpy(h.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    _agree_up_to_binary32_ties(F.bf16_to_f64(out["hb"]), hb_t, h)
    Y = F.bf16_to_f64(out["hb"]) @ wd.astype(np.float64).T
    np.testing.assert_allclose(out["Y"], Y, rtol=1e-13, atol=1e-300)


def _fp4_grid_weight(rng, n, k, S_exp=-12):
    """W = e2m1 * dec(sb) * 2^S_exp with one +-6 per 16-block and one block
    scale 448, so S = 2^S_exp and every code is recovered exactly."""
    nb = k // 16
    sb = rng.integers(0x30, 0x7F, size=(n, nb)).astype(np.uint8)      # normal E4M3 scales
    sb[0, 0] = 0x7E
    q = rng.integers(0, 16, size=(n, k)).astype(np.uint8)
    slot = rng.integers(0, 16, size=(n, nb))
    rows, blks = np.meshgrid(np.arange(n), np.arange(nb), indexing="ij")
    q[rows, blks * 16 + slot] = np.where(rng.integers(0, 2, (n, nb)) > 0, 0x7, 0xF)
    vals = F.E2M1[q] * np.repeat(_torch_e4m3_values(sb), 16, axis=1) * 2.0 ** S_exp
    return q, sb, vals


@pytest.mark.parametrize("seed", [5, 6])
def test_lossless_nvfp4_block(seed):
    rng, d = _lossless_setup(seed, H=64, Iw=32)
    H, Iw = 64, 32
    qg, sbg, wg = _fp4_grid_weight(rng, Iw, H)
    qu, sbu, wu = _fp4_grid_weight(rng, Iw, H)
    qd, sbd, wd = _fp4_grid_weight(rng, H, Iw)
    for q, sb, w in ((qg, sbg, wg), (qu, sbu, wu), (qd, sbd, wd)):
        codes, sbo, S = O.pack_nvfp4(w.astype(np.float32))
        assert S == np.float32(2.0 ** -12)
        assert np.array_equal(sbo, sb)
        # +-0 codes may differ only in sign of zero; compare values
        assert np.array_equal(F.E2M1[codes], F.E2M1[q])
    out = O.block_reference(d["x_bits"], wg.astype(np.float32), wu.astype(np.float32),
                            wd.astype(np.float32), O.PREC_FP4)
    G = d["x"] @ wg.T
    U = d["x"] @ wu.T
    np.testing.assert_allclose(out["h"], _silu_torch(G) * U, rtol=1e-13)
    sh = out["sh"].astype(np.float64)
    Y = (_torch_e4m3_values(out["hq"]) * sh[:, None]) @ wd.T
    np.testing.assert_allclose(out["Y"], Y, rtol=1e-13, atol=1e-300)


# ------------------------------------------------------------------ invariants on workload inputs

@pytest.fixture(scope="module")
def tiny():
    d = I.workload_inputs("tiny_fp8")
    return d


@pytest.mark.parametrize("prec", [O.PREC_FP8, O.PREC_FP8_DOWN_BF16, O.PREC_FP4])
def test_scale_rule_max_code_448(tiny, prec):
    packed = O.pack_block(tiny["w_gate"], tiny["w_up"], tiny["w_down"], prec)
    out = O.forward(tiny["x_bits"], packed)
    for codes in [out["xq"]] + ([out["hq"]] if "hq" in out else []):
        mx = np.max(np.abs(F.dec_e4m3(codes)), axis=1)
        assert np.all(mx == 448.0)
    if prec != O.PREC_FP4:
        for codes, s in (packed["gate"], packed["up"]):
            assert np.all(np.max(np.abs(F.dec_e4m3(codes)), axis=1) == 448.0)
    else:
        for codes, sb, S in (packed["gate"], packed["up"], packed["down"]):
            assert np.all(np.abs(F.dec_e2m1(codes)) <= 6.0)
            assert np.max(F.dec_e4m3(sb)) == 448.0


def test_nvfp4_tensor_scale_and_nearest(tiny):
    w = tiny["w_gate"]
    codes, sb, S = O.pack_nvfp4(w)
    amax = np.float64(np.max(np.abs(w)))
    assert abs(np.float64(S) * 2688.0 - amax) <= amax * 2.0 ** -23
    # every element is the nearest E2M1 grid point at its block's scale
    d = np.repeat(F.dec_e4m3(sb), 16, axis=1) * np.float64(S)
    deq = F.dec_e2m1(codes) * d
    grid = F.E2M1[:8][None, None, :] * d[:, :, None]
    err_best = np.min(np.abs(np.abs(w.astype(np.float64))[:, :, None] - grid), axis=2)
    assert np.all(np.abs(deq - w) <= err_best * (1 + 1e-6) + 1e-30)


def test_fp8_weight_nearest(tiny):
    w = tiny["w_up"]
    codes, s = O.pack_fp8(w)
    deq = F.dec_e4m3(codes) * s[:, None].astype(np.float64)
    # error never exceeds half the E4M3 spacing at the value (relative 2^-4, or 2^-10 * s absolute)
    err = np.abs(deq - w)
    bound = np.maximum(np.abs(w) * 2.0 ** -4, 2.0 ** -10 * s[:, None]) * (1 + 1e-6)
    assert np.all(err <= bound)


def test_zero_row_and_power_of_two_row_scaling(tiny):
    x = tiny["x_bits"].copy()
    x[1] = 0
    xf = F.bf16_to_f64(x)
    xf[2] = xf[2] * 2.0 ** 5                     # exact in bf16
    x2 = _bf16_bits_exact(xf)
    for prec in (O.PREC_FP8, O.PREC_FP8_DOWN_BF16, O.PREC_FP4):
        packed = O.pack_block(tiny["w_gate"], tiny["w_up"], tiny["w_down"], prec)
        a = O.forward(tiny["x_bits"], packed)
        b = O.forward(x2, packed)
        assert b["sx"][1] == 0 and np.all(b["xq"][1] == 0)
        assert np.all(F.bf16_to_f64(b["y"][1]) == 0)
        assert np.array_equal(b["xq"][2], a["xq"][2]) and b["sx"][2] == a["sx"][2] * 32
        assert np.array_equal(b["y"][0], a["y"][0]) and np.array_equal(b["y"][3], a["y"][3])


def test_row_independence():
    d = I.make_inputs(256, 512, 52, x_outliers=True, w_std=0.02, seed=7)
    for prec in (O.PREC_FP8, O.PREC_FP8_DOWN_BF16, O.PREC_FP4):
        packed = O.pack_block(d["w_gate"], d["w_up"], d["w_down"], prec)
        full = O.forward(d["x_bits"], packed)
        part = O.forward(d["x_bits"][:13], packed)
        for key in ("xq", "sx", "y") + (("hb",) if prec == O.PREC_FP8_DOWN_BF16 else ("hq", "sh")):
            assert np.array_equal(full[key][:13], part[key]), (prec, key)


def test_up_projection_is_linear_gate_is_not(tiny):
    # doubling W_up doubles h exactly (same codes, scales x2), hence same hq and
    # sh x2 and y x2; doubling W_gate does not (SiLU is applied to the gate only).
    p1 = O.pack_block(tiny["w_gate"], tiny["w_up"], tiny["w_down"], O.PREC_FP8)
    p2 = O.pack_block(tiny["w_gate"], tiny["w_up"] * 2, tiny["w_down"], O.PREC_FP8)
    p3 = O.pack_block(tiny["w_gate"] * 2, tiny["w_up"], tiny["w_down"], O.PREC_FP8)
    a, b, c = (O.forward(tiny["x_bits"], p) for p in (p1, p2, p3))
    assert np.array_equal(a["hq"], b["hq"]) and np.array_equal(b["sh"], a["sh"] * 2)
    assert np.array_equal(F.bf16_to_f64(b["y"]), 2 * F.bf16_to_f64(a["y"]))
    assert not np.array_equal(F.bf16_to_f64(c["y"]), 2 * F.bf16_to_f64(a["y"]))


def test_silu_identities():
    g = np.array([0.0, 1.0, -1.0, 3.5, -3.5, 40.0, -40.0, 800.0, -800.0])
    s = O.silu(g)
    assert s[0] == 0.0
    assert abs(s[1] - 1.0 / (1.0 + np.exp(-1.0))) < 1e-16
    np.testing.assert_allclose(s[1::2] - s[2::2], g[1::2], rtol=1e-15)   # silu(g) - silu(-g) = g
    assert s[7] == 800.0 and abs(s[8]) < 1e-300
    assert np.all(np.isfinite(s))


def test_quantized_block_close_to_unquantized_mlp(tiny):
    x = F.bf16_to_f64(tiny["x_bits"])
    wg, wu, wd = (tiny[k].astype(np.float64) for k in ("w_gate", "w_up", "w_down"))
    y_ref = (_silu_torch(x @ wg.T) * (x @ wu.T)) @ wd.T
    for prec, hi in ((O.PREC_FP8, 0.08), (O.PREC_FP8_DOWN_BF16, 0.06), (O.PREC_FP4, 0.3)):
        y = F.bf16_to_f64(O.block_reference(tiny["x_bits"], tiny["w_gate"], tiny["w_up"], tiny["w_down"], prec)["y"])
        rel = np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref)
        assert 1e-3 < rel < hi, (prec, rel)


def test_code_sums_exact_vs_rationals():
    # brute force: the fp64 code-domain sum equals the exact rational sum on a small case
    from fractions import Fraction
    rng = np.random.default_rng(9)
    a = rng.integers(0, 255, (3, 40)).astype(np.uint8)
    b = rng.integers(0, 255, (4, 40)).astype(np.uint8)
    a[a == 0x7F] = 0x7E
    b[b == 0x7F] = 0x7E
    a[a == 0xFF] = 0xFE
    b[b == 0xFF] = 0xFE
    got = F.dec_e4m3(a) @ F.dec_e4m3(b).T
    for i in range(3):
        for j in range(4):
            exact = sum(Fraction(float(F.E4M3[a[i, k]])) * Fraction(float(F.E4M3[b[j, k]])) for k in range(40))
            assert Fraction(float(got[i, j])) == exact


# ------------------------------------------------------------------ permutation invariances
#
# Relabelling channels must relabel the results and nothing else.  Hidden
# channels (x columns, gate/up weight columns, down weight rows) permute the
# x codes and the columns of y and leave h unchanged; intermediate channels
# (gate/up weight rows, down weight columns) permute h and its codes and
# leave y unchanged.  The code-domain sums are exact (E4M3 and E2M1 products
# in fp64), so the equalities are bit-exact.  NVFP4 permutes whole 16-input
# blocks, which keeps every block scale's inputs together.  A swapped or
# transposed operand, or a scale or maximum taken along the wrong axis,
# breaks these.

def _block_perm(rng, n, block):
    return (rng.permutation(n // block)[:, None] * block + np.arange(block)[None, :]).reshape(-1)


@pytest.mark.parametrize("prec", [O.PREC_FP8, O.PREC_FP8_DOWN_BF16, O.PREC_FP4])
def test_hidden_channel_permutation(prec):
    d = I.make_inputs(256, 384, 11, x_outliers=True, w_std=0.02, seed=31 + prec)
    rng = np.random.default_rng(5)
    p = _block_perm(rng, 256, 16 if prec == O.PREC_FP4 else 1)
    a = O.block_reference(d["x_bits"], d["w_gate"], d["w_up"], d["w_down"], prec)
    b = O.block_reference(np.ascontiguousarray(d["x_bits"][:, p]), np.ascontiguousarray(d["w_gate"][:, p]),
                          np.ascontiguousarray(d["w_up"][:, p]), np.ascontiguousarray(d["w_down"][p, :]), prec)
    assert np.array_equal(b["xq"], a["xq"][:, p]) and np.array_equal(b["sx"], a["sx"])
    for key in ("hb",) if prec == O.PREC_FP8_DOWN_BF16 else ("hq", "sh"):
        assert np.array_equal(b[key], a[key]), key
    assert np.array_equal(b["y"], a["y"][:, p])


@pytest.mark.parametrize("prec", [O.PREC_FP8, O.PREC_FP8_DOWN_BF16, O.PREC_FP4])
def test_intermediate_channel_permutation(prec):
    d = I.make_inputs(256, 384, 11, x_outliers=True, w_std=0.02, seed=37 + prec)
    rng = np.random.default_rng(6)
    p = _block_perm(rng, 384, 16 if prec == O.PREC_FP4 else 1)
    a = O.block_reference(d["x_bits"], d["w_gate"], d["w_up"], d["w_down"], prec)
    b = O.block_reference(d["x_bits"], np.ascontiguousarray(d["w_gate"][p, :]), np.ascontiguousarray(d["w_up"][p, :]),
                          np.ascontiguousarray(d["w_down"][:, p]), prec)
    assert np.array_equal(b["xq"], a["xq"]) and np.array_equal(b["sx"], a["sx"])
    if prec == O.PREC_FP8_DOWN_BF16:
        assert np.array_equal(b["hb"], a["hb"][:, p])
    else:
        assert np.array_equal(b["hq"], a["hq"][:, p]) and np.array_equal(b["sh"], a["sh"])
    assert np.array_equal(b["y"], a["y"])


# ------------------------------------------------------------------ h requantization from fp64

def test_h_requant_decides_on_fp64_values(golden):
    """The requantization of h takes its codes from the exact fp64 h (hand-
    derived cases 2^-40 off an E4M3 midpoint, where a binary32 rounding of h
    would land on the tie and round to the even code instead)."""
    from conftest import parse_num
    rows = golden("h_requant_fp64_cases.txt")
    vals = np.array([parse_num(v) for v, _, _ in rows])
    want = np.array([int(c, 16) for _, c, _ in rows], dtype=np.uint8)
    assert np.all(vals.astype(np.float32).astype(np.float64) != vals)     # none is a binary32 value
    h = np.concatenate([[448.0], vals])[None, :]
    codes, sh = O.quantize_h_e4m3(h)
    assert sh[0] == np.float32(1.0)
    assert codes[0, 0] == 0x7E
    for (v, _, why), got, exp in zip(rows, codes[0, 1:], want):
        assert got == exp, "%s: got %#x want %#x (%s)" % (v, got, exp, why)


def test_h_requant_scale_rule_and_zero_row():
    # the row maximum is taken on fp64 |h| and the scale stored as float32;
    # a zero row (and a row of -0) gets scale 0 and +0 codes
    h = np.array([[0.0, -0.0, 0.0], [3.0, -7.0, 1.0], [-0.0, -0.0, -0.0]])
    codes, sh = O.quantize_h_e4m3(h)
    assert sh[0] == 0 and sh[2] == 0 and np.all(codes[[0, 2]] == 0)
    assert sh[1] == np.float32(7.0 / 448.0)
    assert codes[1, 1] == 0xFE                          # -amax -> -448 (exact saturation)
    q = np.array([3.0, 1.0]) / np.float64(sh[1])
    assert np.array_equal(codes[1, [0, 2]], F.enc_e4m3(q))


def test_bf16_h_rounds_fp64_directly():
    # bf16(h) in the BF16-down mode is one rounding of the fp64 h: a value
    # 2^-40 above the 1 / 1+2^-7 midpoint goes up; a binary32 rounding first
    # would make it the tie, which goes to the even 1.0
    v = np.array([1.0 + 2.0 ** -8 + 2.0 ** -40, 1.0 + 2.0 ** -8])
    assert np.array_equal(F.rne_bf16(v), np.array([0x3F81, 0x3F80], dtype=np.uint16))
    assert np.array_equal(F.rne_bf16(v.astype(np.float32).astype(np.float64)),
                          np.array([0x3F80, 0x3F80], dtype=np.uint16))


def _tie_block():
    """A 5-input, 3-intermediate block built by hand so that h lands 2^-34
    (relative) past a bf16 and an E4M3 midpoint.  Every x row and weight
    row holds a 448, so every scale is 1 and every code is its value.

      x codes       [448, 256, 16, 2^-9, 0]
      gate rows     [0, 256, 16, 2^-9, 448]  -> G0 = 65536 + 256 + 2^-18
                    [0, 256, 256, 2^-9, 448] -> G1 = 65536 + 4096 + 2^-18
                    [256, 0, 0, 0, 448]      -> G2 = 448 * 256 = 114688
      up rows       [0, 0, 2^-4, 0, 448]     -> U = 16 * 2^-4 = 1 (all three)
    G >= 40, so SiLU(G) = G exactly in fp64, and h = G.
    """
    x = np.array([[448.0, 256.0, 16.0, 2.0 ** -9, 0.0]])
    wg = np.array([[0, 256, 16, 2.0 ** -9, 448], [0, 256, 256, 2.0 ** -9, 448], [256, 0, 0, 0, 448]], np.float32)
    wu = np.tile(np.array([[0, 0, 2.0 ** -4, 0, 448]], np.float32), (3, 1))
    wd = np.eye(5, 3, dtype=np.float32)
    return _bf16_bits_exact(x), wg, wu, wd


def test_tie_block_bf16_h():
    # h0 = 2^16 (1 + 2^-8 + 2^-34): just above the bf16 midpoint of 65536
    # (0x4780) and 66048 (0x4781) -> 0x4781; its float32 rounding (65792) is
    # the tie itself, which would go to the even 0x4780
    x_bits, wg, wu, wd = _tie_block()
    out = O.block_reference(x_bits, wg, wu, wd, O.PREC_FP8_DOWN_BF16)
    assert out["h"][0, 0] == 65792.0 + 2.0 ** -18
    assert list(out["hb"][0]) == [0x4781, 0x4788, 0x47E0]


def test_tie_block_e4m3_h():
    # sh = fl32(114688 / 448) = 256; h1 / sh = 272 + 2^-26, just above the
    # E4M3 midpoint of 256 (0x78) and 288 (0x79) -> 0x79 (float32 would tie
    # to the even 0x78); h0 / sh = 257 + 2^-26 -> 256 (0x78); h2 / sh = 448
    x_bits, wg, wu, wd = _tie_block()
    out = O.block_reference(x_bits, wg, wu, wd, O.PREC_FP8)
    assert out["sh"][0] == np.float32(256.0)
    assert list(out["hq"][0]) == [0x78, 0x79, 0x7E]


# ------------------------------------------------------------------ brute force on 8 x 8 outputs
#
# The projection step (code-domain sum, then the token and column scales)
# against exact rational arithmetic written out as loops over every output
# and input: for E4M3 x E4M3 and E4M3 x (E2M1 x E4M3 block scale) operands
# the fp64 sums are exact, so only the two scale multiplications round (at
# most one unit in the last place each).  A transposed operand, a scale on
# the wrong axis or a dropped block scale breaks these.

@pytest.mark.parametrize("kind", ["fp8", "fp4"])
def test_projection_brute_force_8x8(kind):
    from fractions import Fraction
    rng = np.random.default_rng(21 if kind == "fp8" else 22)
    T, N, K = 8, 8, 32                     # two 16-input NVFP4 blocks per row
    a = rng.integers(0, 255, (T, K)).astype(np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x7E           # no NaN codes
    sa = (rng.random(T) * 0.01 + 1e-4).astype(np.float32)
    if kind == "fp8":
        wc = rng.integers(0, 255, (N, K)).astype(np.uint8)
        wc[(wc & 0x7F) == 0x7F] = 0x7E
        sw = (rng.random(N) * 0.01 + 1e-4).astype(np.float32)
        packed = (wc, sw)
        wval = lambda n, k: Fraction(float(F.E4M3[wc[n, k]]))
        col = lambda n: Fraction(float(sw[n]))
    else:
        wc = rng.integers(0, 16, (N, K)).astype(np.uint8)
        sb = rng.integers(0x08, 0x70, (N, K // 16)).astype(np.uint8)   # positive normal E4M3 block scales
        S = np.float32(0.00123)
        packed = (wc, sb, S)
        wval = lambda n, k: Fraction(float(F.E2M1[wc[n, k]])) * Fraction(float(F.E4M3[sb[n, k // 16]]))
        col = lambda n: Fraction(float(S))
    got = O._projection(F.dec_e4m3(a), sa, packed, kind)
    assert got.shape == (T, N)
    for t in range(T):
        for n in range(N):
            exact = sum(Fraction(float(F.E4M3[a[t, k]])) * wval(n, k) for k in range(K))
            exact *= Fraction(float(sa[t])) * col(n)
            ref = float(exact)
            assert abs(got[t, n] - ref) <= 2 * 2.0 ** -52 * abs(ref) + 1e-300, (t, n, got[t, n], ref)
