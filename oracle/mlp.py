"""The quantized MLP block, written out as its plain definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, step by step, and the passage each step follows:

  pack      Weights are stored in fewer bytes: FP8 E4M3 with one fp32 scale per
            output channel, NVFP4 (E2M1 with one E4M3 scale per 16 inputs and
            one fp32 per-tensor scale), or BF16 for a layer kept at higher
            precision.  ("OCRia 推理栈：单卡 B200 提速近 10 倍", section
            "Reducing the data moved: workload-aware quantization": FP8 halves
            the bytes per weight; precision is mixed per layer across BF16,
            FP8 and NVFP4; sensitive layers stay at higher precision.)
  x-quant   Every row (token) of x is quantized to E4M3 with its own fp32
            scale amax/448 (per-token FP8 activations).  With a smoothed
            blob, x is first multiplied per channel by fl32(1/s[k]) (see
            pack_block and calibrate_smoothing).
  gate/up   G = x W_g^T and U = x W_u^T over all M rows at once: a verify pass
            covers every request's 1 + draft tokens, and the weights are read
            again on every step (section "Generate more tokens per target
            pass: speculative decoding").
  SiLU.up   h = SiLU(G) * U, then h is quantized per token to E4M3 right away
            (German page "Wie es funktioniert": SiLU activation and
            quantization fused so the intermediate never goes to HBM; same in
            the French "Comment cela fonctionne", Spanish "Cómo funciona" and
            Japanese "仕組み").
  down      Y = h W_d^T with the down weights in the precision chosen for that
            layer (FP8, BF16 or NVFP4); y = bf16(Y).

Readings where the pages are silent (all listed with the design notes):
  * scale = fl32(amax / 448); zero amax -> scale 0 and all codes +0.
  * the weights and x are binary32 values (bf16 x, fp32 weights); their codes
    are decided on the binary32 quotient fl32(value / scale), the true
    float32 division both the packer and the x quantization perform.
  * h is the exact (fp64) SiLU(G) * U: its row maximum, its scale and its
    codes E4M3(h / sh) are taken from the fp64 values with no binary32
    rounding in between, and bf16(h) is rounded directly from fp64.
  * scales apply after the integer-code sums (exact algebra for per-row and
    per-column scales); NVFP4 block scales apply inside the sum.
  * in the BF16-down mode h enters the down projection as bf16(h) with no
    FP8 requantization.
Accumulation is fp64; with E4M3/E2M1 operands every product and every partial
sum of the code-domain matmuls is exact in fp64, so the summation order of
the matmul library does not matter.
"""

import numpy as np

from .formats import (E2M1, E4M3, bf16_to_f64, dec_e4m3, enc_e2m1, enc_e4m3,
                      rne_bf16)

PREC_FP8 = 0            # gate/up FP8, down FP8
PREC_FP8_DOWN_BF16 = 1  # gate/up FP8, down BF16 (layer kept at higher precision)
PREC_FP4 = 2            # gate/up/down NVFP4

NVFP4_BLOCK = 16


def _f32(a):
    return np.asarray(a, dtype=np.float64).astype(np.float32)


# ----------------------------------------------------------------------------
# per-row E4M3 quantization (weights per output channel, x and h per token)
# ----------------------------------------------------------------------------


def quantize_rows_e4m3(a):
    """Per-row absmax E4M3 quantization of binary32 values (weights per
    output channel, x per token).

    a: 2-D array whose values are all exactly representable in binary32
    (fp32 weights; bf16 activations, possibly times a float32 multiplier).
    Returns (codes uint8 [R, C], scales float32 [R]) with
    scale = fl32(amax / 448) and codes = E4M3(fl32(value / scale)): the
    quotient is the correctly rounded float32 division of two float32 values.
    """
    a64 = np.asarray(a, dtype=np.float64)
    a32 = a64.astype(np.float32)
    assert np.array_equal(a32.astype(np.float64), a64, equal_nan=True), "values must be binary32"
    amax = np.max(np.abs(a32), axis=1) if a32.shape[1] else np.zeros(a32.shape[0], np.float32)
    scale = _f32(amax.astype(np.float64) / 448.0)
    codes = np.zeros(a32.shape, dtype=np.uint8)
    nz = scale > 0
    if np.any(nz):
        quot = _f32(a32[nz].astype(np.float64) / scale[nz, None].astype(np.float64))
        codes[nz] = enc_e4m3(quot)
    return codes, scale


def quantize_h_e4m3(h):
    """Per-token E4M3 requantization of the intermediate h (fp64 values).

    sh = fl32(max_n |h| / 448) (the scale is stored as float32); codes =
    E4M3(h / sh) with the quotient taken in fp64 from the fp64 h, so no
    binary32 rounding of h or of the quotient comes between the exact
    intermediate and its code.  A zero row gets sh = 0 and codes +0.
    """
    h = np.asarray(h, dtype=np.float64)
    amax = np.max(np.abs(h), axis=1) if h.shape[1] else np.zeros(h.shape[0])
    scale = _f32(amax / 448.0)
    codes = np.zeros(h.shape, dtype=np.uint8)
    nz = scale > 0
    if np.any(nz):
        codes[nz] = enc_e4m3(h[nz] / scale[nz, None].astype(np.float64))
    return codes, scale


# ----------------------------------------------------------------------------
# weight packing (quantization) -- "Reducing the data moved"
# ----------------------------------------------------------------------------


def pack_fp8(w):
    """FP8 E4M3 weights, one fp32 scale per output channel (row of [out, in])."""
    return quantize_rows_e4m3(w)


def pack_bf16(w):
    """BF16 weights (round to nearest even), bit patterns [out, in]."""
    return rne_bf16(np.asarray(w, dtype=np.float32).astype(np.float64))


def pack_nvfp4(w):
    """NVFP4 weights: E2M1 codes, one E4M3 scale per 16 consecutive inputs of
    each output row, one fp32 per-tensor scale.

      S          = fl32(amax(|W|) / (448 * 6))
      sb[n, j]   = E4M3(fl32(amax_j(|W[n, 16j:16j+16]|) / (6 S)))
      q[n, k]    = E2M1(fl32(W[n, k] / (dec(sb[n, k/16]) * S)))
    with codes 0 wherever S or the block scale is 0.
    Returns (codes uint8 [N, K] with one E2M1 code per byte, block scales
    uint8 [N, K/16], S float32).
    """
    w32 = np.asarray(w, dtype=np.float32)
    n, k = w32.shape
    assert k % NVFP4_BLOCK == 0
    amax = np.float32(np.max(np.abs(w32))) if w32.size else np.float32(0)
    S = np.float32(np.float64(amax) / (448.0 * 6.0))
    codes = np.zeros((n, k), dtype=np.uint8)
    sb = np.zeros((n, k // NVFP4_BLOCK), dtype=np.uint8)
    if S > 0:
        blocks = w32.reshape(n, k // NVFP4_BLOCK, NVFP4_BLOCK).astype(np.float64)
        amax_b = np.max(np.abs(blocks), axis=2)
        r = _f32(amax_b / (6.0 * np.float64(S)))
        sb = enc_e4m3(r)
        d = dec_e4m3(sb) * np.float64(S)                # exact product
        ok = d > 0
        quot = np.zeros_like(blocks)
        quot[ok] = blocks[ok] / d[ok][:, None]
        q = enc_e2m1(_f32(quot))
        q[~ok] = 0
        codes = q.reshape(n, k)
    return codes, sb, S


def calibrate_smoothing(x_calib_bits, w_gate, w_up, alpha=0.5):
    """Per-input-channel smoothing factors from calibration activations.

    The pages calibrate the quantization on the workload ("OCRia 推理栈：单卡
    B200 提速近 10 倍", section "Reducing the data moved: workload-aware
    quantization") without giving a rule; this is the published SmoothQuant
    rule: s[k] = amax_x[k]^alpha / amax_w[k]^(1 - alpha), amax_x[k] = max over
    the calibration rows of |x[t, k]|, amax_w[k] = max over the rows of W_gate
    and W_up of |W[n, k]|.  Reading: evaluated in double, rounded once to
    float32; s = 1 where either maximum is 0; clamped to [2^-20, 2^20].
    """
    ax = np.max(np.abs(bf16_to_f64(x_calib_bits)), axis=0)
    wg = np.abs(np.asarray(w_gate, dtype=np.float32).astype(np.float64))
    wu = np.abs(np.asarray(w_up, dtype=np.float32).astype(np.float64))
    aw = np.maximum(wg.max(axis=0), wu.max(axis=0))
    s = np.ones_like(ax)
    ok = (ax > 0) & (aw > 0)
    s[ok] = np.power(ax[ok], float(np.float32(alpha))) / np.power(aw[ok], 1.0 - float(np.float32(alpha)))
    s = np.clip(s, 2.0 ** -20, 2.0 ** 20)
    return s.astype(np.float32)


def pack_block(w_gate, w_up, w_down, prec_mode, smooth=None):
    """Quantize the three projections of one block for `prec_mode`.

    smooth: None, or per-input-channel factors s (float32 [hidden], > 0): the
    gate and up weights are quantized as fl32(W[n, k] s[k]) and the block
    multiplies x by xmul[k] = fl32(1 / s[k]) before quantizing it, which leaves
    x W^T unchanged in exact arithmetic (SmoothQuant's migration of activation
    outliers into the weights).
    """
    H = np.asarray(w_gate).shape[1]
    if smooth is None:
        xmul = np.ones(H, dtype=np.float32)
    else:
        sm = np.asarray(smooth, dtype=np.float32)
        assert sm.shape == (H,) and np.all(sm > 0) and np.all(np.isfinite(sm))
        w_gate = np.asarray(w_gate, dtype=np.float32) * sm[None, :]     # float32 products, RNE
        w_up = np.asarray(w_up, dtype=np.float32) * sm[None, :]
        xmul = np.float32(1.0) / sm
    out = _pack_plain(w_gate, w_up, w_down, prec_mode)
    out["xmul"] = xmul
    return out


def _pack_plain(w_gate, w_up, w_down, prec_mode):
    if prec_mode in (PREC_FP8, PREC_FP8_DOWN_BF16):
        g = pack_fp8(w_gate)
        u = pack_fp8(w_up)
        d = pack_fp8(w_down) if prec_mode == PREC_FP8 else pack_bf16(w_down)
    elif prec_mode == PREC_FP4:
        g, u, d = pack_nvfp4(w_gate), pack_nvfp4(w_up), pack_nvfp4(w_down)
    else:
        raise ValueError("unknown prec_mode %r" % (prec_mode,))
    return {"prec_mode": prec_mode, "gate": g, "up": u, "down": d}


# ----------------------------------------------------------------------------
# dequantized operands (exact fp64 values of the stored weights)
# ----------------------------------------------------------------------------


def fp8_weight_values(packed_fp8):
    """Code values of an FP8 weight (the scale is applied after the sum)."""
    codes, _ = packed_fp8
    return dec_e4m3(codes)


def nvfp4_weight_values(packed_fp4):
    """E2M1 value times its E4M3 block scale (exact); S applies after the sum."""
    codes, sb, _ = packed_fp4
    blk = np.repeat(dec_e4m3(sb), NVFP4_BLOCK, axis=1)
    return E2M1[codes & 0xF] * blk


# ----------------------------------------------------------------------------
# SiLU
# ----------------------------------------------------------------------------


def silu(g):
    """SiLU(g) = g * sigmoid(g) = g / (1 + e^-g); for g < 0 the equivalent
    g e^g / (1 + e^g) avoids overflow of e^-g."""
    g = np.asarray(g, dtype=np.float64)
    out = np.empty_like(g)
    pos = g >= 0
    out[pos] = g[pos] / (1.0 + np.exp(-g[pos]))
    e = np.exp(g[~pos])
    out[~pos] = g[~pos] * e / (1.0 + e)
    return out


# ----------------------------------------------------------------------------
# the block
# ----------------------------------------------------------------------------


def _projection(a_vals, a_scale, w_packed, kind):
    """sum_k a[t,k] w[n,k] in fp64, then the row (token) and column scales."""
    if kind == "fp8":
        acc = a_vals @ fp8_weight_values(w_packed).T
        return acc * a_scale.astype(np.float64)[:, None] * w_packed[1].astype(np.float64)[None, :]
    if kind == "fp4":
        acc = a_vals @ nvfp4_weight_values(w_packed).T
        return acc * a_scale.astype(np.float64)[:, None] * np.float64(w_packed[2])
    raise ValueError(kind)


def forward(x_bits, packed):
    """One MLP block over all M rows.

    x_bits: uint16 [M, H] bfloat16 bit patterns.
    packed: result of pack_block.
    Returns a dict with
      xq (uint8 [M,H]), sx (float32 [M]),
      hq (uint8 [M,I]) and sh (float32 [M])   -- FP8 / FP4 modes,
      hb (uint16 [M,I])                        -- BF16-down mode,
      h  (float64 [M,I]), Y (float64 [M,H]), y (uint16 [M,H]).
    """
    prec = packed["prec_mode"]
    x = bf16_to_f64(x_bits)
    xmul = packed.get("xmul")
    if xmul is not None:
        # x' = fl32(x xmul): a float32 product (x is exact in float32)
        x = (x.astype(np.float32) * np.asarray(xmul, dtype=np.float32)[None, :]).astype(np.float64)
    xq, sx = quantize_rows_e4m3(x)
    X = dec_e4m3(xq)

    kind_gu = "fp4" if prec == PREC_FP4 else "fp8"
    G = _projection(X, sx, packed["gate"], kind_gu)
    U = _projection(X, sx, packed["up"], kind_gu)
    h = silu(G) * U

    out = {"xq": xq, "sx": sx, "h": h}
    if prec == PREC_FP8_DOWN_BF16:
        hb = rne_bf16(h)
        Y = bf16_to_f64(hb) @ bf16_to_f64(packed["down"]).T
        out["hb"] = hb
    else:
        hq, sh = quantize_h_e4m3(h)
        Y = _projection(dec_e4m3(hq), sh, packed["down"], "fp4" if prec == PREC_FP4 else "fp8")
        out["hq"] = hq
        out["sh"] = sh
    out["Y"] = Y
    out["y"] = rne_bf16(Y)
    return out


def block_reference(x_bits, w_gate, w_up, w_down, prec_mode):
    """Pack and run in one call."""
    return forward(x_bits, pack_block(w_gate, w_up, w_down, prec_mode))


def stack_forward(x_bits, packed_layers):
    """L blocks in sequence: block l's bf16 output y is block l+1's x (the
    per-layer precision schedule of "OCRia 推理栈：单卡 B200 提速近 10 倍",
    section "Reducing the data moved: workload-aware quantization", applied
    along a stack).  Returns the list of every block's forward() result."""
    outs = []
    x = x_bits
    for packed in packed_layers:
        o = forward(x, packed)
        outs.append(o)
        x = o["y"]
    return outs
