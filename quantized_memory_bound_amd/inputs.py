"""Seeded synthetic workloads for the quantized MLP block.

The post's workload (document-parsing requests on its own model) and its
calibration data are not available, so every input is synthetic with the
shapes and value distributions of the block configurations below.  This
module only draws random numbers; it holds none of the block's arithmetic.

Draw order from one numpy default_rng(seed): x (float32 normal), the outlier
channel indices (without replacement, round(1% of hidden) of them, applied
as x20 to every row before the bf16 rounding), then W_gate [inter, hidden],
W_up [inter, hidden], W_down [hidden, inter] (float32 normal, std w_std).
x is rounded to bfloat16 by torch's float32 -> bfloat16 cast (round to
nearest even).
"""

import numpy as np

# Block configurations: M = requests x (1 + draft tokens) rows per verify pass.
WORKLOADS = {
    # tiny FP8 block
    "tiny_fp8": dict(hidden=256, inter=512, M=4, prec_mode=0, x_outliers=False, w_std=0.02),
    # plain decode: 16 requests x 1 token, outlier channels in x
    "decode_fp8": dict(hidden=2048, inter=6144, M=16, prec_mode=0, x_outliers=True, w_std=0.02),
    # spec-verify: 16 requests x (1 + 12 draft tokens)
    "spec_verify_fp8": dict(hidden=2048, inter=6144, M=208, prec_mode=0, x_outliers=False, w_std=0.02),
    # 64 requests x 13 tokens, down projection kept in BF16
    "mixed_bf16_down": dict(hidden=4096, inter=12288, M=832, prec_mode=1, x_outliers=True, w_std=0.015),
    # NVFP4 weights, M swept over {1, 13, 52, 208}: leading rows of the M=208 draw
    "nvfp4": dict(hidden=4096, inter=12288, M=208, prec_mode=2, x_outliers=False, w_std=0.015),
}
NVFP4_M_SWEEP = (1, 13, 52, 208)

# Stacks of blocks with a precision mode per layer (0 FP8, 1 FP8 gate/up with
# BF16 down, 2 NVFP4), spec-verify shape: the first and last layers are taken
# as the sensitive ones and keep a BF16 down projection, the others alternate
# FP8 and NVFP4.  Synthetic schedule: the pages name no per-layer assignment.
STACKS = {
    "stack_mixed": dict(hidden=2048, inter=6144, M=208, modes=(1, 0, 2, 0, 2, 0, 2, 1), x_outliers=False,
                        w_std=0.02),
}


def to_bf16_bits(x32):
    """float32 array -> bfloat16 bit patterns (uint16), via torch's RNE cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def make_inputs(hidden, inter, M, x_outliers=False, w_std=0.02, seed=0, with_weights=True):
    """Return dict(x_bits uint16 [M, hidden], w_gate, w_up float32 [inter, hidden],
    w_down float32 [hidden, inter], outliers int array)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, hidden), dtype=np.float32)
    outliers = np.zeros(0, dtype=np.int64)
    if x_outliers:
        n_out = int(round(0.01 * hidden))
        outliers = np.sort(rng.choice(hidden, size=n_out, replace=False))
        x[:, outliers] *= np.float32(20.0)
    out = {"x_bits": to_bf16_bits(x), "outliers": outliers}
    if with_weights:
        out["w_gate"] = rng.standard_normal((inter, hidden), dtype=np.float32) * np.float32(w_std)
        out["w_up"] = rng.standard_normal((inter, hidden), dtype=np.float32) * np.float32(w_std)
        out["w_down"] = rng.standard_normal((hidden, inter), dtype=np.float32) * np.float32(w_std)
    return out


def workload_inputs(name, seed=0, M=None):
    """Inputs of a named workload; M (if given) takes the leading rows."""
    cfg = WORKLOADS[name]
    d = make_inputs(cfg["hidden"], cfg["inter"], cfg["M"], cfg["x_outliers"], cfg["w_std"], seed)
    if M is not None:
        assert M <= cfg["M"]
        d["x_bits"] = d["x_bits"][:M].copy()
    return d


def stack_inputs(name, seed=0):
    """x bits of a named stack and its layers' float32 weights: layer l's
    weights are those make_inputs draws with seed + 1 + l (its one-row x is
    discarded)."""
    cfg = STACKS[name]
    x_bits = make_inputs(cfg["hidden"], cfg["inter"], cfg["M"], cfg["x_outliers"], cfg["w_std"], seed,
                         with_weights=False)["x_bits"]
    layers = []
    for l in range(len(cfg["modes"])):
        d = make_inputs(cfg["hidden"], cfg["inter"], 1, False, cfg["w_std"], seed + 1 + l)
        layers.append((d["w_gate"], d["w_up"], d["w_down"]))
    return x_bits, layers
