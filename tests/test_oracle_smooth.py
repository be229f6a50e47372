"""Pins for the oracle's activation-aware smoothing (CPU only).

Smoothing moves per-input-channel range from x into the gate/up weights:
W'[n,k] = fl32(W[n,k] s[k]), x'[k] = fl32(x[k] fl32(1/s[k])), exact algebra
x' W'^T = x W^T.  Pinned by: s = 1 is the plain block; a constant power of two
s = 2^e changes no code and no result (every scale moves by exactly 2^-+e);
the calibration rule on a hand-computed example; and the purpose of the
method: with outlier input channels the smoothed block is closer to the
unquantized textbook MLP than the plain one.  The host library's calibration
and smoothed packing are compared with the oracle's in test_abi_host.py.
"""

import numpy as np
import pytest
import torch

from oracle import mlp as O
from quantized_memory_bound_amd import inputs as I

MODES = (O.PREC_FP8, O.PREC_FP8_DOWN_BF16, O.PREC_FP4)


@pytest.fixture(scope="module")
def data():
    return I.make_inputs(256, 512, 24, x_outliers=True, w_std=0.05, seed=21)


@pytest.mark.parametrize("prec", MODES)
def test_unit_smoothing_is_the_plain_block(data, prec):
    d = data
    a = O.forward(d["x_bits"], O.pack_block(d["w_gate"], d["w_up"], d["w_down"], prec))
    b = O.forward(d["x_bits"], O.pack_block(d["w_gate"], d["w_up"], d["w_down"], prec,
                                             smooth=np.ones(256, np.float32)))
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["xq"], b["xq"])


@pytest.mark.parametrize("prec", MODES)
@pytest.mark.parametrize("e", [-3, 2])
def test_power_of_two_smoothing_changes_nothing(data, prec, e):
    d = data
    s = np.full(256, 2.0 ** e, np.float32)
    a = O.forward(d["x_bits"], O.pack_block(d["w_gate"], d["w_up"], d["w_down"], prec))
    b = O.forward(d["x_bits"], O.pack_block(d["w_gate"], d["w_up"], d["w_down"], prec, smooth=s))
    assert np.array_equal(a["xq"], b["xq"])
    assert np.array_equal(b["sx"] * np.float32(2.0 ** e), a["sx"])
    assert np.array_equal(a["y"], b["y"])


def test_calibration_rule_by_hand():
    H, Iw = 128, 8
    x = np.zeros((3, H), np.float32)
    x[0, 0], x[1, 0] = 2.0, -8.0          # amax_x[0] = 8
    x[2, 1] = 0.5                          # amax_x[1] = 0.5
    x[:, 3] = 1.0                          # amax_x[3] = 1, but column 3 of W is zero
    x[0, 4] = 1024.0                       # amax_x[4] = 1024 (for the clamp below)
    wg = np.zeros((Iw, H), np.float32)
    wu = np.zeros((Iw, H), np.float32)
    wg[3, 0], wu[5, 0] = 0.5, -2.0         # amax_w[0] = 2
    wg[0, 1] = 0.125                       # amax_w[1] = 0.125
    wu[1, 2] = 1.0                         # channel 2: x is zero
    wg[0, 4] = 2.0 ** -40                  # amax_w[4] = 2^-40
    xb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    s = O.calibrate_smoothing(xb, wg, wu, alpha=0.5)
    assert s[0] == np.float32(2.0)                     # sqrt(8) / sqrt(2)
    assert s[1] == np.float32(2.0)                     # sqrt(0.5) / sqrt(0.125)
    assert s[2] == 1.0 and s[3] == 1.0                 # a zero maximum
    assert s[4] == np.float32(2.0 ** 20)               # sqrt(2^10 / 2^-40) = 2^25, clamped
    s1 = O.calibrate_smoothing(xb, wg, wu, alpha=1.0)
    assert s1[0] == 8.0 and s1[1] == 0.5               # alpha = 1: the activation maxima
    s0 = O.calibrate_smoothing(xb, wg, wu, alpha=0.0)
    assert s0[0] == 0.5 and s0[1] == 8.0               # alpha = 0: 1 / the weight maxima


@pytest.mark.parametrize("prec", MODES)
def test_smoothing_brings_outlier_inputs_closer_to_the_textbook_mlp(prec):
    # x with 1% outlier channels x20 (the decode workload's distribution); the
    # calibration rows are a separate normal draw with the same outlier
    # channels (a property of the model's activations, not of one batch)
    d = I.make_inputs(512, 1024, 64, x_outliers=True, w_std=0.02, seed=5)
    xc = np.random.default_rng(77).standard_normal((256, 512), dtype=np.float32)
    xc[:, d["outliers"]] *= np.float32(20.0)
    calib = I.to_bf16_bits(xc)
    x = O.bf16_to_f64(d["x_bits"])
    wg, wu, wd = (d[k].astype(np.float64) for k in ("w_gate", "w_up", "w_down"))
    ref = (O.silu(x @ wg.T) * (x @ wu.T)) @ wd.T
    s = O.calibrate_smoothing(calib, d["w_gate"], d["w_up"], alpha=0.5)
    plain = O.bf16_to_f64(O.forward(d["x_bits"], O.pack_block(d["w_gate"], d["w_up"], d["w_down"], prec))["y"])
    smooth = O.bf16_to_f64(O.forward(d["x_bits"], O.pack_block(d["w_gate"], d["w_up"], d["w_down"], prec,
                                                               smooth=s))["y"])
    e_plain = np.linalg.norm(plain - ref) / np.linalg.norm(ref)
    e_smooth = np.linalg.norm(smooth - ref) / np.linalg.norm(ref)
    print("normwise error vs textbook MLP: plain %.3e, smoothed %.3e" % (e_plain, e_smooth))
    assert e_smooth < 0.95 * e_plain
