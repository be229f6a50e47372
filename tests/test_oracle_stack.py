"""Pins for the oracle's stack of blocks (CPU only).

A stack applies blocks in sequence, each with its own precision mode; block
l + 1 reads block l's bf16 output.  Pinned by invariants of that definition:
a layer whose down weights are zero outputs zero rows, and every later layer
then sees zero rows and outputs zero rows (so the later layer must read the
earlier layer's output, not the stack's input); rows stay independent along
the stack (permuting the input rows permutes every layer's output rows); a
one-layer stack is the block.
"""

import numpy as np
import pytest

from oracle import mlp as O
from quantized_memory_bound_amd import inputs as I

MODES = (O.PREC_FP8, O.PREC_FP8_DOWN_BF16, O.PREC_FP4)


def _layers(hidden, inter, modes, seed, zero_down=()):
    out = []
    for l, m in enumerate(modes):
        d = I.make_inputs(hidden, inter, 1, w_std=0.05, seed=seed + 17 * l)
        wd = np.zeros_like(d["w_down"]) if l in zero_down else d["w_down"]
        out.append(O.pack_block(d["w_gate"], d["w_up"], wd, m))
    return out


@pytest.fixture(scope="module")
def x_bits():
    return I.make_inputs(128, 256, 9, x_outliers=True, seed=11, with_weights=False)["x_bits"]


def test_one_layer_stack_is_the_block(x_bits):
    layers = _layers(128, 256, (O.PREC_FP8_DOWN_BF16,), 1)
    a = O.stack_forward(x_bits, layers)[-1]["y"]
    b = O.forward(x_bits, layers[0])["y"]
    assert np.array_equal(a, b)


@pytest.mark.parametrize("mode_first", MODES)
def test_zero_layer_zeroes_every_later_layer(x_bits, mode_first):
    modes = (mode_first, O.PREC_FP8, O.PREC_FP4, O.PREC_FP8_DOWN_BF16)
    layers = _layers(128, 256, modes, 2, zero_down=(1,))
    outs = O.stack_forward(x_bits, layers)
    assert np.any(outs[0]["y"] & 0x7FFF)                     # the first layer is not trivial
    for o in outs[1:]:
        assert not np.any(o["y"] & 0x7FFF)                   # +-0 only
    # and the layer after the zero layer quantized all-zero rows: scale 0, codes 0
    assert not np.any(outs[2]["sx"]) and not np.any(outs[2]["xq"])


def test_rows_independent_along_the_stack(x_bits):
    layers = _layers(128, 256, (O.PREC_FP4, O.PREC_FP8, O.PREC_FP8_DOWN_BF16), 3)
    perm = np.random.default_rng(5).permutation(x_bits.shape[0])
    a = O.stack_forward(x_bits, layers)
    b = O.stack_forward(x_bits[perm], layers)
    for oa, ob in zip(a, b):
        assert np.array_equal(oa["y"][perm], ob["y"])
