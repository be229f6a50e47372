"""The oracle's pins must fail for plausible oracle mistakes.

Each case loads a fresh copy of oracle/mlp.py with one mistake planted in its
source text (never in the real module), runs pins of test_oracle_block.py
against the copy (the two channel-permutation pins in all three modes, or the
hand-built tie-block pins of the h requantization), and requires at least one
of them to fail."""

import types

import pytest

import test_oracle_block as T
from oracle import mlp as O

SRC_PATH = O.__file__
PLANTS = {
    # per-row scales taken along the wrong axis (columns)
    "scale_axis": ("amax = np.max(np.abs(a32), axis=1) if a32.shape[1] else np.zeros(a32.shape[0], np.float32)",
                   "amax = (np.max(np.abs(a32), axis=0)[:a32.shape[0]] if a32.shape[0] <= a32.shape[1] "
                   "else np.max(np.abs(a32), axis=1)) if a32.shape[1] else np.zeros(a32.shape[0], np.float32)"),
    # output-channel scales applied to the wrong columns
    "column_scales": ("return acc * a_scale.astype(np.float64)[:, None] * w_packed[1].astype(np.float64)[None, :]",
                      "return acc * a_scale.astype(np.float64)[:, None] * np.sort(w_packed[1]).astype(np.float64)[None, :]"),
    # the down projection's inputs paired with the wrong weight columns
    "down_input_order": ('Y = _projection(dec_e4m3(hq), sh, packed["down"], "fp4" if prec == PREC_FP4 else "fp8")',
                         'Y = _projection(dec_e4m3(hq)[:, ::-1].copy(), sh, packed["down"], '
                         '"fp4" if prec == PREC_FP4 else "fp8")'),
}


def _planted(old, new):
    src = open(SRC_PATH).read()
    assert src.count(old) == 1, "the planted line is no longer in the oracle"
    mod = types.ModuleType("oracle.mlp_planted")
    mod.__file__ = SRC_PATH
    mod.__package__ = "oracle"   # the oracle's relative imports
    exec(compile(src.replace(old, new), SRC_PATH, "exec"), mod.__dict__)
    return mod


# h rounded to binary32 before its decisions (the requantization or the
# bf16 rounding of the BF16-down mode): caught by the hand-built tie block
H_PLANTS = {
    "h_codes_via_binary32": ("codes[nz] = enc_e4m3(h[nz] / scale[nz, None].astype(np.float64))",
                             "codes[nz] = enc_e4m3((h[nz] / scale[nz, None].astype(np.float64))"
                             ".astype(np.float32).astype(np.float64))"),
    "h_amax_via_binary32": ("amax = np.max(np.abs(h), axis=1) if h.shape[1] else np.zeros(h.shape[0])",
                            "h = h.astype(np.float32).astype(np.float64); "
                            "amax = np.max(np.abs(h), axis=1) if h.shape[1] else np.zeros(h.shape[0])"),
    "hb_via_binary32": ("hb = rne_bf16(h)", "hb = rne_bf16(h.astype(np.float32).astype(np.float64))"),
}


@pytest.mark.parametrize("name", sorted(H_PLANTS))
def test_tie_block_pins_catch(name, monkeypatch):
    monkeypatch.setattr(T, "O", _planted(*H_PLANTS[name]))
    caught = 0
    for pin in (T.test_tie_block_bf16_h, T.test_tie_block_e4m3_h):
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught > 0, "planted mistake %s passes the tie-block pins" % name


@pytest.mark.parametrize("name", sorted(PLANTS))
def test_permutation_pins_catch(name, monkeypatch):
    monkeypatch.setattr(T, "O", _planted(*PLANTS[name]))
    caught = 0
    for prec in (O.PREC_FP8, O.PREC_FP8_DOWN_BF16, O.PREC_FP4):
        for pin in (T.test_hidden_channel_permutation, T.test_intermediate_channel_permutation):
            try:
                pin(prec)
            except (AssertionError, ValueError, IndexError):
                caught += 1
    assert caught > 0, "planted mistake %s passes every permutation pin" % name


# mistakes in how the block composes its steps: caught by the lossless-grid
# pins (every quantization exact, so the block must equal the textbook MLP)
COMPOSE_PLANTS = {
    # SiLU applied to the up projection instead of the gate
    "silu_on_up": ("h = silu(G) * U", "h = silu(U) * G"),
    # the gate projection without the token scale
    "gate_without_token_scale": ('G = _projection(X, sx, packed["gate"], kind_gu)',
                                 'G = _projection(X, np.ones_like(sx), packed["gate"], kind_gu)'),
    # the NVFP4 per-tensor scale dropped
    "nvfp4_tensor_scale_dropped": ("return acc * a_scale.astype(np.float64)[:, None] * np.float64(w_packed[2])",
                                   "return acc * a_scale.astype(np.float64)[:, None]"),
}


@pytest.mark.parametrize("name", sorted(COMPOSE_PLANTS))
def test_lossless_pins_catch(name, monkeypatch):
    monkeypatch.setattr(T, "O", _planted(*COMPOSE_PLANTS[name]))
    caught = 0
    for pin in (T.test_lossless_fp8_block_equals_textbook_mlp, T.test_lossless_bf16_down_equals_textbook,
                T.test_lossless_nvfp4_block):
        try:
            pin(0)
        except AssertionError:
            caught += 1
    assert caught > 0, "planted mistake %s passes the lossless-grid pins" % name
