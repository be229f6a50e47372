"""GPU parity: the HIP path (through the C ABI) against the oracle.

Same seeded inputs on both sides.  Small shapes span several tiles and a
ragged tail in every dimension the kernels tile (16-row m-tiles, 128-input
chunks, 8-column gate/up tiles, 16-column down tiles, split-K); the workload
shapes run in the launch configuration the benchmark times, with the oracle
evaluated on all rows or, for the two largest, on sampled rows (the block is
row-independent, so the oracle on a subset of rows is exact for those rows).
"""

import numpy as np
import pytest

from oracle import mlp as O
from quantized_memory_bound_amd import inputs as I
from quantized_memory_bound_amd import ocq
from parity import SH_RTOL, bf16_near_zero, bf16_rank, check_codes, check_y, e4m3_rank

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ocq.lib()


def _to_dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def run_gpu(d, prec, blob=None, x_bits=None):
    """One forward call with every tap set; returns numpy copies."""
    x_bits = d["x_bits"] if x_bits is None else x_bits
    M, H = x_bits.shape
    Iw = d["w_gate"].shape[0]
    if blob is None:
        blob = ocq.pack_weights(d["w_gate"], d["w_up"], d["w_down"], prec)
    x = _to_dev_bf16(x_bits)
    taps = {
        "x_codes": torch.empty((M, H), dtype=torch.uint8, device="cuda"),
        "x_scales": torch.empty(M, dtype=torch.float32, device="cuda"),
        "h_out": torch.empty((M, Iw), dtype=torch.int16 if prec == O.PREC_FP8_DOWN_BF16 else torch.uint8,
                             device="cuda"),
        "h_scales": torch.empty(M, dtype=torch.float32, device="cuda"),
    }
    y = ocq.mlp_forward(blob, x, H, Iw, prec, taps=taps)
    torch.cuda.synchronize()
    out = {"y": y.view(torch.int16).cpu().numpy().view(np.uint16),
           "xq": taps["x_codes"].cpu().numpy(), "sx": taps["x_scales"].cpu().numpy()}
    if prec == O.PREC_FP8_DOWN_BF16:
        out["hb"] = taps["h_out"].cpu().numpy().view(np.uint16)
    else:
        out["hq"] = taps["h_out"].cpu().numpy()
        out["sh"] = taps["h_scales"].cpu().numpy()
    return out, blob


def compare(g, r, prec, rows=None, what=""):
    sel = (lambda a: a[rows]) if rows is not None else (lambda a: a)
    assert np.array_equal(sel(g["xq"]), r["xq"]), what + ": x codes differ"
    assert np.array_equal(sel(g["sx"]), r["sx"]), what + ": x scales differ"
    if prec == O.PREC_FP8_DOWN_BF16:
        check_codes(sel(g["hb"]), r["hb"], bf16_rank, what + " hb", bf16_near_zero(sel(g["hb"]), r["hb"]))
    else:
        check_codes(sel(g["hq"]), r["hq"], e4m3_rank, what + " hq")
        rsh = np.asarray(r["sh"], dtype=np.float64)   # (1e-300 is 0 in float32)
        dsh = np.abs(sel(g["sh"]).astype(np.float64) - rsh) / np.maximum(rsh, 1e-300)
        print("%s sh: max relative difference %.2e" % (what, float(np.max(dsh)) if dsh.size else 0.0))
        np.testing.assert_allclose(sel(g["sh"]), r["sh"], rtol=SH_RTOL, atol=0, err_msg=what + " sh")
    return check_y(sel(g["y"]), r["y"], what + " y")


# the last two take the LDS-tiled kernels for many rows (E4M3 gate/up; BF16
# down): 3 and 4 m-blocks of 208 rows with a ragged last block
SMALL = [(256, 512, 1), (256, 512, 4), (384, 640, 17), (512, 1024, 37), (256, 768, 100), (128, 384, 208),
         (256, 512, 300), (640, 384, 65), (256, 768, 420), (384, 1152, 640)]


# requant 1: h requantized inside the gate/up launch where its grid fits the
# GPU at once (the library's default); 0: the two-pass form everywhere
@pytest.mark.parametrize("requant", [1, 0])
@pytest.mark.parametrize("prec", [0, 1, 2])
@pytest.mark.parametrize("hidden,inter,M", SMALL)
def test_small_shapes(hidden, inter, M, prec, requant):
    print("case hidden=%d inter=%d M=%d prec=%d requant=%d" % (hidden, inter, M, prec, requant), flush=True)
    d = I.make_inputs(hidden, inter, M, x_outliers=True, w_std=0.02, seed=hidden * 7 + inter + M)
    try:
        ocq.set_fused_requant(requant)
        g, _ = run_gpu(d, prec)
    finally:
        ocq.set_fused_requant(ocq.FUSED_REQUANT_DEFAULT)
    r = O.block_reference(d["x_bits"], d["w_gate"], d["w_up"], d["w_down"], prec)
    compare(g, r, prec, what="%dx%d M=%d prec=%d requant=%d" % (hidden, inter, M, prec, requant))


# blobs packed with activation-aware smoothing (factors calibrated on a
# separate draw with the same outlier channels): x is multiplied per channel
# before its quantization; the small shapes, the LDS-tiled kernels (420 rows)
# and the plain decode workload's shape
@pytest.mark.parametrize("prec", [0, 1, 2])
@pytest.mark.parametrize("hidden,inter,M", [(256, 512, 37), (256, 768, 420), (2048, 6144, 16)])
def test_smoothed_blobs(hidden, inter, M, prec):
    print("case smoothed hidden=%d inter=%d M=%d prec=%d" % (hidden, inter, M, prec), flush=True)
    d = I.make_inputs(hidden, inter, M, x_outliers=True, w_std=0.02, seed=hidden + M + prec)
    xc = np.random.default_rng(M + 1).standard_normal((64, hidden), dtype=np.float32)
    xc[:, d["outliers"]] *= np.float32(20.0)
    sm = O.calibrate_smoothing(I.to_bf16_bits(xc), d["w_gate"], d["w_up"], 0.5)
    blob = ocq.pack_weights(d["w_gate"], d["w_up"], d["w_down"], prec, smooth=sm)
    g, _ = run_gpu(d, prec, blob=blob)
    r = O.forward(d["x_bits"], O.pack_block(d["w_gate"], d["w_up"], d["w_down"], prec, smooth=sm))
    compare(g, r, prec, what="smoothed %dx%d M=%d prec=%d" % (hidden, inter, M, prec))


_PACK_CACHE = {}


def _workload(name):
    if name not in _PACK_CACHE:
        d = I.workload_inputs(name)
        cfg = I.WORKLOADS[name]
        _PACK_CACHE[name] = (d, O.pack_block(d["w_gate"], d["w_up"], d["w_down"], cfg["prec_mode"]),
                             ocq.pack_weights(d["w_gate"], d["w_up"], d["w_down"], cfg["prec_mode"]))
    return _PACK_CACHE[name]


@pytest.mark.parametrize("name", ["tiny_fp8", "decode_fp8", "spec_verify_fp8"])
def test_workload_fp8_full(name):
    print("case workload", name, flush=True)
    d, packed, blob = _workload(name)
    g, _ = run_gpu(d, packed["prec_mode"], blob=blob)
    r = O.forward(d["x_bits"], packed)
    rel, mx = compare(g, r, packed["prec_mode"], what=name)
    print("%s: y normwise %.2e, max %.2e" % (name, rel, mx))


def _sample_rows(M, n=48):
    rows = np.unique(np.concatenate([np.linspace(0, M - 1, n).astype(int), np.arange(max(0, M - 5), M)]))
    return rows


def test_workload_mixed_bf16_down_sampled():
    print("case workload mixed_bf16_down", flush=True)
    d, packed, blob = _workload("mixed_bf16_down")
    g, _ = run_gpu(d, packed["prec_mode"], blob=blob)
    rows = _sample_rows(d["x_bits"].shape[0])
    r = O.forward(d["x_bits"][rows], packed)
    compare(g, r, packed["prec_mode"], rows=rows, what="mixed_bf16_down")


@pytest.mark.parametrize("M", I.NVFP4_M_SWEEP)
def test_workload_nvfp4_sweep(M):
    print("case workload nvfp4 M=%d" % M, flush=True)
    d, packed, blob = _workload("nvfp4")
    xb = d["x_bits"][:M]
    g, _ = run_gpu(d, 2, blob=blob, x_bits=xb)
    rows = _sample_rows(M) if M > 64 else None
    r = O.forward(xb[rows] if rows is not None else xb, packed)
    compare(g, r, 2, rows=rows, what="nvfp4 M=%d" % M)


def _stack_layers(hidden, inter, modes, seed):
    ds = [I.make_inputs(hidden, inter, 1, w_std=0.02, seed=seed + 31 * l) for l in range(len(modes))]
    blobs = [ocq.pack_weights(d["w_gate"], d["w_up"], d["w_down"], m) for d, m in zip(ds, modes)]
    packed = [O.pack_block(d["w_gate"], d["w_up"], d["w_down"], m) for d, m in zip(ds, modes)]
    return blobs, packed


# stacks of blocks with a precision mode per layer: every layer's output is
# checked against the oracle block applied to the GPU's own input of that
# layer (the previous layer's GPU output), so differences do not compound;
# even and odd L exercise both placements of the alternating outputs, 420
# rows the LDS-tiled kernels
@pytest.mark.parametrize("hidden,inter,M,modes", [(256, 768, 37, (0, 1, 2, 1)), (256, 768, 420, (1, 0, 2)),
                                                  (384, 640, 5, (2, 2, 0))])
def test_stack_layerwise(hidden, inter, M, modes):
    print("case stack hidden=%d inter=%d M=%d modes=%s" % (hidden, inter, M, modes), flush=True)
    x_bits = I.make_inputs(hidden, inter, M, x_outliers=True, seed=M + 3, with_weights=False)["x_bits"]
    blobs, packed = _stack_layers(hidden, inter, modes, seed=hidden + M)
    x = _to_dev_bf16(x_bits)
    prev = x_bits
    for l in range(1, len(modes) + 1):
        y = ocq.mlp_stack_forward(blobs[:l], modes[:l], x, hidden, inter)
        torch.cuda.synchronize()
        yb = y.view(torch.int16).cpu().numpy().view(np.uint16)
        r = O.forward(prev, packed[l - 1])
        rel, mx = check_y(yb, r["y"], "stack layer %d of %s" % (l, modes))
        prev = yb
    # the whole stack again: same bits (deterministic kernels, same schedule)
    y2 = ocq.mlp_stack_forward(blobs, modes, x, hidden, inter)
    torch.cuda.synchronize()
    assert np.array_equal(y2.view(torch.int16).cpu().numpy().view(np.uint16), prev)


@pytest.mark.parametrize("prec", [0, 1, 2])
def test_deterministic_and_zero_rows(prec):
    print("case determinism prec=%d" % prec, flush=True)
    d = I.make_inputs(512, 1024, 40, x_outliers=True, seed=11)
    d["x_bits"][3] = 0
    d["x_bits"][39] = 0x8000                  # -0.0 row
    g1, blob = run_gpu(d, prec)
    g2, _ = run_gpu(d, prec, blob=blob)
    assert np.array_equal(g1["y"], g2["y"])
    for row in (3, 39):
        assert g1["sx"][row] == 0 and np.all(g1["xq"][row] & 0x7F == 0)
        assert np.all(g1["y"][row] & 0x7FFF == 0)
    r = O.block_reference(d["x_bits"], d["w_gate"], d["w_up"], d["w_down"], prec)
    compare(g1, r, prec, what="zero rows prec=%d" % prec)


# the block is row-wise: the first 13 rows of a 208-row call (13 m-tiles per
# workgroup) against a 13-row call on the same rows (one m-tile per
# workgroup), and a 13-row call against a 16-row call (the same blocking, so
# padding rows must not leak into real ones: bit-exact)
@pytest.mark.parametrize("prec", [0, 1, 2])
def test_row_independence(prec):
    print("case row independence prec=%d" % prec, flush=True)
    d = I.make_inputs(512, 1024, 208, x_outliers=True, seed=21)
    blob = ocq.pack_weights(d["w_gate"], d["w_up"], d["w_down"], prec)
    g208, _ = run_gpu(d, prec, blob=blob)
    g13, _ = run_gpu(d, prec, blob=blob, x_bits=d["x_bits"][:13])
    g16, _ = run_gpu(d, prec, blob=blob, x_bits=d["x_bits"][:16])
    assert np.array_equal(g13["xq"], g208["xq"][:13]) and np.array_equal(g13["sx"], g208["sx"][:13])
    assert np.array_equal(g13["y"], g16["y"][:13]), "rows 13..15 changed rows 0..12"
    r = O.block_reference(d["x_bits"][:13], d["w_gate"], d["w_up"], d["w_down"], prec)
    compare(g13, r, prec, what="M=13 prec=%d" % prec)
    compare(g208, r, prec, rows=slice(0, 13), what="M=208 rows 0..12 prec=%d" % prec)
    check_y(g208["y"][:13], g13["y"], "y of rows 0..12, M=208 against M=13")


# 13-m-tile gate/up with producer waves (H = 2048 or 4096, 113..383 rows):
# every format, one and two m-blocks, padded rows, 1, 2 and 3 weight tiles
# per workgroup (I = 1024, 3200, 6144), bf16 h for a BF16 down projection
@pytest.mark.parametrize("hidden,inter,M,prec", [(2048, 1024, 300, 0), (2048, 3200, 250, 1), (4096, 6144, 208, 0),
                                                 (4096, 3200, 150, 2), (2048, 6144, 120, 1), (2048, 1024, 383, 2)])
def test_gateup_weight_producers(hidden, inter, M, prec):
    print("case producers hidden=%d inter=%d M=%d prec=%d" % (hidden, inter, M, prec), flush=True)
    d = I.make_inputs(hidden, inter, M, x_outliers=True, w_std=0.02, seed=hidden + inter + M + prec)
    g, _ = run_gpu(d, prec)
    r = O.block_reference(d["x_bits"], d["w_gate"], d["w_up"], d["w_down"], prec)
    compare(g, r, prec, what="producers %dx%d M=%d prec=%d" % (hidden, inter, M, prec))


# one workspace for a sequence of calls: different rows each time, and a call
# that takes the LDS-tiled kernels in between
# (H = 2048: the 13-m-tile gate/up with weight producers, one and two
# m-blocks, between skinny calls)
@pytest.mark.parametrize("H,Iw,prec,n,seq", [
    (256, 768, 0, 420, ((0, 16), (16, 32), (0, 420), (100, 116), (200, 213), (0, 16))),
    (2048, 1024, 0, 300, ((0, 208), (0, 16), (0, 300), (100, 113), (40, 248), (0, 13))),
    (2048, 1024, 2, 300, ((0, 300), (7, 20), (0, 208), (0, 52)))])
def test_workspace_reuse(H, Iw, prec, n, seq):
    print("case workspace reuse H=%d prec=%d" % (H, prec), flush=True)
    d = I.make_inputs(H, Iw, n, x_outliers=True, seed=5)
    blob = ocq.pack_weights(d["w_gate"], d["w_up"], d["w_down"], prec)
    nws = max(ocq.workspace_bytes(b - a, H, Iw, prec) for a, b in seq)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    for a, b in seq:
        rows = slice(a, b)
        xb = np.ascontiguousarray(d["x_bits"][rows])
        y = ocq.mlp_forward(blob, _to_dev_bf16(xb), H, Iw, prec, workspace=ws)
        torch.cuda.synchronize()
        r = O.block_reference(xb, d["w_gate"], d["w_up"], d["w_down"], prec)
        check_y(y.view(torch.int16).cpu().numpy().view(np.uint16), r["y"], "rows %s" % rows)


# row counts at the edges of the kernel choice (383 and 384 rows: the last
# skinny shape and the first LDS-tiled one) and the largest M the ABI takes
# (8192 rows: 40 m-blocks of 208 in the LDS-tiled kernels); the oracle runs on
# sampled rows for the largest
@pytest.mark.parametrize("prec", [0, 1, 2])
@pytest.mark.parametrize("M", [383, 384, 8192])
def test_row_count_edges(M, prec):
    print("case rows M=%d prec=%d" % (M, prec), flush=True)
    d = I.make_inputs(256, 768, M, x_outliers=True, w_std=0.02, seed=M + prec)
    g, _ = run_gpu(d, prec)
    rows = _sample_rows(M, 96) if M > 1000 else None
    xb = d["x_bits"][rows] if rows is not None else d["x_bits"]
    r = O.block_reference(xb, d["w_gate"], d["w_up"], d["w_down"], prec)
    compare(g, r, prec, rows=rows, what="M=%d prec=%d" % (M, prec))


def test_check_blob():
    d = I.make_inputs(256, 512, 4, seed=2)
    blob = ocq.pack_weights(d["w_gate"], d["w_up"], d["w_down"], 0)
    ocq.check_blob(blob, 256, 512, 0)
    with pytest.raises(ocq.OcqError) as e:
        ocq.check_blob(blob, 256, 512, 1)
    assert e.value.status == ocq.ERR_BAD_BLOB


def test_binding_rejects_bad_tensors():
    # the binding checks dtype, shape, contiguity and size before the C call
    d = I.make_inputs(256, 512, 4, seed=2)
    blob = ocq.pack_weights(d["w_gate"], d["w_up"], d["w_down"], 0)
    x = _to_dev_bf16(d["x_bits"])
    bad = [dict(x=x.float()), dict(x=x[:, :128].contiguous()), dict(x=torch.cat([x, x], 1)[:, ::2]),
           dict(x=x, y=torch.empty((4, 128), dtype=torch.bfloat16, device="cuda")),
           dict(x=x, blob=blob[:1000]), dict(x=x, taps={"x_codes": torch.empty((4, 256), device="cuda")})]
    for kw in bad:
        args = dict(blob=blob, hidden=256, inter=512, prec_mode=0)
        args.update(kw)
        with pytest.raises(ocq.OcqError):
            ocq.mlp_forward(**args)


# The per-token requantization inside the gate/up kernel (grid-wide row
# maxima, h kept in registers) and the two-pass form (fp32 h to the
# workspace, then k_requant) compute the same h, the same maxima and the
# same codes: every output must be bit-identical.  Shapes: the skinny
# kernels (one pair per wave, and several m-tiles per wave), the 13-m-tile
# kernel with weight producers (E4M3 and NVFP4 weights), the decode and
# spec-verify workloads' shapes, and NVFP4 with six tiles per workgroup.
@pytest.mark.parametrize("H,Iw,M,prec", [(256, 512, 4, 0), (384, 640, 17, 2), (512, 1024, 100, 0),
                                         (2048, 6144, 208, 0), (2048, 6144, 16, 0), (2048, 1024, 150, 2),
                                         (4096, 12288, 52, 2), (256, 768, 208, 0)])
def test_fused_requant_matches_two_pass(H, Iw, M, prec):
    print("case fused requant hidden=%d inter=%d M=%d prec=%d" % (H, Iw, M, prec), flush=True)
    d = I.make_inputs(H, Iw, M, x_outliers=True, w_std=0.02, seed=H + Iw + M + prec)
    blob = ocq.pack_weights(d["w_gate"], d["w_up"], d["w_down"], prec)
    try:
        ocq.set_fused_requant(0)
        g2, _ = run_gpu(d, prec, blob=blob)
        assert ocq.last_requant_in_gateup() == 0
        ocq.set_fused_requant(1)
        g1, _ = run_gpu(d, prec, blob=blob)
        assert ocq.last_requant_in_gateup() == 1   # every grid here fits the GPU at once
    finally:
        ocq.set_fused_requant(ocq.FUSED_REQUANT_DEFAULT)
    for k in ("y", "xq", "sx", "hq", "sh"):
        assert np.array_equal(g1[k], g2[k]), k
    r = O.block_reference(d["x_bits"], d["w_gate"], d["w_up"], d["w_down"], prec)
    compare(g1, r, prec, what="fused %dx%d M=%d prec=%d" % (H, Iw, M, prec))
