"""GPU cases where the arithmetic leaves no room: exact-integer blocks,
lossless-grid blocks in every mode, and the captured-graph path the
benchmark times.

Exact-integer blocks.  x rows hold one 14 and otherwise -1, 0 or +1; every
gate / up / down weight row holds one 14 and otherwise -1, 0 or +1 (BF16
down: small integers).  All row maxima are 14, so every scale is
14 / 448 = 2^-5 and every code is 32 x its value: the quantizations are
exact, every product in the matrix cores is an integer, and every sum stays
far below 2^24, so the fp32 accumulators of the f16 MFMA (gate/up) and the
bf16 MFMA (BF16 down) hold the exact sums.  The gate anchor 14 * 14 = 196
dominates the +-1 terms, so G >= 40 and SiLU(G) = G in fp64 and in the
kernel's fp32 (e^-G is below half a unit of 1.0); h = G U is then an exact
integer.  What must come out bit-exact:
  * x codes and scales, h scales (fl32(max|h| / 448) of the same exact max);
  * bf16(h) and y = bf16(h Wd^T) in the BF16-down mode (exact sums);
  * the h codes: the kernel takes them on the binary32 quotient fl32(h / sh)
    and the oracle on the exact quotient, so they must equal E4M3(fl32(h/sh))
    everywhere and the oracle's codes wherever the two quotients give one
    code (all but a few entries: with integer h, some h / sh fall within a
    float32 rounding of an E4M3 midpoint).
  * y of the FP8-down mode, against the oracle's down projection of the
    GPU's own h codes: the E4M3 products of h codes and weight codes are
    integers here (checked below 2^24 in sum), so the f16 matrix cores' fp32
    sums are exact and y = bf16(fl32(fl32(S sh) sw)) with the exact sum S
    (the kernel applies the row scale, then the column scale, in fp32).
    Against the oracle's y itself the few h codes decided on the other side
    of a midpoint (one step each, within the rule) are amplified here by the
    single large weight in every down row, so that comparison is left to
    the tolerance tests on the workloads' distributions.
"""

import numpy as np
import pytest

from oracle import formats as F
from oracle import mlp as O
from quantized_memory_bound_amd import ocq
from parity import check_y, e4m3_rank

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ocq.lib()


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _anchored(rng, n, k, anchor_col=None, density=0.25, lo=-1, hi=1):
    """n x k integers: one 14 per row (at anchor_col, or a random column >= 1),
    the rest in [lo, hi] at the given density."""
    v = rng.integers(lo, hi + 1, size=(n, k)) * (rng.random((n, k)) < density)
    cols = np.full(n, anchor_col) if anchor_col is not None else rng.integers(1, k, n)
    v[np.arange(n), cols] = 14
    return v.astype(np.float32)


def _exact_inputs(M, H, Iw, prec, seed):
    rng = np.random.default_rng(seed)
    x = _anchored(rng, M, H, anchor_col=0)
    wg = _anchored(rng, Iw, H, anchor_col=0)
    wu = _anchored(rng, Iw, H)
    wu[:, 0] = 0.0                                   # up rows have no share of the x anchor
    if prec == O.PREC_FP8_DOWN_BF16:
        wd = (rng.integers(-4, 5, size=(H, Iw)) * (rng.random((H, Iw)) < 0.25)).astype(np.float32)
    else:
        wd = _anchored(rng, H, Iw)
    G = x.astype(np.float64) @ wg.T.astype(np.float64)
    U = x.astype(np.float64) @ wu.T.astype(np.float64)
    assert G.min() >= 40, "gate anchor must dominate"
    h = G * U
    assert np.abs(h).max() < 2 ** 24
    if prec == O.PREC_FP8_DOWN_BF16:
        hb = F.bf16_to_f64(F.rne_bf16(h))
        assert (np.abs(hb) @ np.abs(wd.T.astype(np.float64))).max() < 2 ** 24
    x_bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return x_bits, wg, wu, wd, h


def _run(blob, x_bits, H, Iw, prec):
    M = x_bits.shape[0]
    taps = {"x_codes": torch.empty((M, H), dtype=torch.uint8, device="cuda"),
            "x_scales": torch.empty(M, dtype=torch.float32, device="cuda"),
            "h_out": torch.empty((M, Iw), dtype=torch.int16 if prec == O.PREC_FP8_DOWN_BF16 else torch.uint8,
                                 device="cuda"),
            "h_scales": torch.empty(M, dtype=torch.float32, device="cuda")}
    y = ocq.mlp_forward(blob, _dev_bf16(x_bits), H, Iw, prec, taps=taps)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in taps.items()}, _bits(y)


# (hidden, inter, M): skinny kernels with a ragged m-tile; the 13-m-tile
# gate/up with weight producers (hidden 2048); the LDS-tiled kernels (420 rows)
EXACT = [(256, 384, 20), (2048, 384, 208), (256, 384, 420)]


@pytest.mark.parametrize("prec", [O.PREC_FP8, O.PREC_FP8_DOWN_BF16])
@pytest.mark.parametrize("H,Iw,M", EXACT)
def test_exact_integer_block(H, Iw, M, prec):
    print("case exact hidden=%d inter=%d M=%d prec=%d" % (H, Iw, M, prec), flush=True)
    x_bits, wg, wu, wd, h = _exact_inputs(M, H, Iw, prec, seed=H + M + prec)
    blob = ocq.pack_weights(wg, wu, wd, prec)
    t, y = _run(blob, x_bits, H, Iw, prec)
    r = O.block_reference(x_bits, wg, wu, wd, prec)
    assert np.array_equal(r["h"], h)                  # the oracle's h is the exact integer product
    assert np.array_equal(t["x_codes"], r["xq"]) and np.array_equal(t["x_scales"], r["sx"])
    assert np.all(r["sx"] == np.float32(2.0 ** -5))
    if prec == O.PREC_FP8_DOWN_BF16:
        assert np.array_equal(t["h_out"].view(np.uint16), r["hb"]), "bf16(h) not bit-exact"
        assert np.array_equal(y, r["y"]), "y not bit-exact (exact bf16 sums)"
        return
    assert np.array_equal(t["h_scales"], r["sh"]), "h scales not bit-exact"
    q32 = (h / r["sh"][:, None].astype(np.float64)).astype(np.float32).astype(np.float64)
    want = F.enc_e4m3(q32)
    assert np.array_equal(e4m3_rank(t["h_out"]), e4m3_rank(want)), "h codes differ from E4M3(fl32(h / sh))"
    same = e4m3_rank(want) == e4m3_rank(r["hq"])
    print("exact h codes: %d of %d entries where the binary32 quotient decides otherwise" %
          (int(np.sum(~same)), same.size))
    assert np.array_equal(e4m3_rank(t["h_out"])[same], e4m3_rank(r["hq"])[same])
    # down projection of the GPU's codes: exact integer sums in fp32
    dq, sw = O.pack_fp8(wd)
    A, W = F.dec_e4m3(t["h_out"]), F.dec_e4m3(dq)
    assert np.all(np.mod(A, 1) == 0) and np.all(np.mod(W, 1) == 0)
    assert (np.abs(A) @ np.abs(W).T).max() < 2 ** 24
    S = (A @ W.T).astype(np.float32)
    y_exp = F.rne_bf16((S * t["h_scales"][:, None]).astype(np.float32).astype(np.float64) * sw[None, :])
    assert np.array_equal(y, y_exp), "y differs from the exact down projection of the GPU's h codes"
    rel, _ = check_y(y, r["y"], "exact-integer y (E4M3 down)", strict=False)
    print("exact-integer y (E4M3 down) against the oracle's y: normwise %.2e" % rel)


# Lossless grids: x and weights are E4M3 values times a power of two with a
# +-448 in every row (NVFP4: E2M1 x E4M3 block scale x 2^-12 with one +-6 per
# block and one 448 scale), so the quantizations are exact and what is left
# is fp32 against fp64 arithmetic in the sums and the SiLU, and the final
# bf16 rounding.  Every projection sums in fp32 (f16 and bf16 matrix cores),
# so y must agree to 2e-4 normwise (a tenth of the general bound): a relative
# difference d in Y flips the bf16 rounding of about d / 2^-8 of the entries,
# each by one unit (2^-8 relative).

def _grid(rng, n, k, lo, hi):
    c = rng.integers(0, 0x7F, size=(n, k)).astype(np.uint8) | (rng.integers(0, 2, (n, k)) * 0x80).astype(np.uint8)
    c[np.arange(n), rng.integers(0, k, n)] = 0x7E
    v = torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return v * np.exp2(rng.integers(lo, hi, n))[:, None]


def _fp4_grid(rng, n, k):
    nb = k // 16
    sb = rng.integers(0x30, 0x7F, size=(n, nb)).astype(np.uint8)
    sb[0, 0] = 0x7E
    q = rng.integers(0, 16, size=(n, k)).astype(np.uint8)
    rows, blks = np.meshgrid(np.arange(n), np.arange(nb), indexing="ij")
    q[rows, blks * 16 + rng.integers(0, 16, size=(n, nb))] = np.where(rng.integers(0, 2, (n, nb)) > 0, 0x7, 0xF)
    return F.E2M1[q] * np.repeat(F.dec_e4m3(sb), 16, axis=1) * 2.0 ** -12


@pytest.mark.parametrize("prec", [O.PREC_FP8, O.PREC_FP8_DOWN_BF16, O.PREC_FP4])
@pytest.mark.parametrize("M", [20, 208])
def test_lossless_grid_inputs_tight(M, prec):
    print("case lossless grid M=%d prec=%d" % (M, prec), flush=True)
    rng = np.random.default_rng(21 + prec)
    H, Iw = (2048, 384) if M == 208 else (256, 384)
    x = _grid(rng, M, H, -9, -5)
    if prec == O.PREC_FP4:
        wg, wu, wd = _fp4_grid(rng, Iw, H), _fp4_grid(rng, Iw, H), _fp4_grid(rng, H, Iw)
    else:
        wg, wu = _grid(rng, Iw, H, -16, -12), _grid(rng, Iw, H, -16, -12)
        wd = _grid(rng, H, Iw, -12, -8)
    x_bits = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    wg, wu, wd = (w.astype(np.float32) for w in (wg, wu, wd))
    blob = ocq.pack_weights(wg, wu, wd, prec)
    t, y = _run(blob, x_bits, H, Iw, prec)
    r = O.block_reference(x_bits, wg, wu, wd, prec)
    assert np.array_equal(t["x_codes"], r["xq"]) and np.array_equal(t["x_scales"], r["sx"])
    rel, mx = check_y(y, r["y"], "lossless y")
    print("lossless M=%d prec=%d: y normwise %.2e, max %.2e" % (M, prec, rel, mx))
    assert rel <= 2e-4


# The path the benchmark times: R calls with R weight copies captured into
# one HIP graph and replayed.  Every replay must reproduce the eager result
# bit for bit (the kernels are deterministic), with eager calls on another
# workspace and host synchronizations between the replays; the eager result
# is held to the oracle by the other parity tests and again here.

@pytest.mark.parametrize("H,Iw,M,prec", [(2048, 6144, 208, 0), (2048, 6144, 16, 0), (512, 1024, 37, 1),
                                         (512, 1024, 52, 2), (256, 768, 420, 0)])
def test_graph_replay_matches_eager(H, Iw, M, prec):
    from quantized_memory_bound_amd import inputs as I
    print("case graph replay hidden=%d inter=%d M=%d prec=%d" % (H, Iw, M, prec), flush=True)
    d = I.make_inputs(H, Iw, M, x_outliers=True, w_std=0.02, seed=H + Iw + M)
    blobs = [ocq.pack_weights(d["w_gate"], d["w_up"], d["w_down"], prec)]
    blobs.append(blobs[0].clone())
    x = _dev_bf16(d["x_bits"])
    ws = torch.empty(ocq.workspace_bytes(M, H, Iw, prec), dtype=torch.uint8, device="cuda")
    y_eager = ocq.mlp_forward(blobs[0], x, H, Iw, prec)
    torch.cuda.synchronize()
    ref = _bits(y_eager)
    r = O.block_reference(d["x_bits"], d["w_gate"], d["w_up"], d["w_down"], prec)
    check_y(ref, r["y"], "eager y")
    yg = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    graph = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=cs):
        for b in blobs:
            ocq.mlp_forward(b, x, H, Iw, prec, y=yg, workspace=ws)
    other = torch.empty(ocq.workspace_bytes(M, H, Iw, prec), dtype=torch.uint8, device="cuda")
    for rep in range(4):
        yg.fill_(0.0)
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(yg), ref), "graph replay %d differs from the eager call" % rep
        # eager work between replays: another call on another workspace
        ocq.mlp_forward(blobs[1], x, H, Iw, prec, workspace=other)
        torch.cuda.synchronize()


def test_graph_captured_stack_matches_eager():
    from quantized_memory_bound_amd import inputs as I
    print("case graph-captured stack", flush=True)
    H, Iw, M, modes = 512, 1024, 40, (1, 0, 2, 0)
    x_bits = I.make_inputs(H, Iw, M, x_outliers=True, seed=9, with_weights=False)["x_bits"]
    ds = [I.make_inputs(H, Iw, 1, w_std=0.02, seed=70 + l) for l in range(len(modes))]
    blobs = [ocq.pack_weights(d["w_gate"], d["w_up"], d["w_down"], m) for d, m in zip(ds, modes)]
    x = _dev_bf16(x_bits)
    y_eager = ocq.mlp_stack_forward(blobs, modes, x, H, Iw)
    torch.cuda.synchronize()
    ref = _bits(y_eager)
    # the last layer against the oracle block on the GPU's own input to it
    # (differences would compound through the quantizations of later layers)
    y_prev = _bits(ocq.mlp_stack_forward(blobs[:-1], modes[:-1], x, H, Iw))
    last = O.pack_block(ds[-1]["w_gate"], ds[-1]["w_up"], ds[-1]["w_down"], modes[-1])
    check_y(ref, O.forward(y_prev, last)["y"], "stack y (eager), last layer against the oracle")
    ws = torch.empty(ocq.stack_workspace_bytes(M, H, Iw, modes), dtype=torch.uint8, device="cuda")
    yg = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        ocq.mlp_stack_forward(blobs, modes, x, H, Iw, y=yg, workspace=ws)
    for rep in range(3):
        yg.fill_(0.0)
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(yg), ref), "stack graph replay %d differs" % rep
        ocq.mlp_stack_forward(blobs, modes, x, H, Iw)
        torch.cuda.synchronize()
