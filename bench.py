#!/usr/bin/env python3
"""Benchmark of the quantized spec-verify MLP block on one MI355X.

A step is one pass of the whole block (x-quant, gate/up + SiLU(gate)*up +
per-token requant, down projection) over one batch of M rows.  Default
workload: hidden 2048, inter 6144, M = 208 rows (16 requests x (1 + 12 draft
tokens)), FP8 E4M3 weights in all three projections, synthetic seeded
inputs (x ~ N(0,1) in bf16, weights ~ N(0, 0.02) quantized per output row).

Timing: R copies of the packed weights are rotated so that R x blob >= 512 MB,
twice the MI355X's 256 MB last-level (Infinity) cache, as consecutive layers
of a model would see.  Inputs are resident in HBM before the timed region.
The stream is pre-filled behind a GPU spin so the K timed steps run back to
back on the GPU (the host-side cost of a call, ~20 us in Python, would
otherwise pace the ~10 us steps).  HIP events bracket the K steps; the
library's stage-event hook brackets the gate/up kernel of every step.

Output: one JSON line (see the field list at the end of main()).
"""

import argparse
import ctypes
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0   # dense fp16 / bf16
MFMA_FP8_PEAK_TFLOPS = 5000.0   # dense fp8
MALL_BYTES = 256 << 20


def alg_bytes(M, H, I, prec):
    """Compulsory traffic of one block: weight codes + weight scales + the
    blob's per-channel x multiplier + x (bf16, read once) + y (bf16, written
    once)."""
    if prec == 0:
        w = 2 * I * H + 2 * I * 4 + H * I + H * 4
    elif prec == 1:
        w = 2 * I * H + 2 * I * 4 + 2 * H * I
    else:
        w = I * H + 2 * I * H // 16 + 8 + H * I // 2 + H * I // 16 + 4
    return w + H * 4 + 2 * M * H * 2


def gateup_alg(M, H, I, prec, requant_inside=False):
    """Gate/up kernel: weight codes + scales + x codes and scales read once
    (h stays on chip in the method, so its spill is not counted), plus the h
    codes and row scales it writes when it requantizes h itself; and flops."""
    if prec in (0, 1):
        w = 2 * I * H + 2 * I * 4
    else:
        w = I * H + 2 * I * H // 16 + 8
    out = M * I + M * 4 if requant_inside else 0
    return w + M * H + M * 4 + out, 2.0 * M * H * 2 * I


class HipEvents:
    """Minimal hipEvent_t access through libamdhip64 (for the library hook)."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        if self.h.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.h.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, e):
        self.h.hipEventDestroy(e)


def _code_only(text):
    """Source text without comments and blank lines (whitespace normalised)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    lines = (re.sub(r"//.*", "", l).split() for l in text.splitlines())
    return "\n".join(" ".join(l) for l in lines if l)


def kernel_source_digest(read=None):
    """Digest of the gate/up kernel's code (comments and blank lines ignored):
    the counters in profiles/ are reported only while it is unchanged.
    read(name) -> text overrides where the sources come from."""
    h = hashlib.sha256()
    for name in ("gemm_gateup.hip", "gemm_core.h", "kcommon.h"):
        if read is not None:
            text = read(name)
        else:
            with open(os.path.join(ROOT, "quantized_memory_bound_amd", "csrc", name)) as f:
                text = f.read()
        h.update(_code_only(text).encode())
    return h.hexdigest()[:16]


def read_traffic(workload, digest):
    """HBM traffic of the gate/up kernel from a committed rocprofv3 --pmc
    summary, if it was taken on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", "gateup_%s_pmc_traffic.txt" % workload)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        for line in f:
            if line.startswith("TRAFFIC_JSON "):
                d = json.loads(line[len("TRAFFIC_JSON "):])
                if d.get("source_digest") == digest:
                    return d.get("bytes_per_dispatch")
    return None


def cpu_baseline(inp, prec, M, seconds):
    """The oracle (plain fp64 numpy) timed on this host's cores on the same
    block: all M rows, pre-packed weights, repeated until `seconds` pass."""
    from threadpoolctl import threadpool_info
    from oracle import mlp as O
    packed = O.pack_block(inp["w_gate"], inp["w_up"], inp["w_down"], prec)
    O.forward(inp["x_bits"], packed)                       # warm caches
    reps, t0 = 0, time.perf_counter()
    while True:
        O.forward(inp["x_bits"], packed)
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = (time.perf_counter() - t0) / reps
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    return dt, reps, threads


def capture_steps(torch, step, n):
    """A HIP graph of steps 0 .. n-1 (None for n = 0), captured on a side stream."""
    if n == 0:
        return None
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        for i in range(n):
            step(i)
    return g


def roofline(nbytes, flops, prec, seconds, traffic):
    """Roofline object of the gate/up kernel.  Binding bound (the larger of
    the two times): HBM at 8 TB/s for the algorithmic bytes, or the matrix
    cores at the peak of the contraction's own type -- E4M3 x E4M3 (FP8,
    5 PFLOP/s) for the E4M3 weights; NVFP4 on its exact dequantized path at
    the fp16 rate (2.5 PFLOP/s).  frac is against the binding bound; the other
    fractions are given beside it, including the f16 peak of the instruction
    the kernel runs (its E4M3 operands are converted exactly to fp16)."""
    mfma_peak = MFMA_F16_PEAK_TFLOPS if prec == 2 else MFMA_FP8_PEAK_TFLOPS
    t_hbm = nbytes / (HBM_PEAK_GBPS * 1e9)
    t_mfma = flops / (mfma_peak * 1e12)
    gbps = nbytes / seconds / 1e9
    tflops = flops / seconds / 1e12
    if t_mfma > t_hbm:
        r = {"bound": "mfma", "achieved": round(tflops, 2), "peak": mfma_peak, "unit": "TFLOP/s",
             "frac": round(tflops / mfma_peak, 4)}
    else:
        r = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
             "frac": round(gbps / HBM_PEAK_GBPS, 4)}
    r["traffic"] = traffic
    r["alg_bytes_per_launch"] = nbytes
    r["alg_flops_per_launch"] = flops
    r["frac_hbm"] = round(gbps / HBM_PEAK_GBPS, 4)
    r["frac_mfma_fp8"] = round(tflops / MFMA_FP8_PEAK_TFLOPS, 4)
    r["frac_mfma_f16"] = round(tflops / MFMA_F16_PEAK_TFLOPS, 4)
    return r


def stream_ceiling(torch, ocq, nbytes, dev, reps=64):
    """GB/s of the library's plain streaming-read kernel reading nbytes per
    launch (rounded to 16 B), launches replayed from a graph over a 1 GiB
    buffer so no read hits the 256 MB last-level cache."""
    n = max(16, nbytes // 16 * 16)
    span = max(1 << 30, 4 * n)
    buf = torch.ones(span, dtype=torch.uint8, device=dev)
    out = torch.empty(2048, dtype=torch.int32, device=dev)
    nslot = span // n
    step = lambda i: ocq.diag_stream_read(buf[(i % nslot) * n:(i % nslot + 1) * n], out, 2048)
    g = capture_steps(torch, step, reps)
    g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    g.replay()
    t1.record()
    torch.cuda.synchronize()
    sec = t0.elapsed_time(t1) * 1e-3 / reps
    del buf
    return n / sec / 1e9


def l2_ceiling(torch, ocq, dev, window=1 << 20, passes=64, blocks=512):
    """GB/s at which L2 feeds the CUs: every workgroup re-reads one 1 MiB
    window (resident in each XCD's L2) with the library's window-read
    kernel; one timed launch after a warm-up launch."""
    buf = torch.ones(window, dtype=torch.uint8, device=dev)
    out = torch.empty(blocks, dtype=torch.int32, device=dev)
    ocq.diag_window_read(buf, window, passes, out, blocks)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    ocq.diag_window_read(buf, window, passes, out, blocks)
    t1.record()
    torch.cuda.synchronize()
    return window * passes * blocks / (t0.elapsed_time(t1) * 1e-3) / 1e9


def mfma_ceiling(torch, ocq, dev, iters=4000, blocks=512):
    """TFLOP/s of independent f16 MFMA 16x16x32 on register operands (two
    8-wave workgroups per CU), one timed launch after a warm-up launch."""
    out = torch.empty(512 * blocks, dtype=torch.float32, device=dev)
    ocq.diag_mfma_rate(iters, out, blocks)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    flops = ocq.diag_mfma_rate(iters, out, blocks)
    t1.record()
    torch.cuda.synchronize()
    return flops / (t0.elapsed_time(t1) * 1e-3) / 1e12


def launch_floor(torch, ocq, reps=200):
    """Seconds per launch of an empty kernel, replayed from a graph."""
    g = capture_steps(torch, lambda i: ocq.diag_empty(), reps)
    g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) * 1e-3 / reps


def vendor_gemm(args, reps=200):
    """Context, not the block: torch's matmul (hipBLASLt) in fp16 and bf16 on
    the workload's two GEMM shapes (M x H x 2I for gate/up, M x I x H for
    down), plain GEMMs on random operands without the block's quantization,
    SiLU epilogue or operand conversions.  One JSON line."""
    import torch
    from quantized_memory_bound_amd import inputs as I
    cfg = I.WORKLOADS[args.workload]
    H, Iw = cfg["hidden"], cfg["inter"]
    M = args.M if args.M is not None else cfg["M"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    torch.manual_seed(0)
    rows = []
    for dt in (torch.float16, torch.bfloat16):
        for what, k, n in (("gate/up", H, 2 * Iw), ("down", Iw, H)):
            a = torch.randn(M, k, device=dev, dtype=dt)
            # weights stored [N, K] as the block stores them (used transposed), or [K, N]
            for layout in ("NK", "KN"):
                b = torch.randn(n, k, device=dev, dtype=dt).t() if layout == "NK" else \
                    torch.randn(k, n, device=dev, dtype=dt)
                for _ in range(10):
                    torch.mm(a, b)
                torch.cuda.synchronize()
                t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                t0.record()
                for _ in range(reps):
                    torch.mm(a, b)
                t1.record()
                torch.cuda.synchronize()
                us = t0.elapsed_time(t1) * 1e3 / reps
                fl = 2.0 * M * k * n
                rows.append({"gemm": what, "dtype": str(dt).split(".")[-1], "weights": layout, "M": M, "K": k, "N": n,
                             "us": round(us, 2), "TFLOPs": round(fl / us / 1e6, 1),
                             "frac_f16_peak": round(fl / us / 1e6 / MFMA_F16_PEAK_TFLOPS, 4)})
                del b
            del a
    print(json.dumps({"vendor_gemm": rows, "workload": args.workload, "reps": reps}))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="spec_verify_fp8",
                    help="a block workload (inputs.WORKLOADS) or a stack of blocks (inputs.STACKS)")
    ap.add_argument("--M", type=int, default=None, help="leading rows of the workload (NVFP4 sweep)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stage-events", action="store_true", help="skip the gate/up kernel timing pass")
    ap.add_argument("--mode", choices=["graph", "eager"], default="graph",
                    help="graph: replay a captured HIP graph of R steps; eager: one call per step")
    ap.add_argument("--fused-requant", type=int, choices=[0, 1], default=1,
                    help="where h is requantized: 1 (the library's default) inside the gate/up kernel where "
                         "its grid fits the GPU at once, 0 in a second kernel")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 256 MiB copy kernel (counter calibration for rocprofv3 --pmc)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="instead of the block: time torch's fp16 / bf16 matmul (the vendor GEMM) on the "
                         "workload's gate/up and down shapes, for context")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: measures one GPU only; the block is row-independent and shards as data "
              "parallel over requests with no exchange between GPUs. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from quantized_memory_bound_amd import inputs as I
    from quantized_memory_bound_amd import ocq

    ocq.set_fused_requant(args.fused_requant)
    if args.vendor_gemm:
        return vendor_gemm(args)
    if args.workload in I.STACKS:
        return run_stack(args)
    cfg = I.WORKLOADS[args.workload]
    H, Iw, prec = cfg["hidden"], cfg["inter"], cfg["prec_mode"]
    inp = I.workload_inputs(args.workload, M=args.M)
    M = inp["x_bits"].shape[0]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    blob0 = ocq.pack_weights(inp["w_gate"], inp["w_up"], inp["w_down"], prec)
    R = max(2, -(-2 * MALL_BYTES // blob0.numel()))
    blobs = [blob0] + [blob0.clone() for _ in range(R - 1)]
    x = torch.from_numpy(inp["x_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(ocq.workspace_bytes(M, H, Iw, prec), dtype=torch.uint8, device=dev)
    if args.copy_calib:
        src = torch.ones(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.add(src, 0, out=dst)
    torch.cuda.synchronize()

    def step(i):
        ocq.mlp_forward(blobs[i % R], x, H, Iw, prec, y=y, workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = args.steps
    ev = HipEvents()

    # --- timed region: K steps, HIP events on the stream the kernels run on
    if args.mode == "graph":
        # one captured graph holds R consecutive steps (one per weight copy),
        # a second one the K mod R steps left over, so exactly K steps run
        full, rest = capture_steps(torch, step, R), capture_steps(torch, step, K % R)
        for g in (full, rest):
            if g is not None:
                g.replay()
        torch.cuda.synchronize()
        t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_start.record()
        for _ in range(K // R):
            full.replay()
        if rest is not None:
            rest.replay()
        t_end.record()
        torch.cuda.synchronize()
    else:
        t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        # keep the GPU busy while the host enqueues the steps (~25 us each)
        torch.cuda._sleep(int(2.4e9 * max(0.02, 30e-6 * K)))
        t_start.record()
        for i in range(K):
            step(i)
        t_end.record()
        torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / K

    # --- gate/up kernel duration: stage events 1 and 2 are recorded by the
    # gate/up launch itself (start and end of that kernel's execution); steps
    # enqueued behind a GPU spin so they run back to back
    gu_ms = None
    gu_how = None
    if not args.no_stage_events:
        Kr = min(256, args.steps)
        ga = [ev.create() for _ in range(Kr)]
        gb = [ev.create() for _ in range(Kr)]
        torch.cuda.synchronize()
        torch.cuda._sleep(int(2.4e9 * 0.02))
        for i in range(Kr):
            ocq.set_stage_events([None, ga[i], gb[i], None, None])
            step(i)
        ocq.set_stage_events(None)
        torch.cuda.synchronize()
        gu = [ev.elapsed_ms(a, b) for a, b in zip(ga, gb)]
        gu_ms = sum(gu) / len(gu)
        gu_how = "start/end events of the gate/up launch, %d eager steps" % len(gu)
        for e in ga + gb:
            ev.destroy(e)

    ab = alg_bytes(M, H, Iw, prec)
    gbps = ab / (ms_step * 1e-3) / 1e9
    tok_s = M / (ms_step * 1e-3)

    inside = ocq.last_requant_in_gateup() == 1
    roof = None
    if gu_ms:
        gbytes, gflops = gateup_alg(M, H, Iw, prec, inside)
        traffic = read_traffic(args.workload if args.M is None else "%s_M%d" % (args.workload, M),
                               kernel_source_digest())
        roof = roofline(gbytes, gflops, prec, gu_ms * 1e-3, traffic)
        roof["kernel"] = ("gate/up GEMM + SiLU*up + per-token requantization" if inside
                          else "gate/up GEMM + SiLU*up + per-token amax")
        roof["us_per_launch"] = round(gu_ms * 1e3, 3)
        roof["timing"] = gu_how
        ceil = stream_ceiling(torch, ocq, gbytes, dev)
        roof["stream_ceiling_GBps"] = round(ceil, 1)
        roof["frac_of_stream_ceiling"] = round(gbytes / (gu_ms * 1e-3) / 1e9 / ceil, 4)
        roof["launch_floor_us"] = round(launch_floor(torch, ocq) * 1e6, 3)
        l2 = l2_ceiling(torch, ocq, dev)
        roof["l2_ceiling_GBps"] = round(l2, 1)
        mf = mfma_ceiling(torch, ocq, dev)
        roof["mfma_f16_ceiling_TFLOPs"] = round(mf, 1)
        roof["frac_of_mfma_f16_ceiling"] = round(gflops / (gu_ms * 1e-3) / 1e12 / mf, 4)

    cpu = None
    if not args.no_cpu_baseline:
        dt, reps, threads = cpu_baseline(inp, prec, M, args.cpu_seconds)
        cpu = {"value": round(ab / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
               "sample": "whole block, all %d rows, weights pre-packed, %d repetitions (%.2f s each)" % (M, reps, dt),
               "tokens_per_s": round(M / dt, 1), "us_per_block": round(dt * 1e6, 1), "cpu_model": cpu_model()}

    prec_name = {0: "fp8_e4m3", 1: "fp8_e4m3 gate/up + bf16 down", 2: "nvfp4 (e2m1 + e4m3 block scales)"}[prec]
    out = {
        "metric": "achieved HBM GB/s (% of peak) + verified tokens/s per MLP block, M=208",
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "mode": args.mode,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3" if prec == 0 else prec_name,
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": {"workload": args.workload, "hidden": H, "inter": Iw, "M": M, "prec_mode": prec_name,
                   "weight_copies_rotated": R, "alg_bytes_per_block": ab,
                   "requant": "inside gate/up" if inside else "separate kernel"},
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "tokens_per_s": round(tok_s, 1),
        "us_per_block": round(ms_step * 1e3, 3),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def run_stack(args):
    """A stack of blocks with a precision mode per layer: a step is one pass
    of the whole stack (block l's output is block l+1's input).  Weight sets
    of the stack are rotated (R x stack bytes >= 512 MB) and R steps replay as
    one captured graph, as for one block."""
    import numpy as np
    import torch
    from quantized_memory_bound_amd import inputs as I
    from quantized_memory_bound_amd import ocq

    cfg = I.STACKS[args.workload]
    H, Iw, M, modes = cfg["hidden"], cfg["inter"], cfg["M"], list(cfg["modes"])
    x_bits, layers = I.stack_inputs(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    blobs0 = [ocq.pack_weights(wg, wu, wd, m) for (wg, wu, wd), m in zip(layers, modes)]
    stack_bytes = sum(b.numel() for b in blobs0)
    R = max(2, -(-2 * MALL_BYTES // stack_bytes))
    sets = [blobs0] + [[b.clone() for b in blobs0] for _ in range(R - 1)]
    x = torch.from_numpy(x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(ocq.stack_workspace_bytes(M, H, Iw, modes), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(i):
        ocq.mlp_stack_forward(sets[i % R], modes, x, H, Iw, y=y, workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    full, rest = capture_steps(torch, step, R), capture_steps(torch, step, K % R)
    for g in (full, rest):
        if g is not None:
            g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(K // R):
        full.replay()
    if rest is not None:
        rest.replay()
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / K

    ab = sum(alg_bytes(M, H, Iw, m) for m in modes)
    gbps = ab / (ms_step * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info
        from oracle import mlp as O
        packed = [O.pack_block(wg, wu, wd, m) for (wg, wu, wd), m in zip(layers, modes)]
        O.stack_forward(x_bits, packed)
        reps, c0 = 0, time.perf_counter()
        while True:
            O.stack_forward(x_bits, packed)
            reps += 1
            if time.perf_counter() - c0 >= args.cpu_seconds:
                break
        dt = (time.perf_counter() - c0) / reps
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
        cpu = {"value": round(ab / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
               "sample": "whole stack, all %d rows, weights pre-packed, %d repetitions (%.2f s each)" % (M, reps, dt),
               "tokens_per_s": round(M / dt, 1), "cpu_model": cpu_model()}
    names = {0: "fp8", 1: "fp8+bf16down", 2: "nvfp4"}
    out = {
        "metric": "achieved HBM GB/s (% of peak) + verified tokens/s per MLP stack (" + str(len(modes)) + " blocks)",
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "mode": "graph",
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "per layer: " + ",".join(names[m] for m in modes),
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": {"workload": args.workload, "hidden": H, "inter": Iw, "M": M, "layers": len(modes),
                   "prec_modes": modes, "weight_sets_rotated": R, "alg_bytes_per_step": ab,
                   "weight_bytes_per_step": stack_bytes},
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "tokens_per_s": round(M / (ms_step * 1e-3), 1),
        "us_per_step": round(ms_step * 1e3, 3),
        "us_per_layer": round(ms_step * 1e3 / len(modes), 3),
        "roofline": None,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
