"""Where the GEMM kernels' time goes: per-wave phase stamps of one workload.

    python -m quantized_memory_bound_amd.build --phase-stamps
    python -m quantized_memory_bound_amd.phase_stamps --workload mixed_bf16_down

Runs the workload's block a few dozen times on cuda:0 with the library built
with phase stamps (libocq_phases.so, or the library OCQ_LIBRARY names) and
prints, from the stamps of the last launch:

* LDS-tiled GEMMs (many rows): per wave, the totals of its waits for its own
  direct-to-LDS loads, of the workgroup barriers, of the MFMA batches (with the
  loads, LDS reads and conversions placed between their MFMAs), of the wait
  for LDS reads after each batch, and of the whole loop, in shader-clock ticks
  per stage; medians over every wave, and per wave slot for the barrier and
  the batches (wave slot w runs on SIMD w mod 4);
* the producer/consumer gate/up (one 208-row block): microseconds from the
  first wave's start to each consumer's loop start, loop end, stored partial
  tiles and end, as medians over the workgroups;
* the x quantization and the requantization: the span from the first
  workgroup's start to the last one's end (its stores landed) and the median
  workgroup's duration, to set beside the kernels' traced durations.

The stamps are only a timing aid; the blocks they time compute the same
results as the plain library (the stamps sit where the waves wait anyway).
"""

import argparse
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
os.environ.setdefault("OCQ_LIBRARY", os.path.join(HERE, "libocq_phases.so"))
sys.path.insert(0, os.path.dirname(HERE))

import numpy as np  # noqa: E402

from quantized_memory_bound_amd import inputs as I  # noqa: E402
from quantized_memory_bound_amd import ocq  # noqa: E402


def lds_tiled_summary(t):
    lines = []
    for k, name in enumerate(("gate/up", "down")):
        b = t[k].astype(np.float64)          # [workgroup][wave][field]
        ok = b[:, :, 4] > 0
        if not ok.any():
            continue
        v = b[ok]
        ns = v[0, 5]
        tot = np.median(v[:, 4])
        lines.append("%s (LDS-tiled): %d waves of the recorded workgroups, %d stages; ticks per stage (medians)"
                     % (name, len(v), ns))
        for j, f in enumerate(("load wait", "barrier", "MFMA batches", "LDS-read wait", "whole loop")):
            lines.append("  %-14s %8.1f  (%5.1f %%)" % (f, np.median(v[:, j]) / ns, 100 * np.median(v[:, j]) / tot))
        rest = v[:, 4] - v[:, :4].sum(axis=1)
        lines.append("  %-14s %8.1f" % ("rest", np.median(rest) / ns))
        full = b[:, :, 4].min(axis=1) > 0
        for j, f in ((1, "barrier"), (2, "MFMA batches")):
            lines.append("  %-14s per wave slot: %s" % (f, " ".join("%.0f" % (np.median(b[full, w, j]) / ns)
                                                                for w in range(8))))
    return lines


def pc_summary(t):
    b = t.astype(np.float64)                 # [workgroup][wave][field]
    n = int((b[:, 0, 0] > 0).sum())
    if n == 0:
        return []
    b = b[:n]
    t0 = b[:, :, 0][b[:, :, 0] > 0].min()
    c = (b[:, :8] - t0) / 100.0              # consumers, microseconds from the first start
    med = np.median
    lines = ["producer/consumer gate/up: %d workgroups; microseconds (medians over workgroups and consumer waves)" % n,
             "  wave start: first 0.00, median %.2f, last %.2f" % (med(c[:, :, 0]), c[:, :, 0].max()),
             "  start -> consumer loop %.2f, loop (with the wait for the first stage) %.2f, partial tiles %.2f, epilogue %.2f"
             % (med(c[:, :, 1] - c[:, :, 0]), med(c[:, :, 2] - c[:, :, 1]), med(c[:, :, 3] - c[:, :, 2]),
                med(c[:, :, 4] - c[:, :, 3]))]
    if (b[:, :, 5:8] > 0).all():             # the launch requantized h itself
        w = (b - t0) / 100.0
        arrive = w[:, :, 5].max(axis=1)      # a workgroup arrives with its last wave
        lines += ["  epilogue with the requantization inside the launch: SiLU and row maxima folded %.2f, wait %.2f,"
                  " row scales %.2f, codes staged %.2f" % (med(c[:, :, 5] - c[:, :, 3]), med(c[:, :, 6] - c[:, :, 5]),
                                                           med(c[:, :, 7] - c[:, :, 6]), med(c[:, :, 4] - c[:, :, 7])),
                  "  workgroup arrival: first %.2f, median %.2f, last %.2f; released from %.2f to %.2f"
                  % (arrive.min(), med(arrive), arrive.max(), c[:, :, 6].min(), c[:, :, 6].max())]
    return lines + ["  last wave end %.2f" % (((b[:, :, 4] - t0) / 100.0).max())]


def quant_summary(t):
    lines = []
    for k, name in enumerate(("x quantization", "requantization")):
        v = t[k].astype(np.float64)
        v = v[v[:, 0] > 0]
        if not len(v):
            continue
        t0 = v[:, 0].min()
        lines.append("%s: %d workgroups; last start %.2f us, median workgroup %.2f us, last end %.2f us after the first start"
                     % (name, len(v), (v[:, 0].max() - t0) / 100.0, np.median(v[:, 1] - v[:, 0]) / 100.0,
                        (v[:, 1].max() - t0) / 100.0))
    return lines


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--workload", default="mixed_bf16_down", choices=sorted(I.WORKLOADS))
    ap.add_argument("--M", type=int, default=None)
    ap.add_argument("--launches", type=int, default=40)
    a = ap.parse_args(argv)
    import torch
    assert torch.cuda.is_available(), "needs a GPU"
    cfg = I.WORKLOADS[a.workload]
    H, Iw, p = cfg["hidden"], cfg["inter"], cfg["prec_mode"]
    d = I.workload_inputs(a.workload, M=a.M)
    blobs = [ocq.pack_weights(d["w_gate"], d["w_up"], d["w_down"], p)]
    blobs += [blobs[0].clone() for _ in range(3)]       # weights not all warm in the caches
    x = torch.from_numpy(d["x_bits"].view(np.int16)).to("cuda").view(torch.bfloat16)
    M = x.shape[0]
    y = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(ocq.workspace_bytes(M, H, Iw, p), dtype=torch.uint8, device="cuda")
    for i in range(a.launches):
        ocq.mlp_forward(blobs[i % len(blobs)], x, H, Iw, p, y=y, workspace=ws)
    torch.cuda.synchronize()
    print("workload %s, M=%d, library %s" % (a.workload, M, ocq.LIB_PATH))
    for line in (lds_tiled_summary(ocq.diag_phase_stamps(0)) + pc_summary(ocq.diag_phase_stamps(1)) +
                 quant_summary(ocq.diag_phase_stamps(2))):
        print(line)


if __name__ == "__main__":
    main()
