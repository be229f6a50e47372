"""The library built with phase stamps (libocq_phases.so) computes what the
plain library computes, bit for bit, and fills its stamp tables.

The stamps only read clocks where the waves wait anyway, so a block run
through either library must give identical x codes, h codes (or bf16 h),
scales and y.  Shapes: the LDS-tiled kernels for many rows (420 rows, BF16
down; the whole-chunk gate/up stages at hidden 256), the producer/consumer
gate/up (208 rows, hidden 2048, FP8; h requantized inside the launch) with
the x quantization.  The stamped library runs in a child process (one
library per process in the binding), which writes its outputs and the stamp
tables to a file.
"""

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

from quantized_memory_bound_amd import inputs as I
from quantized_memory_bound_amd import ocq
from test_gpu_parity import run_gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PHASES = os.path.join(ROOT, "quantized_memory_bound_amd", "libocq_phases.so")

CHILD = r'''
import sys, numpy as np
sys.path.insert(0, sys.argv[1]); sys.path.insert(0, sys.argv[1] + "/tests")
from quantized_memory_bound_amd import inputs as I, ocq
from test_gpu_parity import run_gpu
H, Iw, M, prec, seed, out = int(sys.argv[2]), int(sys.argv[3]), int(sys.argv[4]), int(sys.argv[5]), int(sys.argv[6]), sys.argv[7]
d = I.make_inputs(H, Iw, M, x_outliers=True, w_std=0.02, seed=seed)
g, _ = run_gpu(d, prec)
g.update({"stamps%d" % k: ocq.diag_phase_stamps(k) for k in (0, 1, 2)})
g["lib"] = np.array(ocq.LIB_PATH)
np.savez(out, **g)
'''


@pytest.mark.gpu
@pytest.mark.parametrize("H,Iw,M,prec,family", [(256, 768, 420, 1, 0), (2048, 6144, 208, 0, 1)])
def test_phase_stamped_library_matches_plain(tmp_path, H, Iw, M, prec, family):
    print("case phase stamps hidden=%d inter=%d M=%d prec=%d" % (H, Iw, M, prec), flush=True)
    if not os.path.exists(PHASES):
        pytest.skip("libocq_phases.so is not built (python -m quantized_memory_bound_amd.build --phase-stamps)")
    seed = H + Iw + M
    d = I.make_inputs(H, Iw, M, x_outliers=True, w_std=0.02, seed=seed)
    plain, _ = run_gpu(d, prec)
    out = str(tmp_path / "stamped.npz")
    env = dict(os.environ, OCQ_LIBRARY=PHASES)
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT, str(H), str(Iw), str(M), str(prec), str(seed), out],
                       env=env, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    s = np.load(out)
    assert str(s["lib"]).endswith("libocq_phases.so")
    for k, v in plain.items():
        assert np.array_equal(v, s[k]), k
    # the launched kernels filled their tables: LDS-tiled loop totals, or the
    # producer/consumer and quantization stamps
    if family == 0:
        t = s["stamps0"]
        assert np.all(t[0, 0, :, 4] > 0) and np.all(t[1, 0, :, 4] > 0)   # gate/up and down, workgroup 0
        assert np.all(t[0, 0, :, 5] == H // 128)          # whole-chunk gate/up stages
        assert np.all(t[1, 0, :, 5] == 2 * (Iw // 128))   # down: two stages per chunk
    else:
        t = s["stamps1"]
        assert np.all(t[0, :, 0] > 0) and np.all(t[0, :8, 2] >= t[0, :8, 1])
        # h requantized inside the launch (the default): arrival, release and
        # row scales in that order on every wave
        assert np.all(t[0, :, 5] > 0) and np.all(t[0, :, 6] >= t[0, :, 5]) and np.all(t[0, :, 7] >= t[0, :, 6])
    q = s["stamps2"]
    assert np.all(q[0, :, 1] >= q[0, :, 0]) and (q[0, :, 0] > 0).sum() == M   # one x-quant workgroup per row
