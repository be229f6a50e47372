"""Build the ocq HIP library (libocq.so) in-tree for gfx950.

    python -m quantized_memory_bound_amd.build        # or build() from Python
    python -m quantized_memory_bound_amd.build --phase-stamps

The second form builds libocq_phases.so, the same library with per-wave phase
stamps recorded in the GEMM main loops (ocq_diag_phase_stamps; load it by
setting OCQ_LIBRARY to its path).

Every translation unit is compiled with hipcc for gfx950 (packed fp32
arithmetic disabled), in parallel, then linked into one shared library next
to this file.  The library exports only the C ABI declared in include/ocq.h.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libocq.so")
BUILD_PHASES = os.path.join(HERE, "_build_phases")
LIB_PHASES = os.path.join(HERE, "libocq_phases.so")

SOURCES = ["api.cpp", "pack.cpp", "kernels.hip", "gemm_gateup.hip", "gemm_down.hip", "gemm_large.hip", "diag.hip",
           "noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src, build_dir=BUILD, defines=()):
    out = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + list(defines) + DEVICE + ["-c", os.path.join(CSRC, src), "-o", out]
    if src.endswith(".cpp"):
        cmd = [HIPCC] + COMMON + ["-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, msgs))
    return out, msgs


def build(verbose=False, phase_stamps=False):
    build_dir, lib_path = (BUILD_PHASES, LIB_PHASES) if phase_stamps else (BUILD, LIB)
    defines = ("-DOCQ_PHASE_STAMPS",) if phase_stamps else ()
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(lambda src: _compile(src, build_dir, defines), SOURCES))
    for _, msgs in results:
        if verbose and msgs.strip():
            print(msgs)
    objs = [o for o, _ in results]
    tmp = lib_path + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, phase_stamps="--phase-stamps" in sys.argv))
