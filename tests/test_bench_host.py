"""Host-side checks of bench.py's bookkeeping (no GPU): the digest that ties
the committed traffic counters to the gate/up kernel's code, and the lookup
of those counters."""

import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _sources():
    d = os.path.join(ROOT, "quantized_memory_bound_amd", "csrc")
    return {n: open(os.path.join(d, n)).read() for n in ("gemm_gateup.hip", "gemm_core.h", "kcommon.h")}


def test_digest_ignores_comments_and_blank_lines():
    b, src = _bench(), _sources()
    ref = b.kernel_source_digest(lambda n: src[n])
    assert ref == b.kernel_source_digest()
    edited = dict(src)
    edited["gemm_core.h"] = "// a new comment\n\n" + src["gemm_core.h"].replace("\n", "  \n", 3) + "\n/* block\ncomment */\n"
    assert b.kernel_source_digest(lambda n: edited[n]) == ref


@pytest.mark.parametrize("edit", [lambda t: t.replace("kPcProducers = 4", "kPcProducers = 2", 1),
                                  lambda t: t + "\nstatic int extra_symbol;\n"])
def test_digest_follows_code(edit):
    b, src = _bench(), _sources()
    ref = b.kernel_source_digest(lambda n: src[n])
    edited = dict(src)
    edited["gemm_gateup.hip"] = edit(src["gemm_gateup.hip"])
    assert edited["gemm_gateup.hip"] != src["gemm_gateup.hip"]
    assert b.kernel_source_digest(lambda n: edited[n]) != ref


def test_traffic_lookup_needs_matching_digest():
    b = _bench()
    d = b.kernel_source_digest()
    t = b.read_traffic("spec_verify_fp8", d)
    assert t is None or (isinstance(t, int) and t > 25_000_000)   # at least the algorithmic bytes
    assert b.read_traffic("spec_verify_fp8", "0" * 16) is None
    assert b.read_traffic("no_such_workload", d) is None
