"""Host-side checks of the C-ABI library (no GPU needed).

* the library loads and exports every entry point include/ocq.h declares;
* the host packer's codes and scales equal the oracle's bit for bit (read
  back through ocq_unpack_weights_host, the inverse of the fragment layout);
* argument validation returns the documented status before touching a GPU.
"""

import ctypes
import os
import re
import threading

import numpy as np
import pytest

from oracle import mlp as O
from quantized_memory_bound_amd import inputs as I
from quantized_memory_bound_amd import ocq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    with open(os.path.join(ROOT, "include", "ocq.h")) as f:
        hdr = f.read()
    declared = set(re.findall(r"\b(ocq_[a-z_]+)\s*\(", hdr))
    assert declared == set(ocq.EXPORTS), declared ^ set(ocq.EXPORTS)
    L = ocq.lib()
    for name in declared:
        assert hasattr(L, name), name
    assert ocq.version() >= 10000


def test_phase_stamps_need_the_stamped_build():
    """The plain library reports that it records no phase stamps (before any
    device call), and the arguments are checked first."""
    if os.path.abspath(ocq.LIB_PATH) != os.path.join(ROOT, "quantized_memory_bound_amd", "libocq.so"):
        pytest.skip("another library was selected through OCQ_LIBRARY")
    L = ocq.lib()
    buf = np.zeros(2 * 512 * 8 * 8, dtype=np.uint64)
    assert L.ocq_diag_phase_stamps(3, buf.ctypes.data, buf.nbytes) == ocq.ERR_INVALID_ARG
    assert L.ocq_diag_phase_stamps(-1, buf.ctypes.data, buf.nbytes) == ocq.ERR_INVALID_ARG
    assert L.ocq_diag_phase_stamps(0, None, buf.nbytes) == ocq.ERR_INVALID_ARG
    assert L.ocq_diag_phase_stamps(0, buf.ctypes.data, buf.nbytes - 8) == ocq.ERR_BUFFER_TOO_SMALL
    assert L.ocq_diag_phase_stamps(1, buf.ctypes.data, 512 * 12 * 8 * 8 - 1) == ocq.ERR_BUFFER_TOO_SMALL
    assert L.ocq_diag_phase_stamps(2, buf.ctypes.data, 2 * 1024 * 2 * 8 - 1) == ocq.ERR_BUFFER_TOO_SMALL
    for kernel in (0, 1, 2):
        assert L.ocq_diag_phase_stamps(kernel, buf.ctypes.data, buf.nbytes) == ocq.ERR_UNSUPPORTED
        assert b"phase stamps" in ocq.lib().ocq_last_error()
    assert ocq.PHASE_SHAPES == {0: (2, 512, 8, 8), 1: (512, 12, 8), 2: (2, 1024, 2)}


def test_requant_placement_mode_is_checked():
    """The requantization mode takes 0 or 1; the report of where the last
    call requantized h reads -1 on a thread that made no forward call."""
    L = ocq.lib()
    assert ocq.FUSED_REQUANT_DEFAULT == 1
    for bad in (-1, 2, 100):
        assert L.ocq_set_fused_requant(bad) == ocq.ERR_INVALID_ARG
        assert b"mode" in L.ocq_last_error()
    for good in (0, 1):
        assert L.ocq_set_fused_requant(good) == ocq.OK
    ocq.set_fused_requant(ocq.FUSED_REQUANT_DEFAULT)
    res = []
    t = threading.Thread(target=lambda: res.append(ocq.last_requant_in_gateup()))
    t.start()
    t.join()
    assert res == [-1]


def _packer_vs_oracle(hidden, inter, prec, seed=0, w_std=0.02):
    d = I.make_inputs(hidden, inter, 1, w_std=w_std, seed=seed)
    blob = ocq.pack_weights_host(d["w_gate"], d["w_up"], d["w_down"], prec)
    ref = O.pack_block(d["w_gate"], d["w_up"], d["w_down"], prec)
    for which, key in enumerate(("gate", "up", "down")):
        codes, scales, ts = ocq.unpack_weights_host(blob, which, hidden, inter, prec)
        r = ref[key]
        if prec == O.PREC_FP4:
            assert np.array_equal(codes, r[0]), key
            assert np.array_equal(scales, r[1]), key
            assert np.float32(ts) == r[2], key
        elif prec == O.PREC_FP8_DOWN_BF16 and key == "down":
            assert np.array_equal(codes, r), key
        else:
            assert np.array_equal(codes, r[0]), key
            assert np.array_equal(scales, r[1]), key


@pytest.mark.parametrize("prec", [0, 1, 2])
@pytest.mark.parametrize("hidden,inter", [(256, 512), (384, 640), (128, 1152)])
def test_packer_matches_oracle_small(hidden, inter, prec):
    _packer_vs_oracle(hidden, inter, prec, seed=hidden + inter)


@pytest.mark.parametrize("name", ["decode_fp8", "mixed_bf16_down", "nvfp4"])
def test_packer_matches_oracle_workload_shapes(name):
    cfg = I.WORKLOADS[name]
    _packer_vs_oracle(cfg["hidden"], cfg["inter"], cfg["prec_mode"], seed=0, w_std=cfg["w_std"])


def test_packer_zero_and_outlier_rows():
    hidden, inter = 256, 512
    d = I.make_inputs(hidden, inter, 1, seed=3)
    d["w_gate"][5] = 0.0                       # zero row -> scale 0, codes 0
    d["w_up"][7, 3] = 1e4                      # outlier
    d["w_down"][:, :16] = 0.0                  # zero NVFP4 blocks
    for prec in (0, 1, 2):
        blob = ocq.pack_weights_host(d["w_gate"], d["w_up"], d["w_down"], prec)
        ref = O.pack_block(d["w_gate"], d["w_up"], d["w_down"], prec)
        for which, key in enumerate(("gate", "up", "down")):
            codes, scales, ts = ocq.unpack_weights_host(blob, which, hidden, inter, prec)
            r = ref[key]
            rc = r if (prec == 1 and key == "down") else r[0]
            assert np.array_equal(codes, rc), (prec, key)


def test_packed_and_workspace_sizes():
    assert ocq.packed_bytes(2048, 6144, 0) >= 3 * 2048 * 6144
    assert ocq.packed_bytes(4096, 12288, 2) >= 3 * 4096 * 12288 // 2
    assert ocq.packed_bytes(100, 6144, 0) == 0
    assert ocq.packed_bytes(2048, 6144, 3) == 0
    assert ocq.workspace_bytes(208, 2048, 6144, 0) > 0
    assert ocq.workspace_bytes(0, 2048, 6144, 0) == 0
    assert ocq.workspace_bytes(8193, 2048, 6144, 0) == 0


def _fwd(**kw):
    a = dict(blob=0x10000, nblob=1 << 30, x=0x20000, M=16, hidden=2048, inter=6144, prec=0, y=0x30000,
             ws=0x40000, nws=1 << 30, taps=None, stream=None)
    a.update(kw)
    return ocq.lib().ocq_mlp_forward(a["blob"], a["nblob"], a["x"], a["M"], a["hidden"], a["inter"], a["prec"],
                                     a["y"], a["ws"], a["nws"], a["taps"], a["stream"])


def test_forward_argument_errors():
    assert _fwd(hidden=2000) == ocq.ERR_UNSUPPORTED
    assert _fwd(inter=100) == ocq.ERR_UNSUPPORTED
    assert _fwd(prec=7) == ocq.ERR_INVALID_ARG
    assert _fwd(M=0) == ocq.ERR_INVALID_ARG
    assert _fwd(M=9000) == ocq.ERR_INVALID_ARG
    assert _fwd(x=None) == ocq.ERR_INVALID_ARG
    assert _fwd(y=0x30008) == ocq.ERR_INVALID_ARG          # misaligned
    assert _fwd(nblob=1000) == ocq.ERR_BUFFER_TOO_SMALL
    assert _fwd(nws=1000) == ocq.ERR_BUFFER_TOO_SMALL
    assert "workspace" in ocq.last_error()
    taps = ocq.Taps(0x50004, None, None, None)
    assert _fwd(taps=ctypes.pointer(taps)) == ocq.ERR_INVALID_ARG


def test_pack_argument_errors():
    L = ocq.lib()
    w = np.zeros((512, 256), np.float32)
    out = np.zeros(10, np.uint8)
    assert L.ocq_pack_weights_host(w.ctypes.data, w.ctypes.data, w.ctypes.data, 256, 512, 0, out.ctypes.data, 10) \
        == ocq.ERR_BUFFER_TOO_SMALL
    assert L.ocq_pack_weights_host(None, w.ctypes.data, w.ctypes.data, 256, 512, 0, out.ctypes.data, 10) \
        == ocq.ERR_INVALID_ARG
    assert L.ocq_pack_weights_host(w.ctypes.data, w.ctypes.data, w.ctypes.data, 250, 512, 0, out.ctypes.data, 10) \
        == ocq.ERR_UNSUPPORTED


def test_unpack_rejects_bad_blob():
    d = I.make_inputs(256, 512, 1, seed=1)
    blob = ocq.pack_weights_host(d["w_gate"], d["w_up"], d["w_down"], 0)
    bad = blob.copy()
    bad[0] ^= 0xFF
    with pytest.raises(ocq.OcqError) as e:
        ocq.unpack_weights_host(bad, 0, 256, 512, 0)
    assert e.value.status == ocq.ERR_BAD_BLOB
    with pytest.raises(ocq.OcqError) as e:
        ocq.unpack_weights_host(blob[:1000], 0, 256, 512, 0)
    assert e.value.status == ocq.ERR_BUFFER_TOO_SMALL


def test_forward_without_device_reports_device_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st = _fwd()
    assert st == ocq.ERR_DEVICE, (st, ocq.last_error())


def test_stack_workspace_sizes():
    one = ocq.workspace_bytes(208, 2048, 6144, 0)
    both = ocq.stack_workspace_bytes(208, 2048, 6144, [0, 1, 2])
    assert both >= max(one, ocq.workspace_bytes(208, 2048, 6144, 1)) + 208 * 2048 * 2
    assert ocq.stack_workspace_bytes(208, 2048, 6144, [0, 3]) == 0
    assert ocq.stack_workspace_bytes(0, 2048, 6144, [0]) == 0
    assert ocq.lib().ocq_stack_workspace_bytes(16, 2048, 6144, None, 1) == 0
    assert ocq.stack_workspace_bytes(16, 2048, 6144, []) == 0


def _stack(**kw):
    a = dict(blobs=[0x10000, 0x20000], nblobs=[1 << 30, 1 << 30], modes=[0, 2], x=0x30000, M=16, hidden=2048,
             inter=6144, y=0x40000, ws=0x50000, nws=1 << 30, stream=None)
    a.update(kw)
    n = len(a["modes"])
    blobs = None if a["blobs"] is None else (ctypes.c_void_p * max(1, n))(*a["blobs"])
    sizes = (ctypes.c_size_t * max(1, n))(*a["nblobs"])
    modes = (ctypes.c_int * max(1, n))(*a["modes"])
    return ocq.lib().ocq_mlp_stack_forward(blobs, sizes, modes, a.get("L", n), a["x"], a["M"], a["hidden"],
                                           a["inter"], a["y"], a["ws"], a["nws"], a["stream"])


def test_stack_argument_errors():
    assert _stack(L=0) == ocq.ERR_INVALID_ARG
    assert _stack(L=2000) == ocq.ERR_INVALID_ARG
    assert _stack(blobs=None) == ocq.ERR_INVALID_ARG
    assert _stack(modes=[0, 5]) == ocq.ERR_INVALID_ARG
    assert _stack(hidden=2000) == ocq.ERR_UNSUPPORTED
    assert _stack(M=0) == ocq.ERR_INVALID_ARG
    assert _stack(blobs=[0x10000, 0x20008]) == ocq.ERR_INVALID_ARG      # misaligned
    assert _stack(blobs=[0x10000, 0]) == ocq.ERR_INVALID_ARG
    assert _stack(nblobs=[1 << 30, 1000]) == ocq.ERR_BUFFER_TOO_SMALL
    assert _stack(x=None) == ocq.ERR_INVALID_ARG
    assert _stack(nws=1000) == ocq.ERR_BUFFER_TOO_SMALL
    assert "workspace" in ocq.last_error()


def test_calibration_matches_oracle():
    d = I.make_inputs(384, 640, 40, x_outliers=True, w_std=0.03, seed=9)
    for alpha in (0.0, 0.35, 0.5, 1.0):
        s_lib = ocq.calibrate_smoothing(d["x_bits"], d["w_gate"], d["w_up"], alpha)
        s_ref = O.calibrate_smoothing(d["x_bits"], d["w_gate"], d["w_up"], alpha)
        assert np.array_equal(s_lib, s_ref), alpha


@pytest.mark.parametrize("prec", [0, 1, 2])
def test_smoothed_packer_matches_oracle(prec):
    d = I.make_inputs(256, 512, 32, x_outliers=True, w_std=0.02, seed=prec + 4)
    s = O.calibrate_smoothing(d["x_bits"], d["w_gate"], d["w_up"], 0.5)
    blob = ocq.pack_weights_host(d["w_gate"], d["w_up"], d["w_down"], prec, smooth=s)
    ref = O.pack_block(d["w_gate"], d["w_up"], d["w_down"], prec, smooth=s)
    for which, key in enumerate(("gate", "up", "down")):
        codes, scales, ts = ocq.unpack_weights_host(blob, which, 256, 512, prec)
        r = ref[key]
        if prec == O.PREC_FP4:
            assert np.array_equal(codes, r[0]) and np.array_equal(scales, r[1]) and np.float32(ts) == r[2], key
        elif prec == O.PREC_FP8_DOWN_BF16 and key == "down":
            assert np.array_equal(codes, r), key
        else:
            assert np.array_equal(codes, r[0]) and np.array_equal(scales, r[1]), key
    _, xmul, _ = ocq.unpack_weights_host(blob, 3, 256, 512, prec)
    assert np.array_equal(xmul, ref["xmul"])
    plain = ocq.pack_weights_host(d["w_gate"], d["w_up"], d["w_down"], prec)
    assert np.all(ocq.unpack_weights_host(plain, 3, 256, 512, prec)[1] == 1.0)


def test_smoothing_argument_errors():
    L = ocq.lib()
    w = np.zeros((512, 256), np.float32)
    x = np.zeros((4, 256), np.uint16)
    s = np.ones(256, np.float32)
    out = np.zeros(ocq.packed_bytes(256, 512, 0), np.uint8)
    assert L.ocq_calibrate_smoothing_host(x.ctypes.data, 4, 256, w.ctypes.data, w.ctypes.data, 512, 1.5,
                                          s.ctypes.data) == ocq.ERR_INVALID_ARG
    assert L.ocq_calibrate_smoothing_host(x.ctypes.data, 0, 256, w.ctypes.data, w.ctypes.data, 512, 0.5,
                                          s.ctypes.data) == ocq.ERR_INVALID_ARG
    bad = s.copy()
    bad[7] = 0.0
    assert L.ocq_pack_weights_smoothed_host(w.ctypes.data, w.ctypes.data, w.T.copy().ctypes.data, bad.ctypes.data,
                                            256, 512, 0, out.ctypes.data, out.nbytes) == ocq.ERR_INVALID_ARG
    bad[7] = np.inf
    assert L.ocq_pack_weights_smoothed_host(w.ctypes.data, w.ctypes.data, w.T.copy().ctypes.data, bad.ctypes.data,
                                            256, 512, 0, out.ctypes.data, out.nbytes) == ocq.ERR_INVALID_ARG


def test_binding_rejects_host_tensors():
    import torch
    d = I.make_inputs(256, 512, 4, seed=2)
    x = torch.from_numpy(d["x_bits"].view(np.int16)).view(torch.bfloat16)
    with pytest.raises(ocq.OcqError) as e:
        ocq.mlp_forward(torch.zeros(10, dtype=torch.uint8), x, 256, 512, 0)
    assert e.value.status == ocq.ERR_INVALID_ARG


def test_noalloc_argument_errors():
    # checked before any device call: an invalid shape or M is reported as by
    # ocq_mlp_forward, a call larger than the scratch array as too small
    L = ocq.lib()
    assert L.ocq_noalloc_scratch_bytes() == 32 << 20
    assert L.ocq_mlp_forward_noalloc(0x10000, 1 << 30, 0x20000, 4, 2000, 512, 0, 0x30000, None, None) \
        == ocq.ERR_UNSUPPORTED
    assert L.ocq_mlp_forward_noalloc(0x10000, 1 << 30, 0x20000, 0, 256, 512, 0, 0x30000, None, None) \
        == ocq.ERR_INVALID_ARG
    assert L.ocq_mlp_forward_noalloc(0x10000, 1 << 30, 0x20000, 8192, 4096, 12288, 1, 0x30000, None, None) \
        == ocq.ERR_BUFFER_TOO_SMALL
    assert "no-allocation" in ocq.last_error()
