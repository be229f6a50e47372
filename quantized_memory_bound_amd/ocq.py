"""Python binding of the ocq C ABI (include/ocq.h): argument marshalling only.

Every step of the block runs in the HIP library libocq.so built in-tree next
to this file (``python -m quantized_memory_bound_amd.build``).  There is no
fallback: if the library is missing, every call raises.  PyTorch is used only
for device memory and streams.
"""

import ctypes
import os

import numpy as np

# OCQ_LIBRARY names another build of the library (for instance
# libocq_phases.so, built with --phase-stamps); the default is the in-tree
# libocq.so
LIB_PATH = os.environ.get("OCQ_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libocq.so")

PREC_FP8 = 0
PREC_FP8_DOWN_BF16 = 1
PREC_FP4 = 2

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_DEVICE = -3
ERR_BUFFER_TOO_SMALL = -4
ERR_BAD_BLOB = -5

EXPORTS = ("ocq_version", "ocq_packed_bytes", "ocq_pack_weights_host", "ocq_pack_weights",
           "ocq_unpack_weights_host", "ocq_workspace_bytes", "ocq_mlp_forward", "ocq_check_blob",
           "ocq_set_stage_events", "ocq_last_error", "ocq_stack_workspace_bytes", "ocq_mlp_stack_forward",
           "ocq_calibrate_smoothing_host", "ocq_pack_weights_smoothed_host", "ocq_pack_weights_smoothed",
           "ocq_diag_stream_read", "ocq_diag_window_read", "ocq_diag_mfma_rate", "ocq_diag_empty", "ocq_diag_mfma_dot", "ocq_diag_phase_stamps", "ocq_noalloc_scratch_bytes",
           "ocq_mlp_forward_noalloc", "ocq_set_fused_requant", "ocq_last_requant_in_gateup")


class OcqError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("ocq status %d: %s" % (status, message))
        self.status = status


class Taps(ctypes.Structure):
    _fields_ = [("x_codes", ctypes.c_void_p), ("x_scales", ctypes.c_void_p),
                ("h_out", ctypes.c_void_p), ("h_scales", ctypes.c_void_p)]


_lib = None


def lib():
    """Load libocq.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libocq.so is not built (%s); run python -m quantized_memory_bound_amd.build" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i, f = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_float
    L.ocq_version.argtypes, L.ocq_version.restype = [], i
    L.ocq_last_error.argtypes, L.ocq_last_error.restype = [], ctypes.c_char_p
    L.ocq_packed_bytes.argtypes, L.ocq_packed_bytes.restype = [i, i, i], sz
    L.ocq_pack_weights_host.argtypes = [vp, vp, vp, i, i, i, vp, sz]
    L.ocq_pack_weights_host.restype = i
    L.ocq_pack_weights.argtypes = [vp, vp, vp, i, i, i, vp, sz, vp]
    L.ocq_pack_weights.restype = i
    L.ocq_pack_weights_smoothed_host.argtypes = [vp, vp, vp, vp, i, i, i, vp, sz]
    L.ocq_pack_weights_smoothed_host.restype = i
    L.ocq_pack_weights_smoothed.argtypes = [vp, vp, vp, vp, i, i, i, vp, sz, vp]
    L.ocq_pack_weights_smoothed.restype = i
    L.ocq_calibrate_smoothing_host.argtypes = [vp, i, i, vp, vp, i, f, vp]
    L.ocq_calibrate_smoothing_host.restype = i
    L.ocq_unpack_weights_host.argtypes = [vp, sz, i, vp, vp, ctypes.POINTER(f)]
    L.ocq_unpack_weights_host.restype = i
    L.ocq_workspace_bytes.argtypes, L.ocq_workspace_bytes.restype = [i, i, i, i], sz
    L.ocq_mlp_forward.argtypes = [vp, sz, vp, i, i, i, i, vp, vp, sz, ctypes.POINTER(Taps), vp]
    L.ocq_mlp_forward.restype = i
    L.ocq_check_blob.argtypes, L.ocq_check_blob.restype = [vp, sz, i, i, i, vp], i
    L.ocq_set_stage_events.argtypes, L.ocq_set_stage_events.restype = [ctypes.POINTER(vp), i], i
    ip = ctypes.POINTER(i)
    L.ocq_stack_workspace_bytes.argtypes, L.ocq_stack_workspace_bytes.restype = [i, i, i, ip, i], sz
    L.ocq_mlp_stack_forward.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(sz), ip, i, vp, i, i, i, vp, vp, sz, vp]
    L.ocq_mlp_stack_forward.restype = i
    L.ocq_set_fused_requant.argtypes, L.ocq_set_fused_requant.restype = [i], i
    L.ocq_last_requant_in_gateup.argtypes, L.ocq_last_requant_in_gateup.restype = [], i
    L.ocq_noalloc_scratch_bytes.argtypes, L.ocq_noalloc_scratch_bytes.restype = [], sz
    L.ocq_mlp_forward_noalloc.argtypes = [vp, sz, vp, i, i, i, i, vp, ctypes.POINTER(Taps), vp]
    L.ocq_mlp_forward_noalloc.restype = i
    L.ocq_diag_stream_read.argtypes, L.ocq_diag_stream_read.restype = [vp, sz, vp, i, vp], i
    L.ocq_diag_window_read.argtypes, L.ocq_diag_window_read.restype = [vp, sz, i, vp, i, vp], i
    L.ocq_diag_mfma_rate.argtypes, L.ocq_diag_mfma_rate.restype = [i, vp, i, vp, ctypes.POINTER(ctypes.c_double)], i
    L.ocq_diag_empty.argtypes, L.ocq_diag_empty.restype = [vp], i
    L.ocq_diag_mfma_dot.argtypes, L.ocq_diag_mfma_dot.restype = [i, vp, vp, i, i, i, vp, vp], i
    L.ocq_diag_phase_stamps.argtypes, L.ocq_diag_phase_stamps.restype = [i, vp, sz], i
    _lib = L
    return L


def _check(status):
    if status != OK:
        raise OcqError(status, lib().ocq_last_error().decode())
    return status


def last_error():
    return lib().ocq_last_error().decode()


def version():
    return lib().ocq_version()


def packed_bytes(hidden, inter, prec_mode):
    return lib().ocq_packed_bytes(hidden, inter, prec_mode)


def workspace_bytes(M, hidden, inter, prec_mode):
    return lib().ocq_workspace_bytes(M, hidden, inter, prec_mode)


def _f32c(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def calibrate_smoothing(x_calib_bits, w_gate, w_up, alpha=0.5):
    """Per-input-channel smoothing factors (float32 [hidden]) from calibration
    activations (bf16 bits [rows, hidden]) and the gate/up weights."""
    xb = np.ascontiguousarray(x_calib_bits, dtype=np.uint16)
    wg, wu = _f32c(w_gate), _f32c(w_up)
    inter, hidden = wg.shape
    s = np.empty(hidden, dtype=np.float32)
    _check(lib().ocq_calibrate_smoothing_host(xb.ctypes.data, xb.shape[0], hidden, wg.ctypes.data, wu.ctypes.data,
                                              inter, float(alpha), s.ctypes.data))
    return s


def pack_weights_host(w_gate, w_up, w_down, prec_mode, smooth=None):
    """Quantize + pack on the host; returns the blob as a uint8 numpy array.
    smooth: None or per-input-channel factors (float32 [hidden])."""
    wg, wu, wd = _f32c(w_gate), _f32c(w_up), _f32c(w_down)
    inter, hidden = wg.shape
    n = packed_bytes(hidden, inter, prec_mode)
    if n == 0:
        raise OcqError(ERR_UNSUPPORTED, "invalid shape or prec_mode")
    out = np.empty(n, dtype=np.uint8)
    sm = None if smooth is None else _f32c(smooth)
    _check(lib().ocq_pack_weights_smoothed_host(wg.ctypes.data, wu.ctypes.data, wd.ctypes.data,
                                                None if sm is None else sm.ctypes.data, hidden, inter,
                                                prec_mode, out.ctypes.data, n))
    return out


def unpack_weights_host(blob, which, hidden, inter, prec_mode):
    """Plain-layout codes / scales of one projection from a host blob."""
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    rows, cols = (inter, hidden) if which < 2 else (hidden, inter)
    bf16 = prec_mode == PREC_FP8_DOWN_BF16 and which == 2
    if which == 3:
        xm = np.zeros(hidden, dtype=np.float32)
        _check(lib().ocq_unpack_weights_host(blob.ctypes.data, blob.nbytes, 3, None, xm.ctypes.data, None))
        return None, xm, 0.0
    codes = np.zeros((rows, cols), dtype=np.uint16 if bf16 else np.uint8)
    if prec_mode == PREC_FP4:
        scales = np.zeros((rows, cols // 16), dtype=np.uint8)
    elif bf16:
        scales = None
    else:
        scales = np.zeros(rows, dtype=np.float32)
    ts = ctypes.c_float(0.0)
    _check(lib().ocq_unpack_weights_host(blob.ctypes.data, blob.nbytes, which, codes.ctypes.data,
                                         None if scales is None else scales.ctypes.data, ctypes.byref(ts)))
    return codes, scales, ts.value


def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def pack_weights(w_gate, w_up, w_down, prec_mode, device="cuda", stream=None, smooth=None):
    """Quantize + pack and upload; returns a uint8 torch tensor on `device`.
    smooth: None or per-input-channel factors (float32 [hidden])."""
    import torch
    wg, wu, wd = _f32c(w_gate), _f32c(w_up), _f32c(w_down)
    inter, hidden = wg.shape
    n = packed_bytes(hidden, inter, prec_mode)
    if n == 0:
        raise OcqError(ERR_UNSUPPORTED, "invalid shape or prec_mode")
    blob = torch.empty(n, dtype=torch.uint8, device=device)
    sm = None if smooth is None else _f32c(smooth)
    _check(lib().ocq_pack_weights_smoothed(wg.ctypes.data, wu.ctypes.data, wd.ctypes.data,
                                           None if sm is None else sm.ctypes.data, hidden, inter, prec_mode,
                                           blob.data_ptr(), n, _stream_handle(stream)))
    return blob


FUSED_REQUANT_DEFAULT = 1


def set_fused_requant(mode):
    """Process-wide: requantize h inside the gate/up kernel where its grid
    fits the GPU at once (1 or True, the default), or in a second kernel (0
    or False)."""
    _check(lib().ocq_set_fused_requant(int(mode)))


def last_requant_in_gateup():
    """1 if the last forward call on this thread requantized h inside the
    gate/up kernel, 0 if in a separate kernel, -1 before the first call."""
    return lib().ocq_last_requant_in_gateup()


def set_stage_events(events):
    """events: None (disable) or a list of 5 hipEvent_t handles (int or None)."""
    if events is None:
        _check(lib().ocq_set_stage_events(None, 0))
        return
    arr = (ctypes.c_void_p * 5)(*[e if e else None for e in events])
    _check(lib().ocq_set_stage_events(arr, 5))


def check_blob(blob, hidden, inter, prec_mode, stream=None):
    _check(lib().ocq_check_blob(blob.data_ptr(), blob.numel(), hidden, inter, prec_mode, _stream_handle(stream)))


def _need(t, name, dtype, device, shape=None, min_numel=None):
    """Raise OcqError(ERR_INVALID_ARG) unless t is a contiguous tensor of this
    dtype on this device (and shape / size): the C ABI takes raw pointers and
    would read or write past a tensor of another layout."""
    if t is None or not hasattr(t, "data_ptr"):
        raise OcqError(ERR_INVALID_ARG, "%s must be a tensor" % name)
    if t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise OcqError(ERR_INVALID_ARG, "%s has dtype %s" % (name, t.dtype))
    if t.device != device:
        raise OcqError(ERR_INVALID_ARG, "%s is on %s, not %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise OcqError(ERR_INVALID_ARG, "%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise OcqError(ERR_INVALID_ARG, "%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if min_numel is not None and t.numel() < min_numel:
        raise OcqError(ERR_BUFFER_TOO_SMALL, "%s holds %d elements, needs %d" % (name, t.numel(), min_numel))


def _check_x(x, hidden):
    import torch
    if not hasattr(x, "is_cuda") or not x.is_cuda:
        raise OcqError(ERR_INVALID_ARG, "x must be a CUDA tensor")
    if x.dim() != 2 or x.shape[1] != hidden:
        raise OcqError(ERR_INVALID_ARG, "x must be [M, hidden=%d], got %s" % (hidden, tuple(x.shape)))
    _need(x, "x", torch.bfloat16, x.device)


def _taps_struct(taps, M, hidden, inter, prec_mode, dev):
    """Checked Taps structure (or None) from a dict of optional tensors."""
    import torch
    if not taps:
        return None
    spec = {"x_codes": (torch.uint8, (M, hidden)), "x_scales": (torch.float32, (M,)),
            "h_out": ((torch.int16, torch.uint16) if prec_mode == PREC_FP8_DOWN_BF16 else torch.uint8, (M, inter)),
            "h_scales": (torch.float32, (M,))}
    for k, (dt, shp) in spec.items():
        if taps.get(k) is not None:
            _need(taps[k], "taps[%s]" % k, dt, dev, shape=shp)
    return Taps(*(taps[k].data_ptr() if taps.get(k) is not None else None
                  for k in ("x_codes", "x_scales", "h_out", "h_scales")))


def mlp_forward(blob, x, hidden, inter, prec_mode, y=None, workspace=None, taps=None, stream=None):
    """y = block(x) for x a bf16 [M, hidden] CUDA tensor; returns y (bf16 [M, hidden]).

    taps: optional dict with any of x_codes (uint8 [M, hidden]), x_scales
    (float32 [M]), h_out (uint8 [M, inter]; int16 / uint16 bf16 bits in the
    BF16-down mode) and h_scales (float32 [M]) tensors.  Every tensor must be
    contiguous and on x's device; otherwise OcqError is raised before the call.
    """
    import torch
    _check_x(x, hidden)
    M, dev = x.shape[0], x.device
    _need(blob, "blob", torch.uint8, dev, min_numel=packed_bytes(hidden, inter, prec_mode))
    if y is None:
        y = torch.empty((M, hidden), dtype=torch.bfloat16, device=dev)
    _need(y, "y", torch.bfloat16, dev, shape=(M, hidden))
    if workspace is None:
        workspace = torch.empty(max(1, workspace_bytes(M, hidden, inter, prec_mode)), dtype=torch.uint8,
                                device=dev)
    _need(workspace, "workspace", torch.uint8, dev)
    t = _taps_struct(taps, M, hidden, inter, prec_mode, dev)
    _check(lib().ocq_mlp_forward(blob.data_ptr(), blob.numel(), x.data_ptr(), M, hidden, inter, prec_mode,
                                 y.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                 ctypes.byref(t) if t is not None else None, _stream_handle(stream)))
    return y


def mlp_forward_noalloc(blob, x, hidden, inter, prec_mode, y=None, taps=None, stream=None):
    """As mlp_forward, through the entry point that allocates nothing (its
    workspace is the library's fixed per-device scratch array).  y (bf16
    [M, hidden]) must be given by callers that cannot allocate either."""
    import torch
    _check_x(x, hidden)
    M, dev = x.shape[0], x.device
    _need(blob, "blob", torch.uint8, dev, min_numel=packed_bytes(hidden, inter, prec_mode))
    if y is None:
        y = torch.empty((M, hidden), dtype=torch.bfloat16, device=dev)
    _need(y, "y", torch.bfloat16, dev, shape=(M, hidden))
    t = _taps_struct(taps, M, hidden, inter, prec_mode, dev)
    _check(lib().ocq_mlp_forward_noalloc(blob.data_ptr(), blob.numel(), x.data_ptr(), M, hidden, inter, prec_mode,
                                         y.data_ptr(), ctypes.byref(t) if t is not None else None,
                                         _stream_handle(stream)))
    return y


def noalloc_scratch_bytes():
    return lib().ocq_noalloc_scratch_bytes()


def _int_array(vals):
    return (ctypes.c_int * len(vals))(*[int(v) for v in vals])


def stack_workspace_bytes(M, hidden, inter, prec_modes):
    return lib().ocq_stack_workspace_bytes(M, hidden, inter, _int_array(prec_modes), len(prec_modes))


def mlp_stack_forward(blobs, prec_modes, x, hidden, inter, y=None, workspace=None, stream=None):
    """L blocks in sequence (block l's output is block l+1's input); returns the
    last block's y (bf16 [M, hidden]).  blobs: L uint8 CUDA tensors."""
    import torch
    if len(blobs) != len(prec_modes):
        raise ValueError("one prec_mode per blob")
    _check_x(x, hidden)
    M, dev = x.shape[0], x.device
    for l, (b, m) in enumerate(zip(blobs, prec_modes)):
        _need(b, "blobs[%d]" % l, torch.uint8, dev, min_numel=packed_bytes(hidden, inter, m))
    if y is None:
        y = torch.empty((M, hidden), dtype=torch.bfloat16, device=dev)
    _need(y, "y", torch.bfloat16, dev, shape=(M, hidden))
    if workspace is None:
        workspace = torch.empty(max(1, stack_workspace_bytes(M, hidden, inter, prec_modes)), dtype=torch.uint8,
                                device=dev)
    _need(workspace, "workspace", torch.uint8, dev)
    n = len(blobs)
    ptrs = (ctypes.c_void_p * n)(*[b.data_ptr() for b in blobs])
    sizes = (ctypes.c_size_t * n)(*[b.numel() for b in blobs])
    _check(lib().ocq_mlp_stack_forward(ptrs, sizes, _int_array(prec_modes), n, x.data_ptr(), M, hidden, inter,
                                       y.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                       _stream_handle(stream)))
    return y


class QuantizedMLP:
    """One packed block on the GPU with its workspace, for repeated calls."""

    def __init__(self, w_gate, w_up, w_down, prec_mode, device="cuda"):
        self.inter, self.hidden = np.asarray(w_gate).shape
        self.prec_mode = prec_mode
        self.device = device
        self.blob = pack_weights(w_gate, w_up, w_down, prec_mode, device)
        self._ws = {}

    def workspace(self, M):
        import torch
        if M not in self._ws:
            self._ws[M] = torch.empty(workspace_bytes(M, self.hidden, self.inter, self.prec_mode),
                                      dtype=torch.uint8, device=self.device)
        return self._ws[M]

    def __call__(self, x, y=None, taps=None, stream=None):
        return mlp_forward(self.blob, x, self.hidden, self.inter, self.prec_mode, y=y,
                           workspace=self.workspace(x.shape[0]), taps=taps, stream=stream)


# ---------------------------------------------------------------- measurement helpers

def diag_stream_read(src, out, blocks, stream=None):
    """Read the whole uint8 CUDA tensor src with the library's streaming-read
    kernel (out: int32 / uint8 CUDA tensor of >= 4 * blocks bytes)."""
    import torch
    _need(src, "src", torch.uint8, src.device)
    if out.numel() * out.element_size() < 4 * blocks:
        raise OcqError(ERR_BUFFER_TOO_SMALL, "out holds fewer than 4 * blocks bytes")
    _check(lib().ocq_diag_stream_read(src.data_ptr(), src.numel(), out.data_ptr(), blocks, _stream_handle(stream)))


def diag_window_read(src, window_bytes, passes, out, blocks, stream=None):
    """Every one of `blocks` workgroups reads src[:window_bytes] `passes` times
    (src: uint8 CUDA tensor; out: int32 / uint8 CUDA tensor of >= 4 * blocks
    bytes)."""
    import torch
    _need(src, "src", torch.uint8, src.device)
    if window_bytes > src.numel():
        raise OcqError(ERR_BUFFER_TOO_SMALL, "window larger than src")
    if out.numel() * out.element_size() < 4 * blocks:
        raise OcqError(ERR_BUFFER_TOO_SMALL, "out holds fewer than 4 * blocks bytes")
    _check(lib().ocq_diag_window_read(src.data_ptr(), window_bytes, passes, out.data_ptr(), blocks,
                                      _stream_handle(stream)))


def diag_mfma_rate(iters, out, blocks, stream=None):
    """Launch the matrix-core rate kernel (out: float32 CUDA tensor of >= 512 *
    blocks elements); returns the launch's floating-point operations."""
    import torch
    _need(out, "out", torch.float32, out.device)
    if out.numel() < 512 * blocks:
        raise OcqError(ERR_BUFFER_TOO_SMALL, "out holds fewer than 512 * blocks floats")
    fl = ctypes.c_double()
    _check(lib().ocq_diag_mfma_rate(iters, out.data_ptr(), blocks, _stream_handle(stream), ctypes.byref(fl)))
    return fl.value


def diag_empty(stream=None):
    _check(lib().ocq_diag_empty(_stream_handle(stream)))


PHASE_SHAPES = {0: (2, 512, 8, 8), 1: (512, 12, 8), 2: (2, 1024, 2)}


def diag_phase_stamps(kernel):
    """Phase stamp table of the last launch (kernel 0: LDS-tiled GEMMs,
    kernel 1: producer/consumer gate/up, kernel 2: x quantization and
    requantization) as a uint64 array of shape PHASE_SHAPES[kernel]; needs a
    library built with --phase-stamps."""
    if kernel not in PHASE_SHAPES:
        raise OcqError(ERR_INVALID_ARG, "kernel must be 0, 1 or 2")
    out = np.zeros(PHASE_SHAPES[kernel], dtype=np.uint64)
    _check(lib().ocq_diag_phase_stamps(kernel, out.ctypes.data, out.nbytes))
    return out


def diag_mfma_dot(form, a_codes, b_codes, stream=None):
    """c = dec(a) dec(b)^T (float32 [M, N]) over E4M3 code tensors a [M, K],
    b [N, K] (uint8, CUDA) through matrix-core form 0 (f16), 1 (f8f6f4 K=128)
    or 2 (fp8 K=32)."""
    import torch
    M, K = a_codes.shape
    N = b_codes.shape[0]
    _need(a_codes, "a", torch.uint8, a_codes.device)
    _need(b_codes, "b", torch.uint8, a_codes.device, shape=(N, K))
    c = torch.empty((M, N), dtype=torch.float32, device=a_codes.device)
    _check(lib().ocq_diag_mfma_dot(form, a_codes.data_ptr(), b_codes.data_ptr(), M, N, K, c.data_ptr(),
                                   _stream_handle(stream)))
    return c
