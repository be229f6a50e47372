// C-ABI entry points of the ocq library: argument checks, planning, launches.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "ocq_internal.h"

namespace ocq {

static thread_local std::string g_err;
static thread_local void* g_stage_events[5];
static thread_local bool g_stage_on = false;
static thread_local int g_last_requant = -1;

ocq_status set_error(ocq_status st, const char* msg) {
  g_err = msg ? msg : "";
  return st;
}

static ocq_status set_hip_error(hipError_t e, const char* where) {
  char buf[256];
  std::snprintf(buf, sizeof(buf), "%s: %s (%d)", where, hipGetErrorString(e), (int)e);
  return set_error(OCQ_ERR_DEVICE, buf);
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static ocq_status check_shape(int hidden, int inter, int prec_mode) {
  if (prec_mode < 0 || prec_mode > 2) return set_error(OCQ_ERR_INVALID_ARG, "prec_mode must be 0, 1 or 2");
  if (!shape_ok(hidden, inter))
    return set_error(OCQ_ERR_UNSUPPORTED, "hidden and inter must be multiples of 128 in [128, 65536]");
  return OCQ_OK;
}

}  // namespace ocq

using namespace ocq;

extern "C" {

int ocq_version(void) { return 10000; }

const char* ocq_last_error(void) { return g_err.c_str(); }

int ocq_last_requant_in_gateup(void) { return g_last_requant; }

ocq_status ocq_set_stage_events(void* const* events, int count) {
  g_err.clear();
  if (events == nullptr || count == 0) {
    g_stage_on = false;
    return OCQ_OK;
  }
  if (count != 5) return set_error(OCQ_ERR_INVALID_ARG, "count must be 5 (or 0 to disable)");
  for (int i = 0; i < 5; ++i) g_stage_events[i] = events[i];
  g_stage_on = true;
  return OCQ_OK;
}

ocq_status ocq_set_fused_requant(int mode) {
  g_err.clear();
  if (mode != 0 && mode != 1) return set_error(OCQ_ERR_INVALID_ARG, "fused requantization mode must be 0 or 1");
  set_fused_requant(mode);
  return OCQ_OK;
}

size_t ocq_packed_bytes(int hidden, int inter, int prec_mode) {
  if (prec_mode < 0 || prec_mode > 2 || !shape_ok(hidden, inter)) return 0;
  return blob_layout(hidden, inter, prec_mode).total;
}

ocq_status ocq_pack_weights_smoothed_host(const float* w_gate_host, const float* w_up_host, const float* w_down_host,
                                          const float* smooth_host, int hidden, int inter, int prec_mode,
                                          void* packed_host, size_t packed_bytes) {
  g_err.clear();
  ocq_status st = check_shape(hidden, inter, prec_mode);
  if (st != OCQ_OK) return st;
  if (!w_gate_host || !w_up_host || !w_down_host || !packed_host)
    return set_error(OCQ_ERR_INVALID_ARG, "null weight or output pointer");
  return pack_host(w_gate_host, w_up_host, w_down_host, hidden, inter, prec_mode, smooth_host, (uint8_t*)packed_host,
                   packed_bytes);
}

ocq_status ocq_pack_weights_host(const float* w_gate_host, const float* w_up_host, const float* w_down_host,
                                 int hidden, int inter, int prec_mode, void* packed_host, size_t packed_bytes) {
  return ocq_pack_weights_smoothed_host(w_gate_host, w_up_host, w_down_host, nullptr, hidden, inter, prec_mode,
                                        packed_host, packed_bytes);
}

ocq_status ocq_calibrate_smoothing_host(const void* x_calib_bf16_host, int rows, int hidden, const float* w_gate_host,
                                        const float* w_up_host, int inter, float alpha, float* s_out) {
  g_err.clear();
  if (!shape_ok(hidden, inter))
    return set_error(OCQ_ERR_UNSUPPORTED, "hidden and inter must be multiples of 128 in [128, 65536]");
  if (!x_calib_bf16_host || !w_gate_host || !w_up_host || !s_out || rows < 1)
    return set_error(OCQ_ERR_INVALID_ARG, "null pointer or no calibration rows");
  if (!(alpha >= 0.0f && alpha <= 1.0f)) return set_error(OCQ_ERR_INVALID_ARG, "alpha must be in [0, 1]");
  return calibrate_host((const uint16_t*)x_calib_bf16_host, rows, hidden, w_gate_host, w_up_host, inter, alpha, s_out);
}

ocq_status ocq_pack_weights(const float* w_gate_host, const float* w_up_host, const float* w_down_host, int hidden,
                            int inter, int prec_mode, void* packed_dev, size_t packed_bytes, void* stream) {
  return ocq_pack_weights_smoothed(w_gate_host, w_up_host, w_down_host, nullptr, hidden, inter, prec_mode, packed_dev,
                                   packed_bytes, stream);
}

ocq_status ocq_pack_weights_smoothed(const float* w_gate_host, const float* w_up_host, const float* w_down_host,
                                     const float* smooth_host, int hidden, int inter, int prec_mode, void* packed_dev,
                                     size_t packed_bytes, void* stream) {
  g_err.clear();
  ocq_status st = check_shape(hidden, inter, prec_mode);
  if (st != OCQ_OK) return st;
  if (!w_gate_host || !w_up_host || !w_down_host || !packed_dev)
    return set_error(OCQ_ERR_INVALID_ARG, "null weight or output pointer");
  if (!aligned16(packed_dev)) return set_error(OCQ_ERR_INVALID_ARG, "packed_dev must be 16-byte aligned");
  const size_t need = blob_layout(hidden, inter, prec_mode).total;
  if (packed_bytes < need) return set_error(OCQ_ERR_BUFFER_TOO_SMALL, "packed_bytes < ocq_packed_bytes()");
  std::vector<uint8_t> host(need);
  st = pack_host(w_gate_host, w_up_host, w_down_host, hidden, inter, prec_mode, smooth_host, host.data(), need);
  if (st != OCQ_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(packed_dev, host.data(), need, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return set_hip_error(e, "hipMemcpyAsync(blob)");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return set_hip_error(e, "hipStreamSynchronize(blob copy)");
  return OCQ_OK;
}

ocq_status ocq_unpack_weights_host(const void* packed_host, size_t packed_bytes, int which, void* codes_out,
                                   void* scales_out, float* tensor_scale_out) {
  g_err.clear();
  if (!packed_host) return set_error(OCQ_ERR_INVALID_ARG, "null blob pointer");
  return unpack_host((const uint8_t*)packed_host, packed_bytes, which, codes_out, scales_out, tensor_scale_out);
}

size_t ocq_workspace_bytes(int M, int hidden, int inter, int prec_mode) {
  if (prec_mode < 0 || prec_mode > 2 || !shape_ok(hidden, inter) || M < 1 || M > 8192) return 0;
  return make_plan(M, hidden, inter, prec_mode).total;
}

ocq_status ocq_check_blob(const void* packed_dev, size_t packed_bytes, int hidden, int inter, int prec_mode,
                          void* stream) {
  g_err.clear();
  ocq_status st = check_shape(hidden, inter, prec_mode);
  if (st != OCQ_OK) return st;
  if (!packed_dev) return set_error(OCQ_ERR_INVALID_ARG, "null blob pointer");
  if (packed_bytes < sizeof(BlobHeader)) return set_error(OCQ_ERR_BUFFER_TOO_SMALL, "blob smaller than its header");
  BlobHeader hd;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(&hd, packed_dev, sizeof(hd), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return set_hip_error(e, "reading blob header");
  if (std::memcmp(hd.magic, kBlobMagic, 8) != 0 || hd.version != kBlobVersion)
    return set_error(OCQ_ERR_BAD_BLOB, "bad blob magic or version");
  if (hd.hidden != hidden || hd.inter != inter || hd.prec_mode != prec_mode)
    return set_error(OCQ_ERR_BAD_BLOB, "blob was packed for other dimensions or another prec_mode");
  if (hd.total_bytes != blob_layout(hidden, inter, prec_mode).total || packed_bytes < hd.total_bytes)
    return set_error(OCQ_ERR_BAD_BLOB, "blob size does not match its layout");
  return OCQ_OK;
}

ocq_status ocq_mlp_forward(const void* packed_dev, size_t packed_bytes, const void* x_bf16_dev, int M, int hidden,
                           int inter, int prec_mode, void* y_bf16_dev, void* workspace_dev, size_t workspace_bytes,
                           const ocq_taps* taps, void* stream) {
  g_err.clear();
  ocq_status st = check_shape(hidden, inter, prec_mode);
  if (st != OCQ_OK) return st;
  if (M < 1 || M > 8192) return set_error(OCQ_ERR_INVALID_ARG, "M must be in [1, 8192]");
  if (!packed_dev || !x_bf16_dev || !y_bf16_dev || !workspace_dev)
    return set_error(OCQ_ERR_INVALID_ARG, "null device pointer");
  if (!aligned16(packed_dev) || !aligned16(x_bf16_dev) || !aligned16(y_bf16_dev) || !aligned16(workspace_dev))
    return set_error(OCQ_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  if (packed_bytes < blob_layout(hidden, inter, prec_mode).total)
    return set_error(OCQ_ERR_BUFFER_TOO_SMALL, "packed_bytes < ocq_packed_bytes()");
  const Plan p = make_plan(M, hidden, inter, prec_mode);
  if (workspace_bytes < p.total) return set_error(OCQ_ERR_BUFFER_TOO_SMALL, "workspace_bytes < ocq_workspace_bytes()");
  if (taps) {
    const void* tp[4] = {taps->x_codes, taps->x_scales, taps->h_out, taps->h_scales};
    for (const void* t : tp)
      if (t && !aligned16(t)) return set_error(OCQ_ERR_INVALID_ARG, "tap pointers must be 16-byte aligned");
  }
  FwdArgs a{(const uint8_t*)packed_dev, (const uint16_t*)x_bf16_dev, (uint16_t*)y_bf16_dev, (uint8_t*)workspace_dev,
            stream, g_stage_on ? g_stage_events : nullptr, ocq_taps{}};
  if (taps) a.taps = *taps;
  a.requant_in_gateup = &g_last_requant;
  int rc = launch_forward(p, a);
  if (rc != 0) return set_hip_error((hipError_t)rc, "kernel launch");
  return OCQ_OK;
}

ocq_status ocq_diag_stream_read(const void* src_dev, size_t bytes, void* out_dev, int blocks, void* stream) {
  g_err.clear();
  if (!src_dev || !out_dev || !aligned16(src_dev)) return set_error(OCQ_ERR_INVALID_ARG, "null or misaligned pointer");
  if (bytes == 0 || bytes % 16 || blocks < 1 || blocks > 65536)
    return set_error(OCQ_ERR_INVALID_ARG, "bytes must be a positive multiple of 16, blocks in [1, 65536]");
  int rc = diag_stream_read(src_dev, bytes, out_dev, blocks, stream);
  return rc ? set_hip_error((hipError_t)rc, "kernel launch") : OCQ_OK;
}

ocq_status ocq_diag_window_read(const void* src_dev, size_t window_bytes, int passes, void* out_dev, int blocks,
                                void* stream) {
  g_err.clear();
  if (!src_dev || !out_dev || !aligned16(src_dev)) return set_error(OCQ_ERR_INVALID_ARG, "null or misaligned pointer");
  if (window_bytes < 32768 || window_bytes % 32768 || window_bytes > ((size_t)1 << 30) || passes < 1 ||
      passes > 65536 || blocks < 1 || blocks > 65536)
    return set_error(OCQ_ERR_INVALID_ARG,
                     "window_bytes a multiple of 32768 up to 2^30, passes in [1, 65536], blocks in [1, 65536]");
  int rc = diag_window_read(src_dev, window_bytes, passes, out_dev, blocks, stream);
  return rc ? set_hip_error((hipError_t)rc, "kernel launch") : OCQ_OK;
}

ocq_status ocq_diag_mfma_rate(int iters, void* out_dev, int blocks, void* stream, double* flops) {
  g_err.clear();
  if (!out_dev || iters < 1 || iters > (1 << 20) || blocks < 1 || blocks > 65536)
    return set_error(OCQ_ERR_INVALID_ARG, "out_dev non-null, iters in [1, 2^20], blocks in [1, 65536]");
  if (flops) *flops = (double)diag_mfma_rate_flops(iters, blocks);
  int rc = diag_mfma_rate(iters, (float*)out_dev, blocks, stream);
  return rc ? set_hip_error((hipError_t)rc, "kernel launch") : OCQ_OK;
}

ocq_status ocq_diag_empty(void* stream) {
  g_err.clear();
  int rc = diag_empty(stream);
  return rc ? set_hip_error((hipError_t)rc, "kernel launch") : OCQ_OK;
}

ocq_status ocq_diag_phase_stamps(int kernel, void* host_out, size_t bytes) {
  g_err.clear();
  if (kernel < 0 || kernel > 2) return set_error(OCQ_ERR_INVALID_ARG, "kernel must be 0, 1 or 2");
  if (!host_out) return set_error(OCQ_ERR_INVALID_ARG, "host_out is null");
  const size_t need = kernel == 0 ? kLgPhaseBytes : kernel == 1 ? kPcPhaseBytes : kQPhaseBytes;
  if (bytes < need) return set_error(OCQ_ERR_BUFFER_TOO_SMALL, "host_out smaller than the stamp table");
  const int rc = kernel == 0 ? lg_phase_copy(host_out, bytes)
               : kernel == 1 ? pc_phase_copy(host_out, bytes) : q_phase_copy(host_out, bytes);
  if (rc == -1) return set_error(OCQ_ERR_UNSUPPORTED, "library built without phase stamps (build --phase-stamps)");
  return rc ? set_hip_error((hipError_t)rc, "copy of the stamp table") : OCQ_OK;
}

ocq_status ocq_diag_mfma_dot(int form, const void* a_dev, const void* b_dev, int M, int N, int K, float* c_dev,
                             void* stream) {
  g_err.clear();
  if (form < 0 || form > 2) return set_error(OCQ_ERR_INVALID_ARG, "form must be 0, 1 or 2");
  if (M < 16 || N < 16 || K < 128 || M % 16 || N % 16 || K % 128 || M > 65536 || N > 65536 || K > 65536)
    return set_error(OCQ_ERR_INVALID_ARG, "M, N multiples of 16 and K a multiple of 128, each <= 65536");
  if (!a_dev || !b_dev || !c_dev || !aligned16(a_dev) || !aligned16(b_dev) || !aligned16(c_dev))
    return set_error(OCQ_ERR_INVALID_ARG, "null or misaligned pointer");
  int rc = diag_mfma_dot(form, (const uint8_t*)a_dev, (const uint8_t*)b_dev, M, N, K, c_dev, stream);
  return rc ? set_hip_error((hipError_t)rc, "kernel launch") : OCQ_OK;
}

static size_t stack_ws(int M, int hidden, int inter, const int* modes, int L, size_t* act_off) {
  size_t w = 0;
  for (int l = 0; l < L; ++l) {
    const size_t t = make_plan(M, hidden, inter, modes[l]).total;
    w = t > w ? t : w;
  }
  w = align_up(w);
  if (act_off) *act_off = w;
  return w + align_up((size_t)M * hidden * 2);
}

size_t ocq_stack_workspace_bytes(int M, int hidden, int inter, const int* prec_modes, int L) {
  if (!prec_modes || L < 1 || L > 1024 || M < 1 || M > 8192 || !shape_ok(hidden, inter)) return 0;
  for (int l = 0; l < L; ++l)
    if (prec_modes[l] < 0 || prec_modes[l] > 2) return 0;
  return stack_ws(M, hidden, inter, prec_modes, L, nullptr);
}

ocq_status ocq_mlp_stack_forward(const void* const* packed_devs, const size_t* packed_bytes, const int* prec_modes,
                                 int L, const void* x_bf16_dev, int M, int hidden, int inter, void* y_bf16_dev,
                                 void* workspace_dev, size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (!packed_devs || !packed_bytes || !prec_modes) return set_error(OCQ_ERR_INVALID_ARG, "null host array");
  if (L < 1 || L > 1024) return set_error(OCQ_ERR_INVALID_ARG, "L must be in [1, 1024]");
  if (M < 1 || M > 8192) return set_error(OCQ_ERR_INVALID_ARG, "M must be in [1, 8192]");
  for (int l = 0; l < L; ++l) {
    ocq_status st = check_shape(hidden, inter, prec_modes[l]);
    if (st != OCQ_OK) return st;
    if (!packed_devs[l]) return set_error(OCQ_ERR_INVALID_ARG, "null device pointer");
    if (!aligned16(packed_devs[l])) return set_error(OCQ_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    if (packed_bytes[l] < blob_layout(hidden, inter, prec_modes[l]).total)
      return set_error(OCQ_ERR_BUFFER_TOO_SMALL, "packed_bytes[l] < ocq_packed_bytes()");
  }
  if (!x_bf16_dev || !y_bf16_dev || !workspace_dev) return set_error(OCQ_ERR_INVALID_ARG, "null device pointer");
  if (!aligned16(x_bf16_dev) || !aligned16(y_bf16_dev) || !aligned16(workspace_dev))
    return set_error(OCQ_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  size_t act_off = 0;
  if (workspace_bytes < stack_ws(M, hidden, inter, prec_modes, L, &act_off))
    return set_error(OCQ_ERR_BUFFER_TOO_SMALL, "workspace_bytes < ocq_stack_workspace_bytes()");
  // outputs alternate between y and the workspace's activation buffer so
  // that the last block writes y and no block writes its own input
  uint16_t* act = (uint16_t*)((uint8_t*)workspace_dev + act_off);
  const uint16_t* in = (const uint16_t*)x_bf16_dev;
  for (int l = 0; l < L; ++l) {
    uint16_t* out = ((L - 1 - l) % 2 == 0) ? (uint16_t*)y_bf16_dev : act;
    const Plan p = make_plan(M, hidden, inter, prec_modes[l]);
    FwdArgs a{(const uint8_t*)packed_devs[l], in, out, (uint8_t*)workspace_dev, stream, nullptr, ocq_taps{},
              &g_last_requant};
    int rc = launch_forward(p, a);
    if (rc != 0) return set_hip_error((hipError_t)rc, "kernel launch");
    in = out;
  }
  return OCQ_OK;
}

}  // extern "C"
