// Internal declarations of the ocq library (not part of the C ABI).
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/ocq.h"
#include "ocq_layout.h"

namespace ocq {

// thread-local error message; returns `st` for convenience
ocq_status set_error(ocq_status st, const char* msg);

// host packer (pack.cpp)
// smooth (nullable): per-input-channel factors s[hidden] > 0; the gate/up
// weights are packed as fl32(W[n][k] s[k]) and x is multiplied by fl32(1/s[k])
ocq_status pack_host(const float* wg, const float* wu, const float* wd, int hidden, int inter, int prec,
                     const float* smooth, uint8_t* out, size_t out_bytes);
ocq_status calibrate_host(const uint16_t* x_bf16, int rows, int hidden, const float* wg, const float* wu, int inter,
                          float alpha, float* s_out);
ocq_status unpack_host(const uint8_t* blob, size_t bytes, int which, void* codes_out, void* scales_out,
                       float* tensor_scale_out);
uint8_t host_enc_e4m3(float v);
float host_dec_e4m3(uint8_t c);
uint8_t host_enc_e2m1(float v);
uint16_t host_bf16_rne(float v);

// device pointers of one forward call
struct FwdArgs {
  const uint8_t* blob;
  const uint16_t* x;
  uint16_t* y;
  uint8_t* ws;
  void* stream;
  void* const* stage_events;  // 5 hipEvent_t or NULL
  ocq_taps taps;              // each pointer nullable
  int* requant_in_gateup;     // nullable: set to 1 if the gate/up launch requantized h itself, else 0
};

// enqueue the kernels of one forward call (kernels.hip); returns 0 or a hipError_t value
int launch_forward(const Plan& p, const FwdArgs& a);
// process-wide: where gate/up launches requantize h (ocq_set_fused_requant)
void set_fused_requant(int mode);   // 0 or 1 (ocq_set_fused_requant)

// measurement kernels (diag.hip); return 0 or a hipError_t value
int diag_stream_read(const void* src, size_t bytes, void* out, int nblocks, void* stream);
int diag_window_read(const void* src, size_t window_bytes, int passes, void* out, int nblocks, void* stream);
size_t diag_mfma_rate_flops(int iters, int nblocks);
int diag_mfma_rate(int iters, float* out, int nblocks, void* stream);
int diag_empty(void* stream);
int diag_mfma_dot(int form, const uint8_t* a, const uint8_t* b, int M, int N, int K, float* c, void* stream);

// Per-wave phase stamps of the GEMM main loops, recorded only by a library
// built with OCQ_PHASE_STAMPS, for workgroups below kPhaseWGs: copy the last
// launch's values to host memory of at least the stated bytes.  Return 0, a
// hipError_t value, or -1 when the library was built without the stamps.
constexpr int kPhaseWGs = 512;
constexpr size_t kLgPhaseBytes = (size_t)2 * kPhaseWGs * 8 * 8 * 8;    // gemm_large.hip
constexpr size_t kPcPhaseBytes = (size_t)kPhaseWGs * 12 * 8 * 8;       // gemm_gateup.hip
constexpr int kQPhaseWGs = 1024;
constexpr size_t kQPhaseBytes = (size_t)2 * kQPhaseWGs * 2 * 8;         // kernels.hip
int lg_phase_copy(void* host, size_t bytes);
int pc_phase_copy(void* host, size_t bytes);
int q_phase_copy(void* host, size_t bytes);

}  // namespace ocq
