// Forward call for callers that cannot allocate device memory (code under
// HIP graph capture that may not call hipMalloc, tight serving loops, hosts
// that forbid allocation): the same kernels as ocq_mlp_forward, with the
// workspace taken from a fixed per-device array of kScratchBytes instead of
// a caller buffer.
//
// `scratch` is a host-side stand-in in host code, not a device address:
// its device address is looked up once per device (hipGetSymbolAddress,
// with that device current) and only that address is ever handed to the
// kernels.  Every call on one device shares that device's array, which keeps
// the last call's contents; the kernels never rely on its contents at entry
// (every value they read is written earlier in the same call), and calls
// that overlap on one device (concurrent streams) race on it.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "ocq_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;   // 32 MiB per device
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device ordinal

// Device address of this device's scratch array (looked up on the first
// call on the device, with the device current).  Returns nullptr with the
// error status in *st on failure.
void* scratch_on_current_device(ocq_status* st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    char buf[160];
    std::snprintf(buf, sizeof(buf), "no usable current device (%s, ordinal %d)",
                  e == hipSuccess ? "ok" : hipGetErrorString(e), dev);
    *st = ocq::set_error(OCQ_ERR_DEVICE, buf);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      char buf[160];
      std::snprintf(buf, sizeof(buf), "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      *st = ocq::set_error(OCQ_ERR_DEVICE, buf);
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t ocq_noalloc_scratch_bytes(void) { return kScratchBytes; }

ocq_status ocq_mlp_forward_noalloc(const void* packed_dev, size_t packed_bytes, const void* x_bf16_dev, int M,
                                   int hidden, int inter, int prec_mode, void* y_bf16_dev, const ocq_taps* taps,
                                   void* stream) {
  const size_t need = ocq_workspace_bytes(M, hidden, inter, prec_mode);
  if (need > kScratchBytes) {
    char buf[200];
    std::snprintf(buf, sizeof(buf),
                  "this call needs %zu bytes of workspace; the no-allocation entry point holds %zu per device "
                  "(use ocq_mlp_forward with a caller workspace)", need, kScratchBytes);
    return ocq::set_error(OCQ_ERR_BUFFER_TOO_SMALL, buf);
  }
  if (need == 0)   // invalid shape, mode or M: reported by ocq_mlp_forward's checks, before any device call
    return ocq_mlp_forward(packed_dev, packed_bytes, x_bf16_dev, M, hidden, inter, prec_mode, y_bf16_dev, nullptr, 0,
                           taps, stream);
  ocq_status st = OCQ_OK;
  void* ws = scratch_on_current_device(&st);
  if (!ws) return st;
  return ocq_mlp_forward(packed_dev, packed_bytes, x_bf16_dev, M, hidden, inter, prec_mode, y_bf16_dev, ws,
                         kScratchBytes, taps, stream);
}

}  // extern "C"
