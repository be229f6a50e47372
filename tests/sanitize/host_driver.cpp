// Host-side exercise of the C ABI for a sanitizer build (AddressSanitizer +
// UndefinedBehaviorSanitizer, g++): packing, unpacking, calibration and the
// size queries run in full on random weights of small, ragged shapes in all
// three precision modes; the device entry points are called only with
// arguments they must reject before touching a device.  Exits 0 when every
// status is the expected one; any sanitizer report aborts the run.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "ocq.h"

static int g_fail = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++g_fail;                                                        \
    }                                                                  \
  } while (0)

// counter-based generator (splitmix64) -> roughly normal floats
static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64() {
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static float normalish(float std) {
  float s = 0.f;
  for (int i = 0; i < 4; ++i) s += (float)(next_u64() >> 40) / (float)(1 << 24) - 0.5f;
  return s * std * 1.7320508f;
}
static uint16_t bf16_of(float v) {   // truncation is enough for inputs
  uint32_t b;
  std::memcpy(&b, &v, 4);
  return (uint16_t)(b >> 16);
}

static void exercise_shape(int hidden, int inter, int prec, bool smooth) {
  const size_t nb = ocq_packed_bytes(hidden, inter, prec);
  EXPECT(nb > 0);
  std::vector<float> wg((size_t)inter * hidden), wu(wg.size()), wd((size_t)hidden * inter);
  for (auto& v : wg) v = normalish(0.02f);
  for (auto& v : wu) v = normalish(0.02f);
  for (auto& v : wd) v = normalish(0.02f);
  wg[5] = 0.f;                                   // a few special values
  wu[7] = 1e-30f;
  wd[3] = -3.0f;
  for (int k = 0; k < hidden; ++k) wg[(size_t)1 * hidden + k] = 0.f;   // an all-zero gate row
  std::vector<uint8_t> blob(nb);
  std::vector<float> s(hidden, 1.f);
  if (smooth) {
    const int rows = 24;
    std::vector<uint16_t> x((size_t)rows * hidden);
    for (size_t i = 0; i < x.size(); ++i) x[i] = bf16_of(normalish(1.f) * ((i % hidden) % 37 == 3 ? 20.f : 1.f));
    EXPECT(ocq_calibrate_smoothing_host(x.data(), rows, hidden, wg.data(), wu.data(), inter, 0.5f, s.data()) == OCQ_OK);
    for (float v : s) EXPECT(std::isfinite(v) && v > 0.f);
    EXPECT(ocq_pack_weights_smoothed_host(wg.data(), wu.data(), wd.data(), s.data(), hidden, inter, prec, blob.data(),
                                          nb) == OCQ_OK);
  } else {
    EXPECT(ocq_pack_weights_host(wg.data(), wu.data(), wd.data(), hidden, inter, prec, blob.data(), nb) == OCQ_OK);
  }
  for (int which = 0; which < 3; ++which) {
    const size_t rows = which < 2 ? inter : hidden, cols = which < 2 ? hidden : inter;
    const bool bf16 = prec == OCQ_PREC_FP8_DOWN_BF16 && which == 2;
    std::vector<uint8_t> codes(rows * cols * (bf16 ? 2 : 1));
    std::vector<uint8_t> scales(prec == OCQ_PREC_FP4 ? rows * cols / 16 : rows * 4);
    float ts = -1.f;
    EXPECT(ocq_unpack_weights_host(blob.data(), nb, which, codes.data(), scales.data(), &ts) == OCQ_OK);
    if (prec == OCQ_PREC_FP4) EXPECT(ts > 0.f);
  }
  std::vector<float> xmul(hidden);
  EXPECT(ocq_unpack_weights_host(blob.data(), nb, 3, nullptr, xmul.data(), nullptr) == OCQ_OK);
  if (smooth)
    for (int k = 0; k < hidden; ++k) EXPECT(xmul[k] == 1.0f / s[k]);
  // a truncated blob and a damaged header are rejected
  EXPECT(ocq_unpack_weights_host(blob.data(), 1000, 0, nullptr, nullptr, nullptr) != OCQ_OK);
  std::vector<uint8_t> bad(blob);
  bad[0] ^= 0xFF;
  std::vector<uint8_t> sink((size_t)inter * hidden * 2);
  std::vector<float> ssink((size_t)inter * hidden);
  EXPECT(ocq_unpack_weights_host(bad.data(), nb, 0, sink.data(), ssink.data(), nullptr) == OCQ_ERR_BAD_BLOB);
  // too small an output for the packer
  EXPECT(ocq_pack_weights_host(wg.data(), wu.data(), wd.data(), hidden, inter, prec, blob.data(), nb - 1) ==
         OCQ_ERR_BUFFER_TOO_SMALL);
  EXPECT(ocq_workspace_bytes(208, hidden, inter, prec) > 0);
  EXPECT(ocq_workspace_bytes(0, hidden, inter, prec) == 0);
}

int main() {
  EXPECT(ocq_version() > 0);
  const int shapes[][2] = {{256, 512}, {384, 640}, {128, 1152}};
  for (auto& sh : shapes)
    for (int prec = 0; prec < 3; ++prec) exercise_shape(sh[0], sh[1], prec, false);
  for (int prec = 0; prec < 3; ++prec) exercise_shape(384, 640, prec, true);

  // argument errors, all reported before any device call
  EXPECT(ocq_packed_bytes(100, 6144, 0) == 0);
  EXPECT(ocq_packed_bytes(2048, 6144, 3) == 0);
  EXPECT(ocq_pack_weights_host(nullptr, nullptr, nullptr, 256, 512, 0, nullptr, 0) == OCQ_ERR_INVALID_ARG);
  void* const blob = (void*)0x10000;
  void* const x = (void*)0x20000;
  void* const y = (void*)0x30000;
  void* const ws = (void*)0x40000;
  const size_t big = (size_t)1 << 30;
  EXPECT(ocq_mlp_forward(blob, big, x, 16, 2000, 6144, 0, y, ws, big, nullptr, nullptr) == OCQ_ERR_UNSUPPORTED);
  EXPECT(ocq_mlp_forward(blob, big, x, 16, 2048, 6144, 7, y, ws, big, nullptr, nullptr) == OCQ_ERR_INVALID_ARG);
  EXPECT(ocq_mlp_forward(blob, big, x, 0, 2048, 6144, 0, y, ws, big, nullptr, nullptr) == OCQ_ERR_INVALID_ARG);
  EXPECT(ocq_mlp_forward(blob, big, nullptr, 16, 2048, 6144, 0, y, ws, big, nullptr, nullptr) == OCQ_ERR_INVALID_ARG);
  EXPECT(ocq_mlp_forward(blob, 1000, x, 16, 2048, 6144, 0, y, ws, big, nullptr, nullptr) == OCQ_ERR_BUFFER_TOO_SMALL);
  EXPECT(ocq_mlp_forward(blob, big, x, 16, 2048, 6144, 0, y, ws, 1000, nullptr, nullptr) == OCQ_ERR_BUFFER_TOO_SMALL);
  EXPECT(std::strlen(ocq_last_error()) > 0);
  ocq_taps taps;
  std::memset(&taps, 0, sizeof(taps));
  taps.x_codes = (void*)0x50004;   // misaligned tap
  EXPECT(ocq_mlp_forward(blob, big, x, 16, 2048, 6144, 0, y, ws, big, &taps, nullptr) == OCQ_ERR_INVALID_ARG);
  const void* blobs[2] = {blob, (void*)0x20008};
  const size_t sizes[2] = {big, big};
  const int modes[2] = {0, 2};
  EXPECT(ocq_mlp_stack_forward(blobs, sizes, modes, 2, x, 16, 2048, 6144, y, ws, big, nullptr) == OCQ_ERR_INVALID_ARG);
  EXPECT(ocq_mlp_stack_forward(blobs, sizes, modes, 0, x, 16, 2048, 6144, y, ws, big, nullptr) == OCQ_ERR_INVALID_ARG);
  EXPECT(ocq_stack_workspace_bytes(16, 2048, 6144, nullptr, 1) == 0);
  EXPECT(ocq_stack_workspace_bytes(16, 2048, 6144, modes, 2) > 0);
  EXPECT(ocq_diag_stream_read(nullptr, 16, nullptr, 1, nullptr) == OCQ_ERR_INVALID_ARG);
  EXPECT(ocq_diag_window_read(x, 1000, 1, y, 1, nullptr) == OCQ_ERR_INVALID_ARG);
  EXPECT(ocq_diag_mfma_rate(0, y, 1, nullptr, nullptr) == OCQ_ERR_INVALID_ARG);
  EXPECT(ocq_diag_mfma_dot(3, x, y, 16, 16, 128, (float*)ws, nullptr) == OCQ_ERR_INVALID_ARG);
  {
    std::vector<uint64_t> stamps(2 * 512 * 8 * 8);
    const size_t sb = stamps.size() * sizeof(uint64_t);
    EXPECT(ocq_diag_phase_stamps(3, stamps.data(), sb) == OCQ_ERR_INVALID_ARG);
    EXPECT(ocq_diag_phase_stamps(2, stamps.data(), sb) == OCQ_ERR_UNSUPPORTED);
    EXPECT(ocq_diag_phase_stamps(0, nullptr, sb) == OCQ_ERR_INVALID_ARG);
    EXPECT(ocq_diag_phase_stamps(0, stamps.data(), sb - 1) == OCQ_ERR_BUFFER_TOO_SMALL);
    EXPECT(ocq_diag_phase_stamps(0, stamps.data(), sb) == OCQ_ERR_UNSUPPORTED);
    EXPECT(ocq_diag_phase_stamps(1, stamps.data(), sb) == OCQ_ERR_UNSUPPORTED);
  }
  EXPECT(ocq_set_fused_requant(0) == OCQ_OK);
  EXPECT(ocq_set_fused_requant(1) == OCQ_OK);
  EXPECT(ocq_set_fused_requant(2) == OCQ_ERR_INVALID_ARG);
  EXPECT(ocq_set_fused_requant(-1) == OCQ_ERR_INVALID_ARG);
  EXPECT(ocq_last_requant_in_gateup() == -1);   // no forward call was made
  std::printf("%s (%d failed checks)\n", g_fail ? "FAIL" : "OK", g_fail);
  return g_fail ? 1 : 0;
}
