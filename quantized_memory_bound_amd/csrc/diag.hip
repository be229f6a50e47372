// Measurement kernels: the reference points the block's timings are read
// against (not part of the block).
//
//   k_stream_read  a plain streaming read of a device buffer (16-byte loads,
//                  several in flight per lane), the practical HBM ceiling for
//                  a read of that many bytes in one launch;
//   k_window_read  every workgroup reads the same small window several times
//                  (16-byte loads): with the window resident in L2, the rate
//                  at which L2 feeds the CUs, which bounds kernels whose
//                  workgroups re-read shared operands;
//   k_mfma_rate    independent f16 MFMA 16x16x32 on register operands, the
//                  matrix-core rate the chip sustains (against the published
//                  dense peak);
//   k_empty        an empty kernel, the fixed cost of one launch;
//   k_mfma_dot     C = A B^T over E4M3 codes through one matrix-core
//                  instruction form, with the operand fragment order and the
//                  per-chunk instruction sequence of the block's kernels, so
//                  the accumulation precision of each form can be compared
//                  against exact sums.
#include "kcommon.h"

namespace ocq {
namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;

// Every lane reads kStreamUnroll 16-byte pieces per pass (all requested
// before any is used), xor-folds them and writes one word per workgroup so
// the loads are not dead.  n16: number of 16-byte pieces.
__global__ __launch_bounds__(kStreamThreads) void k_stream_read(const v4i* __restrict__ src, size_t n16,
                                                                 uint32_t* __restrict__ out) {
  const size_t step = (size_t)gridDim.x * kStreamThreads * kStreamUnroll;
  v4i acc = v4i{0, 0, 0, 0};
  for (size_t base = (size_t)blockIdx.x * kStreamThreads * kStreamUnroll + threadIdx.x; base < n16; base += step) {
    v4i v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const size_t i = base + (size_t)u * kStreamThreads;
      v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u];
  }
  uint32_t w = (uint32_t)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
  w = __reduce_or_sync(~0ull, w);
  if (threadIdx.x == 0) out[blockIdx.x] = w;
}

// Every workgroup reads the window [src, src + n16) `passes` times, 8 loads of
// 16 B per lane in flight, starting at a per-workgroup offset (so workgroups
// do not walk the window in lockstep); one word per workgroup is written.
__global__ __launch_bounds__(kStreamThreads) void k_window_read(const v4i* __restrict__ src, size_t n16, int passes,
                                                                 uint32_t* __restrict__ out) {
  constexpr size_t kStep = (size_t)kStreamThreads * kStreamUnroll;
  const size_t n = n16 / kStep * kStep;   // whole passes of the unrolled loop
  const size_t start = ((size_t)blockIdx.x * 37 * kStep) % n;
  v4i acc = v4i{0, 0, 0, 0};
  for (int p = 0; p < passes; ++p) {
    for (size_t base = threadIdx.x; base < n; base += kStep) {
      v4i v[kStreamUnroll];
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) {
        size_t i = start + base + (size_t)u * kStreamThreads;
        i = i < n ? i : i - n;
        v[u] = src[i];
      }
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u];
    }
  }
  uint32_t w = (uint32_t)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
  w = __reduce_or_sync(~0ull, w);
  if (threadIdx.x == 0) out[blockIdx.x] = w;
}

// Each wave keeps kMfmaAcc independent accumulators and issues iters rounds of
// one MFMA on each; every lane writes one float so nothing is dead.
constexpr int kMfmaAcc = 16;
constexpr int kMfmaThreads = 512;
__global__ __launch_bounds__(kMfmaThreads) void k_mfma_rate(int iters, float* __restrict__ out) {
  v8h a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)((threadIdx.x & 7) * 0.125f + i);
    b[i] = (_Float16)(i * 0.0625f);
  }
  v4f acc[kMfmaAcc];
#pragma unroll
  for (int j = 0; j < kMfmaAcc; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kMfmaAcc; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kMfmaAcc; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  out[(size_t)blockIdx.x * kMfmaThreads + threadIdx.x] = s;
}

__global__ void k_empty() {}

// One wave per 16 x 16 output tile.  a: [M][K] codes, b: [N][K] codes
// (row-major); c: [M][N] fp32.  Lane l = 16 g + r loads row r's inputs
// 128 c + 32 g .. +31 of chunk c (two 16-byte units), the order in which the
// block's kernels hold their fragments.
//   form 0: each unit converted exactly to fp16, four MFMA 16x16x32 f16 per chunk
//   form 1: one MFMA 16x16x128 f8f6f4 (E4M3 x E4M3, unit scales) per chunk
//   form 2: four MFMA 16x16x32 fp8 x fp8 per chunk (8 codes per lane each)
template <int FORM>
__global__ __launch_bounds__(64) void k_mfma_dot(const uint8_t* __restrict__ a, const uint8_t* __restrict__ b,
                                                 int N, int K, float* __restrict__ c) {
  const int tn = blockIdx.x, tm = blockIdx.y, lane = threadIdx.x, g = lane >> 4, r = lane & 15;
  const uint8_t* pa = a + (size_t)(tm * 16 + r) * K + 32 * g;
  const uint8_t* pb = b + (size_t)(tn * 16 + r) * K + 32 * g;
  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < K; k0 += kChunk) {
    const v4i a0 = *(const v4i*)(pa + k0), a1 = *(const v4i*)(pa + k0 + 16);
    const v4i b0 = *(const v4i*)(pb + k0), b1 = *(const v4i*)(pb + k0 + 16);
    if constexpr (FORM == 1) {
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(cat(a0, a1), cat(b0, b1), acc, 0, 0, 0, 0, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v4i& ua = i < 2 ? a0 : a1;
        const v4i& ub = i < 2 ? b0 : b1;
        const uint32_t alo = (uint32_t)ua[2 * (i & 1)], ahi = (uint32_t)ua[2 * (i & 1) + 1];
        const uint32_t blo = (uint32_t)ub[2 * (i & 1)], bhi = (uint32_t)ub[2 * (i & 1) + 1];
        if constexpr (FORM == 0) {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(e4m3x8_to_f16(alo, ahi), e4m3x8_to_f16(blo, bhi), acc, 0, 0, 0);
        } else {
          const long la = (long)(((uint64_t)ahi << 32) | alo), lb = (long)(((uint64_t)bhi << 32) | blo);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(la, lb, acc, 0, 0, 0);
        }
      }
    }
  }
  // accumulator: lane holds column r of rows 4 g + i
#pragma unroll
  for (int i = 0; i < 4; ++i) c[(size_t)(tm * 16 + 4 * g + i) * N + tn * 16 + r] = acc[i];
}

}  // namespace

int diag_stream_read(const void* src, size_t bytes, void* out, int nblocks, void* stream) {
  hipLaunchKernelGGL(k_stream_read, dim3(nblocks), dim3(kStreamThreads), 0, (hipStream_t)stream, (const v4i*)src,
                     bytes / 16, (uint32_t*)out);
  return (int)hipGetLastError();
}

int diag_window_read(const void* src, size_t window_bytes, int passes, void* out, int nblocks, void* stream) {
  hipLaunchKernelGGL(k_window_read, dim3(nblocks), dim3(kStreamThreads), 0, (hipStream_t)stream, (const v4i*)src,
                     window_bytes / 16, passes, (uint32_t*)out);
  return (int)hipGetLastError();
}

size_t diag_mfma_rate_flops(int iters, int nblocks) {
  return (size_t)2 * 16 * 16 * 32 * kMfmaAcc * (size_t)iters * (kMfmaThreads / 64) * (size_t)nblocks;
}

int diag_mfma_rate(int iters, float* out, int nblocks, void* stream) {
  hipLaunchKernelGGL(k_mfma_rate, dim3(nblocks), dim3(kMfmaThreads), 0, (hipStream_t)stream, iters, out);
  return (int)hipGetLastError();
}

int diag_empty(void* stream) {
  hipLaunchKernelGGL(k_empty, dim3(1), dim3(64), 0, (hipStream_t)stream);
  return (int)hipGetLastError();
}

int diag_mfma_dot(int form, const uint8_t* a, const uint8_t* b, int M, int N, int K, float* c, void* stream) {
  const dim3 grid(N / 16, M / 16);
  hipStream_t st = (hipStream_t)stream;
  if (form == 0) hipLaunchKernelGGL(k_mfma_dot<0>, grid, dim3(64), 0, st, a, b, N, K, c);
  else if (form == 1) hipLaunchKernelGGL(k_mfma_dot<1>, grid, dim3(64), 0, st, a, b, N, K, c);
  else hipLaunchKernelGGL(k_mfma_dot<2>, grid, dim3(64), 0, st, a, b, N, K, c);
  return (int)hipGetLastError();
}

}  // namespace ocq
