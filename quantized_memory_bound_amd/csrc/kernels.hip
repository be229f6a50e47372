// HIP kernels of the quantized MLP block for CDNA4 (gfx950).
//
// One forward call = four kernels on the caller's stream:
//   k_xquant   per-token E4M3 quantization of x (scale amax/448), zero-padded
//              to whole 16-row tiles; also clears the h-amax accumulators and
//              the split-K arrival counters of this call.
//   k_gateup   G = xq Wg^T, U = xq Wu^T on the matrix cores with exact
//              products and fp32 accumulation: E4M3 codes and NVFP4 weights
//              are converted in registers to fp16 (gfx950 packed converts,
//              exact) and fed to MFMA 16x16x32 f16; fused epilogue
//              h = SiLU(G sx sw_g) * (U sx sw_u) with the per-token |h| max
//              reduced over the wavefront, the workgroup (LDS) and the grid
//              (one atomic max per row and workgroup).  BF16-down mode writes
//              bf16(h) and needs no max.
//   k_requant  hq = E4M3(h / sh), sh = amax / 448 (FP8 / NVFP4 down modes).
//   k_down     Y = hq Wd^T (FP8: MFMA 16x16x128 f8f6f4; BF16: MFMA 16x16x32
//              bf16; NVFP4: fp16 as above), split over the inputs across
//              workgroups; the last workgroup of each output tile to finish
//              sums the split partials in a fixed order (deterministic) and
//              writes y = bf16(Y sh sw_d).
// Cited passages ("OCRia 推理栈：单卡 B200 提速近 10 倍"): "Reducing the data
// moved: workload-aware quantization" (FP8 / NVFP4 / BF16 weights per layer),
// "Generate more tokens per target pass" (M = requests x (1 + drafts) rows
// share one read of the weights); German page "Wie es funktioniert" (SiLU and
// quantization fused, intermediates in registers).
//
// Work decomposition: a workgroup of 4 waves owns T weight tiles (16 output
// rows each) and all rows of one m-block (MT tiles of 16 rows); its waves
// split the input dimension chunk by chunk (chunk = 128 inputs), so every
// weight byte is loaded by exactly one wave, straight from HBM into the MFMA
// operand registers (fragment order, 2 x 16 B per lane per chunk, fully
// coalesced, non-temporal).  The activation rows are read per lane as 32
// contiguous bytes of the row-major buffer.  The four waves' accumulators are
// summed in LDS in wave order (deterministic) before the epilogue.
#include <hip/hip_runtime.h>

#include <cstddef>

#include "ocq_internal.h"

namespace ocq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// ---------------------------------------------------------------- scalar codecs

// E4M3 (OCP FN) code of an fp32 value: nearest, ties to even, saturating at 448.
__device__ __forceinline__ uint32_t enc_e4m3(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t ua = u & 0x7FFFFFFFu;
  const float a = __uint_as_float(ua);
  uint32_t c;
  if (a >= 448.0f) {
    c = 0x7Eu;
  } else if (a < 0.015625f) {                       // subnormal grid 2^-9 (code 8 = 2^-6)
    c = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    const uint32_t e = (ua >> 23) - 120u;           // rebias 127 -> 7
    const uint32_t m = ua & 0x7FFFFFu;
    const uint32_t q = (m + 0x7FFFFu + ((m >> 20) & 1u)) >> 20;
    c = (e << 3) + q;                               // mantissa carry bumps the exponent
  }
  return sign | c;
}

__device__ __forceinline__ float dec_e4m3(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (c & 0x80u) ? -mag : mag;
}

__device__ __forceinline__ uint32_t bf16_bits(float v) {   // round to nearest even (finite v)
  const uint32_t u = __float_as_uint(v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Eight E4M3 codes (two dwords, byte order = element order) -> eight fp16.
// v_cvt_scalef32_pk_f16_fp8 applies only the power-of-two part of its scale,
// so a scale of 1.0 makes the conversion exact (every E4M3 value is an fp16).
__device__ __forceinline__ v8h e4m3x8_to_f16(uint32_t lo, uint32_t hi) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  return v8h{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Eight E2M1 codes (one dword, low nibble first) times an E4M3 block scale
// -> eight fp16, exact: the conversion (scale 1.0) is exact, and E2M1 x E4M3
// products have at most 6 significant bits and lie in [2^-10, 2688].
__device__ __forceinline__ v8h e2m1x8_to_f16(uint32_t d, v2h sb) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 0) * sb;
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 1) * sb;
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 2) * sb;
  const v2h e = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 3) * sb;
  return v8h{a[0], a[1], b[0], b[1], c[0], c[1], e[0], e[1]};
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

template <class T>
__device__ __forceinline__ T ld_nt(const T* p) { return __builtin_nontemporal_load(p); }

// ---------------------------------------------------------------- k_xquant

__global__ __launch_bounds__(kThreads) void k_xquant(const uint16_t* __restrict__ x, int M, int H, int Mpad,
                                                     uint8_t* __restrict__ xq, float* __restrict__ sx,
                                                     uint32_t* __restrict__ amax_h, uint32_t* __restrict__ counters,
                                                     int ncnt) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = blockIdx.x * kThreads + threadIdx.x; i < ncnt; i += gridDim.x * kThreads) counters[i] = 0u;
  const int m = blockIdx.x * kWaves + wave;
  if (m >= Mpad) return;
  uint8_t* qrow = xq + (size_t)m * H;
  if (lane == 0) amax_h[m] = 0u;
  if (m >= M) {                                     // padding row: zero codes, zero scale
    for (int k = lane * 16; k < H; k += 1024) *(v4i*)(qrow + k) = v4i{0, 0, 0, 0};
    if (lane == 0) sx[m] = 0.0f;
    return;
  }
  const uint16_t* xr = x + (size_t)m * H;
  float amax = 0.0f;
  for (int k = lane * 8; k < H; k += 512) {
    const v4i v = *(const v4i*)(xr + k);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = (uint32_t)v[j];
      amax = fmaxf(amax, fabsf(__uint_as_float(w << 16)));
      amax = fmaxf(amax, fabsf(__uint_as_float(w & 0xFFFF0000u)));
    }
  }
  amax = wave_max(amax);
  const float s = amax / 448.0f;
  for (int k = lane * 8; k < H; k += 512) {
    const v4i v = *(const v4i*)(xr + k);
    uint32_t out[2] = {0u, 0u};
    if (s > 0.0f) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = (uint32_t)v[j];
        const uint32_t c0 = enc_e4m3(__uint_as_float(w << 16) / s);
        const uint32_t c1 = enc_e4m3(__uint_as_float(w & 0xFFFF0000u) / s);
        out[j >> 1] |= (c0 | (c1 << 8)) << (16 * (j & 1));
      }
    }
    *(v2u*)(qrow + k) = v2u{out[0], out[1]};
  }
  if (lane == 0) sx[m] = s;
}

// ---------------------------------------------------------------- k_requant

__global__ __launch_bounds__(kThreads) void k_requant(const float* __restrict__ h32,
                                                      const uint32_t* __restrict__ amax_h, int I,
                                                      uint8_t* __restrict__ hq, float* __restrict__ sh) {
  const int m = blockIdx.y;
  const int k = (blockIdx.x * kThreads + threadIdx.x) * 4;
  const float s = __uint_as_float(amax_h[m]) / 448.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0) sh[m] = s;
  if (k >= I) return;
  const v4f v = *(const v4f*)(h32 + (size_t)m * I + k);
  uint32_t out = 0u;
  if (s > 0.0f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) out |= enc_e4m3(v[j] / s) << (8 * j);
  }
  *(uint32_t*)(hq + (size_t)m * I + k) = out;
}

// ---------------------------------------------------------------- matrix-core main loops
//
// All loops accumulate acc[mt][t] (16x16 fp32 tile: lane l holds rows
// 4 (l/16) + i, i = 0..3, column l % 16) over chunks c = c0 + wave, +4, ... < c1.
// A points at row 0 of the m-block; W at the first weight tile of the group.

// FP8 x FP8: one MFMA 16x16x128 f8f6f4 per (m-tile, tile, chunk).  These
// instructions sum their 128 products with ~2^-19 relative error (measured);
// used only for the down projection, whose result is rounded to bf16.
template <int MT, int T>
__device__ __forceinline__ void loop_fp8(const uint8_t* __restrict__ A, int lda, const uint8_t* __restrict__ W,
                                         size_t tile_stride, int c0, int c1, v4f (&acc)[MT][T]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint8_t* arow = A + (size_t)(lane & 15) * lda + 32 * (lane >> 4);
  const uint8_t* wl = W + lane * 16;
#pragma unroll 1
  for (int c = c0 + wave; c < c1; c += kWaves) {
    v8i a[MT], b[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const uint8_t* q = wl + t * tile_stride + (size_t)c * 2048;
      const v4i lo = ld_nt((const v4i*)q), hi = ld_nt((const v4i*)(q + 1024));
      b[t] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const v4i* p = (const v4i*)(arow + (size_t)mt * 16 * lda + c * 128);
      const v4i lo = p[0], hi = p[1];
      a[mt] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < T; ++t)
        acc[mt][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[mt], b[t], acc[mt][t], 0, 0, 0, 0, 0, 0);
  }
}

// FP8 x FP8 with exact products and fp32 accumulation: both operands are
// converted in registers to fp16 and multiplied with MFMA 16x16x32 f16 (four
// per chunk; sub-step i covers k = 32 g + 8 i .. +8 of each lane's 32 bytes).
// Used where a code is decided on the result (gate/up -> h -> E4M3 codes):
// the FP8 matrix-core instructions sum their products with about 2^-19
// relative error (measured), too coarse for the code-parity bar.
template <int MT, int T>
__device__ __forceinline__ void loop_fp8_exact(const uint8_t* __restrict__ A, int lda, const uint8_t* __restrict__ W,
                                               size_t tile_stride, int c0, int c1, v4f (&acc)[MT][T]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint8_t* arow = A + (size_t)(lane & 15) * lda + 32 * (lane >> 4);
  const uint8_t* wl = W + lane * 16;
#pragma unroll 1
  for (int c = c0 + wave; c < c1; c += kWaves) {
    v8i a[MT], b[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const uint8_t* q = wl + t * tile_stride + (size_t)c * 2048;
      const v4i lo = ld_nt((const v4i*)q), hi = ld_nt((const v4i*)(q + 1024));
      b[t] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const v4i* p = (const v4i*)(arow + (size_t)mt * 16 * lda + c * 128);
      const v4i lo = p[0], hi = p[1];
      a[mt] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v8h bh[T];
#pragma unroll
      for (int t = 0; t < T; ++t) bh[t] = e4m3x8_to_f16((uint32_t)b[t][2 * i], (uint32_t)b[t][2 * i + 1]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const v8h ah = e4m3x8_to_f16((uint32_t)a[mt][2 * i], (uint32_t)a[mt][2 * i + 1]);
#pragma unroll
        for (int t = 0; t < T; ++t)
          acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh[t], acc[mt][t], 0, 0, 0);
      }
    }
  }
}

// BF16 x BF16: four MFMA 16x16x32 per chunk (sub-step i covers k = 32 g + 8 i .. +8)
template <int MT, int T>
__device__ __forceinline__ void loop_bf16(const uint16_t* __restrict__ A, int lda, const uint8_t* __restrict__ W,
                                          size_t tile_stride, int c0, int c1, v4f (&acc)[MT][T]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint16_t* arow = A + (size_t)(lane & 15) * lda + 32 * (lane >> 4);
  const uint8_t* wl = W + lane * 16;
#pragma unroll 1
  for (int c = c0 + wave; c < c1; c += kWaves) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v8bf a[MT], b[T];
#pragma unroll
      for (int t = 0; t < T; ++t)
        b[t] = __builtin_bit_cast(v8bf, ld_nt((const v4i*)(wl + t * tile_stride + ((size_t)c * 4 + i) * 1024)));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        a[mt] = __builtin_bit_cast(v8bf, *(const v4i*)(arow + (size_t)mt * 16 * lda + c * 128 + 8 * i));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < T; ++t)
          acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt], b[t], acc[mt][t], 0, 0, 0);
    }
  }
}

// E4M3 activations x NVFP4 weights: both dequantized in registers to fp16
// (exact, see e2m1x8_to_f16), four MFMA 16x16x32 f16 per chunk.  Wb points at
// the block-scale groups of the first tile of the group; tile_stride /
// btile_stride are per-tile byte strides.
template <int MT, int T>
__device__ __forceinline__ void loop_fp4(const uint8_t* __restrict__ A, int lda, const uint8_t* __restrict__ W,
                                         size_t tile_stride, const uint8_t* __restrict__ Wb, size_t btile_stride,
                                         int c0, int c1, v4f (&acc)[MT][T]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint8_t* arow = A + (size_t)(lane & 15) * lda + 32 * (lane >> 4);
  const uint8_t* wl = W + lane * 16;
  const uint8_t* bl = Wb + lane * 16;
#pragma unroll 1
  for (int c = c0 + wave; c < c1; c += kWaves) {
    v4i wq[T];
    v2h s0[T], s1[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      wq[t] = ld_nt((const v4i*)(wl + t * tile_stride + (size_t)c * 1024));
      const uint8_t* sp = bl + t * btile_stride + (size_t)(c >> 3) * 1024 + 2 * (c & 7);
      const v2h sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)sp[0] | ((uint32_t)sp[1] << 8), 1.0f, false);
      s0[t] = v2h{sc[0], sc[0]};
      s1[t] = v2h{sc[1], sc[1]};
    }
    v8i araw[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const v4i* p = (const v4i*)(arow + (size_t)mt * 16 * lda + c * 128);
      const v4i lo = p[0], hi = p[1];
      araw[mt] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v8h b[T];
#pragma unroll
      for (int t = 0; t < T; ++t) b[t] = e2m1x8_to_f16((uint32_t)wq[t][i], i < 2 ? s0[t] : s1[t]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const v8h a = e4m3x8_to_f16((uint32_t)araw[mt][2 * i], (uint32_t)araw[mt][2 * i + 1]);
#pragma unroll
        for (int t = 0; t < T; ++t)
          acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[t], acc[mt][t], 0, 0, 0);
      }
    }
  }
}

// ---------------------------------------------------------------- cross-wave reduction

// LDS layout [wave][pair p][i][lane]; pair p = mt * T + t
template <int MT, int T>
__device__ __forceinline__ void stash_acc(const v4f (&acc)[MT][T], float* red) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[((wave * MT * T + mt * T + t) * 4 + i) * 64 + lane] = acc[mt][t][i];
}

__device__ __forceinline__ float red_sum(const float* red, int PT, int p, int i, int ln) {
  float s = red[((0 * PT + p) * 4 + i) * 64 + ln];
  s += red[((1 * PT + p) * 4 + i) * 64 + ln];
  s += red[((2 * PT + p) * 4 + i) * 64 + ln];
  s += red[((3 * PT + p) * 4 + i) * 64 + ln];
  return s;
}

// ---------------------------------------------------------------- k_gateup

enum GUKind { kGU_FP8 = 0, kGU_FP4 = 1 };

struct GateUpArgs {
  const uint8_t* xq;        // [Mpad][H] E4M3 codes
  const float* sx;          // [Mpad]
  const uint8_t* wcodes;    // interleaved gate/up fragments
  const float* wscales;     // FP8: [2][I] per-row scales
  const uint8_t* wbscales;  // NVFP4: block-scale groups
  const float* tscales;     // NVFP4: blob header s_gate, s_up
  float* h32;               // [Mpad][I] (FP8 / NVFP4 down modes)
  uint16_t* hb;             // [Mpad][I] bf16 (BF16-down mode)
  uint32_t* amax_h;         // [Mpad] float bits of max |h|
  int H, I, n_mb;
};

template <int MT, int T, int KIND, bool BF16H>
__global__ __launch_bounds__(kThreads, 1) void k_gateup(GateUpArgs g) {
  extern __shared__ float red[];
  __shared__ uint32_t s_amax[16 * MT];
  const int mb = blockIdx.x % g.n_mb, ng = blockIdx.x / g.n_mb;
  const int C = g.H / kChunk;
  const int row0 = mb * MT * 16;
  for (int i = threadIdx.x; i < 16 * MT; i += kThreads) s_amax[i] = 0u;

  v4f acc[MT][T];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[mt][t] = v4f{0.f, 0.f, 0.f, 0.f};

  if constexpr (KIND == kGU_FP8) {
    const size_t ts = (size_t)C * 2048;
    loop_fp8_exact<MT, T>(g.xq + (size_t)row0 * g.H, g.H, g.wcodes + (size_t)ng * T * ts, ts, 0, C, acc);
  } else {
    const size_t ts = (size_t)C * 1024, bts = (size_t)((g.H / kChunk + 7) / 8) * 1024;
    loop_fp4<MT, T>(g.xq + (size_t)row0 * g.H, g.H, g.wcodes + (size_t)ng * T * ts, ts,
                    g.wbscales + (size_t)ng * T * bts, bts, 0, C, acc);
  }
  stash_acc<MT, T>(acc, red);
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, gq = lane >> 4, r = lane & 15;
  float sg = 0.f, su = 0.f;
  if constexpr (KIND == kGU_FP4) { sg = g.tscales[0]; su = g.tscales[1]; }
  for (int p = wave; p < MT * T; p += kWaves) {
    const int mt = p / T, t = p % T;
    const int n = (ng * T + t) * 8 + (r & 7);
    float cg = sg, cu = su;
    if constexpr (KIND == kGU_FP8) { cg = g.wscales[n]; cu = g.wscales[g.I + n]; }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = row0 + mt * 16 + 4 * gq + i;
      float hv = 0.f;
      if (r < 8) {
        const float xs = g.sx[m];
        const float gv = red_sum(red, MT * T, p, i, lane) * xs * cg;
        const float uv = red_sum(red, MT * T, p, i, lane + 8) * xs * cu;
        hv = silu(gv) * uv;
        if constexpr (BF16H) g.hb[(size_t)m * g.I + n] = (uint16_t)bf16_bits(hv);
        else g.h32[(size_t)m * g.I + n] = hv;
      }
      if constexpr (!BF16H) {
        float am = fabsf(hv);
        am = fmaxf(am, __shfl_xor(am, 1));
        am = fmaxf(am, __shfl_xor(am, 2));
        am = fmaxf(am, __shfl_xor(am, 4));
        if (r == 0 && am > 0.f) atomicMax(&s_amax[mt * 16 + 4 * gq + i], __float_as_uint(am));
      }
    }
  }
  if constexpr (!BF16H) {
    __syncthreads();
    for (int i = threadIdx.x; i < 16 * MT; i += kThreads)
      if (s_amax[i]) __hip_atomic_fetch_max(&g.amax_h[row0 + i], s_amax[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------- k_down

enum DNKind { kDN_FP8 = 0, kDN_BF16 = 1, kDN_FP4 = 2 };

struct DownArgs {
  const void* A;            // hq [Mpad][I] codes (FP8 / NVFP4) or hb bf16 (BF16)
  const float* sh;          // [Mpad] (FP8 / NVFP4)
  const uint8_t* wcodes;
  const float* wscales;     // FP8: [H]
  const uint8_t* wbscales;  // NVFP4 block-scale groups
  const float* tscale;      // NVFP4: blob header s_down
  float* part;              // [nsplit][Mpad][H]
  uint32_t* counters;       // [n_mb][ngroups]
  uint16_t* y;              // [M][H]
  int H, I, M, Mpad, n_mb, ngroups, cps, nsplit;
};

template <int MT, int T, int KIND>
__global__ __launch_bounds__(kThreads, 1) void k_down(DownArgs d) {
  extern __shared__ float red[];
  __shared__ int s_last;
  const int mb = blockIdx.x % d.n_mb;
  const int rest = blockIdx.x / d.n_mb;
  const int ng = rest % d.ngroups, sp = rest / d.ngroups;
  const int C = d.I / kChunk;
  const int c0 = sp * d.cps, c1 = min(C, c0 + d.cps);
  const int row0 = mb * MT * 16;

  v4f acc[MT][T];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[mt][t] = v4f{0.f, 0.f, 0.f, 0.f};

  if constexpr (KIND == kDN_FP8) {
    const size_t ts = (size_t)C * 2048;
    loop_fp8<MT, T>((const uint8_t*)d.A + (size_t)row0 * d.I, d.I, d.wcodes + (size_t)ng * T * ts, ts, c0, c1, acc);
  } else if constexpr (KIND == kDN_BF16) {
    const size_t ts = (size_t)C * 4096;
    loop_bf16<MT, T>((const uint16_t*)d.A + (size_t)row0 * d.I, d.I, d.wcodes + (size_t)ng * T * ts, ts, c0, c1, acc);
  } else {
    const size_t ts = (size_t)C * 1024, bts = (size_t)((d.I / kChunk + 7) / 8) * 1024;
    loop_fp4<MT, T>((const uint8_t*)d.A + (size_t)row0 * d.I, d.I, d.wcodes + (size_t)ng * T * ts, ts,
                    d.wbscales + (size_t)ng * T * bts, bts, c0, c1, acc);
  }
  stash_acc<MT, T>(acc, red);
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, gq = lane >> 4, r = lane & 15;
  float tsd = 1.0f;
  if constexpr (KIND == kDN_FP4) tsd = d.tscale[0];
  for (int p = wave; p < MT * T; p += kWaves) {
    const int mt = p / T, t = p % T;
    const int j = (ng * T + t) * 16 + r;
    float cs = tsd;
    if constexpr (KIND == kDN_FP8) cs = d.wscales[j];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = row0 + mt * 16 + 4 * gq + i;
      const float v = red_sum(red, MT * T, p, i, lane);
      if (d.nsplit == 1) {
        if (m < d.M) {
          const float rs = KIND == kDN_BF16 ? 1.0f : d.sh[m];
          d.y[(size_t)m * d.H + j] = (uint16_t)bf16_bits(v * rs * cs);
        }
      } else {
        d.part[((size_t)sp * d.Mpad + m) * d.H + j] = v;
      }
    }
  }
  if (d.nsplit == 1) return;

  // split-K: the last workgroup to arrive for this (m-block, output group)
  // sums the partials in split order
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = atomicAdd(&d.counters[mb * d.ngroups + ng], 1u);
    s_last = prev == (unsigned)(d.nsplit - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  for (int p = wave; p < MT * T; p += kWaves) {
    const int mt = p / T, t = p % T;
    const int j = (ng * T + t) * 16 + r;
    float cs = tsd;
    if constexpr (KIND == kDN_FP8) cs = d.wscales[j];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = row0 + mt * 16 + 4 * gq + i;
      if (m >= d.M) continue;
      float v = 0.f;
      for (int s2 = 0; s2 < d.nsplit; ++s2) v += __builtin_nontemporal_load(&d.part[((size_t)s2 * d.Mpad + m) * d.H + j]);
      const float rs = KIND == kDN_BF16 ? 1.0f : d.sh[m];
      d.y[(size_t)m * d.H + j] = (uint16_t)bf16_bits(v * rs * cs);
    }
  }
}

// ---------------------------------------------------------------- dispatch tables

template <int MT, int T, int KIND, bool BF16H>
hipError_t launch_gateup_t(const GateUpArgs& g, int grid, hipStream_t st) {
  auto fn = k_gateup<MT, T, KIND, BF16H>;
  const size_t lds = (size_t)kWaves * MT * T * 256 * sizeof(float);
  hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(kThreads), lds, st, g);
  return hipGetLastError();
}

template <int MT, int T, int KIND>
hipError_t launch_down_t(const DownArgs& d, int grid, hipStream_t st) {
  auto fn = k_down<MT, T, KIND>;
  const size_t lds = (size_t)kWaves * MT * T * 256 * sizeof(float);
  hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(kThreads), lds, st, d);
  return hipGetLastError();
}

template <int KIND, bool BF16H, int MT>
hipError_t gateup_T(const GateUpArgs& g, int T, int grid, hipStream_t st) {
  switch (T) {
    case 1: return launch_gateup_t<MT, 1, KIND, BF16H>(g, grid, st);
    case 2: return launch_gateup_t<MT, 2, KIND, BF16H>(g, grid, st);
    case 3: return launch_gateup_t<MT, 3, KIND, BF16H>(g, grid, st);
  }
  return hipErrorInvalidValue;
}

template <int KIND, bool BF16H>
hipError_t gateup_dispatch(const GateUpArgs& g, int MT, int T, int grid, hipStream_t st) {
  switch (MT) {
    case 1: return gateup_T<KIND, BF16H, 1>(g, T, grid, st);
    case 2: return gateup_T<KIND, BF16H, 2>(g, T, grid, st);
    case 4: return gateup_T<KIND, BF16H, 4>(g, T, grid, st);
    case 7: return gateup_T<KIND, BF16H, 7>(g, T, grid, st);
    case 13: return gateup_T<KIND, BF16H, 13>(g, T, grid, st);
  }
  return hipErrorInvalidValue;
}

template <int KIND, int MT>
hipError_t down_T(const DownArgs& d, int T, int grid, hipStream_t st) {
  switch (T) {
    case 1: return launch_down_t<MT, 1, KIND>(d, grid, st);
    case 2: return launch_down_t<MT, 2, KIND>(d, grid, st);
    case 3: return launch_down_t<MT, 3, KIND>(d, grid, st);
    case 4: if constexpr (MT * 4 <= 39) return launch_down_t<MT, 4, KIND>(d, grid, st); else break;
    case 8: if constexpr (MT * 8 <= 39) return launch_down_t<MT, 8, KIND>(d, grid, st); else break;
  }
  return hipErrorInvalidValue;
}

template <int KIND>
hipError_t down_dispatch(const DownArgs& d, int MT, int T, int grid, hipStream_t st) {
  switch (MT) {
    case 1: return down_T<KIND, 1>(d, T, grid, st);
    case 2: return down_T<KIND, 2>(d, T, grid, st);
    case 4: return down_T<KIND, 4>(d, T, grid, st);
    case 7: return down_T<KIND, 7>(d, T, grid, st);
    case 13: return down_T<KIND, 13>(d, T, grid, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// ---------------------------------------------------------------- forward

int launch_forward(const Plan& p, const FwdArgs& a) {
  hipStream_t st = (hipStream_t)a.stream;
  const BlobLayout L = blob_layout(p.hidden, p.inter, p.prec);
  uint8_t* ws = a.ws;
  uint8_t* xq = ws + p.off_xq;
  float* sx = (float*)(ws + p.off_sx);
  uint32_t* amax = (uint32_t*)(ws + p.off_amax);
  float* h32 = (float*)(ws + p.off_h32);
  uint8_t* hq = ws + p.off_hq;
  uint16_t* hb = (uint16_t*)(ws + p.off_hb);
  float* sh = (float*)(ws + p.off_sh);
  float* part = (float*)(ws + p.off_part);
  uint32_t* cnt = (uint32_t*)(ws + p.off_cnt);
  const int ncnt = p.n_mblocks * p.ngroups2;

  hipLaunchKernelGGL(k_xquant, dim3((p.Mpad + kWaves - 1) / kWaves), dim3(kThreads), 0, st, a.x, p.M, p.hidden,
                     p.Mpad, xq, sx, amax, cnt, ncnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;

  GateUpArgs g{};
  g.xq = xq; g.sx = sx;
  g.wcodes = a.blob + L.off_gu_codes;
  g.wscales = (const float*)(a.blob + L.off_gu_scales);
  g.wbscales = a.blob + L.off_gu_bscales;
  g.tscales = (const float*)(a.blob + offsetof(BlobHeader, s_gate));
  g.h32 = h32; g.hb = hb; g.amax_h = amax;
  g.H = p.hidden; g.I = p.inter; g.n_mb = p.n_mblocks;
  const int grid1 = p.ngroups1 * p.n_mblocks;
  if (p.prec == kFP8) e = gateup_dispatch<kGU_FP8, false>(g, p.MT, p.T1, grid1, st);
  else if (p.prec == kFP8DownBF16) e = gateup_dispatch<kGU_FP8, true>(g, p.MT, p.T1, grid1, st);
  else e = gateup_dispatch<kGU_FP4, false>(g, p.MT, p.T1, grid1, st);
  if (e != hipSuccess) return (int)e;

  if (p.prec != kFP8DownBF16) {
    hipLaunchKernelGGL(k_requant, dim3((p.inter + 1023) / 1024, p.Mpad), dim3(kThreads), 0, st, h32, amax, p.inter,
                       hq, sh);
    e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }

  DownArgs d{};
  d.A = p.prec == kFP8DownBF16 ? (const void*)hb : (const void*)hq;
  d.sh = sh;
  d.wcodes = a.blob + L.off_dn_codes;
  d.wscales = (const float*)(a.blob + L.off_dn_scales);
  d.wbscales = a.blob + L.off_dn_bscales;
  d.tscale = (const float*)(a.blob + offsetof(BlobHeader, s_down));
  d.part = part; d.counters = cnt; d.y = a.y;
  d.H = p.hidden; d.I = p.inter; d.M = p.M; d.Mpad = p.Mpad; d.n_mb = p.n_mblocks;
  d.ngroups = p.ngroups2; d.cps = p.chunks_per_split2; d.nsplit = p.nsplit2;
  const int grid2 = p.n_mblocks * p.ngroups2 * p.nsplit2;
  if (p.prec == kFP8) e = down_dispatch<kDN_FP8>(d, p.MT, p.T2, grid2, st);
  else if (p.prec == kFP8DownBF16) e = down_dispatch<kDN_BF16>(d, p.MT, p.T2, grid2, st);
  else e = down_dispatch<kDN_FP4>(d, p.MT, p.T2, grid2, st);
  return (int)e;
}

}  // namespace ocq
