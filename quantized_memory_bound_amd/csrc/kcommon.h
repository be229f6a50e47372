// Device-side building blocks shared by the ocq kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstddef>
#include <cstdint>

#include "ocq_internal.h"

namespace ocq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- arguments

// Activation operands (x, h) are stored in MFMA fragment order: blocks of 16
// rows x 128 inputs, block (mt, c) at (mt * C + c) * BLK bytes, and inside a
// block [unit][lane][16 B] where lane l = 16 g + r carries row r and inputs
// 128 c + 32 g .. +32 (the same k-ranges as the weight fragments).  E4M3 codes:
// BLK = 2048, 2 units (code j in unit j / 16); 16-bit values (fp16 / bf16):
// BLK = 4096, 4 units (value j in unit j / 8).  One 16 B load per lane then
// reads 1 KB of contiguous memory.
__device__ __forceinline__ size_t frag_off8(int m, int k, int C) {   // byte offset of code (m, k)
  const int mt = m >> 4, r = m & 15, c = k >> 7, g = (k >> 5) & 3, j = k & 31;
  return ((size_t)(mt * C + c) * 2 + (j >> 4)) * 1024 + (16 * g + r) * 16 + (j & 15);
}
__device__ __forceinline__ size_t frag_off16(int m, int k, int C) {  // element offset of value (m, k)
  const int mt = m >> 4, r = m & 15, c = k >> 7, g = (k >> 5) & 3, j = k & 31;
  return (((size_t)(mt * C + c) * 4 + (j >> 3)) * 64 + (16 * g + r)) * 8 + (j & 7);
}

struct GateUpArgs {
  const uint8_t* xq;        // E4M3 codes of x, fragment order, Mpad rows
  const float* sx;          // [Mpad]
  const uint8_t* wcodes;    // interleaved gate/up fragments
  const float* wscales;     // FP8: [2][I] per-row scales
  const uint8_t* wbscales;  // NVFP4: block-scale groups
  const float* tscales;     // NVFP4: blob header s_gate, s_up
  float* h32;               // FP8 / NVFP4 down modes: [I / 8][Mpad][8]: each 8-column tile
                            // of h is one contiguous [row][8] block
  uint16_t* hb;             // bf16(h), fragment order (BF16-down mode)
  uint16_t* tap_hb;         // optional plain [M][I] copy of bf16(h) (BF16-down mode)
  float* amax_part;         // [Mpad][ngroups] max |h| of each row over each workgroup's columns
  // per-token requantization inside the gate/up kernel (fused launches only):
  uint32_t* amax_g;         // [kAmaxSlots][Mpad] max |h| of each row (float bits, atomic max) over the
                            // workgroups of each copy, zeroed by the x quantization
  uint32_t* sync;           // [kSyncWords]: [0] arrival count, [1] wait time-out flag, release flags at
                            // kGoStride (1 + k), zeroed by the x quantization
  uint8_t* hq;              // E4M3 codes of h, fragment order, Mpad rows
  float* sh;                // [Mpad] row scales
  uint8_t* tap_hq;          // optional plain [M][I] copy of the codes
  float* tap_sh;            // optional plain [M] copy of the scales
  int H, I, M, n_mb, Mpad;
};

struct DownArgs {
  const void* A;            // hq codes (FP8 / NVFP4) or bf16(h) (BF16), fragment order
  const float* sh;          // [Mpad] (FP8 / NVFP4)
  const uint8_t* wcodes;
  const float* wscales;     // FP8: [H]
  const uint8_t* wbscales;  // NVFP4 block-scale groups
  const float* tscale;      // NVFP4: blob header s_down
  uint16_t* y;              // [M][H]
  const uint32_t* sync;     // gate/up wait flags (sync[1] != 0: the fused requantization timed out)
  int H, I, M, n_mb, ngroups;
};

// Events recorded by a launch itself at the kernel's start and end (nullable).
struct LaunchEvents {
  hipEvent_t start = nullptr, end = nullptr;
};

template <class K, class... Args>
inline void launch_kernel(K fn, dim3 grid, dim3 block, size_t lds, hipStream_t st, const LaunchEvents& ev,
                          Args... args) {
  if (ev.start || ev.end) hipExtLaunchKernelGGL(fn, grid, block, (uint32_t)lds, st, ev.start, ev.end, 0, args...);
  else hipLaunchKernelGGL(fn, grid, block, lds, st, args...);
}

// A kernel that uses more than 64 KB of dynamic LDS must be allowed it on
// each device it runs on (the attribute belongs to the device's copy of the
// kernel).  `done` holds one bit per device ordinal (< 64) on which it has
// been set; two threads racing only repeat the call.
inline hipError_t allow_lds(const void* fn, size_t bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
  if (bit && (done.load(std::memory_order_relaxed) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_relaxed);
  return e;
}

// fused: in (may the kernel requantize h itself) / out (did it)
hipError_t launch_gateup(const Plan& p, const GateUpArgs& g, hipStream_t st, const LaunchEvents& ev, bool& fused);
hipError_t launch_down(const Plan& p, const DownArgs& d, hipStream_t st);

constexpr int kMaxDevices = 64;

// Workgroups of kernel fn (threads per workgroup, dynamic LDS bytes) that
// can be resident at once on the current device: occupancy per CU times the
// CU count, cached per device ordinal in cap (0 = not yet known, -1 = none).
inline int resident_capacity(const void* fn, int threads, size_t lds, std::atomic<int> (&cap)[kMaxDevices]) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int c = cap[dev].load(std::memory_order_relaxed);
  if (c != 0) return c;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  c = per_cu * cus > 0 ? per_cu * cus : -1;
  cap[dev].store(c, std::memory_order_relaxed);
  return c;
}
hipError_t launch_gateup_large(const Plan& p, const GateUpArgs& g, hipStream_t st, const LaunchEvents& ev);
hipError_t launch_down_large(const Plan& p, const DownArgs& d, hipStream_t st);

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

// Eight E4M3 codes of fl32(v[j] / s) for s > 0 with rcp = fl32(1 / s), two
// dwords in element order: the same codes as enc_e4m3(v[j] / s).
//   * q = v rcp is within 2.5 units in the last place of fl32(v / s) (two
//     roundings of relative size 2^-24 each), so both round to the same E4M3
//     code unless a decision boundary lies that close: in the normal range a
//     midpoint has low 20 mantissa bits 0x80000 (tested with a window of
//     +-3 units); in the subnormal range (|q| < 2^-6, grid 2^-9) a midpoint
//     is an odd multiple of 2^-10, i.e. fract(|q| 2^9) = 1/2 (tested with a
//     window of 2^-19, more than 2.5 units there).  If any of the eight is
//     that close, all eight take the exact quotient (one branch, rarely taken).
//   * Clamped to +-448, the hardware conversion (nearest even, sign kept for
//     zero) gives the saturating code; checked equal to enc_e4m3 on every
//     midpoint +-3 units, the subnormals, both zeros and random values.
__device__ __forceinline__ v2u e4m3x8_quot(const float (&v)[8], float s, float rcp) {
  float q[8];
  bool near = false;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    q[j] = v[j] * rcp;
    const float t = fabsf(q[j]) * 512.0f;
    near |= (t < 8.0f) & (fabsf(__builtin_amdgcn_fractf(t) - 0.5f) < 0x1p-19f);
    near |= (__float_as_uint(q[j]) & 0xFFFFFu) - 0x7FFFDu <= 6u;
  }
  if (near) {
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = v[j] / s;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) q[j] = __builtin_amdgcn_fmed3f(q[j], -448.0f, 448.0f);
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], hi, true);
  return v2u{(uint32_t)lo, (uint32_t)hi};
}

// N E4M3 codes (low bytes) of fl32(v[j] / s) for s > 0 with rcp = fl32(1 / s):
// the rule of e4m3x8_quot (same window test, same fallback to the exact
// quotients, same saturating hardware conversion) for the N values of one
// row.  The exact quotients stay behind a branch that a wave skips unless
// one of its lanes needs them (computed unconditionally, the divisions were
// most of the in-launch requantization's vector work).
template <int N>
__device__ __forceinline__ void e4m3_quotN(const float (&v)[N], float s, float rcp, uint32_t (&c)[N]) {
  float q[N];
  bool near = false;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    q[j] = v[j] * rcp;
    const float t = fabsf(q[j]) * 512.0f;
    near |= (t < 8.0f) & (fabsf(__builtin_amdgcn_fractf(t) - 0.5f) < 0x1p-19f);
    near |= (__float_as_uint(q[j]) & 0xFFFFFu) - 0x7FFFDu <= 6u;
  }
  if (near) {
    asm volatile("");   // not speculated: the block has a side effect
#pragma unroll
    for (int j = 0; j < N; ++j) q[j] = v[j] / s;
  }
#pragma unroll
  for (int j = 0; j < N; ++j)
    c[j] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(q[j], -448.0f, 448.0f), 0.0f, 0, false) &
           0xFFu;
}

// One E4M3 code (low byte) of fl32(v / s) for s > 0 with rcp = fl32(1 / s):
// the single-value form of e4m3x8_quot (same window test, same fallback to
// the exact quotient, same saturating hardware conversion).
__device__ __forceinline__ uint32_t e4m3_quot1(float v, float s, float rcp) {
  float q = v * rcp;
  const float t = fabsf(q) * 512.0f;
  const bool near = (((int)(t < 8.0f) & (int)(fabsf(__builtin_amdgcn_fractf(t) - 0.5f) < 0x1p-19f)) |
                     (int)((__float_as_uint(q) & 0xFFFFFu) - 0x7FFFDu <= 6u)) != 0;   // no branch
  if (near) q = v / s;
  q = __builtin_amdgcn_fmed3f(q, -448.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q, 0.0f, 0, false) & 0xFFu;
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

// two E4M3 block scales (bytes of a 16-bit value) -> broadcast fp16 pairs
__device__ __forceinline__ void e4m3x2_scales(uint32_t two, v2h& s0, v2h& s1) {
  const v2h sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(two, 1.0f, false);
  s0 = v2h{sc[0], sc[0]};
  s1 = v2h{sc[1], sc[1]};
}

// SiLU(g) = g / (1 + e^-g) through the hardware exp2 and reciprocal (each
// about one unit in the last place of fp32): for h that is requantized to
// E4M3, whose 3-bit mantissa makes such a difference change a code only right
// next to a rounding midpoint.  e^-g overflowing to +inf gives -0 for very
// negative g.
__device__ __forceinline__ float silu_rcp(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// The same with the quotient refined by one residual step, q = q0 + (g - d q0) / d
// (the reciprocal's error no longer reaches the result, which is then the
// correctly rounded quotient but in rare cases), for the bf16 h of a BF16 down
// projection: its 8-bit mantissa makes a unit-in-the-last-place difference
// change bf16(h) far more often than an E4M3 code.  Cheaper than the IEEE
// division sequence (no scaling steps: d lies in [1, +inf]).
__device__ __forceinline__ float silu_div(float g) {
  const float d = 1.0f + __expf(-g);
  const float r = __builtin_amdgcn_rcpf(d);
  const float q0 = g * r;
  const float q = __builtin_fmaf(__builtin_fmaf(-d, q0, g), r, q0);
  return d == __builtin_inff() ? q0 : q;   // d = +inf: q0 = -0 (the refinement would be NaN)
}

// Cross-lane moves inside 16-lane rows through DPP (no LDS round trip).
// CTRL: 0x128 row_ror:8 (lane r <- r ^ 8), 0xB1 quad_perm [1,0,3,2] (r ^ 1),
// 0x4E quad_perm [2,3,0,1] (r ^ 2), 0x141 row_half_mirror (r <- 7 - r in
// each half-row).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// maximum over each group of 8 lanes (lanes 8k .. 8k+7)
__device__ __forceinline__ float max8(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  return fmaxf(v, dpp<0x141>(v));
}

// maximum over the wave, returned in every lane: 16-lane rows through DPP
// (0x140 row_mirror, r <- 15 - r), then the four row results via readlane
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(max8(v), dpp<0x140>(max8(v)));
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

template <class T>
__device__ __forceinline__ T ld_nt(const T* p) { return __builtin_nontemporal_load(p); }

// Workgroup barrier for LDS exchanges only: waits for this wave's LDS
// operations, not for its outstanding global stores (a __syncthreads() is a
// workgroup-scope release and would wait for those too).  Correct where no
// wave of the workgroup reads what the others stored to global memory.  The
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ v8i cat(v4i lo, v4i hi) {
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// ---------------------------------------------------------------- weight operand formats
//
// Weight tiles are 16 output rows; a chunk is 128 inputs.  Per format: bytes of
// one tile-chunk in the blob, and the matrix-core instruction used.
enum BFmt {
  kB_FP8_F16 = 1,   // E4M3 codes converted to fp16, MFMA 16x16x32 f16 (four per chunk)
  kB_BF16 = 2,      // bf16, MFMA 16x16x32 bf16 (four per chunk)
  kB_FP4_F16 = 3    // NVFP4 codes x block scale converted to fp16, MFMA 16x16x32 f16
};

template <int BF> struct Fmt;
// kA16: the activation operand is bf16 (BF16 down projection) rather than
// E4M3 codes (converted to fp16 in registers for the f16 formats).
template <> struct Fmt<kB_FP8_F16> { static constexpr int kGlobal = 2048, kUnits = 2, kLds = 4096; static constexpr bool kA16 = false; };
template <> struct Fmt<kB_BF16> { static constexpr int kGlobal = 4096, kUnits = 4, kLds = 4096; static constexpr bool kA16 = true; };
template <> struct Fmt<kB_FP4_F16> { static constexpr int kGlobal = 1024, kUnits = 1, kLds = 4096; static constexpr bool kA16 = false; };

template <int BF>
struct AGeom {
  static constexpr int kUnits = Fmt<BF>::kA16 ? 4 : 2;   // 16 B units per lane per chunk
  static constexpr int kBlk = kUnits * 1024;             // bytes per (m-tile, chunk) block
};

// One chunk's activation fragment of one m-tile for one lane
template <int BF>
struct AFrag {
  v4i q[AGeom<BF>::kUnits];
};

// p points at this lane's 16 B of unit 0 of the (m-tile, chunk) block
template <int BF>
__device__ __forceinline__ void load_a(AFrag<BF>& f, const uint8_t* p) {
#pragma unroll
  for (int u = 0; u < AGeom<BF>::kUnits; ++u) f.q[u] = *(const v4i*)(p + u * 1024);
}

}  // namespace ocq
