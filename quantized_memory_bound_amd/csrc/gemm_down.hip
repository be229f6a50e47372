// Down projection Y = A Wd^T, y = bf16(Y sh[m] sw_d[j]).
//
// A is the requantized h (E4M3 codes, FP8 and NVFP4 modes) or bf16(h) (BF16
// mode, a layer kept at higher precision: "OCRia 推理栈：单卡 B200 提速近 10 倍",
// section "Reducing the data moved: workload-aware quantization").  E4M3 and
// NVFP4 operands are converted exactly to fp16 in registers and summed by the
// f16 matrix cores in fp32: the E4M3 matrix-core forms sum their products
// with an error up to about 2^-15 of the sum of their magnitudes, which the
// exact-integer case of the pages' definition does not allow.
//
// One workgroup owns MT m-tiles x T output tiles over the whole input range;
// its NW waves take the 128-input chunks round-robin (every load of a wave is
// issued D chunks ahead, no workgroup barrier in the loop) and the NW partial
// tiles are summed in LDS in wave order, so the result is deterministic and no
// workgroup ever waits for another.  Workgroups that share weight tiles (same
// column group, different m-blocks) are numbered 8 apart, so the hardware's
// round-robin placement puts them on one XCD, where the second read of a
// weight tile hits that XCD's L2.
#include "gemm_core.h"

namespace ocq {
namespace {

template <int BF>
__device__ __forceinline__ float col_scale(const DownArgs& d, int j) {
  if constexpr (BF == kB_FP8_F16) return d.wscales[j];
  else if constexpr (BF == kB_FP4_F16) return d.tscale[0];
  else return 1.0f;
}

template <int BF>
__device__ __forceinline__ float row_scale(const DownArgs& d, int m) {
  if constexpr (BF == kB_BF16) return 1.0f;
  else return d.sh[m];
}

// workgroup -> (m-block, column group)
__device__ __forceinline__ void down_block(const DownArgs& d, int& mb, int& ng) {
  const int b = blockIdx.x;
  if (d.ngroups % 8 == 0) {
    const int q = b >> 3;
    mb = q % d.n_mb;
    ng = (q / d.n_mb) * 8 + (b & 7);
  } else {
    mb = b % d.n_mb;
    ng = b / d.n_mb;
  }
}

template <int BF, int MT, int T, int NW, int D>
__global__ __launch_bounds__(64 * NW) void ks_down(DownArgs d) {
  extern __shared__ v4f red[];
  int mb, ng;
  down_block(d, mb, ng);
  const int C = d.I / kChunk;
  const int row0 = mb * MT * 16;
  const size_t wt = (size_t)C * Fmt<BF>::kGlobal, bt = (size_t)((C + 7) / 8) * 1024;
  const LanePtrs lp = lane_ptrs<BF>((const uint8_t*)d.A + (size_t)(row0 / 16) * C * AGeom<BF>::kBlk, d.I, MT,
                                    d.wcodes + (size_t)ng * T * wt, wt, d.wbscales + (size_t)ng * T * bt, bt);
  v4f acc[MT][T];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[mt][t] = v4f{0.f, 0.f, 0.f, 0.f};
  ks_mainloop<BF, MT, T, NW, D, false>(lp, __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), 0, C, acc);
  ks_stash<MT, T>(acc, red);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, gq = lane >> 4, r = lane & 15;
  // a fused requantization whose grid-wide wait timed out left h codes of
  // undefined value: the output is NaN rather than plausible numbers
  const bool bad = d.sync != nullptr && d.sync[1] != 0u;
  for (int q = wave; q < MT * T; q += NW) {
    const int mt = q / T, t = q % T;
    const int j = (ng * T + t) * 16 + r;
    const int mbase = row0 + mt * 16 + 4 * gq;
    float rs[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) rs[i] = row_scale<BF>(d, mbase + i);   // rows < Mpad: always readable
    const float cs = col_scale<BF>(d, j);
    const v4f v = ks_sum<NW>(red, MT * T, 0, 1, q, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (mbase + i < d.M) d.y[(size_t)(mbase + i) * d.H + j] = bad ? (uint16_t)0x7FC0u : (uint16_t)bf16_bits(v[i] * rs[i] * cs);
  }
}

// ---------------------------------------------------------------- dispatch

// registers of one chunk's operands (A and B fragments) per lane
template <int BF, int MT, int T>
constexpr int chunk_vgprs() {
  return 4 * (MT * AGeom<BF>::kUnits + T * Fmt<BF>::kUnits);
}

template <int BF, int MT, int T, int NW, int D>
hipError_t go_d(const DownArgs& d, int grid, hipStream_t st) {
  auto fn = ks_down<BF, MT, T, NW, D>;
  const size_t lds = (size_t)NW * MT * T * 256 * sizeof(float);
  static std::atomic<uint64_t> lds_set{0};
  if (hipError_t e = allow_lds((const void*)fn, lds, lds_set); e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(64 * NW), lds, st, d);
  return hipGetLastError();
}

// Eight waves (two per SIMD) unless one chunk's operands need more than 64
// registers, then four; the prefetch depth is what fits in about 160 (eight
// waves; 128 when the operands are converted to fp16 in registers) or 320
// (four waves) registers, at most 3, preferring a depth that divides the
// per-wave chunk count (no zero-weight padding iterations).  A workgroup of
// one 16 x 16 E4M3 tile (few rows: 128 workgroups for 2048 outputs) runs
// sixteen waves with every chunk in flight at once.
template <int BF, int MT, int T>
hipError_t go(const DownArgs& d, int grid, hipStream_t st) {
  constexpr int CV = chunk_vgprs<BF, MT, T>();
  constexpr bool ONE = BF == kB_FP8_F16 && MT * T == 1;
  constexpr int NW = CV > 64 ? 4 : (ONE ? 16 : 8);
  constexpr int BUDGET = NW == 4 ? 320 : (BF == kB_BF16 ? 160 : 128);
  constexpr int DMAX = ONE ? 3 : (BUDGET / CV >= 3 ? 3 : (BUDGET / CV >= 2 ? 2 : 1));
  const int nk = (d.I / kChunk + NW - 1) / NW;
  if constexpr (DMAX >= 3) {
    if (nk % 3 == 0 || nk % 2 != 0) return go_d<BF, MT, T, NW, 3>(d, grid, st);
  }
  if constexpr (DMAX >= 2) {
    if (nk >= 2) return go_d<BF, MT, T, NW, 2>(d, grid, st);
  }
  return go_d<BF, MT, T, NW, 1>(d, grid, st);
}

template <int BF, int MT>
hipError_t go_t(const DownArgs& d, int T, int grid, hipStream_t st) {
  switch (T) {
    case 1: return go<BF, MT, 1>(d, grid, st);
    case 2: return go<BF, MT, 2>(d, grid, st);
    case 4: return go<BF, MT, 4>(d, grid, st);
  }
  return hipErrorInvalidValue;
}

template <int BF>
hipError_t go_mt(const DownArgs& d, int MT, int T, int grid, hipStream_t st) {
  switch (MT) {
    case 1: return go_t<BF, 1>(d, T, grid, st);
    case 2: return go_t<BF, 2>(d, T, grid, st);
    case 4: return go_t<BF, 4>(d, T, grid, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_down(const Plan& p, const DownArgs& d, hipStream_t st) {
  if (p.lg2) return launch_down_large(p, d, st);
  const int grid = p.n_mb2 * p.ngroups2;
  if (p.prec == kFP8) return go_mt<kB_FP8_F16>(d, p.MT2, p.T2, grid, st);
  if (p.prec == kFP8DownBF16) return go_mt<kB_BF16>(d, p.MT2, p.T2, grid, st);
  return go_mt<kB_FP4_F16>(d, p.MT2, p.T2, grid, st);
}

}  // namespace ocq
