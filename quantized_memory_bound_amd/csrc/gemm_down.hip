// Down projection Y = A Wd^T, y = bf16(Y sh[m] sw_d[j]).
//
// A is the requantized h (E4M3 codes, FP8 and NVFP4 modes) or bf16(h) (BF16
// mode, a layer kept at higher precision: "OCRia 推理栈：单卡 B200 提速近 10 倍",
// section "Reducing the data moved: workload-aware quantization").  The
// input range is split across workgroups when there are too few output tiles
// to fill the GPU; each split writes an fp32 partial tile, and the last
// workgroup of an output group to arrive sums the partials in split order
// (deterministic) and applies the scales.
#include "gemm_core.h"

namespace ocq {
namespace {

constexpr int kKsWaves = 8;

template <int BF>
__device__ __forceinline__ float col_scale(const DownArgs& d, int j) {
  if constexpr (BF == kB_FP8) return d.wscales[j];
  else if constexpr (BF == kB_FP4_F16) return d.tscale[0];
  else return 1.0f;
}

template <int BF>
__device__ __forceinline__ float row_scale(const DownArgs& d, int m) {
  if constexpr (BF == kB_BF16) return 1.0f;
  else return d.sh[m];
}

// Store one finished 16x16 tile (value v at this lane) as y or as a partial.
template <int BF>
__device__ __forceinline__ void down_store(const DownArgs& d, const v4f& v, int m_base, int tile, int sp) {
  const int lane = threadIdx.x & 63, gq = lane >> 4, r = lane & 15;
  const int j = tile * 16 + r;
  if (d.nsplit == 1) {
    const float cs = col_scale<BF>(d, j);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m_base + 4 * gq + i;
      if (m < d.M) d.y[(size_t)m * d.H + j] = (uint16_t)bf16_bits(v[i] * row_scale<BF>(d, m) * cs);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) d.part[((size_t)sp * d.Mpad + m_base + 4 * gq + i) * d.pp + j] = v[i];
  }
}

// Arrival count of a split; the last arriver sums all partials of the
// group's tiles (rows row0 .. row0 + 16 MT, T tiles) in split order.
template <int BF, int MT, int T>
__device__ __forceinline__ void down_finish_split(const DownArgs& d, int mb, int ng, int row0) {
  __shared__ int s_last;
  // drain this workgroup's partial stores to L2, then one agent-scope
  // release (L2 write-back) before the arrival; the last arriver acquires
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const unsigned prev = __hip_atomic_fetch_add(&d.counters[mb * d.ngroups + ng], 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (unsigned)(d.nsplit - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  // items: (row, 4 consecutive columns); up to 8 items per thread, all split
  // loads of an item issued before they are summed
  constexpr int kCols4 = T * 4;
  const int nitems = 16 * MT * kCols4;
  const int col0 = ng * T * 16;
  for (int base = 0; base < nitems; base += 8 * (int)blockDim.x) {
    v4f s[8];
    int m_of[8], c_of[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int it = base + q * (int)blockDim.x + (int)threadIdx.x;
      m_of[q] = row0 + it / kCols4;
      c_of[q] = col0 + (it % kCols4) * 4;
      s[q] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    for (int sp = 0; sp < d.nsplit; ++sp) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int it = base + q * (int)blockDim.x + (int)threadIdx.x;
        if (it < nitems && m_of[q] < d.M)
          s[q] += __builtin_nontemporal_load((const v4f*)(d.part + ((size_t)sp * d.Mpad + m_of[q]) * d.pp + c_of[q]));
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int it = base + q * (int)blockDim.x + (int)threadIdx.x;
      const int m = m_of[q];
      if (it < nitems && m < d.M) {
        const float rs = row_scale<BF>(d, m);
        uint32_t o[2];
#pragma unroll
        for (int e = 0; e < 2; ++e)
          o[e] = bf16_bits(s[q][2 * e] * rs * col_scale<BF>(d, c_of[q] + 2 * e)) |
                 (bf16_bits(s[q][2 * e + 1] * rs * col_scale<BF>(d, c_of[q] + 2 * e + 1)) << 16);
        *(v2u*)(d.y + (size_t)m * d.H + c_of[q]) = v2u{o[0], o[1]};
      }
    }
  }
}

// ---- K-split (few rows)
template <int BF, int MT, int T>
__global__ __launch_bounds__(64 * kKsWaves) void ks_down(DownArgs d) {
  extern __shared__ float red[];
  const int mb = blockIdx.x % d.n_mb;
  const int rest = blockIdx.x / d.n_mb;
  const int ng = rest % d.ngroups, sp = rest / d.ngroups;
  const int C = d.I / kChunk;
  const int c0 = sp * d.cps, c1 = min(C, c0 + d.cps);
  const int row0 = mb * MT * 16;
  const size_t wt = (size_t)C * Fmt<BF>::kGlobal, bt = (size_t)((C + 7) / 8) * 1024;
  const LanePtrs lp = lane_ptrs<BF>((const uint8_t*)d.A + (size_t)(row0 / 16) * C * AGeom<BF>::kBlk, d.I,
                                    d.wcodes + (size_t)ng * T * wt, wt, d.wbscales + (size_t)ng * T * bt, bt);
  v4f acc[MT][T];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[mt][t] = v4f{0.f, 0.f, 0.f, 0.f};
  ks_mainloop<BF, MT, T, kKsWaves>(lp, c0, c1, acc);
  ks_stash<MT, T>(acc, red);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int p = wave; p < MT * T; p += kKsWaves) {
    v4f v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = ks_sum<kKsWaves>(red, MT * T, p, i, lane);
    down_store<BF>(d, v, row0 + (p / T) * 16, ng * T + p % T, sp);
  }
  if (d.nsplit > 1) down_finish_split<BF, MT, T>(d, mb, ng, row0);
}

// ---- M-split (many rows)
template <int BF, int MT, int T>
__global__ __launch_bounds__(64 * kMsWaves) void ms_down(DownArgs d) {
  using G = MsGeom<BF, MT, T>;
  __shared__ v4i lds[2 * G::SLOT / 16];
  const int mb = blockIdx.x % d.n_mb;
  const int rest = blockIdx.x / d.n_mb;
  const int ng = rest % d.ngroups, sp = rest / d.ngroups;
  const int C = d.I / kChunk;
  const int c0 = sp * d.cps, c1 = min(C, c0 + d.cps);
  const int row0 = mb * MT * 16;
  const size_t wt = (size_t)C * Fmt<BF>::kGlobal, bt = (size_t)((C + 7) / 8) * 1024;
  const LanePtrs lp = lane_ptrs<BF>((const uint8_t*)d.A + (size_t)(row0 / 16) * C * AGeom<BF>::kBlk, d.I,
                                    d.wcodes + (size_t)ng * T * wt, wt, d.wbscales + (size_t)ng * T * bt, bt);
  v4f acc[G::MTW][T];
#pragma unroll
  for (int j = 0; j < G::MTW; ++j)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[j][t] = v4f{0.f, 0.f, 0.f, 0.f};
  ms_mainloop<BF, MT, T>(lp, c0, c1, lds, acc);
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < G::MTW; ++j) {
    const int mt = wave + kMsWaves * j;
    if (mt < MT)
#pragma unroll
      for (int t = 0; t < T; ++t) down_store<BF>(d, acc[j][t], row0 + mt * 16, ng * T + t, sp);
  }
  if (d.nsplit > 1) down_finish_split<BF, MT, T>(d, mb, ng, row0);
}

// ---------------------------------------------------------------- dispatch

template <int BF, int MT, int T>
hipError_t go(const DownArgs& d, int grid, hipStream_t st) {
  if constexpr (MT <= 4) {
    auto fn = ks_down<BF, MT, T>;
    const size_t lds = (size_t)kKsWaves * MT * T * 256 * sizeof(float);
    static bool attr = false;   // idempotent; a race only repeats the call
    if (!attr) {
      hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      attr = true;
    }
    hipLaunchKernelGGL(fn, dim3(grid), dim3(64 * kKsWaves), lds, st, d);
  } else {
    hipLaunchKernelGGL((ms_down<BF, MT, T>), dim3(grid), dim3(64 * kMsWaves), 0, st, d);
  }
  return hipGetLastError();
}

template <int BF, int MT>
hipError_t go_t(const DownArgs& d, int T, int grid, hipStream_t st) {
  switch (T) {
    case 1: return go<BF, MT, 1>(d, grid, st);
    case 2: return go<BF, MT, 2>(d, grid, st);
  }
  return hipErrorInvalidValue;
}

template <int BF>
hipError_t go_mt(const DownArgs& d, int MT, int T, int grid, hipStream_t st) {
  switch (MT) {
    case 1: return go_t<BF, 1>(d, T, grid, st);
    case 2: return go_t<BF, 2>(d, T, grid, st);
    case 4: return go_t<BF, 4>(d, T, grid, st);
    case 7: return go_t<BF, 7>(d, T, grid, st);
    case 13: return go_t<BF, 13>(d, T, grid, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_down(const Plan& p, const DownArgs& d, hipStream_t st) {
  const int grid = p.n_mblocks * p.ngroups2 * p.nsplit2;
  if (p.prec == kFP8) return go_mt<kB_FP8>(d, p.MT, p.T2, grid, st);
  if (p.prec == kFP8DownBF16) return go_mt<kB_BF16>(d, p.MT, p.T2, grid, st);
  return go_mt<kB_FP4_F16>(d, p.MT, p.T2, grid, st);
}

}  // namespace ocq
