// Matrix-core main loop of the skinny GEMMs (activations [rows x K] times
// weight tiles [16 x K]).
//
// A workgroup owns a block of m-tiles (16 rows each) x T weight tiles and the
// whole input range.  Its waves form an MS x KS grid: wave (ms, ks) holds the
// accumulators of m-tiles ms*MTW .. ms*MTW+MTW-1 and runs over the chunks
// (128 inputs) ks, ks+KS, ks+2KS, ...  Every wave loads its own operand
// fragments straight from memory into registers (16 B per lane per load,
// weights non-temporal), D chunks ahead, and converts them to the matrix-core
// format in registers; there is no LDS traffic and no barrier in the loop, so
// the waves never wait for each other.  Each (row, input) and each (weight
// row, input) pair is loaded by exactly one wave of the workgroup when MS = 1,
// weights by MS waves otherwise.  After the loop the KS partial tiles of every
// m-tile are summed in LDS in a fixed order (deterministic).
//
// Accumulator layout (MFMA 16x16 fp32): lane l holds rows 4 (l/16) + i,
// i = 0..3, of column l % 16 of the tile.
#pragma once
#include "kcommon.h"

namespace ocq {

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt for vector-memory count <= N only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14; expcnt 6:4 and lgkmcnt 11:8 left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ---------------------------------------------------------------- per-chunk registers (K-split)

template <int BF, int MT, int T>
struct ChunkRegs {
  AFrag<BF> a[MT];
  v4i b[T][Fmt<BF>::kUnits];
  uint32_t sb[T];
};

// Global operand pointers of one lane.
struct LanePtrs {
  const uint8_t* a;    // activation block (first m-tile, chunk 0) + lane * 16 (fragment order)
  size_t a_mt_stride;  // bytes between m-tiles (all chunks of 16 rows)
  int a_chunk;         // bytes per (m-tile, chunk) block
  int a_nvalid;        // m-tiles of this wave that exist; later ones reload the last
  const uint8_t* w;    // weight tile 0 of the group, + lane * 16
  size_t w_tile;       // bytes per weight tile
  const uint8_t* wb;   // NVFP4 block-scale groups of tile 0, + lane * 16
  size_t wb_tile;
};

// A: fragment-ordered activations of the wave's first m-tile, K inputs;
// nvalid: wave-uniform count of its m-tiles that exist
template <int BF>
__device__ __forceinline__ LanePtrs lane_ptrs(const void* A, int K, int nvalid, const uint8_t* W, size_t w_tile,
                                              const uint8_t* Wb, size_t wb_tile) {
  const int lane = threadIdx.x & 63;
  LanePtrs p;
  p.a = (const uint8_t*)A + lane * 16;
  p.a_chunk = AGeom<BF>::kBlk;
  p.a_mt_stride = (size_t)(K / kChunk) * AGeom<BF>::kBlk;
  p.a_nvalid = nvalid;
  p.w = W + lane * 16;
  p.w_tile = w_tile;
  p.wb = Wb + lane * 16;
  p.wb_tile = wb_tile;
  return p;
}

// WNT: weight loads carry the non-temporal hint.  Right when every weight
// byte is read by one workgroup only; where several workgroups on one XCD
// share weight tiles (the down projection's m-blocks) plain loads keep the
// lines in L2 for the others.
template <int BF, int MT, int T, bool WNT = true>
__device__ __forceinline__ void load_chunk(ChunkRegs<BF, MT, T>& r, const LanePtrs& p, int c) {
#pragma unroll
  for (int t = 0; t < T; ++t) {
#pragma unroll
    for (int u = 0; u < Fmt<BF>::kUnits; ++u) {
      const v4i* q = (const v4i*)(p.w + t * p.w_tile + (size_t)c * Fmt<BF>::kGlobal + u * 1024);
      r.b[t][u] = WNT ? ld_nt(q) : *q;
    }
    if constexpr (BF == kB_FP4_F16)
      r.sb[t] = *(const uint16_t*)(p.wb + t * p.wb_tile + (size_t)(c >> 3) * 1024 + 2 * (c & 7));
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    load_a<BF>(r.a[mt], p.a + (mt < p.a_nvalid ? mt : p.a_nvalid - 1) * p.a_mt_stride + (size_t)c * p.a_chunk);
}

// B operand of tile t, sub-step i, from raw registers
template <int BF, int MT, int T>
__device__ __forceinline__ auto b_from_regs(const ChunkRegs<BF, MT, T>& r, int t, int i) {
  if constexpr (BF == kB_FP8_F16) {
    const v4i& w = r.b[t][i >> 1];
    return e4m3x8_to_f16((uint32_t)w[2 * (i & 1)], (uint32_t)w[2 * (i & 1) + 1]);
  } else if constexpr (BF == kB_BF16) {
    return __builtin_bit_cast(v8bf, r.b[t][i]);
  } else {
    v2h s0, s1;
    e4m3x2_scales(r.sb[t], s0, s1);
    return e2m1x8_to_f16((uint32_t)r.b[t][0][i], i < 2 ? s0 : s1);
  }
}

// acc[j][t] += A[j] x B[t] over one chunk (all NMT m-tiles; padding tiles
// hold duplicate data and are discarded by the caller)
// (MFMA 16x16x32 f16 on exact fp16 conversions of E4M3 / E2M1 operands, or
// 16x16x32 bf16; four sub-steps of 32 inputs per chunk)
template <int BF, int NMT, int T, class BGet>
__device__ __forceinline__ void compute_chunk(v4f (&acc)[NMT][T], const AFrag<BF> (&a)[NMT], int, BGet bget) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    decltype(bget(0, 0)) b[T];
#pragma unroll
    for (int t = 0; t < T; ++t) b[t] = bget(t, i);
#pragma unroll
    for (int j = 0; j < NMT; ++j) {
      if constexpr (BF == kB_BF16) {
        const v8bf av = __builtin_bit_cast(v8bf, a[j].q[i]);
#pragma unroll
        for (int t = 0; t < T; ++t) acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b[t], acc[j][t], 0, 0, 0);
      } else {
        const v4i& w = a[j].q[i >> 1];
        const v8h av = e4m3x8_to_f16((uint32_t)w[2 * (i & 1)], (uint32_t)w[2 * (i & 1) + 1]);
#pragma unroll
        for (int t = 0; t < T; ++t) acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, b[t], acc[j][t], 0, 0, 0);
      }
    }
  }
}

// ---------------------------------------------------------------- software pipeline
//
// Runs proc(d, k) for k = 0 .. n-1 with chunk k held in register buffer
// d = k % D, refilling buffer d with chunk k + D right after it is consumed.
// When n is a positive multiple of D the prologue and every steady-state
// refill are unconditional and the last group is peeled, so the compiler sees
// the same sequence of outstanding loads on every path into the loop and
// waits only for the buffer it is about to use (a conditional load would make
// it wait for all outstanding loads).  Other n take the general loop.
template <int D, class Load, class Proc>
__device__ __forceinline__ void pipelined(int n, Load load, Proc proc) {
  if (n >= D && n % D == 0) {
#pragma unroll
    for (int d = 0; d < D; ++d) load(d, d);
    for (int g = 0; g + D < n; g += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        proc(d, g + d);
        load(d, g + d + D);
      }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) proc(d, n - D + d);
  } else {
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (d < n) load(d, d);
    for (int g = 0; g < n; g += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        if (g + d < n) {
          proc(d, g + d);
          if (g + d + D < n) load(d, g + d + D);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- K-split main loop

template <int BF, int MT, int T>
__device__ __forceinline__ void zero_b(ChunkRegs<BF, MT, T>& r) {
#pragma unroll
  for (int t = 0; t < T; ++t) {
#pragma unroll
    for (int u = 0; u < Fmt<BF>::kUnits; ++u) r.b[t][u] = v4i{0, 0, 0, 0};
    r.sb[t] = 0u;
  }
}

// Every wave runs the same number of iterations, rounded up to a multiple of
// the prefetch depth D (D chunks in flight); a chunk index past the range is
// clamped to the last chunk for the loads and its weight operand is zeroed,
// so no load depends on the wave or the iteration.  kidx: the wave's K-split
// index (wave-uniform), KS: number of K-split waves.
template <int BF, int MT, int T, int KS, int D, bool WNT = true>
__device__ __forceinline__ void ks_mainloop(const LanePtrs& p, int kidx, int c0, int c1, v4f (&acc)[MT][T]) {
  const int nk = ((c1 - c0 + KS - 1) / KS + D - 1) / D * D;
  ChunkRegs<BF, MT, T> r[D];
  pipelined<D>(
      nk,
      [&](int d, int k) {
        const int c = c0 + kidx + k * KS;
        load_chunk<BF, MT, T, WNT>(r[d], p, c < c1 ? c : c1 - 1);
      },
      [&](int d, int k) {
        if (c0 + kidx + k * KS >= c1) zero_b(r[d]);
        compute_chunk<BF, MT, T>(acc, r[d].a, MT, [&](int t, int i) { return b_from_regs(r[d], t, i); });
      });
}

// Main loop for the f16-converting formats with E4M3 activations (gate/up),
// for waves that hold many m-tiles and cannot afford a second register copy
// of a chunk.  Each operand fragment is two 16 B units per lane: unit 0 feeds
// sub-steps 0-1, unit 1 sub-steps 2-3.  As soon as a unit has been consumed
// its registers are reloaded in place: activations with the next chunk,
// weights with the chunk after next (two weight buffers alternate), so the
// L2 latency of the activations and the HBM latency of the weights are
// covered by the remaining work of the current chunk.  NVFP4 weights are one
// unit per tile, reloaded after sub-step 3.  Scheduling fences keep every
// reload at the point where its unit is free, so the compiler neither
// hoists it (which would need more registers) nor waits on it early.  EXACT:
// every wave has the same even number of chunks (no padding chunk, no
// zeroing); otherwise the count is rounded up to even, chunk indices past the
// range are clamped for the loads and their weight operand is zeroed.
// NK > 0: every wave has exactly NK chunks and the loop is fully unrolled, so
// the compiler knows which loads each wait is for (across a loop back-edge it
// waits for all of them).
template <int BF, int MT, int T, int KS, bool EXACT, int NK = 0>
__device__ __forceinline__ void ks_mainloop_roll(const LanePtrs& p, int kidx, int c0, int c1, v4f (&acc)[MT][T]) {
  static_assert(BF == kB_FP8_F16 || BF == kB_FP4_F16, "f16-converting weight formats only");
  constexpr int UB = Fmt<BF>::kUnits;
  const int nk = NK > 0 ? NK : ((c1 - c0 + KS - 1) / KS + 1) / 2 * 2;
  auto cidx = [&](int k) { const int c = c0 + kidx + k * KS; return c < c1 ? c : c1 - 1; };
  auto a_ld = [&](int mt, int c, int u) {
    return *(const v4i*)(p.a + (mt < p.a_nvalid ? mt : p.a_nvalid - 1) * p.a_mt_stride + (size_t)c * p.a_chunk +
                         u * 1024);
  };
  auto b_ld = [&](int t, int c, int u) {   // plain loads (measured faster than non-temporal here)
    return *(const v4i*)(p.w + t * p.w_tile + (size_t)c * Fmt<BF>::kGlobal + u * 1024);
  };
  auto sb_ld = [&](int t, int c) {
    return (uint32_t) * (const uint16_t*)(p.wb + t * p.wb_tile + (size_t)(c >> 3) * 1024 + 2 * (c & 7));
  };
  v4i a[MT][2];
  v4i b[2][T][UB];
  uint32_t sb[2][T];
#pragma unroll
  for (int d = 0; d < 2; ++d)
#pragma unroll
    for (int t = 0; t < T; ++t) {
#pragma unroll
      for (int u = 0; u < UB; ++u) b[d][t][u] = b_ld(t, cidx(d), u);
      sb[d][t] = BF == kB_FP4_F16 ? sb_ld(t, cidx(d)) : 0u;
    }
#pragma unroll
  for (int j = 0; j < MT; ++j) {
    a[j][0] = a_ld(j, cidx(0), 0);
    a[j][1] = a_ld(j, cidx(0), 1);
  }
#pragma unroll
  for (int k0 = 0; k0 < (NK > 0 ? NK : nk); k0 += 2) {
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const int k = k0 + d;
      const int cn = cidx(k + 1), cb = cidx(k + 2);
      if constexpr (!EXACT) {
        if (c0 + kidx + k * KS >= c1) {
#pragma unroll
          for (int t = 0; t < T; ++t)
#pragma unroll
            for (int u = 0; u < UB; ++u) b[d][t][u] = v4i{0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v8h bv[T];
#pragma unroll
        for (int t = 0; t < T; ++t) {
          if constexpr (BF == kB_FP8_F16) {
            const v4i& w = b[d][t][i >> 1];
            bv[t] = e4m3x8_to_f16((uint32_t)w[2 * (i & 1)], (uint32_t)w[2 * (i & 1) + 1]);
          } else {
            v2h s0, s1;
            e4m3x2_scales(sb[d][t], s0, s1);
            bv[t] = e2m1x8_to_f16((uint32_t)b[d][t][0][i], i < 2 ? s0 : s1);
          }
        }
#pragma unroll
        for (int j = 0; j < MT; ++j) {
          const v4i& w = a[j][i >> 1];
          const v8h av = e4m3x8_to_f16((uint32_t)w[2 * (i & 1)], (uint32_t)w[2 * (i & 1) + 1]);
#pragma unroll
          for (int t = 0; t < T; ++t) acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv[t], acc[j][t], 0, 0, 0);
        }
        if (i == 1 || i == 3) {
          const int u = i >> 1;
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int j = 0; j < MT; ++j) a[j][u] = a_ld(j, cn, u);
          if constexpr (BF == kB_FP8_F16) {
#pragma unroll
            for (int t = 0; t < T; ++t) b[d][t][u] = b_ld(t, cb, u);
          } else if (i == 3) {
#pragma unroll
            for (int t = 0; t < T; ++t) {
              b[d][t][0] = b_ld(t, cb, 0);
              sb[d][t] = sb_ld(t, cb);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- gate/up epilogue

// Epilogue of one 16x16 gate/up tile pair for one m-tile: v = accumulated tile (gate
// in lanes r < 8, up in lanes r + 8 of each 16-lane row, rows 4 gq + i),
// m_base = first row of the m-tile, n = column of h.  One DPP exchange gives
// gate lane r the up values of rows 0, 2 and up lane r + 8 the gate values of
// rows 1, 3, so every lane evaluates two of the four h values: value e is row
// 4 gq + 2 e (gate lanes) or 4 gq + 2 e + 1 (up lanes).  Each 16-lane group
// then stores two adjacent rows of the tile's 8 columns: 64 contiguous bytes
// of the [tile][row][8] h32 block.  amax[e] accumulates |h| of value e.
// SKIP_PAD: rows >= M (padding, never read back) store no h32.
// h = SiLU(G) U of the lane's two values (value e: row 4 gq + 2 e of the
// m-tile for gate lanes, 4 gq + 2 e + 1 for up lanes; column r % 8 of the
// tile), from the accumulated tile v, the lane's row scales xs and the
// column's gate / up scales.  BF16H: the exact-division SiLU (h becomes bf16).
template <bool BF16H>
__device__ __forceinline__ void gateup_tile_h(const v4f v, const v4f xs, float cg, float cu, float (&hv)[2]) {
  const bool lo = (threadIdx.x & 15) < 8;
  // gate lanes send G of rows 1, 3 and receive U of rows 0, 2
  const float p0 = dpp<0x128>(lo ? v[1] : v[0]);
  const float p1 = dpp<0x128>(lo ? v[3] : v[2]);
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    // selects, not a lane-dependent array index, which would put xs and v in
    // scratch memory
    const float vi = lo ? v[2 * e] : v[2 * e + 1];
    const float xi = lo ? xs[2 * e] : xs[2 * e + 1];
    const float gv = lo ? vi : (e ? p1 : p0);
    const float uv = lo ? (e ? p1 : p0) : vi;
    const float ga = gv * xi * cg;
    hv[e] = (BF16H ? silu_div(ga) : silu_rcp(ga)) * (uv * xi * cu);
  }
}

// row (within the m-tile) of the lane's value e in gateup_tile_h
__device__ __forceinline__ int gateup_value_row(int e) {
  const int lane = threadIdx.x & 63;
  return 4 * (lane >> 4) + 2 * e + ((lane & 8) ? 1 : 0);
}

template <bool BF16H, int T, bool SKIP_PAD = false>
__device__ __forceinline__ void gateup_tile_epilogue(const GateUpArgs& g, const v4f v, const v4f xs,
                                                     float cg, float cu, int m_base, int ng, int t,
                                                     float (&amax)[2]) {
  const int lane = threadIdx.x & 63;
  const int c = lane & 7, n = (ng * T + t) * 8 + c;
  float h[2];
  gateup_tile_h<BF16H>(v, xs, cg, cu, h);
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const float hv = h[e];
    const int m = m_base + gateup_value_row(e);
    if constexpr (BF16H) {
      const uint16_t hb = (uint16_t)bf16_bits(hv);
      g.hb[frag_off16(m, n, g.I / 128)] = hb;
      if (g.tap_hb && m < g.M) g.tap_hb[(size_t)m * g.I + n] = hb;
    } else {
      if (!SKIP_PAD || m < g.M) g.h32[((size_t)(ng * T + t) * g.Mpad + m) * 8 + c] = hv;
      amax[e] = fmaxf(amax[e], fabsf(hv));
    }
  }
}

// ---------------------------------------------------------------- per-token requantization inside gate/up
//
// The row scale sh = max_n |h| / 448 spans the columns of every gate/up
// workgroup.  When the whole grid is resident at once (checked on the host
// before such a launch), each workgroup folds its row maxima into one of the
// kAmaxSlots copies of amax_g with device-scope atomic maxima, arrives at a
// device-scope counter and waits for every workgroup to arrive (the last to
// arrive sets the kGoCopies release flags, each polled by a few workgroups);
// it then combines the copies for its rows and quantizes the h values it has
// kept in registers, so h never goes to memory (the
// German page "Wie es funktioniert": SiLU and quantization fused, the
// intermediate kept on chip).  Device-scope atomics and loads are coherent
// across the XCDs' L2 caches, so no cache write-back or invalidation is
// needed: a wave's atomics are complete once it has waited for its vector
// memory counter, which every wave does before its workgroup arrives.  The
// wait is bounded (kGridWaitTicks of the 100 MHz clock): if the grid is not
// all resident (the GPU shared with other work) the waiting workgroups set
// sync[1] and go on, and the down projection then writes NaN for y.

constexpr uint64_t kGridWaitTicks = 10000000;   // 0.1 s

// Returns the value the atomic replaced: the returning form of the atomic,
// whose result arrives only once the maximum has been performed.  Callers
// OR the results together and hand them to grid_arrive_and_wait, which waits
// for them before the workgroup arrives.
__device__ __forceinline__ uint32_t amax_atomic(const GateUpArgs& g, int m, float a) {
  uint32_t* copy = g.amax_g + (size_t)(blockIdx.x % kAmaxSlots) * g.Mpad;
  // |h| >= +0: the float order is the unsigned order of the bits
  return __hip_atomic_fetch_max(copy + m, __float_as_uint(a), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every wave of the workgroup calls this (two workgroup barriers inside);
// seen: the OR of the wave's amax_atomic results (0 if it made none).  Also
// clears the workgroup's nrows row maxima rmax in LDS for grid_row_maxima.
__device__ __forceinline__ void grid_arrive_and_wait(uint32_t* sync, uint32_t nwg, uint32_t seen, float* rmax,
                                                     int nrows) {
  asm volatile("" ::"v"(seen));   // the results have arrived: this wave's maxima are performed
  wait_vm<0>();
  for (int i = threadIdx.x; i < nrows; i += blockDim.x) rmax[i] = 0.0f;
  lds_barrier();                  // ... and those of every wave of the workgroup
  if (threadIdx.x < 64) {          // wave 0
    uint32_t last = 0u;
    if (threadIdx.x == 0) {
      const uint32_t G = kArriveGroups, grp = blockIdx.x % G;
      const uint32_t members = nwg / G + (grp < nwg % G ? 1u : 0u);
      uint32_t* gc = sync + kGoStride * (1 + kGoCopies + grp);
      if (__hip_atomic_fetch_add(gc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == members - 1) {
        const uint32_t groups = nwg < G ? nwg : G;   // the last of its group arrives for the group
        last = __hip_atomic_fetch_add(sync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == groups - 1 ? 1u : 0u;
      }
    }
    last = __builtin_amdgcn_readfirstlane(last);
    if (last) {                   // every other workgroup has arrived: release them
      if (threadIdx.x < kGoCopies)
        __hip_atomic_store(sync + kGoStride * (1 + threadIdx.x), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (threadIdx.x == 0) {
      const uint32_t* go = sync + kGoStride * (1 + blockIdx.x % kGoCopies);
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (__hip_atomic_load(go, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
        __builtin_amdgcn_s_sleep(1);
        if (__builtin_amdgcn_s_memrealtime() - t0 > kGridWaitTicks) {
          __hip_atomic_store(sync + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
  }
  lds_barrier();
}

// Row scale s = fl32(a / 448) of a row whose maximum |h| is a, and its
// reciprocal (0 for a zero row)
__device__ __forceinline__ void row_scale_of(float a, float& s, float& rcp) {
  s = a / 448.0f;
  rcp = s > 0.0f ? 1.0f / s : 0.0f;
}

// After grid_arrive_and_wait, by every thread of the workgroup (NT threads):
// the maxima of its ROWS rows from row0 over the kAmaxSlots copies, into
// rs[0, ROWS) in LDS (cleared by grid_arrive_and_wait), then each row's scale
// s = fl32(max / 448) in rs[r] and its reciprocal in rs[ROWS + r] (computed
// once per row here instead of by every lane that quantizes a value of the
// row).  The threads share the ROWS x kAmaxSlots loads, all requested before
// the first is used; returns after a workgroup barrier.
template <int NT, int ROWS>
__device__ __forceinline__ void grid_row_maxima(const GateUpArgs& g, int row0, float* rs) {
  constexpr int PER = (ROWS * kAmaxSlots + NT - 1) / NT, n = ROWS * kAmaxSlots;
  uint32_t v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = threadIdx.x + j * NT, rl = i % ROWS, k = i / ROWS;
    v[j] = i < n ? __hip_atomic_load(g.amax_g + (size_t)k * g.Mpad + row0 + rl, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT)
                 : 0u;
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = threadIdx.x + j * NT;
    if (i < n) __hip_atomic_fetch_max((uint32_t*)rs + i % ROWS, v[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  lds_barrier();
  for (int rl = threadIdx.x; rl < ROWS; rl += NT) row_scale_of(rs[rl], rs[rl], rs[ROWS + rl]);
  lds_barrier();
}

// E4M3 code of the lane's value hv into the LDS stage [row][ncols] bytes of
// the workgroup's block (rl: row within the block; col: column within the
// block) with the row's scale s and its reciprocal (a zero row gets code 0)
__device__ __forceinline__ void stage_code(uint8_t* stage, int ncols, int rl, int col, float hv, float s, float rcp) {
  stage[rl * ncols + col] = (uint8_t)(s > 0.0f ? e4m3_quot1(hv, s, rcp) : 0u);
}

// The same for the lane's N values of row rl in columns col0 + 8 j
template <int N>
__device__ __forceinline__ void stage_codes(uint8_t* stage, int ncols, int rl, int col0, const float (&hv)[N], float s,
                                            float rcp) {
  uint32_t c[N];
  e4m3_quotN<N>(hv, s, rcp, c);
#pragma unroll
  for (int j = 0; j < N; ++j) stage[rl * ncols + col0 + 8 * j] = (uint8_t)(s > 0.0f ? c[j] : 0u);
}

// Write-out of a fused requantization, by every thread of the workgroup
// (nthreads): the staged codes of rows [row0, row0 + nrows) x columns
// [n0, n0 + ncols) as 8-byte pieces in the down projection's fragment order
// and to the plain tap; the row scales rs of those rows (scales: one
// workgroup per m-block); and zero codes and scales for the rows [rows_end, Mpad) that
// lie past every gate/up m-block but inside the down projection's
// (last_mb: the workgroups of the last m-block, each for its own columns).
__device__ __forceinline__ void fused_write_out(const GateUpArgs& g, const uint8_t* stage, const float* rs,
                                                int row0, int nrows, int n0, int ncols, bool scales, bool last_mb,
                                                int rows_end, int nthreads) {
  const int C = g.I / kChunk, per_row = ncols / 8;
  for (int p = threadIdx.x; p < nrows * per_row; p += nthreads) {
    const int rl = p / per_row, t = p % per_row, m = row0 + rl, n = n0 + 8 * t;
    const v2u w = *(const v2u*)(stage + rl * ncols + 8 * t);
    *(v2u*)(g.hq + frag_off8(m, n, C)) = w;
    if (g.tap_hq && m < g.M) *(v2u*)(g.tap_hq + (size_t)m * g.I + n) = w;
  }
  if (scales) {
    for (int rl = threadIdx.x; rl < nrows; rl += nthreads) {
      const int m = row0 + rl;
      const float s = rs[rl];
      g.sh[m] = s;
      if (g.tap_sh && m < g.M) g.tap_sh[m] = s;
    }
  }
  if (last_mb) {
    for (int p = threadIdx.x; p < (g.Mpad - rows_end) * per_row; p += nthreads) {
      const int m = rows_end + p / per_row, n = n0 + 8 * (p % per_row);
      *(v2u*)(g.hq + frag_off8(m, n, C)) = v2u{0u, 0u};
      if (scales && p % per_row == 0) g.sh[m] = 0.0f;
    }
  }
}

// LDS partial tiles [wave][pair][lane], 16 B each (one ds_write_b128 per
// tile); returns after a workgroup barrier
template <int MT, int T>
__device__ __forceinline__ void ks_stash(const v4f (&acc)[MT][T], v4f* red) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < T; ++t) red[(wave * MT * T + mt * T + t) * 64 + lane] = acc[mt][t];
  lds_barrier();   // no wave reads what another stored to global memory
}

// sum of pair p (lane ln) over the KS waves w0, w0 + ws, ... in wave order
template <int KS>
__device__ __forceinline__ v4f ks_sum(const v4f* red, int PT, int w0, int ws, int p, int ln) {
  v4f s = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < KS; ++k) s += red[((w0 + k * ws) * PT + p) * 64 + ln];
  return s;
}

}  // namespace ocq
