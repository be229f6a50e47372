// Gate/up projection + fused SiLU(gate) * up epilogue.
//
// G = xq Wg^T and U = xq Wu^T with exact products and fp32 accumulation
// (operands converted in registers to fp16; MFMA 16x16x32 f16), then
// h = SiLU(G sx sw_g) * (U sx sw_u) per element, with the row maximum of |h|
// over the workgroup's columns written to amax_part[row][group] (reduced by
// the requantization), or bf16(h) written for a BF16 down projection.
// ("OCRia 推理栈：单卡 B200 提速近 10 倍", German page "Wie es funktioniert":
// SiLU fused with the quantization, intermediates in registers; section
// "Reducing the data moved": FP8 / NVFP4 weights.)
//
// Gate/up tiles interleave 8 gate and 8 up rows, so in an accumulator tile
// lane r (< 8) holds G and lane r + 8 holds U of the same output column.
#include "gemm_core.h"

namespace ocq {

#ifdef OCQ_PHASE_STAMPS
// Time stamps (100 MHz clock, s_memrealtime) of the last launch of the
// producer/consumer gate/up, built only with OCQ_PHASE_STAMPS:
// [workgroup < 512][wave: 8 consumers, then 4 producers][entry, consumer loop
// start, loop end, K halves' partial tiles stored, wave end; with the
// requantization inside the launch also: row maxima folded (arrival), grid
// released, row scales ready].  Producer waves record entry, wave end and
// the last three.
__device__ uint64_t g_pc_phases[kPhaseWGs][12][8];
static_assert(sizeof(g_pc_phases) == kPcPhaseBytes, "layout stated in ocq_internal.h");
__device__ __forceinline__ void pc_stamp(int wave, int i) {
  const uint64_t t = __builtin_amdgcn_s_memrealtime();
  if ((threadIdx.x & 63) == 0 && blockIdx.x < kPhaseWGs) g_pc_phases[blockIdx.x][wave][i] = t;
}
#define OCQ_PC_STAMP(w, i) pc_stamp(w, i)
#else
#define OCQ_PC_STAMP(w, i)
#endif

namespace {

// Epilogue operands of one lane, loaded together before they are used:
// row scales sx of the lane's 4 rows of each of Q m-tiles, and the gate / up
// column scales of its column in each of the T tiles.
template <int Q, int T>
struct EpiScales {
  v4f xs[Q];   // vectors: element selects stay in registers
  float cg[T], cu[T];
};

// q_of(j): row block (m-tile index from row0) of the wave's j-th epilogue m-tile
template <int BF, int Q, int T, class QOf>
__device__ __forceinline__ void load_epi(EpiScales<Q, T>& e, const GateUpArgs& g, int row0, int tile0, QOf q_of) {
  const int lane = threadIdx.x & 63, gq = lane >> 4, r = lane & 15;
#pragma unroll
  for (int j = 0; j < Q; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) e.xs[j][i] = g.sx[row0 + q_of(j) * 16 + 4 * gq + i];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    if constexpr (BF == kB_FP4_F16) {
      e.cg[t] = g.tscales[0];
      e.cu[t] = g.tscales[1];
    } else {
      const int n = (tile0 + t) * 8 + (r & 7);
      e.cg[t] = g.wscales[n];
      e.cu[t] = g.wscales[g.I + n];
    }
  }
}

// workgroup -> (m-block, column group); groups shared by several m-blocks are
// numbered 8 apart (one XCD under round-robin placement) when possible
__device__ __forceinline__ void gateup_block(const GateUpArgs& g, int ngroups, int& mb, int& ng) {
  const int b = blockIdx.x;
  if (g.n_mb > 1 && ngroups % 8 == 0) {
    const int q = b >> 3;
    mb = q % g.n_mb;
    ng = (q / g.n_mb) * 8 + (b & 7);
  } else {
    mb = b % g.n_mb;
    ng = b / g.n_mb;
  }
}

// MT m-tiles per workgroup, MS x KS waves, MTW = ceil(MT / MS) m-tiles per wave
// D > 0: prefetch depth of ks_mainloop; D = -1: ks_mainloop_roll with
// padding chunks; D <= -2: ks_mainloop_roll with exactly -D chunks per wave.
// FUSED: the per-token requantization of h happens here (grid-wide row
// maxima, codes written by this kernel; see gemm_core.h), else fp32 h and
// per-workgroup row maxima go to the workspace for k_requant.
template <int BF, int MT, int T, int MS, int KS, int D, bool BF16H, bool FUSED>
__global__ __launch_bounds__(64 * MS * KS) void ks_gateup(GateUpArgs g) {
  static_assert(!(FUSED && BF16H), "the BF16-down mode has no requantization");
  constexpr int MTW = (MT + MS - 1) / MS;
  extern __shared__ v4f red4[];
  __shared__ float s_rmax[FUSED ? 2 * MT * 16 : 1];   // FUSED: the rows' scales and their reciprocals
  int mb, ng;
  gateup_block(g, (g.I / 8) / T, mb, ng);
  const int C = g.H / kChunk;
  const int row0 = mb * MT * 16;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int ms = wave % MS, kidx = wave / MS;
  const int nvalid = MT - ms * MTW < MTW ? MT - ms * MTW : MTW;
  const size_t wt = (size_t)C * Fmt<BF>::kGlobal, bt = (size_t)((C + 7) / 8) * 1024;
  const LanePtrs lp = lane_ptrs<BF>(g.xq + (size_t)(row0 / 16 + ms * MTW) * C * AGeom<BF>::kBlk, g.H, nvalid,
                                    g.wcodes + (size_t)ng * T * wt, wt, g.wbscales + (size_t)ng * T * bt, bt);
  v4f acc[MTW][T];
#pragma unroll
  for (int j = 0; j < MTW; ++j)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[j][t] = v4f{0.f, 0.f, 0.f, 0.f};
  // the epilogue's scales are requested before the main loop, so their
  // latency is hidden behind it (after it for the loop with padding chunks,
  // which has no registers to spare)
  constexpr int NW = MS * KS, Q = (MT + NW - 1) / NW;
  constexpr bool SPLIT = MS == 1 && MT * T <= NW;   // one (m-tile, tile) pair per wave
  EpiScales<Q, T> es;
  auto q_of = [&](int j) { return wave + NW * j < MT ? wave + NW * j : wave; };
  if constexpr (D != -1 && !SPLIT) load_epi<BF, Q, T>(es, g, row0, ng * T, q_of);
  // SPLIT: this wave's pair (m-tile sq, tile st) and its scales
  const int sq = SPLIT && wave < MT * T ? wave / T : 0, st = SPLIT && wave < MT * T ? wave % T : 0;
  v4f sxs = v4f{0.f, 0.f, 0.f, 0.f};
  float scg = 0.f, scu = 0.f;
  if constexpr (SPLIT) {
    if (wave < MT * T) {
      if constexpr (BF == kB_FP4_F16) {
        scg = g.tscales[0];
        scu = g.tscales[1];
      } else {
        scg = g.wscales[(ng * T + st) * 8 + (lane & 7)];
        scu = g.wscales[g.I + (ng * T + st) * 8 + (lane & 7)];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sxs[i] = g.sx[row0 + sq * 16 + 4 * (lane >> 4) + i];
    }
  }
  if constexpr (D == -1) ks_mainloop_roll<BF, MTW, T, KS, false>(lp, kidx, 0, C, acc);
  else if constexpr (D < -1) ks_mainloop_roll<BF, MTW, T, KS, true, -D>(lp, kidx, 0, C, acc);
  else ks_mainloop<BF, MTW, T, KS, D>(lp, kidx, 0, C, acc);

  if constexpr (SPLIT) {
    // Few (m-tile, tile) pairs: all partial tiles go through LDS at once
    // ([wave][m-tile][tile][lane]) and wave i finishes pair i; the T waves of
    // an m-tile then combine their rows' maxima in LDS, and the first of them
    // writes one partial per row for the workgroup.
    __shared__ float s_am[8][16];
#pragma unroll
    for (int j = 0; j < MT; ++j)
#pragma unroll
      for (int t = 0; t < T; ++t) red4[((wave * MT + j) * T + t) * 64 + lane] = acc[j][t];
    lds_barrier();
    float hv[2] = {0.f, 0.f};   // FUSED: the lane's two h values of the wave's pair
    uint32_t seen = 0u;
    if (wave < MT * T) {
      const int q = sq, t = st;
      v4f v = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) v += red4[((ks * MT + q) * T + t) * 64 + lane];
      const int n0 = ng * T + t;
      float am[2] = {0.f, 0.f};
      if constexpr (FUSED) {
        gateup_tile_h<false>(v, sxs, scg, scu, hv);
        am[0] = fabsf(hv[0]);
        am[1] = fabsf(hv[1]);
      } else {
        // padding rows (>= M) are never read back: their h is not stored
        gateup_tile_epilogue<BF16H, 1, true>(g, v, sxs, scg, scu, row0 + q * 16, n0, 0, am);
      }
      if constexpr (!BF16H) {
#pragma unroll
        for (int e = 0; e < 2; ++e) am[e] = max8(am[e]);
        if ((lane & 7) == 0) {   // lane 16 gq (rows 0, 2) and 16 gq + 8 (rows 1, 3) of 4 gq ..
          const int r = 4 * (lane >> 4) + ((lane & 8) ? 1 : 0);
#pragma unroll
          for (int e = 0; e < 2; ++e) s_am[wave][r + 2 * e] = am[e];
        }
      }
    }
    if constexpr (!BF16H) {
      lds_barrier();
      if (wave < MT * T && st == 0 && lane < 16) {
        float a = s_am[wave][lane];
#pragma unroll
        for (int t = 1; t < T; ++t) a = fmaxf(a, s_am[wave + t][lane]);
        const int m = row0 + sq * 16 + lane;
        if (m < g.M) {
          if constexpr (FUSED) seen = amax_atomic(g, m, a);
          else g.amax_part[(size_t)m * ((g.I / 8) / T) + ng] = a;
        }
      }
    }
    if constexpr (FUSED) {
      grid_arrive_and_wait(g.sync, gridDim.x, seen, s_rmax, MT * 16);
      grid_row_maxima<64 * NW, MT * 16>(g, row0, s_rmax);
      uint8_t* stage = (uint8_t*)red4;   // every partial tile was read before the barriers
      constexpr int NC = T * 8;
      if (wave < MT * T) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int rl = sq * 16 + gateup_value_row(e);
          const float sc = s_rmax[rl], rcp = s_rmax[MT * 16 + rl];
          stage_code(stage, NC, rl, st * 8 + (lane & 7), hv[e], sc, rcp);
        }
      }
      lds_barrier();
      fused_write_out(g, stage, s_rmax, row0, MT * 16, ng * NC, NC, ng == 0, mb == g.n_mb - 1, g.n_mb * MT * 16,
                      64 * NW);
    }
    return;
  }
  // Epilogue, one wave per m-tile (rows are owned by exactly one wave, so the
  // row maxima need no cross-wave combination).  The partial tiles go through
  // LDS one weight tile t at a time ([wave][m-tile][lane] 16 B each, NW * MTW
  // KB per tile, two regions used alternately so a tile's partials can be
  // written while the previous tile's are still being read: one barrier per
  // tile); m-tile q = (ms, j) was accumulated by waves ms, ms + MS, ...
  if constexpr (D == -1) load_epi<BF, Q, T>(es, g, row0, ng * T, q_of);
  float amax[Q][2];
#pragma unroll
  for (int jq = 0; jq < Q; ++jq) amax[jq][0] = amax[jq][1] = 0.f;
  float hvq[FUSED ? Q : 1][FUSED ? T : 1][2];   // FUSED: the wave's h values, kept for the requantization
#pragma unroll
  for (int t = 0; t < T; ++t) {
    // region t & 1 was last read for tile t - 2, before every wave passed the
    // barrier of tile t - 1
    v4f* red = red4 + (t & 1) * (NW * MTW * 64);
#pragma unroll
    for (int j = 0; j < MTW; ++j) red[(wave * MTW + j) * 64 + lane] = acc[j][t];
    lds_barrier();
#pragma unroll
    for (int jq = 0; jq < Q; ++jq) {
      const int q = wave + NW * jq;
      if (q < MT) {
        const int qm = q / MTW, qj = q % MTW;
        v4f v = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) v += red[((qm + MS * ks) * MTW + qj) * 64 + lane];
        if constexpr (FUSED) {
          gateup_tile_h<false>(v, es.xs[jq], es.cg[t], es.cu[t], hvq[jq][t]);
          amax[jq][0] = fmaxf(amax[jq][0], fabsf(hvq[jq][t][0]));
          amax[jq][1] = fmaxf(amax[jq][1], fabsf(hvq[jq][t][1]));
        } else {
          gateup_tile_epilogue<BF16H, T>(g, v, es.xs[jq], es.cg[t], es.cu[t], row0 + q * 16, ng, t, amax[jq]);
        }
      }
    }
  }
  uint32_t seen = 0u;
  if constexpr (!BF16H) {
    const int ngroups = (g.I / 8) / T;
#pragma unroll
    for (int jq = 0; jq < Q; ++jq) {
      const int q = wave + NW * jq;
      if (q < MT) {
#pragma unroll
        for (int e = 0; e < 2; ++e) amax[jq][e] = max8(amax[jq][e]);
        if ((lane & 7) == 0) {      // lane 16 gq (rows 0, 2) and 16 gq + 8 (rows 1, 3)
          const int m = row0 + q * 16 + 4 * (lane >> 4) + ((lane & 8) ? 1 : 0);
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            if constexpr (FUSED) {
              if (m + 2 * e < g.M) seen |= amax_atomic(g, m + 2 * e, amax[jq][e]);
            } else {
              g.amax_part[(size_t)(m + 2 * e) * ngroups + ng] = amax[jq][e];
            }
          }
        }
      }
    }
  }
  if constexpr (FUSED) {
    grid_arrive_and_wait(g.sync, gridDim.x, seen, s_rmax, MT * 16);
    grid_row_maxima<64 * NW, MT * 16>(g, row0, s_rmax);
    uint8_t* stage = (uint8_t*)red4;   // the last tile's partials were read before the barriers
    constexpr int NC = T * 8;
#pragma unroll
    for (int jq = 0; jq < Q; ++jq) {
      const int q = wave + NW * jq;
      if (q < MT) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int rl = q * 16 + gateup_value_row(e);
          const float sc = s_rmax[rl], rcp = s_rmax[MT * 16 + rl];
          float hvt[T];
#pragma unroll
          for (int t = 0; t < T; ++t) hvt[t] = hvq[jq][t][e];
          stage_codes<T>(stage, NC, rl, lane & 7, hvt, sc, rcp);
        }
      }
    }
    lds_barrier();
    fused_write_out(g, stage, s_rmax, row0, MT * 16, ng * NC, NC, ng == 0, mb == g.n_mb - 1, g.n_mb * MT * 16,
                    64 * NW);
  }
}

// ---------------------------------------------------------------- 13 m-tiles, weights through LDS
//
// For one 208-row m-block the skinny kernel's waves stall on the weight
// stream (a wave's loads complete in issue order, so the activations it
// needs next wait behind the weights it requested earlier), and each of its
// two wave rows converts the same weights to fp16.  Here the roles are split.
// Four producer waves (one per SIMD) load the workgroup's weight tiles (E4M3,
// or E2M1 with their E4M3 block scales) in stages of 2 chunks, one stage
// ahead, convert each unit once to fp16 and write it to a two-slot LDS ring;
// a workgroup barrier publishes each stage.  Eight consumer waves load only
// activations (one chunk ahead, in registers), read fp16 weights from LDS
// and run the MFMAs: wave (ms, kidx) holds m-tiles 0-3 (ms = 0) or
// 1 + 3 ms .. 3 + 3 ms and the chunks kidx, kidx + 2, ...  Every barrier is
// passed by all twelve waves in the same order: one per stage, one after the
// main loop, one after the partial tiles are stored.
constexpr int kPcConsumers = 8, kPcProducers = 4;

template <int BF_, int T_, int C_>
struct Pc {
  static constexpr int BF = BF_, C = C_, T = T_;       // weight format, chunks of 128 inputs, weight tiles
  static constexpr int CPS = 2;                        // chunks per stage (one per consumer wave)
  static constexpr int NS = C / CPS;                   // stages
  static constexpr int NK = C / 2;                     // chunks per consumer wave
  static constexpr int UB = Fmt<BF>::kUnits;           // weight units (1 KB) per tile and chunk
  static constexpr int US = CPS * T * UB;              // weight units per stage
  static constexpr int PPW = (US + kPcProducers - 1) / kPcProducers;   // loads per producer wave and stage
  static constexpr int PW = 1;                         // stages loaded ahead of the one being converted
  static constexpr int W = PW + 1;                     // register buffers of a producer (stages)
  static constexpr int SLOT = CPS * T * 4 * 1024;      // fp16 units of a stage: [chunk][tile][sub-step]
  static constexpr int RED = kPcConsumers * 4 * 1024;  // epilogue partials of one weight tile (all T stored at once)
  static constexpr int LDS = 2 * SLOT > T * RED ? 2 * SLOT : T * RED;
  static_assert(BF == kB_FP8_F16 || BF == kB_FP4_F16, "E4M3 or NVFP4 weights");
  static_assert(W * PPW < 64 && PPW * kPcProducers - US <= kPcProducers, "loads per producer");
  static_assert(CPS % 2 == 0 && C % CPS == 0, "stages of whole chunk pairs");
  static_assert(LDS <= 160 * 1024, "LDS of one CU");
};

// fp16 unit of (chunk c, tile t, sub-step i) in the ring (lane part excluded)
template <class P>
__device__ __forceinline__ int pc_f16_unit(int c, int t, int i) {
  return ((c / P::CPS) & 1) * P::SLOT + ((((c % P::CPS) * P::T) + t) * 4 + i) * 1024;
}

template <int BF, int T, int C>
__device__ __forceinline__ void pc_producer(const GateUpArgs& g, uint8_t* lds, int ng, int p) {
  using P = Pc<BF, T, C>;
  const int lane = threadIdx.x & 63;
  const size_t wt = (size_t)C * Fmt<BF>::kGlobal, bt = (size_t)((C + 7) / 8) * 1024;
  const uint8_t* w = g.wcodes + (size_t)ng * T * wt + lane * 16;
  const uint8_t* wb = g.wbscales + (size_t)ng * T * bt + lane * 16;
  // unit x of a stage: chunk x / (T UB) of the stage, tile (x / UB) % T,
  // unit x % UB of the tile's chunk; NVFP4 units also take the lane's two
  // E4M3 block scales (inputs 0-15 and 16-31 of each 32-input sub-step pair)
  v4i r[P::W][P::PPW];
  uint32_t rs[P::W][P::PPW];
  // Every load is unconditional (a unit past the stage's last reloads one
  // that exists and is not written): a load under a branch would make the
  // compiler wait for every outstanding load where the branches join, so
  // stage s + 1 would have landed before stage s is published.
  auto load = [&](int b, int s) {
#pragma unroll
    for (int q = 0; q < P::PPW; ++q) {
      const int x0 = p + q * kPcProducers;
      const int x = P::US % kPcProducers == 0 || x0 < P::US ? x0 : x0 - kPcProducers;
      const int cc = x / (T * P::UB), t = (x / P::UB) % T, u = x % P::UB, c = P::CPS * s + cc;
      r[b][q] = *(const v4i*)(w + t * wt + (size_t)c * Fmt<BF>::kGlobal + u * 1024);
      if constexpr (BF == kB_FP4_F16)
        rs[b][q] = *(const uint16_t*)(wb + t * bt + (size_t)(c >> 3) * 1024 + 2 * (c & 7));
    }
  };
  // stage 0 alone first: requested together with later stages it would
  // land only once most of them had (the memory system does not serve a
  // burst in issue order), and every consumer waits for it
  load(0, 0);
#pragma unroll
  for (int s = 0; s < P::NS; ++s) {
    // slot s % 2 held stage s - 2, which every consumer finished before
    // passing barrier s - 1
    uint8_t* slot = lds + (s & 1) * P::SLOT + lane * 16;
#pragma unroll
    for (int q = 0; q < P::PPW; ++q) {
      const int x = p + q * kPcProducers;
      if (P::US % kPcProducers == 0 || x < P::US) {
        const int cc = x / (T * P::UB), t = (x / P::UB) % T, u = x % P::UB;
        const v4i& v = r[s % P::W][q];
        uint8_t* dst = slot + ((cc * T) + t) * 4 * 1024;
        if constexpr (BF == kB_FP8_F16) {
#pragma unroll
          for (int h = 0; h < 2; ++h)
            *(v8h*)(dst + (2 * u + h) * 1024) = e4m3x8_to_f16((uint32_t)v[2 * h], (uint32_t)v[2 * h + 1]);
        } else {
          v2h s0, s1;
          e4m3x2_scales(rs[s % P::W][q], s0, s1);
#pragma unroll
          for (int i = 0; i < 4; ++i) *(v8h*)(dst + i * 1024) = e2m1x8_to_f16((uint32_t)v[i], i < 2 ? s0 : s1);
        }
      }
    }
#pragma unroll
    for (int n = s + 1; n <= s + P::PW; ++n)
      if (n < P::NS && (s == 0 || n == s + P::PW)) load(n % P::W, n);
    lds_barrier();   // stage s published
  }
  lds_barrier();   // after the main loop
  lds_barrier();   // partial tiles stored
}

template <int BF, int NV, int T, int C, bool BF16H, bool FUSED>
__device__ __forceinline__ void pc_consumer(const GateUpArgs& g, uint8_t* lds, float* rmax, int row0, int ng, int wave,
                                            int mt0) {
  using P = Pc<BF, T, C>;
  constexpr int MT = 13, Q = 2;
  const int lane = threadIdx.x & 63, kidx = wave & 1;
  const size_t a_mt = (size_t)P::C * AGeom<kB_FP8_F16>::kBlk;
  const uint8_t* abase = g.xq + (size_t)(row0 / 16 + mt0) * a_mt + lane * 16;
  const uint8_t* lbase = lds + lane * 16;
  auto a_ld = [&](int j, int c, int u) {
    return *(const v4i*)(abase + j * a_mt + (size_t)c * AGeom<kB_FP8_F16>::kBlk + u * 1024);
  };
  auto b_rd = [&](v8h (&d)[T], int c, int i) {
#pragma unroll
    for (int t = 0; t < T; ++t) d[t] = *(const v8h*)(lbase + pc_f16_unit<P>(c, t, i));
  };
  // epilogue: this wave finishes m-tiles q = wave and wave + 8 (if < 13);
  // their scales are requested before the main loop
  EpiScales<Q, T> es;
  auto q_of = [&](int j) { return wave + kPcConsumers * j < MT ? wave + kPcConsumers * j : wave; };
  load_epi<BF, Q, T>(es, g, row0, ng * T, q_of);

  v4f acc[NV][T];
#pragma unroll
  for (int j = 0; j < NV; ++j)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[j][t] = v4f{0.f, 0.f, 0.f, 0.f};
  v4i a[NV][2];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    a[j][0] = a_ld(j, kidx, 0);
    a[j][1] = a_ld(j, kidx, 1);
  }
  // fp16 weights of two sub-steps: the next one is read while the current
  // one's MFMAs run
  OCQ_PC_STAMP(wave, 1);
  v8h bq[2][T];
#pragma unroll
  for (int k = 0; k < P::NK; ++k) {
    const int c = kidx + 2 * k;
    constexpr int KPS = P::CPS / 2;   // chunks per consumer wave and stage
    if (k % KPS == 0) {   // stage k / KPS published
      lds_barrier();
      b_rd(bq[0], c, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if (i < 3) b_rd(bq[(i + 1) & 1], c, i + 1);
      else if ((k + 1) % KPS != 0) b_rd(bq[0], c + 2, 0);   // next chunk, same stage
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const v4i& w = a[j][i >> 1];
        const v8h av = e4m3x8_to_f16((uint32_t)w[2 * (i & 1)], (uint32_t)w[2 * (i & 1) + 1]);
#pragma unroll
        for (int t = 0; t < T; ++t) acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bq[i & 1][t], acc[j][t], 0, 0, 0);
      }
      if ((i == 1 || i == 3) && k + 1 < P::NK) {
        // unit i / 2 of the activations is free: load the next chunk's
        const int u = i >> 1;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NV; ++j) a[j][u] = a_ld(j, c + 2, u);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // Epilogue: every partial tile to LDS at once ([wave][m-tile][tile][lane],
  // one barrier), then the wave that owns m-tile q sums its two K halves
  // (wave 2 ms, then 2 ms + 1) tile by tile.
  OCQ_PC_STAMP(wave, 2);
  lds_barrier();   // every consumer is done with the weights; the ring is reused
  float amax[Q][2];
#pragma unroll
  for (int jq = 0; jq < Q; ++jq) amax[jq][0] = amax[jq][1] = 0.f;
  float hvq[FUSED ? Q : 1][FUSED ? T : 1][2];   // FUSED: the wave's h values, kept for the requantization
  v4f* red = (v4f*)lds;   // [wave][m-tile slot][tile][lane]
#pragma unroll
  for (int j = 0; j < NV; ++j)
#pragma unroll
    for (int t = 0; t < T; ++t) red[((wave * 4 + j) * T + t) * 64 + lane] = acc[j][t];
  lds_barrier();
  OCQ_PC_STAMP(wave, 3);
#pragma unroll
  for (int jq = 0; jq < Q; ++jq) {
    const int q = wave + kPcConsumers * jq;
    if (q < MT) {
      const int msq = q < 4 ? 0 : (q - 1) / 3, jj = q < 4 ? q : (q - 1) % 3;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const v4f v = red[(((2 * msq) * 4 + jj) * T + t) * 64 + lane] + red[(((2 * msq + 1) * 4 + jj) * T + t) * 64 + lane];
        if constexpr (FUSED) {
          gateup_tile_h<false>(v, es.xs[jq], es.cg[t], es.cu[t], hvq[jq][t]);
          amax[jq][0] = fmaxf(amax[jq][0], fabsf(hvq[jq][t][0]));
          amax[jq][1] = fmaxf(amax[jq][1], fabsf(hvq[jq][t][1]));
        } else {
          gateup_tile_epilogue<BF16H, T>(g, v, es.xs[jq], es.cg[t], es.cu[t], row0 + q * 16, ng, t, amax[jq]);
        }
      }
    }
  }
  uint32_t seen = 0u;
  if constexpr (!BF16H) {
    const int ngroups = (g.I / 8) / T;
#pragma unroll
    for (int jq = 0; jq < Q; ++jq) {
      const int q = wave + kPcConsumers * jq;
      if (q < MT) {
#pragma unroll
        for (int e = 0; e < 2; ++e) amax[jq][e] = max8(amax[jq][e]);
        if ((lane & 7) == 0) {      // lane 16 gq (rows 0, 2) and 16 gq + 8 (rows 1, 3)
          const int m = row0 + q * 16 + 4 * (lane >> 4) + ((lane & 8) ? 1 : 0);
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            if constexpr (FUSED) {
              if (m + 2 * e < g.M) seen |= amax_atomic(g, m + 2 * e, amax[jq][e]);
            } else {
              g.amax_part[(size_t)(m + 2 * e) * ngroups + ng] = amax[jq][e];
            }
          }
        }
      }
    }
  }
  if constexpr (FUSED) {
    // every wave of the workgroup (producers too) arrives here; afterwards
    // the codes go to an LDS stage [208 rows][T * 8 columns]
    OCQ_PC_STAMP(wave, 5);
    grid_arrive_and_wait(g.sync, gridDim.x, seen, rmax, MT * 16);
    OCQ_PC_STAMP(wave, 6);
    grid_row_maxima<64 * (kPcConsumers + kPcProducers), MT * 16>(g, row0, rmax);
    OCQ_PC_STAMP(wave, 7);
    uint8_t* stage = lds;
    constexpr int NC = T * 8;
#pragma unroll
    for (int jq = 0; jq < Q; ++jq) {
      const int q = wave + kPcConsumers * jq;
      if (q < MT) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int rl = q * 16 + gateup_value_row(e);
          const float sc = rmax[rl], rcp = rmax[MT * 16 + rl];
          float hvt[T];
#pragma unroll
          for (int t = 0; t < T; ++t) hvt[t] = hvq[jq][t][e];
          stage_codes<T>(stage, NC, rl, lane & 7, hvt, sc, rcp);
        }
      }
    }
  }
}

template <int BF, int T, int C, bool BF16H, bool FUSED>
__global__ __launch_bounds__(64 * (kPcConsumers + kPcProducers)) void pc_gateup(GateUpArgs g) {
  static_assert(!(FUSED && BF16H), "the BF16-down mode has no requantization");
  extern __shared__ v4f pc_lds[];
  __shared__ float s_rmax[FUSED ? 2 * 13 * 16 : 1];   // FUSED: the rows' scales and their reciprocals
  uint8_t* lds = (uint8_t*)pc_lds;
  int mb, ng;
  gateup_block(g, (g.I / 8) / T, mb, ng);
  const int row0 = mb * 13 * 16;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  OCQ_PC_STAMP(wave, 0);
  if (wave >= kPcConsumers) {
    pc_producer<BF, T, C>(g, lds, ng, wave - kPcConsumers);
    if constexpr (FUSED) {
      OCQ_PC_STAMP(wave, 5);
      grid_arrive_and_wait(g.sync, gridDim.x, 0u, s_rmax, 13 * 16);
      OCQ_PC_STAMP(wave, 6);
      grid_row_maxima<64 * (kPcConsumers + kPcProducers), 13 * 16>(g, row0, s_rmax);
      OCQ_PC_STAMP(wave, 7);
    }
  } else if (wave < 2) {
    pc_consumer<BF, 4, T, C, BF16H, FUSED>(g, lds, s_rmax, row0, ng, wave, 0);
  } else {
    pc_consumer<BF, 3, T, C, BF16H, FUSED>(g, lds, s_rmax, row0, ng, wave, 1 + 3 * (wave >> 1));
  }
#ifdef OCQ_PHASE_STAMPS
  __builtin_amdgcn_s_waitcnt(0);
  OCQ_PC_STAMP(wave, 4);
#endif
  if constexpr (FUSED) {
    lds_barrier();   // every code staged
    constexpr int NC = T * 8;
    fused_write_out(g, lds, s_rmax, row0, 13 * 16, ng * NC, NC, ng == 0, mb == g.n_mb - 1, g.n_mb * 13 * 16,
                    64 * (kPcConsumers + kPcProducers));
  }
}

template <int BF, int T, int C, bool BF16H, bool FUSED>
hipError_t launch_pc(const GateUpArgs& g, int grid, hipStream_t st, const LaunchEvents& ev) {
  auto fn = pc_gateup<BF, T, C, BF16H, FUSED>;
  constexpr size_t lds = Pc<BF, T, C>::LDS;
  static std::atomic<uint64_t> lds_set{0};
  if (hipError_t e = allow_lds((const void*)fn, lds, lds_set); e != hipSuccess) return e;
  launch_kernel(fn, dim3(grid), dim3(64 * (kPcConsumers + kPcProducers)), lds, st, ev, g);
  return hipGetLastError();
}

// ---------------------------------------------------------------- dispatch

// The fused variant of a launch is used only if the whole grid can be
// resident at once (its workgroups wait for each other); otherwise, and for
// the BF16-down mode, the unfused one, followed by k_requant.  `fused`: in,
// may the launch fuse; out, did it.
template <class KF, class KU>
hipError_t launch_either(KF fused_fn, KU plain_fn, int threads, size_t lds, const GateUpArgs& g, int grid,
                         hipStream_t st, const LaunchEvents& ev, bool& fused, std::atomic<uint64_t>& lds_f,
                         std::atomic<uint64_t>& lds_u, std::atomic<int> (&cap)[kMaxDevices]) {
  if (fused) {
    if (hipError_t e = allow_lds((const void*)fused_fn, lds, lds_f); e != hipSuccess) return e;
    if (resident_capacity((const void*)fused_fn, threads, lds, cap) >= grid) {
      launch_kernel(fused_fn, dim3(grid), dim3(threads), lds, st, ev, g);
      return hipGetLastError();
    }
    fused = false;
  }
  if (hipError_t e = allow_lds((const void*)plain_fn, lds, lds_u); e != hipSuccess) return e;
  launch_kernel(plain_fn, dim3(grid), dim3(threads), lds, st, ev, g);
  return hipGetLastError();
}

template <int BF, bool BF16H, int MT, int T, int MS, int KS, int D>
hipError_t launch_ks(const GateUpArgs& g, int grid, hipStream_t st, const LaunchEvents& ev, bool& fused) {
  constexpr int MTW = (MT + MS - 1) / MS;
  // partial tiles in LDS (also the stage of a fused requantization's codes)
  const size_t lds = (size_t)(MS == 1 && MT * T <= MS * KS ? T : (T > 1 ? 2 : 1)) * MS * KS * MTW * 64 * sizeof(v4f);
  static std::atomic<uint64_t> lds_f{0}, lds_u{0};
  static std::atomic<int> cap[kMaxDevices];
  fused = fused && !BF16H;
  return launch_either(ks_gateup<BF, MT, T, MS, KS, D, BF16H, !BF16H>, ks_gateup<BF, MT, T, MS, KS, D, BF16H, false>,
                       64 * MS * KS, lds, g, grid, st, ev, fused, lds_f, lds_u, cap);
}

template <int BF, int T, int C, bool BF16H>
hipError_t launch_pc(const GateUpArgs& g, int grid, hipStream_t st, const LaunchEvents& ev, bool& fused) {
  constexpr size_t lds = Pc<BF, T, C>::LDS;
  static std::atomic<uint64_t> lds_f{0}, lds_u{0};
  static std::atomic<int> cap[kMaxDevices];
  fused = fused && !BF16H;
  return launch_either(pc_gateup<BF, T, C, BF16H, !BF16H>, pc_gateup<BF, T, C, BF16H, false>,
                       64 * (kPcConsumers + kPcProducers), lds, g, grid, st, ev, fused, lds_f, lds_u, cap);
}

// Eight waves (two per SIMD: each CU keeps enough operand loads in flight)
// in an MS x KS grid: up to 7 m-tiles all eight split K; 13 m-tiles, 2 x 4
// (each wave 7 m-tiles).  Up to 4 m-tiles a wave keeps two whole chunks in
// flight; with 7 m-tiles per wave the operands are reloaded in place unit by
// unit (ks_mainloop_roll), which fits the 256 registers a wave has at two
// waves per SIMD.
template <int BF, bool BF16H, int MT, int T>
hipError_t go(const GateUpArgs& g, int grid, hipStream_t st, const LaunchEvents& ev, bool& fused) {
  constexpr int MS = MT >= 13 ? 2 : 1;
  constexpr int KS = 8 / MS;
  constexpr int MTW = (MT + MS - 1) / MS;
  const int C = g.H / kChunk;
  // six NVFP4 tiles of 1-4 m-tiles: one chunk in flight per wave (two
  // would not fit the registers of two waves per SIMD)
  if constexpr ((BF == kB_FP8_F16 || BF == kB_FP4_F16) && MT == 13 && T <= 3) {
    if (C == 16) return launch_pc<BF, T, 16, BF16H>(g, grid, st, ev, fused);
    if (C == 32) return launch_pc<BF, T, 32, BF16H>(g, grid, st, ev, fused);
  }
  if constexpr (T == 6) return launch_ks<BF, BF16H, MT, T, MS, KS, 1>(g, grid, st, ev, fused);
  else if constexpr (MTW <= 4) return launch_ks<BF, BF16H, MT, T, MS, KS, 2>(g, grid, st, ev, fused);
  else if (C == 4 * KS) return launch_ks<BF, BF16H, MT, T, MS, KS, -4>(g, grid, st, ev, fused);
  else if (C == 8 * KS) return launch_ks<BF, BF16H, MT, T, MS, KS, -8>(g, grid, st, ev, fused);
  else return launch_ks<BF, BF16H, MT, T, MS, KS, -1>(g, grid, st, ev, fused);
}

template <int BF, bool BF16H, int MT>
hipError_t go_t(const GateUpArgs& g, int T, int grid, hipStream_t st, const LaunchEvents& ev, bool& fused) {
  switch (T) {
    case 1: return go<BF, BF16H, MT, 1>(g, grid, st, ev, fused);
    case 2: return go<BF, BF16H, MT, 2>(g, grid, st, ev, fused);
    case 3: return go<BF, BF16H, MT, 3>(g, grid, st, ev, fused);
    case 6:
      if constexpr (BF == kB_FP4_F16 && MT <= 4) return go<BF, BF16H, MT, 6>(g, grid, st, ev, fused);
  }
  return hipErrorInvalidValue;
}

template <int BF, bool BF16H>
hipError_t go_mt(const GateUpArgs& g, int MT, int T, int grid, hipStream_t st, const LaunchEvents& ev, bool& fused) {
  switch (MT) {
    case 1: return go_t<BF, BF16H, 1>(g, T, grid, st, ev, fused);
    case 2: return go_t<BF, BF16H, 2>(g, T, grid, st, ev, fused);
    case 4: return go_t<BF, BF16H, 4>(g, T, grid, st, ev, fused);
    case 7: return go_t<BF, BF16H, 7>(g, T, grid, st, ev, fused);
    case 13: return go_t<BF, BF16H, 13>(g, T, grid, st, ev, fused);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int pc_phase_copy(void* host, size_t bytes) {
#ifdef OCQ_PHASE_STAMPS
  if (bytes < sizeof(g_pc_phases)) return (int)hipErrorInvalidValue;
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_pc_phases), sizeof(g_pc_phases));
#else
  (void)host; (void)bytes;
  return -1;
#endif
}

hipError_t launch_gateup(const Plan& p, const GateUpArgs& g, hipStream_t st, const LaunchEvents& ev, bool& fused) {
  if (p.lg1) {
    fused = false;
    return launch_gateup_large(p, g, st, ev);
  }
  const int grid = p.ngroups1 * p.n_mblocks;
  if (p.prec == kFP8) return go_mt<kB_FP8_F16, false>(g, p.MT, p.T1, grid, st, ev, fused);
  if (p.prec == kFP8DownBF16) {
    fused = false;
    return go_mt<kB_FP8_F16, true>(g, p.MT, p.T1, grid, st, ev, fused);
  }
  return go_mt<kB_FP4_F16, false>(g, p.MT, p.T1, grid, st, ev, fused);
}

}  // namespace ocq
