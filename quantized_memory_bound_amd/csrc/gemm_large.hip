// LDS-tiled GEMMs for many rows (large verify batches).
//
// With several 208-row m-blocks the skinny kernels pull the activations
// through every CU once per small weight group.  Here a workgroup owns RM
// m-tiles x RT weight tiles over the whole input range and both operands pass
// through LDS once per workgroup:
//
//   * a stage is UPS 1 KB units (16 B per lane of a fragment) of every m-tile
//     and every weight tile; stages stream into an NSTG-deep LDS ring with
//     direct-to-LDS loads, every wave issuing a fixed share, so the buffering
//     costs no registers;
//   * one workgroup barrier per stage: before it each wave waits until its own
//     loads of the stage have landed (a fixed count per wave), after it every
//     wave reads its MTW m-tiles x TW tiles of the stage from LDS, converts
//     E4M3 to fp16 in registers where needed and runs the MFMAs;
//   * KW waves share each output tile and split every stage's unit positions
//     (KW > 1: one LDS reduction after the loop, fixed order).
//
// Gate/up: E4M3 weights x E4M3 activations through MFMA 16x16x32 f16 (exact
// products, fp32 sums); the activations arrive as fp16 values of their codes
// (written so by the x quantization), which saves the four waves that share
// an m-tile converting it each,
// then SiLU(gate) * up, stored as by the skinny gate/up epilogue (fp32 h and
// per-row partial maxima for the E4M3 / NVFP4 down modes, bf16(h) in fragment
// order for the BF16 down mode).  Down, BF16 mode (a layer kept at higher
// precision: "OCRia 推理栈：单卡 B200 提速近 10 倍", section "Reducing the data
// moved: workload-aware quantization"): bf16(h) x bf16 weights through MFMA
// 16x16x32 bf16, y = bf16(Y).
#include <type_traits>

#include "gemm_core.h"

namespace ocq {

#ifdef OCQ_PHASE_STAMPS
// Per-wave phase totals of the last launch of each LDS-tiled kernel (built
// only with OCQ_PHASE_STAMPS): [gate/up, down][workgroup < 512][wave < 8]
// [load wait, barrier, MFMA batches, LDS-read wait after the batches, whole
// loop, stages] in shader-clock ticks (s_memtime), the time stamps placed
// where the waves wait for LDS reads anyway.
__device__ uint64_t g_lg_phases[2][kPhaseWGs][8][8];
static_assert(sizeof(g_lg_phases) == kLgPhaseBytes, "layout stated in ocq_internal.h");
#endif

namespace {

// Geometry of one LDS-tiled kernel.  BF: weight format (kB_FP8_F16: E4M3
// codes, two MFMA sub-steps per unit; kB_BF16: one).  A16: the activations
// are 16-bit values in fragment order (one unit per sub-step: AU units per
// weight unit) rather than E4M3 codes.  NSTG: ring depth in stages.
template <int BF_, bool A16_, int RM_, int RT_, int WM_, int WT_, int KW_, int UPS_, int NSTG_>
struct Lg {
  static constexpr int BF = BF_, RM = RM_, RT = RT_, WM = WM_, WT = WT_, KW = KW_, UPS = UPS_, NSTG = NSTG_;
  static constexpr bool A16 = A16_;
  static constexpr int NW = WM * WT * KW;
  static constexpr int MTW = (RM + WM - 1) / WM;     // m-tiles per wave (the last may be padding)
  static constexpr int TW = RT / WT;                 // weight tiles per wave
  static constexpr int SUB = BF == kB_BF16 ? 1 : 2;  // MFMA sub-steps (32 inputs each) per weight unit
  static constexpr int AU = A16 ? SUB : 1;           // activation units per weight unit
  static constexpr int AW = RM * AU;                 // activation units per unit position (a wave's
                                                     // m-tiles past RM read the last one)
  static constexpr int UT = AW + RT;                 // units per unit position: activations, then weights
  static constexpr int NU = UPS * UT;                // units per stage
  static constexpr int PW = (NU + NW - 1) / NW;      // loads per wave per stage (a surplus one repeats a unit)
  static constexpr int UPC = 4 / SUB;                // weight units per 128-input chunk
  static constexpr int SPC = UPC / UPS;              // stages per chunk
  static constexpr int UPK = UPS / KW;               // unit positions of a stage per K-wave
  static constexpr int A_BLK = A16 ? 4096 : 2048;    // activation bytes per (m-tile, chunk)
  static constexpr int LDS = NSTG * NU * 1024;
  static constexpr int THREADS = 64 * NW;
  static_assert(BF == kB_FP8_F16 || (BF == kB_BF16 && A16), "formats");
  static_assert(RT % WT == 0, "weight tiles split evenly over the wave columns");
  static_assert(UPC % UPS == 0 && UPS % KW == 0, "stage and K-wave split of a chunk");
  static constexpr int NPU = A16 ? SUB : 1;          // pieces (MFMA batches) per unit position
  static constexpr int NP = NPU * UPK;               // pieces per stage
  static_assert(NSTG >= 2 && PW >= 2 && (NSTG - 1) * PW < 64, "outstanding loads within the vmcnt range");
  static_assert((KW - 1) * WM * WT * MTW * TW * 1024 <= LDS, "reduction fits the ring");
  static_assert(LDS <= 160 * 1024, "LDS of one CU");
};

// This wave's load sources.  Load q of every stage fetches unit x = wave +
// q NW of the stage: unit position x / UT, then (m-tile, activation unit) or
// weight tile by x % UT.  Which operand, m-tile (those past nva reload the
// last; their results are dropped), sub-unit and tile a load slot reads is
// the same in every stage, so it is resolved once here; per stage only the
// chunk and the first unit position move the sources, by one offset per
// operand (a few scalar instructions per stage instead of the whole index
// arithmetic per load).  a: activation block of the workgroup's first m-tile,
// w: weight tile 0 (both + lane * 16).
template <class G>
struct LgSrc {
  const uint8_t* p[G::PW];   // the slot's unit at chunk 0, unit position 0
  bool act[G::PW];           // activation unit (else weight)
};

template <class G>
__device__ __forceinline__ LgSrc<G> lg_sources(const uint8_t* a, int nva, size_t a_mt, const uint8_t* w,
                                               size_t w_tile, int wave) {
  LgSrc<G> r;
#pragma unroll
  for (int q = 0; q < G::PW; ++q) {
    const int x0 = wave + q * G::NW;
    const int x = x0 < G::NU ? x0 : G::NU - 1;   // a surplus load slot repeats the stage's last unit
    const int uu = x / G::UT, y = x % G::UT;
    r.act[q] = y < G::AW;
    if (y < G::AW) {
      const int mt = y / G::AU < nva ? y / G::AU : nva - 1;
      r.p[q] = a + mt * a_mt + (size_t)(uu * G::AU + y % G::AU) * 1024;
    } else {
      r.p[q] = w + (y - G::AW) * w_tile + (size_t)uu * 1024;
    }
  }
  return r;
}

// Issue load q of stage s into `slot` (the stage's LDS slot).  Every wave
// issues PW loads per stage: a surplus one repeats the stage's last unit, the
// same bytes to the same place, so no branch depends on the wave.
template <class G>
__device__ __forceinline__ void lg_issue_one(const LgSrc<G>& src, int s, uint8_t* slot, int wave, int q) {
  const int c = s / G::SPC, u0 = (s % G::SPC) * G::UPS;
  const size_t off_a = (size_t)c * G::A_BLK + (size_t)u0 * G::AU * 1024;
  const size_t off_w = (size_t)c * Fmt<G::BF>::kGlobal + (size_t)u0 * 1024;
  int x = wave + q * G::NW;   // wave-uniform
  x = x < G::NU ? x : G::NU - 1;
  __builtin_amdgcn_global_load_lds((const void*)(src.p[q] + (src.act[q] ? off_a : off_w)),
                                   (lds_void*)(slot + x * 1024), 16, 0, 0);
}

template <class G>
__device__ __forceinline__ void lg_issue(const LgSrc<G>& src, int s, uint8_t* slot, int wave) {
#pragma unroll
  for (int q = 0; q < G::PW; ++q) lg_issue_one<G>(src, s, slot, wave, q);
}

// wait until at most K stages of this wave's loads are outstanding
// (every wave issues PW loads per stage, the surplus ones repeating an
// existing unit, so that the loads can sit between MFMAs without a branch)
template <class G, int K>
__device__ __forceinline__ void lg_wait() {
  wait_vm<K * G::PW>();
}

// Operand registers of one piece of a wave's work: its MTW activation
// units and (once per stage) its TW weight units.  A piece is one sub-step
// for 16-bit activations (units hold one sub-step each), else a whole unit.
template <class G>
struct LgFrag {
  v4i a[G::MTW];
};
template <class G>
struct LgWFrag {
  v4i b[G::TW];
};

// LDS offsets (lane part excluded) in a stage slot: activation unit of the
// wave's m-tile j (wave row wm; an m-tile slot past RM reads the last m-tile,
// its results are dropped) for sub-step qa, and weight unit of the wave's
// tile t (wave column wt), both of the stage's unit position up
template <class G>
__device__ __forceinline__ int lg_a_unit(int up, int wm, int j, int qa) {
  const int mt = wm * G::MTW + j < G::RM ? wm * G::MTW + j : G::RM - 1;
  return ((up * G::UT + mt * G::AU) + qa) * 1024;
}
template <class G>
__device__ __forceinline__ int lg_b_unit(int up, int wt, int t) {
  return (up * G::UT + G::AW + wt * G::TW + t) * 1024;
}

// LDS reads of sub-step qa of unit position up in the stage at `base` (lane
// offset included)
template <class G>
__device__ __forceinline__ void lg_read_a(LgFrag<G>& f, const uint8_t* base, int up, int wm, int qa) {
#pragma unroll
  for (int j = 0; j < G::MTW; ++j) f.a[j] = *(const v4i*)(base + lg_a_unit<G>(up, wm, j, qa));
}
template <class G>
__device__ __forceinline__ void lg_read_b(LgWFrag<G>& f, const uint8_t* base, int up, int wt) {
#pragma unroll
  for (int t = 0; t < G::TW; ++t) f.b[t] = *(const v4i*)(base + lg_b_unit<G>(up, wt, t));
}

// MFMAs of one piece.  A lane's 16 B of a weight unit: E4M3 codes of two
// sub-steps (bytes 0-7, 8-15) or bf16 values of one; 16-bit activations hold
// one sub-step per unit, E4M3 ones two like the weights.  Both operands order
// the inputs of a sub-step alike, so each sub-step is one MFMA over 32 inputs.
// hook(k) runs after the piece's k-th MFMA (it issues the stage's loads).
template <class G, class Hook>
__device__ __forceinline__ void lg_mfma(const LgFrag<G>& fa, const LgWFrag<G>& fb, int qa,
                                        v4f (&acc)[G::MTW][G::TW], Hook hook) {
  if constexpr (G::BF == kB_BF16) {
#pragma unroll
    for (int j = 0; j < G::MTW; ++j) {
      const v8bf av = __builtin_bit_cast(v8bf, fa.a[j]);
#pragma unroll
      for (int t = 0; t < G::TW; ++t) {
        acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(v8bf, fb.b[t]), acc[j][t], 0, 0, 0);
        hook(j * G::TW + t);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else {
#pragma unroll
    for (int ii = 0; ii < (G::A16 ? 1 : G::SUB); ++ii) {
      const int i = G::A16 ? qa : ii;
      v8h bv[G::TW];
#pragma unroll
      for (int t = 0; t < G::TW; ++t) bv[t] = e4m3x8_to_f16((uint32_t)fb.b[t][2 * i], (uint32_t)fb.b[t][2 * i + 1]);
#pragma unroll
      for (int j = 0; j < G::MTW; ++j) {
        v8h av;
        if constexpr (G::A16) av = __builtin_bit_cast(v8h, fa.a[j]);
        else av = e4m3x8_to_f16((uint32_t)fa.a[j][2 * i], (uint32_t)fa.a[j][2 * i + 1]);
#pragma unroll
        for (int t = 0; t < G::TW; ++t) {
          acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv[t], acc[j][t], 0, 0, 0);
          hook((ii * G::MTW + j) * G::TW + t);
        }
      }
    }
  }
}

// Gate/up with 16-bit activations: the MFMAs of one piece take B already in
// fp16 (bh_cur) and the E4M3 B of the next piece (sub-step i_next of fb_next)
// is converted between them, so the converts issue while the matrix core runs
// instead of ahead of the batch.  Conversion u follows MFMA 12 + 3 u: late
// enough for B read from LDS during the first MFMAs of the batch.
template <class G, class Hook>
__device__ __forceinline__ void lg_mfma_pipelined(const LgFrag<G>& fa, const v8h (&bh_cur)[G::TW],
                                                  const LgWFrag<G>& fb_next, int i_next, v8h (&bh_next)[G::TW],
                                                  v4f (&acc)[G::MTW][G::TW], Hook hook) {
  static_assert(G::MTW * G::TW >= 12 + 3 * G::TW - 2, "room to interleave the conversions");
#pragma unroll
  for (int j = 0; j < G::MTW; ++j) {
#pragma unroll
    for (int t = 0; t < G::TW; ++t) {
      acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, fa.a[j]), bh_cur[t], acc[j][t], 0, 0, 0);
      const int k = j * G::TW + t;
      if (k >= 12 && k % 3 == 0 && (k - 12) / 3 < G::TW) {
        const int u = (k - 12) / 3;
        bh_next[u] = e4m3x8_to_f16((uint32_t)fb_next.b[u][2 * i_next], (uint32_t)fb_next.b[u][2 * i_next + 1]);
        asm volatile("" : "+v"(bh_next[u]));   // keep the conversion here (not sunk to its use)
      }
      hook(k);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Tell the compiler's wait tracking that this wave has no LDS or scalar-memory
// access outstanding.  It cannot see the wait inside lds_barrier (inline asm),
// and with more LDS reads in flight than the counter can name it falls back to
// waiting for all of them, which would hold each piece's MFMAs until the next
// piece's reads had landed.  Placed where everything issued before has long
// completed (after a barrier, after a piece's MFMA issue), it costs nothing and
// lets the reads of the next piece overlap the MFMAs of the current one.
__device__ __forceinline__ void lgkm_settled() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// acc over all NS stages (NS even).  All NSTG slots are filled up front.  A
// stage holds UPK unit positions per K-wave, each processed in NPU pieces
// (MFMA batches); the workgroup barrier sits at the start of a stage's last
// piece: by then every wave has finished its LDS reads of the stage (the
// last piece's operands were read during the piece before), so stage
// s + NSTG goes into that slot, and the loads of stage s + 1 have landed, so
// the last piece reads the first operands of stage s + 1.  Stage indices past
// the last are clamped (the loads repeat the last stage into a slot whose
// reads are over, and the reads after the last stage fetch registers nobody
// uses), so every wave has the same number of loads outstanding at each wait.
// Register ping-pong: the LDS reads of the next piece are issued among the
// MFMAs of the current one, which never wait for them.  On return no load
// of the wave is outstanding.
template <class G>
__device__ __forceinline__ void lg_mainloop(const uint8_t* a, int nva, size_t a_mt, const uint8_t* w, size_t w_tile,
                                            int NS, uint8_t* lds, int wave, int wm, int wt, int kw,
                                            v4f (&acc)[G::MTW][G::TW]) {
  constexpr int NP = G::NP, NPU = G::NPU;
  static_assert(NP == 1 || NP % 2 == 0, "operand buffers alternate with the pieces or the stages");
  const int lane = threadIdx.x & 63;
  auto slot = [&](int s) { return lds + (size_t)(s % G::NSTG) * G::NU * 1024 + lane * 16; };
  const LgSrc<G> src = lg_sources<G>(a, nva, a_mt, w, w_tile, wave);
  auto issue = [&](int s) {
    lg_issue<G>(src, s < NS ? s : NS - 1, lds + (size_t)(s % G::NSTG) * G::NU * 1024, wave);
  };
#pragma unroll
  for (int s = 0; s < G::NSTG; ++s) issue(s);
  lg_wait<G, G::NSTG - 1>();
  lds_barrier();
  // lgkmcnt(0) through the builtin as well: the compiler's wait tracking
  // does not see the one inside the barrier, and would otherwise treat
  // earlier scalar loads as pending in the loop and wait for every LDS read
  __builtin_amdgcn_s_waitcnt(0xC07F);
  LgFrag<G> fa[2];
  LgWFrag<G> fb[2];
  lg_read_a<G>(fa[0], slot(0), kw * G::UPK, wm, 0);
  lg_read_b<G>(fb[0], slot(0), kw * G::UPK, wt);
  constexpr bool PIPE = G::BF == kB_FP8_F16 && G::A16;
  v8h bh[2][G::TW];
  if constexpr (PIPE) {
#pragma unroll
    for (int t = 0; t < G::TW; ++t) bh[0][t] = e4m3x8_to_f16((uint32_t)fb[0].b[t][0], (uint32_t)fb[0].b[t][1]);
  }
  // MFMAs of a piece, and the spacing of the stage's loads between those of
  // its last piece
  constexpr int NM = G::MTW * G::TW * (G::A16 ? 1 : G::SUB);
  constexpr int LSTEP = 2 * G::PW <= NM ? 2 : 1;
  static_assert(LSTEP * G::PW <= NM, "every load of a stage between two MFMAs of its last piece");
#ifdef OCQ_PHASE_STAMPS
  uint64_t p_vm = 0, p_bar = 0, p_mma = 0, p_set = 0;
#endif
  // one stage; E = s % 2 (compile-time)
  auto stage = [&](int s, auto ec) {
    constexpr int E = decltype(ec)::value;
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const int up = q / NPU, qa = q % NPU;                    // this piece: unit position, sub-step
      const int qn = q + 1 < NP ? q + 1 : 0;                   // the next piece (this stage or the next)
      const int upn = qn / NPU, qan = qn % NPU;
      const bool newu = qan == 0;                              // ... starts a unit position
      const int cur = NP % 2 == 0 ? q % 2 : E;                 // A buffers: by piece, or by stage
      const int bcur = (E * G::UPK + up) % 2, bnext = (E * G::UPK + up + 1) % 2;   // B buffers: by unit position
#ifdef OCQ_PHASE_STAMPS
      uint64_t t_s;
      if (q + 1 == NP) {
        const uint64_t ta = __builtin_amdgcn_s_memtime();
        lg_wait<G, G::NSTG - 2>();
        const uint64_t tb = __builtin_amdgcn_s_memtime();
        lds_barrier();
        lgkm_settled();
        t_s = __builtin_amdgcn_s_memtime();
        p_vm += tb - ta;
        p_bar += t_s - tb;
      } else {
        t_s = __builtin_amdgcn_s_memtime();
      }
#else
      if (q + 1 == NP) {   // also after the last stage: no branch, so no conservative wait at a join
        lg_wait<G, G::NSTG - 2>();
        lds_barrier();
        lgkm_settled();
      }
#endif
      // the next piece's LDS reads, one after each of the first MFMAs
      const uint8_t* rbase = slot(q + 1 < NP ? s : s + 1);
      const int rup = kw * G::UPK + upn;
      constexpr int NR = G::MTW + G::TW;
      // fences: the compiler would otherwise sink the reads to their uses
      __builtin_amdgcn_sched_barrier(0);
      // The next piece's LDS reads and, after the barrier, the loads of stage
      // s + NSTG go between this piece's MFMAs (reads after the first MFMAs,
      // loads after every LSTEP-th one): issued together ahead of the batch
      // they held the matrix cores idle (about 9 CU cycles per load).
      const int sl = s + G::NSTG < NS ? s + G::NSTG : NS - 1;
      uint8_t* dst = lds + (size_t)((s + G::NSTG) % G::NSTG) * G::NU * 1024;
      auto loads = [&](int k) {
        if (k < G::MTW) {
          fa[1 - cur].a[k] = *(const v4i*)(rbase + lg_a_unit<G>(rup, wm, k, qan));
        } else if (newu && k < NR) {
          fb[bnext].b[k - G::MTW] = *(const v4i*)(rbase + lg_b_unit<G>(rup, wt, k - G::MTW));
        }
        if (q + 1 == NP && k % LSTEP == LSTEP - 1 && k / LSTEP < G::PW) lg_issue_one<G>(src, sl, dst, wave, k / LSTEP);
      };
      // gate/up: the wave's MFMA batch at raised priority, so that of the two
      // waves on a SIMD the one issuing matrix work keeps the issue slots
      // (M=832 gate/up 149.8 -> 146.6 us in kernel traces of alternating runs
      // on one box; no gain for the BF16 down projection, whose batches are
      // shorter: 14 MFMAs against 21)
      if constexpr (PIPE) __builtin_amdgcn_s_setprio(1);
      if constexpr (PIPE) {
        lg_mfma_pipelined<G>(fa[cur], bh[q % 2], fb[newu ? bnext : bcur], qan, bh[(q + 1) % 2], acc, loads);
      } else {
        lg_mfma<G>(fa[cur], fb[bcur], qa, acc, loads);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (PIPE) __builtin_amdgcn_s_setprio(0);
#ifdef OCQ_PHASE_STAMPS
      const uint64_t t_e = __builtin_amdgcn_s_memtime();
      lgkm_settled();
      p_mma += t_e - t_s;
      p_set += __builtin_amdgcn_s_memtime() - t_e;
#else
      lgkm_settled();
#endif
    }
  };
#ifdef OCQ_PHASE_STAMPS
  const uint64_t t_loop0 = __builtin_amdgcn_s_memtime();
#endif
  for (int s = 0; s < NS; s += 2) {
    lgkm_settled();
    stage(s, std::integral_constant<int, 0>{});
    stage(s + 1, std::integral_constant<int, 1>{});
  }
  wait_vm<0>();
#ifdef OCQ_PHASE_STAMPS
  const uint64_t t_loop1 = __builtin_amdgcn_s_memtime();
  __builtin_amdgcn_s_waitcnt(0xC07F);
  if (lane == 0 && blockIdx.x < kPhaseWGs && wave < 8) {
    uint64_t* o = g_lg_phases[G::BF == kB_BF16 ? 1 : 0][blockIdx.x][wave];
    o[0] = p_vm; o[1] = p_bar; o[2] = p_mma; o[3] = p_set; o[4] = t_loop1 - t_loop0; o[5] = (uint64_t)NS;
  }
#endif
}

// Sum the KW partial tiles into the kw = 0 waves in a fixed order, reusing
// the ring once every wave has finished reading it.
template <class G>
__device__ __forceinline__ void lg_reduce(uint8_t* lds, int wmt, int kw, v4f (&acc)[G::MTW][G::TW]) {
  if constexpr (G::KW > 1) {
    const int lane = threadIdx.x & 63;
    v4f* red = (v4f*)lds;
    auto at = [&](int k, int j, int t) { return (((k * G::WM * G::WT + wmt) * G::MTW + j) * G::TW + t) * 64 + lane; };
    lds_barrier();
    if (kw > 0) {
#pragma unroll
      for (int j = 0; j < G::MTW; ++j)
#pragma unroll
        for (int t = 0; t < G::TW; ++t) red[at(kw - 1, j, t)] = acc[j][t];
    }
    lds_barrier();
    if (kw == 0) {
#pragma unroll
      for (int k = 1; k < G::KW; ++k)
#pragma unroll
        for (int j = 0; j < G::MTW; ++j)
#pragma unroll
          for (int t = 0; t < G::TW; ++t) acc[j][t] += red[at(k - 1, j, t)];
    }
  }
}

// workgroup -> (m-block, column group); groups shared by the m-blocks are
// numbered 8 apart (one XCD under round-robin placement) when possible
__device__ __forceinline__ void lg_block(int n_mb, int ngroups, int& mb, int& ng) {
  const int b = blockIdx.x;
  if (ngroups % 8 == 0) {
    const int q = b >> 3;
    mb = q % n_mb;
    ng = (q / n_mb) * 8 + (b & 7);
  } else {
    mb = b % n_mb;
    ng = b / n_mb;
  }
}

// ---------------------------------------------------------------- gate/up

constexpr size_t kLgScaleBytes = 2048;   // epilogue scales behind the gate/up ring

template <class G, bool BF16H>
__global__ __launch_bounds__(G::THREADS) void lg_gateup(GateUpArgs g) {
  extern __shared__ float lds_f[];
  uint8_t* lds = (uint8_t*)lds_f;
  const int ngroups = (g.I / 8) / G::RT;
  int mb, ng;
  lg_block(g.n_mb, ngroups, mb, ng);
  const int C = g.H / kChunk;
  const int row0 = mb * G::RM * 16;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave % G::WM, wt = (wave / G::WM) % G::WT, kw = wave / (G::WM * G::WT);
  const int left = g.Mpad / 16 - row0 / 16;
  const int nva = left < G::RM ? left : G::RM;
  const size_t wtile = (size_t)C * Fmt<G::BF>::kGlobal;
  // the epilogue's scales (the workgroup's row scales of x, then the gate
  // and up column scales) go to LDS behind the ring with direct-to-LDS loads
  // issued before the ring's: the first stage's wait covers them, and the
  // epilogue reads them without a global round trip
  float* sc = (float*)(lds + G::LDS);
  constexpr int kRows = G::RM * 16, kCols = G::RT * 8;
  static_assert(kRows + 2 * kCols <= kLgScaleBytes / 4, "scale area");
  if (wave * 64 < kRows + 2 * kCols) {
    const int k = wave * 64 + lane;
    const float* src = k < kRows ? g.sx + row0 + (k < nva * 16 ? k : 0)
                     : k < kRows + kCols ? g.wscales + ng * kCols + (k - kRows)
                     : k < kRows + 2 * kCols ? g.wscales + g.I + ng * kCols + (k - kRows - kCols) : g.sx + row0;
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(sc + wave * 64), 4, 0, 0);
  }
  v4f acc[G::MTW][G::TW];
#pragma unroll
  for (int j = 0; j < G::MTW; ++j)
#pragma unroll
    for (int t = 0; t < G::TW; ++t) acc[j][t] = v4f{0.f, 0.f, 0.f, 0.f};
  lg_mainloop<G>(g.xq + (size_t)(row0 / 16) * C * G::A_BLK + lane * 16, nva, (size_t)C * G::A_BLK,
                 g.wcodes + (size_t)ng * G::RT * wtile + lane * 16, wtile, C * G::SPC, lds, wave, wm, wt, kw, acc);
  lg_reduce<G>(lds, wave % (G::WM * G::WT), kw, acc);
  if (kw > 0) return;

  // epilogue: m-tiles wm*MTW + j (those that exist) x tiles tile0 + t.  The
  // pairing of gate and up lanes and the h32 layout ([tile][row][8]) are
  // those of the skinny gate/up epilogue.
  const int tile0 = ng * G::RT + wt * G::TW;
  const int r = lane & 15, c = r & 7;
  const bool lo = r < 8;
  float cg[G::TW], cu[G::TW];
#pragma unroll
  for (int t = 0; t < G::TW; ++t) {
    const int k = (wt * G::TW + t) * 8 + c;   // column of the workgroup's group
    cg[t] = sc[kRows + k];
    cu[t] = sc[kRows + kCols + k];
  }
  const int ngp = ngroups * G::WT;   // partial row maxima per row
  // bf16(h) goes through LDS: each lane holds 2 of the 4 rows x 8 channels of
  // a tile's value group, so storing it directly would be 2-byte stores
  // spread over many lines; staged as [m-tile][row][tile][8 channels] per
  // wave, each lane then writes 16 B (8 channels of one row) to the fragment
  // order and the row-major tap.
  constexpr int kStage = G::MTW * 16 * G::TW * 16;   // bytes per wave
  static_assert(!BF16H || G::NW * kStage <= G::LDS, "staging fits the ring");
  uint16_t* st = (uint16_t*)(lds + (size_t)wave * kStage);
  if constexpr (BF16H) lds_barrier();   // every wave is done reading the ring
#pragma unroll
  for (int j = 0; j < G::MTW; ++j) {
    const int mt = wm * G::MTW + j;
    if (mt >= nva) break;
    const int m_base = row0 + mt * 16 + 4 * (lane >> 4);
    v4f xs;
#pragma unroll
    for (int i = 0; i < 4; ++i) xs[i] = sc[m_base - row0 + i];
    float amax[2] = {0.f, 0.f};
#pragma unroll
    for (int t = 0; t < G::TW; ++t) {
      const int tile = tile0 + t;
      const v4f& v = acc[j][t];
      const float p0 = dpp<0x128>(lo ? v[1] : v[0]);
      const float p1 = dpp<0x128>(lo ? v[3] : v[2]);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int i = 2 * e + (lo ? 0 : 1);
        const float vi = lo ? v[2 * e] : v[2 * e + 1];
        const float xi = lo ? xs[2 * e] : xs[2 * e + 1];
        const float gv = lo ? vi : (e ? p1 : p0);
        const float uv = lo ? (e ? p1 : p0) : vi;
        const float ga = gv * xi * cg[t];
        const float hv = (BF16H ? silu_div(ga) : silu_rcp(ga)) * (uv * xi * cu[t]);
        const int m = m_base + i;
        if constexpr (BF16H) {
          st[((j * 16 + (m - row0 - mt * 16)) * G::TW + t) * 8 + c] = (uint16_t)bf16_bits(hv);
        } else {
          g.h32[((size_t)tile * g.Mpad + m) * 8 + c] = hv;
          amax[e] = fmaxf(amax[e], fabsf(hv));
        }
      }
    }
    if constexpr (!BF16H) {
#pragma unroll
      for (int e = 0; e < 2; ++e) amax[e] = max8(amax[e]);
      if ((lane & 7) == 0) {   // lanes 16 gq (rows 0, 2) and 16 gq + 8 (rows 1, 3)
        const int m = m_base + ((lane & 8) ? 1 : 0);
#pragma unroll
        for (int e = 0; e < 2; ++e) g.amax_part[(size_t)(m + 2 * e) * ngp + ng * G::WT + wt] = amax[e];
      }
    }
  }
  if constexpr (BF16H) {
    // the wave reads back what it staged (its own LDS accesses complete in order)
    constexpr int kItems = G::MTW * 16 * G::TW;   // (m-tile, row, tile) groups of 8 channels
    const int C128 = g.I / 128;
#pragma unroll
    for (int k0 = 0; k0 < kItems; k0 += 64) {
      const int k = k0 + lane;
      const int j = k / (16 * G::TW), rr = (k / G::TW) % 16, t = k % G::TW;
      const int mt = wm * G::MTW + j;
      if (k < kItems && mt < nva) {
        const v4i d = *(const v4i*)(st + (size_t)k * 8);
        const int m = row0 + mt * 16 + rr, n0 = (tile0 + t) * 8;
        *(v4i*)(g.hb + frag_off16(m, n0, C128)) = d;
        if (g.tap_hb && m < g.M) *(v4i*)(g.tap_hb + (size_t)m * g.I + n0) = d;
      }
    }
  }
}

// ---------------------------------------------------------------- down, BF16 mode

template <class G>
__global__ __launch_bounds__(G::THREADS) void lg_down_bf16(DownArgs d) {
  extern __shared__ float lds_f[];
  uint8_t* lds = (uint8_t*)lds_f;
  const int ngroups = (d.H / 16) / G::RT;
  int mb, ng;
  lg_block(d.n_mb, ngroups, mb, ng);
  const int C = d.I / kChunk;
  const int row0 = mb * G::RM * 16;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave % G::WM, wt = (wave / G::WM) % G::WT, kw = wave / (G::WM * G::WT);
  const int left = (d.M + 15) / 16 - row0 / 16;
  const int nva = left < G::RM ? left : G::RM;
  const size_t wtile = (size_t)C * Fmt<G::BF>::kGlobal;
  v4f acc[G::MTW][G::TW];
#pragma unroll
  for (int j = 0; j < G::MTW; ++j)
#pragma unroll
    for (int t = 0; t < G::TW; ++t) acc[j][t] = v4f{0.f, 0.f, 0.f, 0.f};
  lg_mainloop<G>((const uint8_t*)d.A + (size_t)(row0 / 16) * C * G::A_BLK + lane * 16, nva, (size_t)C * G::A_BLK,
                 d.wcodes + (size_t)ng * G::RT * wtile + lane * 16, wtile, C * G::SPC, lds, wave, wm, wt, kw, acc);
  lg_reduce<G>(lds, wave % (G::WM * G::WT), kw, acc);
  if (kw > 0) return;
  const int r = lane & 15;
#pragma unroll
  for (int j = 0; j < G::MTW; ++j) {
    const int mt = wm * G::MTW + j;
    if (mt >= nva) break;
#pragma unroll
    for (int t = 0; t < G::TW; ++t) {
      const int col = (ng * G::RT + wt * G::TW + t) * 16 + r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = row0 + mt * 16 + 4 * (lane >> 4) + i;
        if (m < d.M) d.y[(size_t)m * d.H + col] = (uint16_t)bf16_bits(acc[j][t][i]);
      }
    }
  }
}

template <class G, class Arg>
hipError_t lg_launch(void (*fn)(Arg), int grid, const Arg& arg, hipStream_t st, std::atomic<uint64_t>& lds_set,
                     const LaunchEvents& ev = LaunchEvents{}, size_t lds = G::LDS) {
  if (hipError_t e = allow_lds((const void*)fn, lds, lds_set); e != hipSuccess) return e;
  launch_kernel(fn, dim3(grid), dim3(G::THREADS), lds, st, ev, arg);
  return hipGetLastError();
}

// gate/up: 13 m-tiles x 12 tiles per workgroup; 2 x 4 waves of 7 m-tiles x 3
// tiles.  A stage is one whole chunk (two weight unit positions, 128 inputs,
// 76 KB) in a two-stage ring, so that each workgroup barrier is shared by
// twice the matrix work of a one-unit stage (the per-stage cost of the
// barrier, its wait for the slower wave of each SIMD and the restart was
// about a third of the stage); with an odd chunk count, one unit position
// per stage in a three-stage ring.
using GUL2 = Lg<kB_FP8_F16, true, kLgRM, kLgRT1, 2, kLgWT1, 1, 2, 2>;
using GUL = Lg<kB_FP8_F16, true, kLgRM, kLgRT1, 2, kLgWT1, 1, 1, 3>;
// down: 7 m-tiles x 8 tiles per workgroup (112 rows x 128 columns: more
// multiply-adds per staged byte than 208 x 64); 1 x 4 waves of 7 m-tiles x 2
// tiles, each pair of K-waves splitting the two unit positions of a stage (64
// inputs), four stages (120 KB).  Whole-chunk stages in a two-stage ring were
// slower here (M=832: 94 -> 127 us): the weight loads, which come from HBM,
// then have one short stage to land instead of three.
using GDL = Lg<kB_BF16, true, kLgRM2, kLgRT2, 1, 4, 2, 2, 4>;

}  // namespace

int lg_phase_copy(void* host, size_t bytes) {
#ifdef OCQ_PHASE_STAMPS
  if (bytes < sizeof(g_lg_phases)) return (int)hipErrorInvalidValue;
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_lg_phases), sizeof(g_lg_phases));
#else
  (void)host; (void)bytes;
  return -1;
#endif
}

hipError_t launch_gateup_large(const Plan& p, const GateUpArgs& g, hipStream_t st, const LaunchEvents& ev) {
  if ((p.inter / 8) % GUL::RT || p.hidden % kChunk) return hipErrorInvalidValue;
  const int grid = p.n_mblocks * ((p.inter / 8) / GUL::RT);
  // stages are processed in pairs: a whole-chunk stage needs an even chunk count
  const bool whole = (p.hidden / kChunk) % 2 == 0;
  if (p.prec == kFP8DownBF16) {
    static std::atomic<uint64_t> lds_set{0}, lds_set2{0};
    if (whole) return lg_launch<GUL2>(lg_gateup<GUL2, true>, grid, g, st, lds_set2, ev, GUL2::LDS + kLgScaleBytes);
    return lg_launch<GUL>(lg_gateup<GUL, true>, grid, g, st, lds_set, ev, GUL::LDS + kLgScaleBytes);
  }
  static std::atomic<uint64_t> lds_set{0}, lds_set2{0};
  if (whole) return lg_launch<GUL2>(lg_gateup<GUL2, false>, grid, g, st, lds_set2, ev, GUL2::LDS + kLgScaleBytes);
  return lg_launch<GUL>(lg_gateup<GUL, false>, grid, g, st, lds_set, ev, GUL::LDS + kLgScaleBytes);
}

hipError_t launch_down_large(const Plan& p, const DownArgs& d, hipStream_t st) {
  if ((p.hidden / 16) % GDL::RT || p.inter % kChunk || p.prec != kFP8DownBF16) return hipErrorInvalidValue;
  const int grid = p.n_mb2 * ((p.hidden / 16) / GDL::RT);
  static std::atomic<uint64_t> lds_set{0};
  return lg_launch<GDL>(lg_down_bf16<GDL>, grid, d, st, lds_set);
}

}  // namespace ocq
