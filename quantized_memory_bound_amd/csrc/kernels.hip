// HIP kernels of the quantized MLP block for CDNA4 (gfx950): x quantization,
// h requantization and the forward launch sequence.  The two matrix-core
// stages live in gemm_gateup.hip and gemm_down.hip (main loops in
// gemm_core.h).
//
// One forward call = three kernels on the caller's stream:
//   k_xquant   per-token E4M3 quantization of x (scale amax/448), zero rows
//              up to whole m-blocks.
//   gate/up    G = xq Wg^T, U = xq Wu^T (exact products, fp32 accumulation),
//              h = SiLU(G sx sw_g) * (U sx sw_u), and in the same launch the
//              per-token requantization sh = max|h| / 448, hq = E4M3(h / sh)
//              (row maxima across workgroups through device-scope atomics,
//              h kept in registers), or bf16(h) for a BF16 down projection.
//   down       Y = hq Wd^T (or bf16(h) Wd^T), y = bf16(Y sh sw_d).
// Where the gate/up grid cannot be resident all at once (several m-blocks,
// the LDS-tiled kernels for many rows), it writes fp32 h and per-workgroup
// row maxima instead and a fourth kernel, k_requant, quantizes.
// Cited passages ("OCRia 推理栈：单卡 B200 提速近 10 倍"): "Reducing the data
// moved: workload-aware quantization" (FP8 / NVFP4 / BF16 weights per layer),
// "Generate more tokens per target pass" (M = requests x (1 + drafts) rows
// share one read of the weights); German page "Wie es funktioniert" (SiLU and
// quantization fused, intermediates kept on chip).
#include "kcommon.h"

namespace ocq {

#ifdef OCQ_PHASE_STAMPS
// Start and end (100 MHz clock) of every workgroup of the last x-quant and
// requantization launches, built only with OCQ_PHASE_STAMPS:
// [x-quant, requant][workgroup < 1024][start, end after its stores landed].
__device__ uint64_t g_q_phases[2][kQPhaseWGs][2];
static_assert(sizeof(g_q_phases) == kQPhaseBytes, "layout stated in ocq_internal.h");
#define OCQ_Q_START() const uint64_t q_t0 = __builtin_amdgcn_s_memrealtime()
#define OCQ_Q_END(k)                                                                        \
  do {                                                                                      \
    __builtin_amdgcn_s_waitcnt(0);                                                          \
    if (threadIdx.x == 0 && blockIdx.x < kQPhaseWGs) {                                      \
      g_q_phases[k][blockIdx.x][0] = q_t0;                                                  \
      g_q_phases[k][blockIdx.x][1] = __builtin_amdgcn_s_memrealtime();                      \
    }                                                                                       \
  } while (0)
#else
#define OCQ_Q_START()
#define OCQ_Q_END(k)
#endif

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// Row-per-workgroup kernels write one row's pieces of 16-row fragment blocks.
// Workgroup b handles row 16 mt + r (and slice `rest`) with
//   b = ((rest * G + mt / 8) * 16 + r) * 8 + mt % 8,   G = ceil(mtiles / 8),
// so the 16 rows of an m-tile are 8 workgroups apart: under round-robin
// placement they run on one XCD and complete every cache line of their
// blocks in that XCD's L2.  Returns false for the unused slots of the last
// group of 8 m-tiles.
__device__ __forceinline__ bool tile_row_of(int b, int mtiles, int& m, int& rest) {
  const int G = (mtiles + 7) / 8;
  const int x = b & 7, r = (b >> 3) & 15, q = b >> 7;
  const int mt = (q % G) * 8 + x;
  rest = q / G;
  m = mt * 16 + r;
  return mt < mtiles;
}

inline int tile_row_grid(int mtiles, int nrest) { return (mtiles + 7) / 8 * 128 * nrest; }

// ---------------------------------------------------------------- k_xquant

// One workgroup per row (all 256 threads), so the row's loads are all in
// flight at once; |x| max reduced over the wavefront, then across the four
// waves in LDS.  Codes go to the fragment-ordered operand buffer (8
// consecutive inputs = 8 contiguous bytes there), or with f16 set their exact
// fp16 values in the 16-bit fragment order (16 contiguous bytes); rows
// M..Mpad-1 are written as zero codes with scale 0.  x is first multiplied by
// the blob's per-channel multiplier xmul (1 unless packed with smoothing):
// x'[k] = fl32(x[k] xmul[k]), and x' is what is quantized.  tap_q / tap_s (nullable) receive the plain
// [M][H] codes and [M] scales.
__global__ __launch_bounds__(kThreads) void k_xquant(const uint16_t* __restrict__ x, const float* __restrict__ xmul,
                                                     int M, int H, int Mpad,
                                                     uint8_t* __restrict__ xq, int f16, float* __restrict__ sx,
                                                     uint8_t* __restrict__ tap_q, float* __restrict__ tap_s,
                                                     uint32_t* __restrict__ amax_g, uint32_t* __restrict__ sync) {
  __shared__ float s_max[kWaves];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  OCQ_Q_START();
  int m, rest;
  if (!tile_row_of(blockIdx.x, Mpad / 16, m, rest)) return;
  const int C = H / 128;
  // the next kernel's grid-wide row maxima (every copy), arrival counts and release flags start at zero
  if (threadIdx.x < kAmaxSlots) amax_g[(size_t)threadIdx.x * Mpad + m] = 0u;
  if (m == 0 && threadIdx.x < 2) sync[threadIdx.x] = 0u;
  if (m == 0 && threadIdx.x < kGoCopies + kArriveGroups) sync[kGoStride * (1 + threadIdx.x)] = 0u;
  if (m >= M) {                                     // padding row: zero codes, zero scale
    for (int k = threadIdx.x * 8; k < H; k += kThreads * 8) {
      if (f16) *(v4i*)((uint16_t*)xq + frag_off16(m, k, C)) = v4i{0, 0, 0, 0};
      else *(v2u*)(xq + frag_off8(m, k, C)) = v2u{0u, 0u};
    }
    if (threadIdx.x == 0) sx[m] = 0.0f;
    return;
  }
  const uint16_t* xr = x + (size_t)m * H;
  constexpr int kReg = 4;                           // 8 bf16 per load, up to 4 loads held per thread
  v4i v[kReg];
  float amax = 0.0f;
  for (int base = 0; base < H; base += kThreads * 8 * kReg) {
#pragma unroll
    for (int j = 0; j < kReg; ++j) {
      const int k = base + (j * kThreads + threadIdx.x) * 8;
      v[j] = k < H ? *(const v4i*)(xr + k) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < kReg; ++j) {
      const int k = base + (j * kThreads + threadIdx.x) * 8;
      if (k >= H) continue;
      const v4f m0 = *(const v4f*)(xmul + k), m1 = *(const v4f*)(xmul + k + 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t w = (uint32_t)v[j][q];
        const float ma = q < 2 ? m0[2 * q] : m1[2 * q - 4], mb = q < 2 ? m0[2 * q + 1] : m1[2 * q - 3];
        amax = fmaxf(amax, fabsf(__uint_as_float(w << 16) * ma));
        amax = fmaxf(amax, fabsf(__uint_as_float(w & 0xFFFF0000u) * mb));
      }
    }
  }
  amax = wave_max(amax);
  if (lane == 0) s_max[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  const float s = amax / 448.0f;
  const float rcp = s > 0.0f ? 1.0f / s : 0.0f;
  for (int base = 0; base < H; base += kThreads * 8 * kReg) {
    if (base > 0 || H > kThreads * 8 * kReg) {      // reload unless the whole row is still in registers
#pragma unroll
      for (int j = 0; j < kReg; ++j) {
        const int k = base + (j * kThreads + threadIdx.x) * 8;
        v[j] = k < H ? *(const v4i*)(xr + k) : v4i{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int j = 0; j < kReg; ++j) {
      const int k = base + (j * kThreads + threadIdx.x) * 8;
      if (k >= H) continue;
      uint32_t out[2] = {0u, 0u};
      if (s > 0.0f) {
        const v4f m0 = *(const v4f*)(xmul + k), m1 = *(const v4f*)(xmul + k + 4);
        float p[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t w = (uint32_t)v[j][q];
          p[2 * q] = __uint_as_float(w << 16) * (q < 2 ? m0[2 * q] : m1[2 * q - 4]);
          p[2 * q + 1] = __uint_as_float(w & 0xFFFF0000u) * (q < 2 ? m0[2 * q + 1] : m1[2 * q - 3]);
        }
        const v2u c = e4m3x8_quot(p, s, rcp);
        out[0] = c[0];
        out[1] = c[1];
      }
      if (f16) *(v8h*)((uint16_t*)xq + frag_off16(m, k, C)) = e4m3x8_to_f16(out[0], out[1]);
      else *(v2u*)(xq + frag_off8(m, k, C)) = v2u{out[0], out[1]};
      if (tap_q) *(v2u*)(tap_q + (size_t)m * H + k) = v2u{out[0], out[1]};
    }
  }
  if (threadIdx.x == 0) {
    sx[m] = s;
    if (tap_s) tap_s[m] = s;
  }
  OCQ_Q_END(0);
}

// ---------------------------------------------------------------- k_requant

// amax_part[m][g] holds the |h| maximum of row m over the columns of gate/up
// partial g; every block first reduces the row's ngroups partial maxima.
// Rows M..Mpad-1 (padding, possibly beyond the gate/up m-blocks) get zero
// codes and scale 0 without reading h.  Each thread quantizes 8 consecutive
// columns (one 32-byte piece of an 8-column h32 tile) into 8 contiguous bytes
// of the fragment-ordered operand buffer of the down projection.  tap_q /
// tap_s (nullable) receive the plain [M][I] codes and [M] scales.
constexpr int kRqCols = 8 * kThreads;   // columns of a row per workgroup

__global__ __launch_bounds__(kThreads) void k_requant(const float* __restrict__ h32,
                                                      const float* __restrict__ amax_part, int ngroups, int M,
                                                      int Mpad, int I, uint8_t* __restrict__ hq,
                                                      float* __restrict__ sh, uint8_t* __restrict__ tap_q,
                                                      float* __restrict__ tap_s) {
  __shared__ float s_max[kWaves];
  int m, xb;
  OCQ_Q_START();
  if (!tile_row_of(blockIdx.x, Mpad / 16, m, xb)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int k = xb * kRqCols + threadIdx.x * 8;
  const bool has = k < I;
  if (m >= M) {
    if (xb == 0 && threadIdx.x == 0) sh[m] = 0.0f;
    if (has) *(v2u*)(hq + frag_off8(m, k, I / 128)) = v2u{0u, 0u};
    return;
  }
  // the thread's 8 values of h are requested before the row maximum, so the
  // loads are in flight together (h32: each 8-column tile is a [Mpad][8] block)
  v4f v0 = v4f{0.f, 0.f, 0.f, 0.f}, v1 = v0;
  if (has) {
    const float* src = h32 + ((size_t)(k / 8) * Mpad + m) * 8;
    v0 = *(const v4f*)src;
    v1 = *(const v4f*)(src + 4);
  }
  // up to 8 partials per thread requested together
  float a = 0.0f;
  const float* ap = amax_part + (size_t)m * ngroups;
  if (ngroups <= kThreads) {
    if (threadIdx.x < ngroups) a = ap[threadIdx.x];
  } else for (int g0 = 0; g0 < ngroups; g0 += 8 * kThreads) {
    float t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int g = g0 + u * kThreads + threadIdx.x;
      t[u] = g < ngroups ? ap[g] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) a = fmaxf(a, t[u]);
  }
  a = wave_max(a);
  if (lane == 0) s_max[wave] = a;
  __syncthreads();
  a = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  const float s = a / 448.0f;
  if (xb == 0 && threadIdx.x == 0) {
    sh[m] = s;
    if (tap_s) tap_s[m] = s;
  }
  if (!has) return;
  v2u out = v2u{0u, 0u};
  if (s > 0.0f) {
    const float p[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    out = e4m3x8_quot(p, s, 1.0f / s);
  }
  *(v2u*)(hq + frag_off8(m, k, I / 128)) = out;
  if (tap_q) *(v2u*)(tap_q + (size_t)m * I + k) = out;
  OCQ_Q_END(1);
}

}  // namespace

// ---------------------------------------------------------------- forward

// Where h is requantized: 1 (default) inside the gate/up kernel where its
// grid is resident at once, 0 in a second kernel.  Measured on MI355X (graph
// replays, one box at a time), the in-launch form saves 0.3-1.2 us per block:
// spec-verify 35.2 -> 34.7 us, decode 20.6 -> 19.4 us, NVFP4 M=1 28.4 ->
// 27.5 us.
static std::atomic<int> g_fused_requant{1};

void set_fused_requant(int mode) { g_fused_requant.store(mode, std::memory_order_relaxed); }

static inline void stage(const FwdArgs& a, int i) {
  if (a.stage_events && a.stage_events[i]) (void)hipEventRecord((hipEvent_t)a.stage_events[i], (hipStream_t)a.stream);
}

int q_phase_copy(void* host, size_t bytes) {
#ifdef OCQ_PHASE_STAMPS
  if (bytes < sizeof(g_q_phases)) return (int)hipErrorInvalidValue;
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_q_phases), sizeof(g_q_phases));
#else
  (void)host; (void)bytes;
  return -1;
#endif
}

int launch_forward(const Plan& p, const FwdArgs& a) {
  hipStream_t st = (hipStream_t)a.stream;
  const BlobLayout L = blob_layout(p.hidden, p.inter, p.prec);
  uint8_t* ws = a.ws;
  uint8_t* xq = ws + p.off_xq;
  float* sx = (float*)(ws + p.off_sx);
  float* amax_part = (float*)(ws + p.off_amax);
  float* h32 = (float*)(ws + p.off_h32);
  uint8_t* hq = ws + p.off_hq;
  uint16_t* hb = (uint16_t*)(ws + p.off_hb);
  float* sh = (float*)(ws + p.off_sh);
  uint32_t* amax_g = (uint32_t*)(ws + p.off_amaxg);
  uint32_t* sync = (uint32_t*)(ws + p.off_sync);

  stage(a, 0);
  const bool bf16_down = p.prec == kFP8DownBF16;
  hipLaunchKernelGGL(k_xquant, dim3(tile_row_grid(p.Mpad / 16, 1)), dim3(kThreads), 0, st, a.x,
                     (const float*)(a.blob + L.off_xmul), p.M, p.hidden, p.Mpad, xq, p.lg1, sx,
                     (uint8_t*)a.taps.x_codes, (float*)a.taps.x_scales, amax_g, sync);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;

  GateUpArgs g{};
  g.xq = xq; g.sx = sx;
  g.wcodes = a.blob + L.off_gu_codes;
  g.wscales = (const float*)(a.blob + L.off_gu_scales);
  g.wbscales = a.blob + L.off_gu_bscales;
  g.tscales = (const float*)(a.blob + offsetof(BlobHeader, s_gate));
  g.h32 = h32; g.hb = hb; g.amax_part = amax_part;
  g.tap_hb = bf16_down ? (uint16_t*)a.taps.h_out : nullptr;
  g.amax_g = amax_g; g.sync = sync; g.hq = hq; g.sh = sh;
  g.tap_hq = bf16_down ? nullptr : (uint8_t*)a.taps.h_out;
  g.tap_sh = (float*)a.taps.h_scales;
  g.H = p.hidden; g.I = p.inter; g.M = p.M; g.n_mb = p.n_mblocks; g.Mpad = p.Mpad;
  LaunchEvents gev;   // stage events 1 and 2 are taken by the gate/up launch itself
  if (a.stage_events) {
    gev.start = (hipEvent_t)a.stage_events[1];
    gev.end = (hipEvent_t)a.stage_events[2];
  }
  bool fused = !bf16_down && g_fused_requant.load(std::memory_order_relaxed) != 0;
  e = launch_gateup(p, g, st, gev, fused);
  if (e != hipSuccess) return (int)e;
  if (a.requant_in_gateup) *a.requant_in_gateup = fused ? 1 : 0;

  if (!bf16_down && !fused) {
    hipLaunchKernelGGL(k_requant, dim3(tile_row_grid(p.Mpad / 16, (p.inter + kRqCols - 1) / kRqCols)),
                       dim3(kThreads), 0, st,
                       h32, amax_part,
                       p.namax, p.M, p.Mpad, p.inter, hq, sh, (uint8_t*)a.taps.h_out,
                       (float*)a.taps.h_scales);
    e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }

  stage(a, 3);
  DownArgs d{};
  d.A = bf16_down ? (const void*)hb : (const void*)hq;
  d.sh = sh;
  d.wcodes = a.blob + L.off_dn_codes;
  d.wscales = (const float*)(a.blob + L.off_dn_scales);
  d.wbscales = a.blob + L.off_dn_bscales;
  d.tscale = (const float*)(a.blob + offsetof(BlobHeader, s_down));
  d.y = a.y;
  d.sync = sync;
  d.H = p.hidden; d.I = p.inter; d.M = p.M; d.n_mb = p.n_mb2; d.ngroups = p.ngroups2;
  e = launch_down(p, d, st);
  stage(a, 4);
  return (int)e;
}

}  // namespace ocq
