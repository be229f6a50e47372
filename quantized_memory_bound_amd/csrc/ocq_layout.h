// Packed-weight blob layout and workspace layout shared by the host packer,
// the C-ABI entry points and the HIP kernels.
//
// Fragment order.  The matrix cores take, per 16x16xK product, one operand
// fragment per lane.  Every weight projection is cut into "tiles" of 16
// output rows and "chunks" of 128 input columns.  Lane l = 16 g + r (g = 0..3,
// r = 0..15) of a wave holds row r of the tile and the 32 consecutive inputs
// k = 128 c + 32 g + j, j = 0..31, of chunk c.  Activations are read with the
// same per-lane k-ranges from fragment-ordered activation buffers (written so
// by the quantization kernels), so the two operands agree on which k each
// lane/byte carries and the hardware sums the same products as the plain
// definition.
//
//   FP8 chunk  (2048 B): [half h = 0,1][lane][16 B]   byte j of lane l at
//                        h = j / 16, offset (h * 64 + l) * 16 + j % 16.
//   BF16 chunk (4096 B): [sub i = 0..3][lane][16 B]   bf16 element j at
//                        i = j / 8, offset (i * 64 + l) * 16 + 2 * (j % 8).
//   FP4 chunk  (1024 B): [lane][16 B]                 E2M1 code j in byte j/2,
//                        low nibble for even j.
//   FP4 block scales: per tile, groups of 8 chunks, [lane][8 chunks x 2 B]
//                        (1024 B per group); byte 2 (c % 8) + b is the E4M3
//                        scale of inputs 128 c + 32 g + 16 b .. +16.
//
// Gate/up tiles interleave the two projections: tile t holds gate rows
// 8t..8t+7 (tile rows 0..7) and up rows 8t..8t+7 (tile rows 8..15), so one
// output fragment carries both values of the SiLU(gate) * up product.
// Down tiles hold 16 consecutive output rows of W_down.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <initializer_list>

namespace ocq {

constexpr uint32_t kBlobVersion = 2;
constexpr char kBlobMagic[8] = {'O', 'C', 'Q', 'B', 'L', 'O', 'B', '1'};
constexpr int kChunk = 128;           // inputs per chunk
constexpr int kTileRows = 16;         // output rows per tile
constexpr size_t kAlign = 256;

inline size_t align_up(size_t v, size_t a = kAlign) { return (v + a - 1) / a * a; }

enum Prec { kFP8 = 0, kFP8DownBF16 = 1, kFP4 = 2 };
enum WeightKind { kWFP8 = 0, kWBF16 = 1, kWFP4 = 2 };

struct BlobHeader {
  char magic[8];
  uint32_t version;
  int32_t hidden, inter, prec_mode;
  // byte offsets from the blob start
  uint64_t off_gu_codes, off_gu_scales, off_gu_bscales;
  uint64_t off_dn_codes, off_dn_scales, off_dn_bscales;
  uint64_t off_xmul;           // fp32 [hidden]: x is multiplied by it before its quantization
  uint64_t total_bytes;
  float s_gate, s_up, s_down;  // NVFP4 per-tensor scales (0 otherwise)
  uint8_t pad[256 - 8 - 4 - 12 - 8 * 8 - 12];
};
static_assert(sizeof(BlobHeader) == 256, "header is 256 bytes");

// bytes of a projection's codes / scale sections with `rows` outputs, `cols` inputs
inline size_t codes_bytes(WeightKind k, size_t rows, size_t cols) {
  switch (k) {
    case kWFP8: return rows * cols;
    case kWBF16: return rows * cols * 2;
    case kWFP4: return rows * cols / 2;
  }
  return 0;
}
inline size_t chunk_groups(size_t cols) { return (cols / kChunk + 7) / 8; }
inline size_t bscale_bytes(WeightKind k, size_t rows, size_t cols) {
  return k == kWFP4 ? (rows / kTileRows) * chunk_groups(cols) * 1024 : 0;
}

struct BlobLayout {
  WeightKind gu, dn;
  uint64_t off_gu_codes, off_gu_scales, off_gu_bscales;
  uint64_t off_dn_codes, off_dn_scales, off_dn_bscales;
  uint64_t off_xmul;
  uint64_t total;
};

inline bool shape_ok(int hidden, int inter) {
  return hidden >= 128 && inter >= 128 && hidden <= 65536 && inter <= 65536 &&
         hidden % kChunk == 0 && inter % kChunk == 0;
}

inline BlobLayout blob_layout(int hidden, int inter, int prec) {
  BlobLayout L{};
  L.gu = prec == kFP4 ? kWFP4 : kWFP8;
  L.dn = prec == kFP4 ? kWFP4 : (prec == kFP8DownBF16 ? kWBF16 : kWFP8);
  size_t H = hidden, I = inter;
  size_t o = align_up(sizeof(BlobHeader));
  L.off_gu_codes = o;   o = align_up(o + codes_bytes(L.gu, 2 * I, H));
  L.off_gu_scales = o;  o = align_up(o + (L.gu == kWFP8 ? 2 * I * sizeof(float) : 0));
  L.off_gu_bscales = o; o = align_up(o + bscale_bytes(L.gu, 2 * I, H));
  L.off_dn_codes = o;   o = align_up(o + codes_bytes(L.dn, H, I));
  L.off_dn_scales = o;  o = align_up(o + (L.dn == kWFP8 ? H * sizeof(float) : 0));
  L.off_dn_bscales = o; o = align_up(o + bscale_bytes(L.dn, H, I));
  // per-input-channel multiplier of x (1 everywhere unless packed with smoothing)
  L.off_xmul = o;       o = align_up(o + H * sizeof(float));
  L.total = o;
  return L;
}

// ---------------------------------------------------------------------------
// Execution plan and workspace
// ---------------------------------------------------------------------------

// m-tiles (16 rows each) per gate/up workgroup; instantiated template values
constexpr int kMTChoices[] = {1, 2, 4, 7, 13};
constexpr int kMTMax = 13;
// In-launch requantization: the row maxima are folded with atomics into
// kAmaxSlots copies (workgroup b into copy b % kAmaxSlots), so that no
// address takes more than a few of them; workgroups arrive on kArriveGroups
// group counters (b % kArriveGroups), the last of each group on the top
// counter; the release of the grid-wide wait is broadcast through kGoCopies
// flags, each polled by a few workgroups.  Counters and flags lie kGoStride
// words apart (each on its own 128-byte line).
constexpr int kAmaxSlots = 32;
constexpr int kGoCopies = 32, kArriveGroups = 16, kGoStride = 32;
// [0] top arrivals, [1] time-out, release flags, group arrivals
constexpr int kSyncWords = kGoStride * (1 + kGoCopies + kArriveGroups);

// LDS-tiled kernels for many rows; chosen from kLgMinRows rows on
constexpr int kLgRM = 13;        // gate/up: m-tiles per workgroup
constexpr int kLgRT1 = 12;       // gate/up: interleaved tiles per workgroup
constexpr int kLgWT1 = 4;        // gate/up: wave columns (partial row maxima per workgroup)
constexpr int kLgRT2 = 8;        // down: output tiles per workgroup
constexpr int kLgRM2 = 7;        // down: m-tiles per workgroup
constexpr int kLgMinRows = 384;

struct Plan {
  int M, hidden, inter, prec;
  int Mpad;        // rows of every activation buffer (covers both projections' m-blocks)
  // gate/up kernel: n_mblocks m-blocks of MT m-tiles x ngroups1 groups of T1 tiles
  int MT, n_mblocks, T1, ngroups1;
  // down kernel: n_mb2 m-blocks of MT2 m-tiles x ngroups2 groups of T2 tiles,
  // every workgroup over the whole input range
  int MT2, n_mb2, T2, ngroups2;
  // LDS-tiled kernels selected (gate/up, down)
  int lg1, lg2;
  // partial maxima of |h| per row written by the gate/up kernel: one per
  // workgroup (skinny kernels) or per wave column (LDS-tiled kernel)
  int namax;
  // workspace offsets (xq, hq, hb are fragment-ordered operand buffers of Mpad rows);
  // amaxg / sync: grid-wide row maxima and the arrival counter of a gate/up
  // launch that requantizes h itself
  size_t off_xq, off_sx, off_amax, off_h32, off_hq, off_hb, off_sh, off_amaxg, off_sync, total;
};

inline int pick_mt(int M) {
  int need = (M + 15) / 16;
  for (int c : kMTChoices)
    if (c >= need) return c;
  return kMTMax;
}

// Down projection blocking.  Each workgroup reads its rows' activations and
// its tiles' weights over the whole input range once, so the bytes it pulls
// through its CU are inter * (rows * act_bytes + cols * w_bytes); the choice
// minimises that per-CU volume (times the number of workgroup waves over the
// 256 CUs) plus the matrix-core time of the padded rows.
inline void pick_down(Plan& p) {
  const int mtiles = (p.M + 15) / 16, ntiles = p.hidden / 16;
  const double ea = p.prec == kFP8DownBF16 ? 2.0 : 1.0;
  const double eb = p.prec == kFP8DownBF16 ? 2.0 : (p.prec == kFP4 ? 0.5 + 1.0 / 16 : 1.0);
  double best = 1e30;
  for (int mt : {1, 2, 4}) {
    for (int t : {1, 2, 4}) {
      if (ntiles % t) continue;
      const int nmb = (mtiles + mt - 1) / mt, ng = ntiles / t;
      const double wgs = (double)nmb * ng;
      const double waves = wgs <= 256 ? 1.0 : (double)((nmb * ng + 255) / 256);
      const double l1 = (double)p.inter * 16.0 * (mt * ea + t * eb);           // bytes per workgroup
      const double mm = (double)p.inter * 16.0 * 16.0 * mt * t;   // 16-bit MACs per workgroup
      // per CU: ~150 GB/s through L1; ~4 TMAC/s of 16-bit matrix work (us)
      double cost = waves * (l1 / 150e3 + mm / 4e6);
      if (wgs < 128) cost *= 128.0 / wgs;                                    // too few CUs streaming
      if (cost < best * 0.999) {
        best = cost;
        p.MT2 = mt; p.T2 = t; p.n_mb2 = nmb; p.ngroups2 = ng;
      }
    }
  }
}

inline Plan make_plan(int M, int hidden, int inter, int prec) {
  Plan p{};
  p.M = M; p.hidden = hidden; p.inter = inter; p.prec = prec;
  p.MT = pick_mt(M);
  int rows_per_block = 16 * p.MT;
  p.n_mblocks = (M + rows_per_block - 1) / rows_per_block;
  // gate/up: tiles of 8 gate + 8 up columns; 3 tiles per workgroup when that
  // still gives >= 192 workgroups (one per CU at the configured sizes); 6 for
  // NVFP4 with 1-4 m-tiles, whose workgroups hold one per CU (512 workgroups of
  // 3 tiles would run in two rounds with 2-4 m-tiles; with one m-tile, two per
  // CU, the six-tile workgroups measured 2 % faster at M = 1 and 13)
  int nt1 = inter / 8;
  p.T1 = 1;
  for (int t : {6, 3, 2}) {
    if (nt1 % t == 0 && nt1 / t >= 192 && (t < 6 || (prec == kFP4 && p.MT <= 4))) { p.T1 = t; break; }
  }
  p.ngroups1 = nt1 / p.T1;
  p.namax = p.ngroups1;
  pick_down(p);
  const bool many = M >= kLgMinRows;
  p.lg1 = many && (prec == kFP8 || prec == kFP8DownBF16) && nt1 % kLgRT1 == 0 && hidden >= 256;
  if (p.lg1) {
    p.MT = kLgRM;
    p.n_mblocks = (M + 16 * kLgRM - 1) / (16 * kLgRM);
    p.T1 = kLgRT1;
    p.ngroups1 = nt1 / kLgRT1;
    p.namax = p.ngroups1 * kLgWT1;
  }
  p.lg2 = many && prec == kFP8DownBF16 && (hidden / 16) % kLgRT2 == 0 && inter >= 256;
  if (p.lg2) {
    p.MT2 = kLgRM2;
    p.T2 = kLgRT2;
    p.n_mb2 = (M + 16 * kLgRM2 - 1) / (16 * kLgRM2);
    p.ngroups2 = hidden / 16 / kLgRT2;
  }
  const int rows1 = p.n_mblocks * 16 * p.MT, rows2 = p.n_mb2 * 16 * p.MT2;
  p.Mpad = rows1 > rows2 ? rows1 : rows2;
  // workspace
  size_t Mp = p.Mpad;
  size_t o = 0;
  p.off_xq = o;   o = align_up(o + Mp * hidden * (p.lg1 ? 2 : 1));   // E4M3 codes, or their fp16 values
  p.off_sx = o;   o = align_up(o + Mp * 4);
  p.off_amax = o; o = align_up(o + (size_t)p.namax * Mp * 4);   // partial row maxima of |h|
  p.off_h32 = o;  o = align_up(o + (prec == kFP8DownBF16 ? 0 : Mp * inter * 4));   // [inter / 8][Mpad][8]
  p.off_hq = o;   o = align_up(o + (prec == kFP8DownBF16 ? 0 : Mp * inter));
  p.off_hb = o;   o = align_up(o + (prec == kFP8DownBF16 ? Mp * inter * 2 : 0));
  p.off_sh = o;   o = align_up(o + Mp * 4);
  p.off_amaxg = o; o = align_up(o + (size_t)kAmaxSlots * Mp * 4);
  p.off_sync = o; o = align_up(o + (size_t)kSyncWords * 4);
  p.total = o;
  return p;
}

}  // namespace ocq
