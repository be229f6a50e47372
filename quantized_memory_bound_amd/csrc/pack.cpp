// Host-side weight quantizer and packer (no GPU involved).
//
// Quantization rules ("OCRia 推理栈：单卡 B200 提速近 10 倍", section "Reducing
// the data moved: workload-aware quantization": FP8 halves the bytes per
// weight; layers mix BF16, FP8 and NVFP4; sensitive layers stay BF16):
//   FP8   per output row: s = fl32(amax / 448), code = E4M3(fl32(w / s)).
//   BF16  round to nearest even.
//   NVFP4 S = fl32(amax / 2688) per tensor; per 16 consecutive inputs of a row
//         sb = E4M3(fl32(amax_b / (6 S))); code = E2M1(fl32(w / (dec(sb) S))).
//   Zero scale -> all codes 0.  Encoders: nearest, ties to even, saturating.
// The codes are then written in the fragment order described in ocq_layout.h.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "ocq_internal.h"

namespace ocq {

// ---- scalar codecs (host) --------------------------------------------------

uint8_t host_enc_e4m3(float v) {
  uint32_t u;
  std::memcpy(&u, &v, 4);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t ua = u & 0x7FFFFFFFu;
  float a;
  std::memcpy(&a, &ua, 4);
  uint32_t c;
  if (a >= 448.0f) {
    c = 0x7E;                                     // saturate at 448
  } else if (a < 0.015625f) {                     // below 2^-6: subnormal grid of 2^-9
    c = (uint32_t)std::nearbyint(a * 512.0f);     // exact scaling; ties to even (default mode)
  } else {
    uint32_t e = (ua >> 23) - 127 + 7;            // biased E4M3 exponent, 1..15
    uint32_t m = ua & 0x7FFFFFu;
    uint32_t q = (m + 0x7FFFFu + ((m >> 20) & 1u)) >> 20;   // 3-bit mantissa, RNE
    c = (e << 3) + q;                             // q == 8 carries into the exponent
  }
  return (uint8_t)(sign | c);
}

float host_dec_e4m3(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  float mag = e == 0 ? std::ldexp((float)m, -9) : std::ldexp(1.0f + m / 8.0f, e - 7);
  return s ? -mag : mag;
}

uint8_t host_enc_e2m1(float v) {
  uint32_t u;
  std::memcpy(&u, &v, 4);
  uint8_t sign = (u >> 31) ? 0x8 : 0x0;
  float a = std::fabs(v);
  // thresholds are the midpoints of 0,.5,1,1.5,2,3,4,6; '>' where the lower
  // neighbour has the even code, '>=' where the upper one has
  uint8_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
              (a >= 3.5f) + (a > 5.0f);
  return (uint8_t)(sign | c);
}

uint16_t host_bf16_rne(float v) {
  uint32_t u;
  std::memcpy(&u, &v, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---- plain-layout quantizers -------------------------------------------------

struct FP8Plain { std::vector<uint8_t> codes; std::vector<float> scales; };
struct FP4Plain { std::vector<uint8_t> codes; std::vector<uint8_t> bscales; float S; };

static FP8Plain quant_fp8_rows(const float* w, size_t rows, size_t cols) {
  FP8Plain r;
  r.codes.assign(rows * cols, 0);
  r.scales.assign(rows, 0.0f);
  for (size_t n = 0; n < rows; ++n) {
    const float* row = w + n * cols;
    float amax = 0.0f;
    for (size_t k = 0; k < cols; ++k) amax = std::fmax(amax, std::fabs(row[k]));
    float s = amax / 448.0f;
    r.scales[n] = s;
    if (s > 0.0f)
      for (size_t k = 0; k < cols; ++k) r.codes[n * cols + k] = host_enc_e4m3(row[k] / s);
  }
  return r;
}

static FP4Plain quant_nvfp4(const float* w, size_t rows, size_t cols) {
  FP4Plain r;
  size_t nb = cols / 16;
  r.codes.assign(rows * cols, 0);
  r.bscales.assign(rows * nb, 0);
  float amax = 0.0f;
  for (size_t i = 0; i < rows * cols; ++i) amax = std::fmax(amax, std::fabs(w[i]));
  r.S = amax / 2688.0f;                               // 448 * 6
  if (!(r.S > 0.0f)) return r;
  double six_S = 6.0 * (double)r.S;                   // exact in binary64
  for (size_t n = 0; n < rows; ++n) {
    for (size_t b = 0; b < nb; ++b) {
      const float* blk = w + n * cols + b * 16;
      float ab = 0.0f;
      for (int j = 0; j < 16; ++j) ab = std::fmax(ab, std::fabs(blk[j]));
      uint8_t sb = host_enc_e4m3((float)((double)ab / six_S));
      r.bscales[n * nb + b] = sb;
      double d = (double)host_dec_e4m3(sb) * (double)r.S;   // exact product
      if (d > 0.0)
        for (int j = 0; j < 16; ++j) r.codes[n * cols + b * 16 + j] = host_enc_e2m1((float)((double)blk[j] / d));
    }
  }
  return r;
}

// ---- fragment writers ----------------------------------------------------------

// source row of tile row rr in tile t: interleaved gate/up or plain
static inline size_t src_row(bool interleaved, size_t t, int rr, size_t half_rows, int* which) {
  if (!interleaved) { *which = 0; return t * 16 + rr; }
  *which = rr < 8 ? 0 : 1;
  return t * 8 + (rr & 7);
  (void)half_rows;
}

static void write_fp8_frags(uint8_t* dst, const uint8_t* a, const uint8_t* b, bool inter, size_t ntiles,
                            size_t cols) {
  size_t C = cols / kChunk;
  for (size_t t = 0; t < ntiles; ++t)
    for (size_t c = 0; c < C; ++c)
      for (int l = 0; l < 64; ++l) {
        int g = l >> 4, r = l & 15, which;
        size_t row = src_row(inter, t, r, 0, &which);
        const uint8_t* src = (which ? b : a) + row * cols + c * kChunk + 32 * g;
        uint8_t* base = dst + (t * C + c) * 2048;
        for (int j = 0; j < 32; ++j) base[((j >> 4) * 64 + l) * 16 + (j & 15)] = src[j];
      }
}

static void write_bf16_frags(uint8_t* dst, const uint16_t* a, size_t ntiles, size_t cols) {
  size_t C = cols / kChunk;
  for (size_t t = 0; t < ntiles; ++t)
    for (size_t c = 0; c < C; ++c)
      for (int l = 0; l < 64; ++l) {
        int g = l >> 4, r = l & 15;
        const uint16_t* src = a + (t * 16 + r) * cols + c * kChunk + 32 * g;
        uint8_t* base = dst + (t * C + c) * 4096;
        for (int j = 0; j < 32; ++j) std::memcpy(base + ((j >> 3) * 64 + l) * 16 + 2 * (j & 7), src + j, 2);
      }
}

static void write_fp4_frags(uint8_t* dst, uint8_t* bdst, const FP4Plain& a, const FP4Plain* b, bool inter,
                            size_t ntiles, size_t cols) {
  size_t C = cols / kChunk, CG = chunk_groups(cols), nb = cols / 16;
  for (size_t t = 0; t < ntiles; ++t)
    for (size_t c = 0; c < C; ++c)
      for (int l = 0; l < 64; ++l) {
        int g = l >> 4, r = l & 15, which;
        size_t row = src_row(inter, t, r, 0, &which);
        const FP4Plain& P = which ? *b : a;
        const uint8_t* src = P.codes.data() + row * cols + c * kChunk + 32 * g;
        uint8_t* base = dst + (t * C + c) * 1024 + l * 16;
        for (int j = 0; j < 16; ++j) base[j] = (uint8_t)((src[2 * j] & 0xF) | ((src[2 * j + 1] & 0xF) << 4));
        uint8_t* sb = bdst + (t * CG + c / 8) * 1024 + l * 16 + 2 * (c % 8);
        for (int bb = 0; bb < 2; ++bb) sb[bb] = P.bscales[row * nb + 8 * c + 2 * g + bb];
      }
}

static void read_fp8_frags(const uint8_t* src, uint8_t* a, uint8_t* b, bool inter, size_t ntiles, size_t cols) {
  size_t C = cols / kChunk;
  for (size_t t = 0; t < ntiles; ++t)
    for (size_t c = 0; c < C; ++c)
      for (int l = 0; l < 64; ++l) {
        int g = l >> 4, r = l & 15, which;
        size_t row = src_row(inter, t, r, 0, &which);
        uint8_t* d = (which ? b : a);
        if (!d) continue;
        d += row * cols + c * kChunk + 32 * g;
        const uint8_t* base = src + (t * C + c) * 2048;
        for (int j = 0; j < 32; ++j) d[j] = base[((j >> 4) * 64 + l) * 16 + (j & 15)];
      }
}

// ---- entry points (host) ----------------------------------------------------

ocq_status pack_host(const float* wg, const float* wu, const float* wd, int hidden, int inter, int prec,
                     const float* smooth, uint8_t* out, size_t out_bytes) {
  BlobLayout L = blob_layout(hidden, inter, prec);
  if (out_bytes < L.total) return set_error(OCQ_ERR_BUFFER_TOO_SMALL, "packed buffer smaller than ocq_packed_bytes");
  size_t H = hidden, I = inter;
  // per-input-channel smoothing: W'[n][k] = fl32(W[n][k] s[k]) for gate and up,
  // x'[k] = fl32(x[k] fl32(1 / s[k])) at run time
  std::vector<float> sg, su;
  if (smooth) {
    for (size_t k = 0; k < H; ++k)
      if (!(smooth[k] > 0.0f) || !std::isfinite(smooth[k]))
        return set_error(OCQ_ERR_INVALID_ARG, "smoothing factors must be finite and > 0");
    sg.resize(I * H);
    su.resize(I * H);
    for (size_t n = 0; n < I; ++n)
      for (size_t k = 0; k < H; ++k) {
        sg[n * H + k] = wg[n * H + k] * smooth[k];
        su[n * H + k] = wu[n * H + k] * smooth[k];
      }
    wg = sg.data();
    wu = su.data();
  }
  std::memset(out, 0, L.total);
  BlobHeader hd{};
  std::memcpy(hd.magic, kBlobMagic, 8);
  hd.version = kBlobVersion;
  hd.hidden = hidden; hd.inter = inter; hd.prec_mode = prec;
  hd.off_gu_codes = L.off_gu_codes; hd.off_gu_scales = L.off_gu_scales; hd.off_gu_bscales = L.off_gu_bscales;
  hd.off_dn_codes = L.off_dn_codes; hd.off_dn_scales = L.off_dn_scales; hd.off_dn_bscales = L.off_dn_bscales;
  hd.off_xmul = L.off_xmul;
  hd.total_bytes = L.total;
  float* xmul = reinterpret_cast<float*>(out + L.off_xmul);
  for (size_t k = 0; k < H; ++k) xmul[k] = smooth ? 1.0f / smooth[k] : 1.0f;
  if (L.gu == kWFP8) {
    FP8Plain g = quant_fp8_rows(wg, I, H), u = quant_fp8_rows(wu, I, H);
    write_fp8_frags(out + L.off_gu_codes, g.codes.data(), u.codes.data(), true, I / 8, H);
    float* sc = reinterpret_cast<float*>(out + L.off_gu_scales);
    std::memcpy(sc, g.scales.data(), I * 4);
    std::memcpy(sc + I, u.scales.data(), I * 4);
  } else {
    FP4Plain g = quant_nvfp4(wg, I, H), u = quant_nvfp4(wu, I, H);
    write_fp4_frags(out + L.off_gu_codes, out + L.off_gu_bscales, g, &u, true, I / 8, H);
    hd.s_gate = g.S; hd.s_up = u.S;
  }
  if (L.dn == kWFP8) {
    FP8Plain d = quant_fp8_rows(wd, H, I);
    write_fp8_frags(out + L.off_dn_codes, d.codes.data(), nullptr, false, H / 16, I);
    std::memcpy(out + L.off_dn_scales, d.scales.data(), H * 4);
  } else if (L.dn == kWBF16) {
    std::vector<uint16_t> b(H * I);
    for (size_t i = 0; i < H * I; ++i) b[i] = host_bf16_rne(wd[i]);
    write_bf16_frags(out + L.off_dn_codes, b.data(), H / 16, I);
  } else {
    FP4Plain d = quant_nvfp4(wd, H, I);
    write_fp4_frags(out + L.off_dn_codes, out + L.off_dn_bscales, d, nullptr, false, H / 16, I);
    hd.s_down = d.S;
  }
  std::memcpy(out, &hd, sizeof(hd));
  return OCQ_OK;
}

// Smoothing factors from calibration activations (SmoothQuant's rule):
// s[k] = amax_x[k]^alpha / amax_w[k]^(1 - alpha), amax_x over the calibration
// rows of x, amax_w over the rows of both gate and up; evaluated in double and
// rounded once to float; 1 where either maximum is 0; clamped to [2^-20, 2^20].
ocq_status calibrate_host(const uint16_t* x_bf16, int rows, int hidden, const float* wg, const float* wu, int inter,
                          float alpha, float* s_out) {
  const size_t H = hidden, I = inter;
  std::vector<float> ax(H, 0.0f), aw(H, 0.0f);
  for (size_t t = 0; t < (size_t)rows; ++t)
    for (size_t k = 0; k < H; ++k) {
      uint32_t b = (uint32_t)x_bf16[t * H + k] << 16;
      float v;
      std::memcpy(&v, &b, 4);
      ax[k] = std::max(ax[k], std::fabs(v));
    }
  for (size_t n = 0; n < I; ++n)
    for (size_t k = 0; k < H; ++k)
      aw[k] = std::max(aw[k], std::max(std::fabs(wg[n * H + k]), std::fabs(wu[n * H + k])));
  for (size_t k = 0; k < H; ++k) {
    double v = 1.0;
    if (ax[k] > 0.0f && aw[k] > 0.0f) v = std::pow((double)ax[k], (double)alpha) / std::pow((double)aw[k], 1.0 - alpha);
    v = std::min(std::max(v, 0x1p-20), 0x1p20);
    s_out[k] = (float)v;
  }
  return OCQ_OK;
}

ocq_status unpack_host(const uint8_t* blob, size_t bytes, int which, void* codes_out, void* scales_out,
                       float* tensor_scale_out) {
  if (bytes < sizeof(BlobHeader)) return set_error(OCQ_ERR_BUFFER_TOO_SMALL, "blob smaller than its header");
  BlobHeader hd;
  std::memcpy(&hd, blob, sizeof(hd));
  if (std::memcmp(hd.magic, kBlobMagic, 8) != 0 || hd.version != kBlobVersion)
    return set_error(OCQ_ERR_BAD_BLOB, "bad blob magic or version");
  if (!shape_ok(hd.hidden, hd.inter) || hd.prec_mode < 0 || hd.prec_mode > 2)
    return set_error(OCQ_ERR_BAD_BLOB, "blob header holds an invalid shape or mode");
  BlobLayout L = blob_layout(hd.hidden, hd.inter, hd.prec_mode);
  if (bytes < L.total) return set_error(OCQ_ERR_BUFFER_TOO_SMALL, "blob smaller than its layout");
  size_t H = hd.hidden, I = hd.inter;
  if (which == 3) {   // the x multiplier (1 / smoothing factor per input channel)
    if (!scales_out) return set_error(OCQ_ERR_INVALID_ARG, "which = 3 needs scales_out");
    std::memcpy(scales_out, blob + L.off_xmul, H * 4);
    if (tensor_scale_out) *tensor_scale_out = 0.0f;
    return OCQ_OK;
  }
  if (which < 0 || which > 2 || !codes_out) return set_error(OCQ_ERR_INVALID_ARG, "which must be 0..3, codes_out non-null");
  bool gu = which < 2;
  WeightKind k = gu ? L.gu : L.dn;
  size_t rows = gu ? I : H, cols = gu ? H : I;
  if (tensor_scale_out) *tensor_scale_out = 0.0f;
  if (k == kWFP8) {
    if (gu) {
      read_fp8_frags(blob + L.off_gu_codes, which == 0 ? (uint8_t*)codes_out : nullptr,
                     which == 1 ? (uint8_t*)codes_out : nullptr, true, I / 8, H);
      if (scales_out) std::memcpy(scales_out, blob + L.off_gu_scales + (which == 1 ? I * 4 : 0), I * 4);
    } else {
      read_fp8_frags(blob + L.off_dn_codes, (uint8_t*)codes_out, nullptr, false, H / 16, I);
      if (scales_out) std::memcpy(scales_out, blob + L.off_dn_scales, H * 4);
    }
  } else if (k == kWBF16) {
    size_t C = cols / kChunk;
    uint16_t* d = (uint16_t*)codes_out;
    const uint8_t* src = blob + L.off_dn_codes;
    for (size_t t = 0; t < rows / 16; ++t)
      for (size_t c = 0; c < C; ++c)
        for (int l = 0; l < 64; ++l) {
          int g = l >> 4, r = l & 15;
          for (int j = 0; j < 32; ++j)
            std::memcpy(d + (t * 16 + r) * cols + c * kChunk + 32 * g + j,
                        src + (t * C + c) * 4096 + ((j >> 3) * 64 + l) * 16 + 2 * (j & 7), 2);
        }
  } else {
    size_t C = cols / kChunk, CG = chunk_groups(cols), nb = cols / 16;
    const uint8_t* src = blob + (gu ? L.off_gu_codes : L.off_dn_codes);
    const uint8_t* bsrc = blob + (gu ? L.off_gu_bscales : L.off_dn_bscales);
    uint8_t* d = (uint8_t*)codes_out;
    uint8_t* sbo = (uint8_t*)scales_out;
    size_t ntiles = gu ? I / 8 : H / 16;
    for (size_t t = 0; t < ntiles; ++t)
      for (size_t c = 0; c < C; ++c)
        for (int l = 0; l < 64; ++l) {
          int g = l >> 4, r = l & 15, w;
          size_t row = src_row(gu, t, r, 0, &w);
          if (gu && w != which) continue;
          const uint8_t* base = src + (t * C + c) * 1024 + l * 16;
          for (int j = 0; j < 32; ++j)
            d[row * cols + c * kChunk + 32 * g + j] = (base[j / 2] >> (4 * (j & 1))) & 0xF;
          if (sbo) {
            const uint8_t* sb = bsrc + (t * CG + c / 8) * 1024 + l * 16 + 2 * (c % 8);
            sbo[row * nb + 8 * c + 2 * g] = sb[0];
            sbo[row * nb + 8 * c + 2 * g + 1] = sb[1];
          }
        }
    if (tensor_scale_out) *tensor_scale_out = which == 0 ? hd.s_gate : which == 1 ? hd.s_up : hd.s_down;
  }
  return OCQ_OK;
}

}  // namespace ocq
