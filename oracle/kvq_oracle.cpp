// kvq_oracle.cpp — plain, slow, single-threaded CPU oracle for the block-quantized
// KV cache and single-query decode attention.
//
// TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or call this
// file: only the test suite, the smoke check and the benchmark's CPU-baseline leg do.
// It shares no code, header, table or helper with the HIP library; it needs libc/libm.
//
// Sources (three web pages on DeepSeek-R1 inference optimisation):
//   [Pg1] "第一章：DeepSeek R1推理模型性能跃迁全景概览" (aicoding.csdn.net), §2.2
//         "KV Cache动态压缩策略": INT8 KV codes whose scales come from a pre-pass that
//         takes the extreme values of each chunk.
//   [Pg2] "DeepSeek-R1推理延迟骤降41.8%？独家披露3类硬件感知调度策略" (jsqmd.com), §2.1
//         "基于A100显存带宽瓶颈的KV Cache分块压缩策略", sub-section "分块量化压缩设计"
//         and its quantize_block generator: 4-bit codes, one scale per 64-token block
//         equal to the block's absolute maximum divided by 7.5, codes rounded and
//         clamped to [-8, 7].
//   [Pg3] "DeepSeek R1性能优化有哪些技巧" (ddd.cn), §一 "精度与量化": an FP8 KV cache.
//   Attention itself is not written out on the pages; the plain definition used here is
//   textbook scaled dot-product attention (Vaswani et al., 2017) over the dequantized
//   cache, for one query token.
//
// Readings taken where the pages are silent or garbled:
//   * a block is 64 consecutive tokens of ONE (sequence, head) row, all head_dim
//     channels together (the listing flattens heads, the prose says per block);
//   * rounding is round-half-to-even (the listing's torch.round), never half-away;
//   * all scale arithmetic is IEEE binary32 with round-to-nearest division;
//   * the INT8 scheme is asymmetric per 64-token chunk: s = (max - min) / 255,
//     zp = round(-min / s), code = clamp(round(x / s) + zp, 0, 255), the integer
//     zero-point added after rounding; -0.0 zero-points are stored as +0.0;
//   * degenerate blocks: int4 absmax 0 -> s = 0, codes 0; uint8 with max == min == c:
//     c == 0 -> s = 0, zp = 0, codes 0; otherwise the range is widened to include 0;
//   * int4 packing: each code c is stored as the offset-binary nibble c + 8 (0..15);
//     byte k of a token's row holds channel 2k in bits 0-3 and channel 2k+1 in bits 4-7;
//   * bytes of tokens at or past the length inside the last block are 0;
//   * cache layout: codes [B][H][max_blocks][64][D/2 or D] bytes, scales and zero
//     points [B][H][max_blocks] binary32;
//   * a row of length 0 attends to nothing; its output is defined as all zeros;
//   * the FP8 scheme (the pages name FP8 KV without its scaling) mirrors the 4-bit
//     one: per 64-token block s = absmax / 448 (448 = the largest finite E4M3
//     magnitude), code = the E4M3 value nearest to x / s (ties to even mantissa, the
//     sign kept, so -0 and negative values that round to zero give 0x80), 0 when s = 0;
//     one byte per channel, [token][channel].
//
// Build: g++ -std=c++17 -O2 -fPIC -shared -ffp-contract=off (no fast-math), x86-64 SSE
// arithmetic (binary32 operations round once, to nearest-even).

#include <cfenv>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

constexpr int kBlock = 64;  // tokens per quantization block ([Pg2] §2.1, block_size=64)

// IEEE 754 binary16 -> value, straight from the format definition: 1 sign bit,
// 5 exponent bits (bias 15), 10 fraction bits; exponent 0 encodes f * 2^-24.
// Every binary16 value is exactly representable in binary32 and binary64.
double half_value(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int e = (h >> 10) & 0x1F;
  const int f = h & 0x3FF;
  double mag;
  if (e == 0) {
    mag = std::ldexp(static_cast<double>(f), -24);
  } else if (e == 31) {
    mag = f ? NAN : INFINITY;
  } else {
    mag = std::ldexp(static_cast<double>(1024 + f), e - 25);
  }
  return sign ? -mag : mag;
}

float half_to_f32(uint16_t h) { return static_cast<float>(half_value(h)); }

// Round to nearest integer, ties to even (the default FE_TONEAREST mode).
float round_half_even(float v) { return std::nearbyint(v); }

struct RowIn {  // one (sequence, head) row of fp16 input: element (t, d) at p[t*st + d]
  const uint16_t* p;
  int64_t st;
};

// ---- 4-bit symmetric block ([Pg2] §2.1) -------------------------------------------
// codes: 64 * D/2 bytes for this block; ntok valid tokens starting at token `first`.
void quantize_block_int4(RowIn x, int first, int ntok, int D, uint8_t* codes,
                         float* scale, float* zero) {
  // step 1: the block's absolute maximum over its valid tokens and all channels
  float a = 0.0f;
  for (int t = 0; t < ntok; ++t)
    for (int d = 0; d < D; ++d) {
      const float v = std::fabs(half_to_f32(x.p[(first + t) * x.st + d]));
      if (v > a) a = v;
    }
  // step 2: scale = absmax / 7.5 (one binary32 division)
  const float s = (a == 0.0f) ? 0.0f : a / 7.5f;
  // step 3: code = clamp(round(x / s), -8, 7) (0 when s = 0), stored as c + 8, two per byte
  std::memset(codes, 0, static_cast<size_t>(kBlock) * (D / 2));
  for (int t = 0; t < ntok; ++t)
    for (int d = 0; d < D; ++d) {
      int c = 0;
      if (s != 0.0f) {
        const float q = half_to_f32(x.p[(first + t) * x.st + d]) / s;
        c = static_cast<int>(round_half_even(q));
        if (c < -8) c = -8;
        if (c > 7) c = 7;
      }
      const uint8_t nib = static_cast<uint8_t>(c + 8);
      uint8_t& byte = codes[t * (D / 2) + d / 2];
      byte |= (d % 2 == 0) ? nib : static_cast<uint8_t>(nib << 4);
    }
  *scale = s;
  *zero = 0.0f;
}

// ---- 8-bit asymmetric chunk ([Pg1] §2.2, per-chunk extremes) -----------------------
void quantize_block_uint8(RowIn x, int first, int ntok, int D, uint8_t* codes,
                          float* scale, float* zero) {
  // step 1: the chunk's minimum and maximum
  float mn = INFINITY, mx = -INFINITY;
  for (int t = 0; t < ntok; ++t)
    for (int d = 0; d < D; ++d) {
      const float v = half_to_f32(x.p[(first + t) * x.st + d]);
      if (v < mn) mn = v;
      if (v > mx) mx = v;
    }
  std::memset(codes, 0, static_cast<size_t>(kBlock) * D);
  if (mx == mn) {  // degenerate chunk: every element equal
    if (mx == 0.0f) {
      *scale = 0.0f;
      *zero = 0.0f;
      return;
    }
    if (mn > 0.0f) mn = 0.0f;
    if (mx < 0.0f) mx = 0.0f;
  }
  // step 2: s = (max - min) / 255, two binary32 operations in that order
  const float range = mx - mn;
  const float s = range / 255.0f;
  // step 3: zero point = round(-min / s), kept as +0.0 when it rounds to zero
  const float zp = round_half_even(-mn / s) + 0.0f;
  const int zpi = static_cast<int>(zp);
  // step 4: code = clamp(round(x / s) + zp, 0, 255), integer add after rounding
  for (int t = 0; t < ntok; ++t)
    for (int d = 0; d < D; ++d) {
      const float q = half_to_f32(x.p[(first + t) * x.st + d]) / s;
      int c = static_cast<int>(round_half_even(q)) + zpi;
      if (c < 0) c = 0;
      if (c > 255) c = 255;
      codes[t * D + d] = static_cast<uint8_t>(c);
    }
  *scale = s;
  *zero = zp;
}

// ---- 8-bit floating-point block: FP8 E4M3 ([Pg3] §一) ------------------------------
// E4M3 ("fn" variant of the OCP 8-bit floating-point formats): 1 sign bit, 4 exponent
// bits with bias 7, 3 fraction bits. Exponent field 0 encodes (m/8) * 2^-6; otherwise
// (1 + m/8) * 2^(e-7). S.1111.111 is NaN, there are no infinities, so the largest
// finite magnitude is 1.75 * 2^8 = 448 (code 0x7E).
double e4m3_value(uint8_t c) {
  const int e = (c >> 3) & 15, m = c & 7;
  const double v = (e == 0) ? std::ldexp(m / 8.0, -6) : std::ldexp(1.0 + m / 8.0, e - 7);
  return (c & 0x80) ? -v : v;
}

// The code of the finite E4M3 value nearest to q (|q| finite): the 127 non-negative
// finite codes are searched in order, a tie goes to the even code (whose fraction is
// even), and the sign bit is q's. Beyond 448 the nearest finite value is 448.
uint8_t e4m3_code(float q) {
  const double a = std::fabs(static_cast<double>(q));
  int best = 0;
  double best_d = a;  // distance to code 0 (value 0)
  for (int c = 1; c <= 0x7E; ++c) {
    const double d = std::fabs(e4m3_value(static_cast<uint8_t>(c)) - a);
    if (d < best_d || (d == best_d && c % 2 == 0)) {
      best = c;
      best_d = d;
    }
  }
  return static_cast<uint8_t>(best | (std::signbit(q) ? 0x80 : 0));
}

void quantize_block_fp8(RowIn x, int first, int ntok, int D, uint8_t* codes, float* scale,
                        float* zero) {
  // step 1: the block's absolute maximum over its valid tokens and all channels
  float a = 0.0f;
  for (int t = 0; t < ntok; ++t)
    for (int d = 0; d < D; ++d) {
      const float v = std::fabs(half_to_f32(x.p[(first + t) * x.st + d]));
      if (v > a) a = v;
    }
  // step 2: scale = absmax / 448 (one binary32 division)
  const float s = (a == 0.0f) ? 0.0f : a / 448.0f;
  // step 3: code = nearest E4M3 value of x / s (0 when s = 0), one byte per channel
  std::memset(codes, 0, static_cast<size_t>(kBlock) * D);
  for (int t = 0; t < ntok; ++t)
    for (int d = 0; d < D; ++d)
      codes[t * D + d] =
          (s == 0.0f) ? 0 : e4m3_code(half_to_f32(x.p[(first + t) * x.st + d]) / s);
  *scale = s;
  *zero = 0.0f;
}

void quantize_block(int scheme, RowIn x, int first, int ntok, int D, uint8_t* codes,
                    float* scale, float* zero) {
  if (scheme == 0)
    quantize_block_int4(x, first, ntok, D, codes, scale, zero);
  else if (scheme == 1)
    quantize_block_uint8(x, first, ntok, D, codes, scale, zero);
  else
    quantize_block_fp8(x, first, ntok, D, codes, scale, zero);
}

int row_bytes(int scheme, int D) { return scheme == 0 ? D / 2 : D; }

bool shape_ok(int scheme, int B, int H, int D, int max_blocks) {
  return (scheme == 0 || scheme == 1 || scheme == 2) && B > 0 && H > 0 && D > 0 &&
         D % 2 == 0 && max_blocks > 0;
}

// Dequantized value of channel d of token t in block j of row r (binary64, exact).
double dequant(int scheme, int D, int max_blocks, const uint8_t* codes, const float* scale,
               const float* zero, int64_t r, int t, int d) {
  const int j = t / kBlock, tt = t % kBlock;
  const int64_t blk = r * max_blocks + j;
  const uint8_t* row = codes + (blk * kBlock + tt) * static_cast<int64_t>(row_bytes(scheme, D));
  const double s = static_cast<double>(scale[blk]);
  if (scheme == 0) {
    const int nib = (d % 2 == 0) ? (row[d / 2] & 0x0F) : (row[d / 2] >> 4);
    return static_cast<double>(nib - 8) * s;  // offset-binary nibble
  }
  if (scheme == 2) return e4m3_value(row[d]) * s;
  return (static_cast<double>(row[d]) - static_cast<double>(zero[blk])) * s;
}

}  // namespace

extern "C" {

int oracle_version(void) { return 2; }

// FP8 E4M3 codes of binary32 values (nearest, ties to even, saturating) and the values
// of codes (binary64, exact).
void oracle_e4m3_code(const float* in, uint8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_code(in[i]);
}
void oracle_e4m3_value(const uint8_t* in, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_value(in[i]);
}

// binary16 bit patterns -> binary32 values (exact).
void oracle_half_to_float(const uint16_t* in, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = half_to_f32(in[i]);
}

// Quantizes every block [0, ceil(len_b/64)) of every row (b, h) of k and v.
// k, v: binary16, element (b, t, h, d) at base[b*sb + t*st + h*sh + d].
// Outputs use the cache layout in the header comment; blocks at or past
// ceil(len_b/64) are left untouched. Returns 0, or -1 on a bad shape or length.
int oracle_quantize_cache(int scheme, int B, int H, int D, int max_blocks,
                          const uint16_t* k, const uint16_t* v, int64_t sb, int64_t st,
                          int64_t sh, const int32_t* lens, uint8_t* k_codes,
                          uint8_t* v_codes, float* k_scale, float* v_scale, float* k_zero,
                          float* v_zero) {
  if (!shape_ok(scheme, B, H, D, max_blocks)) return -1;
  if (scheme == 1 && (!k_zero || !v_zero)) return -1;
  if (std::fegetround() != FE_TONEAREST) return -1;
  const int64_t rb = row_bytes(scheme, D);
  for (int b = 0; b < B; ++b) {
    const int len = lens[b];
    if (len < 0 || len > max_blocks * kBlock) return -1;
    const int nb = (len + kBlock - 1) / kBlock;
    for (int h = 0; h < H; ++h) {
      const int64_t r = static_cast<int64_t>(b) * H + h;
      for (int tensor = 0; tensor < 2; ++tensor) {
        const uint16_t* src = tensor == 0 ? k : v;
        uint8_t* codes = tensor == 0 ? k_codes : v_codes;
        float* scale = tensor == 0 ? k_scale : v_scale;
        float* zero = tensor == 0 ? k_zero : v_zero;
        RowIn x{src + b * sb + h * sh, st};
        for (int j = 0; j < nb; ++j) {
          const int first = j * kBlock;
          const int ntok = (len - first < kBlock) ? len - first : kBlock;
          const int64_t blk = r * max_blocks + j;
          uint8_t* out = codes + blk * kBlock * rb;
          float zdummy;
          float* zp = zero ? zero + blk : &zdummy;
          quantize_block(scheme, x, first, ntok, D, out, scale + blk, zp);
        }
      }
    }
  }
  return 0;
}

// Appending one token to a row is defined as re-quantizing that row's tail block over
// its valid tokens after the append. This re-runs the block quantizer on block
// (new_len-1)/64 of every row, reading the full fp16 history (same layout as above).
int oracle_append(int scheme, int B, int H, int D, int max_blocks, const uint16_t* k,
                  const uint16_t* v, int64_t sb, int64_t st, int64_t sh,
                  const int32_t* new_lens, uint8_t* k_codes, uint8_t* v_codes,
                  float* k_scale, float* v_scale, float* k_zero, float* v_zero) {
  if (!shape_ok(scheme, B, H, D, max_blocks)) return -1;
  if (scheme == 1 && (!k_zero || !v_zero)) return -1;
  if (std::fegetround() != FE_TONEAREST) return -1;
  const int64_t rb = row_bytes(scheme, D);
  for (int b = 0; b < B; ++b) {
    const int len = new_lens[b];
    if (len < 1 || len > max_blocks * kBlock) return -1;
    const int j = (len - 1) / kBlock;
    const int first = j * kBlock;
    const int ntok = len - first;
    for (int h = 0; h < H; ++h) {
      const int64_t blk = (static_cast<int64_t>(b) * H + h) * max_blocks + j;
      for (int tensor = 0; tensor < 2; ++tensor) {
        const uint16_t* src = tensor == 0 ? k : v;
        RowIn x{src + b * sb + h * sh, st};
        uint8_t* out = (tensor == 0 ? k_codes : v_codes) + blk * kBlock * rb;
        float* scale = (tensor == 0 ? k_scale : v_scale) + blk;
        float* zero = tensor == 0 ? k_zero : v_zero;
        float zdummy;
        float* zp = zero ? zero + blk : &zdummy;
        quantize_block(scheme, x, first, ntok, D, out, scale, zp);
      }
    }
  }
  return 0;
}

// Decode attention for rows [row_begin, row_end) of the flattened (b, h) index, in
// binary64 over the dequantized cache:
//   s_t = sm * sum_d q_d * K^_{t,d},  p_t = exp(s_t - max_t s_t),
//   o_d = sum_t p_t * V^_{t,d} / sum_t p_t,   t < len_b.
// q: binary16 [B][H][D]; out: binary64 [B][H][D] (only the requested rows written).
int oracle_attention(int scheme, int B, int H, int D, int max_blocks,
                     const uint8_t* k_codes, const uint8_t* v_codes, const float* k_scale,
                     const float* v_scale, const float* k_zero, const float* v_zero,
                     const int32_t* lens, const uint16_t* q, double sm_scale,
                     int64_t row_begin, int64_t row_end, double* out) {
  if (!shape_ok(scheme, B, H, D, max_blocks)) return -1;
  if (scheme == 1 && (!k_zero || !v_zero)) return -1;
  const int64_t rows = static_cast<int64_t>(B) * H;
  if (row_begin < 0 || row_end > rows || row_begin > row_end) return -1;
  for (int64_t r = row_begin; r < row_end; ++r) {
    const int b = static_cast<int>(r / H);
    const int len = lens[b];
    if (len < 0 || len > max_blocks * kBlock) return -1;
    double* o = out + r * D;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    if (len == 0) continue;
    std::vector<double> qd(D);
    for (int d = 0; d < D; ++d) qd[d] = half_value(q[r * D + d]);
    // pass 1: scores and their maximum
    std::vector<double> s(len);
    double m = -INFINITY;
    for (int t = 0; t < len; ++t) {
      double acc = 0.0;
      for (int d = 0; d < D; ++d)
        acc += qd[d] * dequant(scheme, D, max_blocks, k_codes, k_scale, k_zero, r, t, d);
      s[t] = sm_scale * acc;
      if (s[t] > m) m = s[t];
    }
    // pass 2: normalized weights and the weighted sum of V
    double l = 0.0;
    for (int t = 0; t < len; ++t) {
      const double p = std::exp(s[t] - m);
      l += p;
      for (int d = 0; d < D; ++d)
        o[d] += p * dequant(scheme, D, max_blocks, v_codes, v_scale, v_zero, r, t, d);
    }
    for (int d = 0; d < D; ++d) o[d] /= l;
  }
  return 0;
}

}  // extern "C"
