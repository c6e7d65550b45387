// kvq_device.h — device-side helpers shared by the libkvq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int kBlock = 64;  // tokens per quantization block
constexpr int kWave = 64;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// ---- DPP lane exchanges (all 64 lanes active) --------------------------------------
// quad_perm [1,0,3,2] / [2,3,0,1]; row_half_mirror (lane i of each 8 <- 7-i);
// row_mirror (lane i of each 16 <- 15-i).
constexpr int kDppQuadXor1 = 0xB1;
constexpr int kDppQuadXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// max(v, dpp<CTRL>(v)) as one v_max_f32 with a DPP source operand. Written through
// fmaxf, the exchange takes a separate v_mov_b32_dpp (after a move of the old value,
// since the compiler cannot see that every source lane is valid) and an IEEE-mode
// canonicalisation of the moved value before the max: four instructions per step.
// s_nop 1 gives the two wait states a DPP read needs after a VALU write of its source.
template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
  float r;
  if constexpr (CTRL == kDppQuadXor1)
    asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
        : "=v"(r) : "v"(v));
  else if constexpr (CTRL == kDppQuadXor2)
    asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
        : "=v"(r) : "v"(v));
  else if constexpr (CTRL == kDppHalfMirror)
    asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 row_half_mirror row_mask:0xf bank_mask:0xf"
        : "=v"(r) : "v"(v));
  else if constexpr (CTRL == kDppRowMirror)
    asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 row_mirror row_mask:0xf bank_mask:0xf"
        : "=v"(r) : "v"(v));
  else
    static_assert(CTRL == kDppQuadXor1, "unsupported DPP control");
  return r;
}

// Sum over each group of N consecutive lanes (N in {1, 2, 4, 8}); every lane of the
// group receives the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp<kDppQuadXor1>(v);
  if constexpr (N >= 4) v += dpp<kDppQuadXor2>(v);
  if constexpr (N >= 8) v += dpp<kDppHalfMirror>(v);
  static_assert(N <= 8, "group too wide");
  return v;
}

// Maximum over the whole wave, returned uniformly.
__device__ __forceinline__ float wave_max(float v) {
  v = dpp_max<kDppQuadXor1>(v);
  v = dpp_max<kDppQuadXor2>(v);
  v = dpp_max<kDppHalfMirror>(v);
  v = dpp_max<kDppRowMirror>(v);
  const int iv = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}


// ---- fp16 helpers -------------------------------------------------------------------
__device__ __forceinline__ float h2f_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(half2_t, w).x);
}
__device__ __forceinline__ float h2f_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(half2_t, w).y);
}

// 8 fp16 values held in a 16-byte load -> binary32 (exact, subnormals included).
__device__ __forceinline__ void unpack8(const uint4& r, float (&x)[8]) {
  x[0] = h2f_lo(r.x); x[1] = h2f_hi(r.x);
  x[2] = h2f_lo(r.y); x[3] = h2f_hi(r.y);
  x[4] = h2f_lo(r.z); x[5] = h2f_hi(r.z);
  x[6] = h2f_lo(r.w); x[7] = h2f_hi(r.w);
}

// ---- block statistics and scales (IEEE binary32, round-to-nearest) ------------------
// int4: s = absmax / 7.5 (0 for an all-zero block).
__device__ __forceinline__ float int4_scale(float absmax) {
  return absmax == 0.0f ? 0.0f : absmax / 7.5f;
}

// uint8: s = (max - min) / 255, zp = rint(-min / s) + 0.0 with the degenerate-chunk
// rule (all elements equal to c: c == 0 -> s = zp = 0; else widen the range to 0).
__device__ __forceinline__ void uint8_scale_zero(float mn, float mx, float& s, float& zp) {
  if (mx == mn) {
    if (mx == 0.0f) {
      s = 0.0f;
      zp = 0.0f;
      return;
    }
    mn = fminf(mn, 0.0f);
    mx = fmaxf(mx, 0.0f);
  }
  const float range = mx - mn;
  s = range / 255.0f;
  zp = __builtin_rintf(-mn / s) + 0.0f;
}

// ---- codes: rounding decisions on the quotient x / s --------------------------------
// Every code is a rounding decision on the correctly rounded quotient RN(x / s). It is
// taken on q = RN(x * r), r = RN(1 / s), one multiply instead of a division:
// q = (x / s)(1 + e1)(1 + e2) and RN(x / s) = (x / s)(1 + e3), |ei| <= 2^-24, so
// |q - RN(x / s)| < 2^-22 |q|. When q lies farther than 2^-20 |q| from every decision
// boundary, both round to the same code; otherwise the division is done. (q - rint(q) and
// the distance to the boundary are exact by Sterbenz's lemma, and 2^-20 |q| is a
// power-of-two scaling; the compiler may fuse q - rint(q) with the product into one
// FMA, x * r - rint(q) rounded once, which moves the tested distance by at most
// 2^-24 |q| + 2^-25: inside the 2^-20 |q| - 2^-22 |q| of slack wherever a boundary is
// near, since there |q| >= 1/2.) The slow path is taken for
// about one value in 10^5 and for a block's extreme element, whose quotient sits on a
// boundary (7.5 for int4).
struct Divisor {
  float s, r;
  __device__ explicit Divisor(float s_) : s(s_), r(s_ == 0.0f ? 0.0f : 1.0f / s_) {}
};

// rint(q), q = RN(x * r); `near` is or-ed with whether rint(RN(x / s)) may differ.
__device__ __forceinline__ float rint_quotient_fast(float x, const Divisor& d, bool& near) {
  const float q = x * d.r;
  const float c = __builtin_rintf(q);
  near |= !(0.5f - fabsf(q - c) > fabsf(q) * 0x1p-20f);
  return c;
}


// FP8 E4M3 (OCP "fn": bias 7, subnormals (m/8)*2^-6, largest finite 448 = code 0x7E):
// s = absmax / 448 (0 for an all-zero block); the code of x is the E4M3 value nearest
// to x / s with ties to the even code, the sign kept, saturating at 448.
__device__ __forceinline__ float fp8_scale(float absmax) {
  return absmax == 0.0f ? 0.0f : absmax / 448.0f;
}

// The E4M3 codes of 8 values are taken by the hardware conversion v_cvt_pk_fp8_f32 (two
// values per instruction), which on gfx950 rounds a binary32 value to the nearest OCP
// E4M3 value with ties to even, keeps the sign (so -0 and negative values that round to
// zero give 0x80) and produces the subnormals m/8 * 2^-6. Its input is the quotient
// RN(x / s) clamped to +-448, so that values the scheme saturates (|x / s| can exceed 448
// by a rounding error) convert to 0x7E / 0xFE instead of overflowing to NaN.
//
// The quotient is not divided out for every value: q = RN(x * r), r = RN(1 / s), lies
// within 2^-22 (relative) of RN(x / s), so RN(x / s) lies between q * (1 - 2^-21) and
// q * (1 + 2^-21) (each product rounded, which moves it by at most 2^-24 relative), and
// the conversion and the clamp are monotonic: where both ends of that interval give the
// same code, it is the code of RN(x / s). Only when one of the 8 values' ends differ
// (its quotient next to the midpoint between two E4M3 values, or to 448) are the 8
// quotients divided out. Bit-exact against the oracle's search over all codes on every
// rounding decision (ties, subnormals, signed zeros, 448: GPU test).
__device__ __forceinline__ float fp8_clamp(float q) {
  return __builtin_amdgcn_fmed3f(q, -448.0f, 448.0f);
}

__device__ __forceinline__ uint2 fp8_codes8(const float (&q)[8]) {
  int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);  // bytes 0, 1
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w0, true);      // bytes 2, 3
  int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], w1, true);
  return make_uint2(static_cast<uint32_t>(w0), static_cast<uint32_t>(w1));
}

// 8 values -> 8 bytes of FP8 codes (x[i] in byte i). T: float, or _Float16 (the
// quotient then takes the fp16 operand as it is, as in pack_int4x8, but with a -0
// addend: fma(x, r, -0) = RN(x * r) with the product's sign, which the code keeps; the
// addend is hidden from the compiler, which would otherwise turn the FMA back into a
// multiply of the converted value).
template <class T>
__device__ __forceinline__ uint2 pack_fp8x8(const T (&x)[8], const Divisor& d) {
  if (d.s == 0.0f) return make_uint2(0u, 0u);
  float neg_zero = -0.0f;
  asm("" : "+v"(neg_zero));
  float lo[8], hi[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float q = __builtin_fmaf(static_cast<float>(x[i]), d.r, neg_zero);
    lo[i] = fp8_clamp(q * (1.0f - 0x1p-21f));
    hi[i] = fp8_clamp(q * (1.0f + 0x1p-21f));
  }
  const uint2 a = fp8_codes8(lo);
  const uint2 b = fp8_codes8(hi);
  if (a.x == b.x && a.y == b.y) return a;
  // Only the values whose two ends' codes differ are divided out, one at a time: the
  // two ends of the 8K workload's fp16 values differ for about 6 values in 10^4, so a
  // division of all 8 values whenever one differed ran in about a quarter of a wave's
  // passes (the other values keep lo, whose code is theirs).
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    q[i] = lo[i];
    const uint32_t wa = i < 4 ? a.x : a.y, wb = i < 4 ? b.x : b.y;
    if (((wa ^ wb) >> (8 * (i % 4))) & 0xFFu) q[i] = fp8_clamp(static_cast<float>(x[i]) / d.s);
  }
  return fp8_codes8(q);
}

// The packers below code 8 values with the multiply. The int4 packer takes one branch,
// for all 8, in the rare case that one of them needs the division; the uint8 and FP8
// packers, whose quotients sit near a boundary far more often, divide each such value
// on its own.

// 8 values -> 4 bytes of int4 nibbles c + 8 (x[i] in bits 4i .. 4i+3; for 8 consecutive
// channels: channel 2k in the low nibble of byte k).
// The quotient q = RN(x * r) is clamped to [-8, 7] first (rounding and a clamp to
// integer bounds commute, and above 7 or below -8 every quotient near q gives the same
// clamped code), then added to 1.5 * 2^23 + 8: in that binade the ulp is 1, so the add
// rounds to the nearest integer with ties to even (1.5 * 2^23 + 8 is even), t =
// 1.5 * 2^23 + 8 + rint(qc) exactly, and the low byte of t's bit pattern is the nibble
// rint(qc) + 8 (the constant's low 22 bits are zero). t - (1.5 * 2^23 + 8) = rint(qc)
// and qc - rint(qc) are exact (Sterbenz), and a block's quotients satisfy
// |q| <= 7.5 (1 + 2^-22), so the test |qc - rint(qc)| < 1/2 - 2^-17 keeps q farther
// than 2^-20 |q| from every boundary, as the division-free rule above requires.
// T: float, or _Float16 (the product then takes the fp16 operand as it is, one
// mixed-precision FMA with a +0 addend: the same rounding decision on q, and a zero
// product of either sign gives code 8).
template <class T>
__device__ __forceinline__ uint32_t pack_int4x8(const T (&x)[8], const Divisor& d) {
  if (d.s == 0.0f) return 0x88888888u;
  constexpr float kMagic = 12582920.0f;  // 1.5 * 2^23 + 8
  float t[8];
  bool near = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float q = __builtin_fmaf(static_cast<float>(x[i]), d.r, 0.0f);
    const float qc = __builtin_amdgcn_fmed3f(q, -8.0f, 7.0f);
    t[i] = qc + kMagic;
    near |= !(fabsf(qc - (t[i] - kMagic)) < 0.5f - 0x1p-17f);
  }
  if (near) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      t[i] = __builtin_amdgcn_fmed3f(__builtin_rintf(static_cast<float>(x[i]) / d.s), -8.0f,
                                     7.0f) +
             kMagic;
  }
  uint32_t b[4];  // byte k in the low 8 bits of b[k]
#pragma unroll
  for (int k = 0; k < 4; ++k)
    b[k] = (__builtin_bit_cast(uint32_t, t[2 * k + 1]) << 4) |
           __builtin_bit_cast(uint32_t, t[2 * k]);
  return __builtin_amdgcn_perm(b[1], b[0], 0x0C0C0400u) |
         __builtin_amdgcn_perm(b[3], b[2], 0x04000C0Cu);
}

// 8 values -> 8 bytes of uint8 codes (x[i] in byte i). T as for pack_int4x8.
// The code clamp(rint(q) + zp, 0, 255) is taken as in pack_int4x8: q is clamped to
// [-zp, 255 - zp] (integer bounds), then added to 1.5 * 2^23 + zp, exact for |zp| <
// 2^21 (fp16 inputs give |zp| <= 255 * 2^11), whose sum is 1.5 * 2^23 + zp + rint(qc)
// with rint(qc) + zp in the low byte. Where 1.5 * 2^23 + zp is odd a tie would round
// the other way, but a tie is always near and recomputed. The distance test is the
// relative one above, 2^-20 |qc| (|qc| <= |q| where q is not clamped, and a clamped q
// gives a code no nearby quotient changes).
template <class T>
__device__ __forceinline__ uint2 pack_uint8x8(const T (&x)[8], const Divisor& d, int zpi) {
  if (d.s == 0.0f) return make_uint2(0u, 0u);
  uint32_t b[8];
  if (zpi > -(1 << 21) && zpi < (1 << 21)) {  // uniform over the block
    const float zp = static_cast<float>(zpi);
    const float magic = 12582912.0f + zp;  // 1.5 * 2^23 + zp
    // Each value is divided out on its own where it is near: fp16 inputs put quotients
    // on a rounding boundary far more often than random values would (a quotient
    // 255 x / (max - min) of two fp16 values is often exactly a half-integer), and a
    // branch over all 8 values made the whole wave divide all 8 whenever one lane had
    // one near value.
    float t[8];
    bool near[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q = __builtin_fmaf(static_cast<float>(x[i]), d.r, 0.0f);
      const float qc = __builtin_amdgcn_fmed3f(q, -zp, 255.0f - zp);
      t[i] = qc + magic;
      near[i] = !(__builtin_fmaf(fabsf(qc), 0x1p-20f, fabsf(qc - (t[i] - magic))) < 0.5f);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (near[i])
        t[i] = __builtin_amdgcn_fmed3f(__builtin_rintf(static_cast<float>(x[i]) / d.s), -zp,
                                       255.0f - zp) +
               magic;
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = __builtin_bit_cast(uint32_t, t[i]);
  } else {
    float c[8];
    bool near = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = rint_quotient_fast(static_cast<float>(x[i]), d, near);
    if (near) {
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = __builtin_rintf(static_cast<float>(x[i]) / d.s);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int v = static_cast<int>(c[i]) + zpi;
      b[i] = static_cast<uint32_t>(v < 0 ? 0 : (v > 255 ? 255 : v));
    }
  }
  // byte i of the result = the low byte of b[i]
  return make_uint2(__builtin_amdgcn_perm(b[1], b[0], 0x0C0C0400u) |
                        __builtin_amdgcn_perm(b[3], b[2], 0x04000C0Cu),
                    __builtin_amdgcn_perm(b[5], b[4], 0x0C0C0400u) |
                        __builtin_amdgcn_perm(b[7], b[6], 0x04000C0Cu));
}

// ---- int4 cache block layout ---------------------------------------------------------
// An int4 block (64 tokens x D channels, one K and one V region of 32*D bytes each) is
// stored in the operand order of v_mfma_f32_16x16x32_f16, so that a lane's 16-byte
// loads are exactly its matrix-core fragments. Lane l (0..63) owns F = D/8 dwords per
// region, dword f at byte ((f / 4) * 64 + l) * 16 + (f % 4) * 4; each dword holds 8
// offset-binary nibbles (code + 8), nibble q in bits 4q..4q+3.
//   K (B operand of QK^T, K = channels, N = tokens): f = nt * (D/32) + ks,
//     nibble q = channel 32*ks + 8*(l/16) + q of token 16*nt + (l%16).
//   V (B operand of P.V, K = tokens, N = channels): f = 2*nt + ks,
//     nibble q = token 32*ks + 8*(l/16) + q of channel 16*nt + (l%16).
__device__ __forceinline__ uint32_t int4_dword_offset(int lane, int f) {
  return static_cast<uint32_t>(((f >> 2) * 64 + lane) * 16 + (f & 3) * 4);
}

// Index of block j of row (b, h) in the code, scale and zero-point arrays: dense
// [B][H][max_blocks], or, with a block table, [num_pages][H] at the page the table
// gives for (b, j), clamped to the pool.
__device__ __forceinline__ int64_t block_slot(const int32_t* table, int num_pages, int heads,
                                              int max_blocks, int b, int h, int j) {
  if (table == nullptr) return (static_cast<int64_t>(b) * heads + h) * max_blocks + j;
  int p = table[static_cast<int64_t>(b) * max_blocks + j];
  p = p < 0 ? 0 : (p >= num_pages ? num_pages - 1 : p);
  return static_cast<int64_t>(p) * heads + h;
}

// Word 3 of a raw buffer resource on gfx9-family chips (32-bit data format, no
// swizzle): loads past num_records return zeros and access no memory.
constexpr int kBufferRsrcWord3 = 0x00020000;

// 16-byte store of a value (component by component, so that a uint4 held in a register
// array is never copied out of memory).
// Non-temporal: the decode step's code stores come at the very end of the kernel, which
// completes only once they have reached memory; marked streaming they do not wait in the
// L2 for the end-of-kernel write-back (8K int4 step 43.4 -> 42.8 us).
__device__ __forceinline__ void store_b128(uint8_t* p, const uint4& v) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}

// 16-byte load through a buffer resource at voffset (per lane) + soffset (uniform);
// AUX = cache policy bits (2: non-temporal).
template <int AUX>
__device__ __forceinline__ uint4 load_b128(__amdgpu_buffer_rsrc_t rsrc, int voffset, int soffset) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voffset, soffset, AUX);
  return make_uint4(v.x, v.y, v.z, v.w);
}

}  // namespace kvq
