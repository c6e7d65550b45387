// kvq_quant.hip — block quantization of the KV cache (prefill and per-token append).
//
// Formats follow page "DeepSeek-R1推理延迟骤降41.8%？独家披露3类硬件感知调度策略" §2.1
// ("分块量化压缩设计": 4-bit codes, one scale per 64-token block = absmax / 7.5, codes
// rounded and clamped to [-8, 7]), page "第一章：DeepSeek R1推理模型性能跃迁全景概览"
// §2.2 (INT8 codes with scales from each chunk's extremes; asymmetric min/max reading)
// and page "DeepSeek R1性能优化有哪些技巧" §一 (an FP8 KV cache; here E4M3 codes with a
// 4-bit-style per-block scale, absmax / 448).
//
// One 256-thread workgroup owns one 64-token block of one (sequence, head, K|V) row.
// Each thread holds 8 channels of one token per 16-byte load, so every wave-wide load
// instruction reads whole token rows (coalesced). The block statistic is reduced with
// DPP inside each wave and through LDS across the 4 waves. Each code is the rounding
// (half to even) of the correctly rounded binary32 quotient x / s, taken from the
// scale's reciprocal where that provably decides the same code and from the division
// otherwise (the encoders in kvq_device.h).
// uint8 codes are written in natural order ([token][channel]); int4 blocks are staged
// in LDS and written in the matrix-core fragment order described in kvq_device.h, one
// 16-byte store per thread.
#include "kvq_append.h"

namespace kvq {
namespace {

// ---- prefill: grid (blocks, heads, batch * 2) ---------------------------------------
template <int SCHEME, int D>
__global__ __launch_bounds__(kThreads) void quantize_blocks_kernel(QuantArgs a) {
  using G = QGeo<SCHEME, D>;
  __shared__ float red[2 * kWaves];
  __shared__ __align__(16) _Float16 xs[SCHEME == KVQ_INT4_SYM ? kBlock * D : 8];
  const int j = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z >> 1;
  const int kv = blockIdx.z & 1;
  const int cap = a.max_blocks * kBlock;
  int len = a.seq_lens[b];
  len = len < 0 ? 0 : len;
  len = min(len, min(a.max_len, cap));
  const int nb = (len + kBlock - 1) / kBlock;
  if (j >= nb) return;  // uniform over the workgroup
  const int ntok = min(kBlock, len - j * kBlock);

  const int tid = threadIdx.x;
  const int tr = tid / G::kThreadsPerToken;
  const int chunk = tid % G::kThreadsPerToken;
  const uint16_t* src = (kv ? a.v : a.k) + static_cast<int64_t>(b) * a.stride_b +
                        static_cast<int64_t>(h) * a.stride_h +
                        static_cast<int64_t>(j) * kBlock * a.stride_t + chunk * 8;

  uint4 raw[G::kPasses];
  // The block statistics are taken on the fp16 values as loaded, with no binary32 copy
  // of them: the absmax schemes (int4, FP8) on the bit patterns (with the sign bit
  // cleared, the patterns of finite values order as unsigned integers the way the
  // values do, two per packed max; tokens past the block's end load as zeros, which
  // cannot raise it), uint8 with packed fp16 min and max over the tokens that exist.
  // The codes take the fp16 values as operands (int4: staged in LDS first).
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  u16x2 amax_bits = {0, 0};
  h2 mn2 = {__builtin_inff16(), __builtin_inff16()};
  h2 mx2 = {-__builtin_inff16(), -__builtin_inff16()};
  // All of the thread's loads are requested before any is used (a use between them made
  // the compiler wait for each load before requesting the next).
#pragma unroll
  for (int p = 0; p < G::kPasses; ++p) {
    const int t = p * G::kTokensPerPass + tr;
    // the fp16 inputs are read once: non-temporal loads (8K workload, all blocks: uint8
    // 384 -> 326 us, FP8 464 -> 456 us, int4 unchanged at about 340 us)
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    v4u r4 = {0u, 0u, 0u, 0u};
    if (t < ntok)
      r4 = __builtin_nontemporal_load(
          reinterpret_cast<const v4u*>(src + static_cast<int64_t>(t) * a.stride_t));
    raw[p] = make_uint4(r4.x, r4.y, r4.z, r4.w);
  }
#pragma unroll
  for (int p = 0; p < G::kPasses; ++p) {
    const int t = p * G::kTokensPerPass + tr;
    if constexpr (SCHEME == KVQ_INT4_SYM)
      *reinterpret_cast<uint4*>(xs + t * D + chunk * 8) = raw[p];
    const uint32_t w[4] = {raw[p].x, raw[p].y, raw[p].z, raw[p].w};
    if constexpr (SCHEME != KVQ_UINT8_ASYM) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        amax_bits = __builtin_elementwise_max(
            amax_bits, __builtin_bit_cast(u16x2, w[k] & 0x7FFF7FFFu));
    } else if (t < ntok) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        mn2 = __builtin_elementwise_min(mn2, __builtin_bit_cast(h2, w[k]));
        mx2 = __builtin_elementwise_max(mx2, __builtin_bit_cast(h2, w[k]));
      }
    }
  }
  float amax = 0.0f, mn = 0.0f, mx = 0.0f;
  if constexpr (SCHEME != KVQ_UINT8_ASYM) {
    const unsigned short bits = amax_bits.x > amax_bits.y ? amax_bits.x : amax_bits.y;
    amax = static_cast<float>(__builtin_bit_cast(_Float16, bits));
  } else {
    mn = fminf(static_cast<float>(mn2.x), static_cast<float>(mn2.y));
    mx = fmaxf(static_cast<float>(mx2.x), static_cast<float>(mx2.y));
  }

  float s, zp = 0.0f;
  if constexpr (SCHEME != KVQ_UINT8_ASYM) {  // absmax schemes
    float st[1] = {amax};
    block_max<1>(st, red);
    s = SCHEME == KVQ_INT4_SYM ? int4_scale(st[0]) : fp8_scale(st[0]);
  } else {
    float st[2] = {-mn, mx};
    block_max<2>(st, red);
    uint8_scale_zero(-st[0], st[1], s, zp);
  }
  const int zpi = static_cast<int>(zp);
  const Divisor dv(s);

  const int64_t row = static_cast<int64_t>(b) * a.heads + h;
  const int64_t blk = block_slot(a.block_table, a.num_pages, a.heads, a.max_blocks, b, h, j);
  uint8_t* codes = (kv ? a.v_codes : a.k_codes) + blk * kBlock * G::kRowBytes;
  if constexpr (SCHEME == KVQ_INT4_SYM) {
    int4_write_block_from<D>(xs, ntok, dv, kv != 0, codes, tid);  // block_max synced xs
  } else {
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p) {
      const int t = p * G::kTokensPerPass + tr;
      typedef _Float16 h8 __attribute__((ext_vector_type(8)));
      const h8 v = __builtin_bit_cast(h8, raw[p]);
      _Float16 xh[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) xh[i] = v[i];
      store_codes<SCHEME, D>(codes + t * G::kRowBytes, chunk, xh, dv, zpi, t < ntok);
    }
  }
  if (tid == 0) {
    (kv ? a.v_scale : a.k_scale)[blk] = s;
    float* zero = kv ? a.v_zero : a.k_zero;
    if (zero) zero[blk] = zp;
  }
  // Stage the fp16 values of an open tail block for later appends.
  uint16_t* tail = kv ? a.v_tail : a.k_tail;
  if (ntok < kBlock && tail) {
    uint16_t* trow = tail + row * kBlock * D + chunk * 8;
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p) {
      const int t = p * G::kTokensPerPass + tr;
      *reinterpret_cast<uint4*>(trow + t * D) = raw[p];
    }
  }
}

// ---- append one token per sequence: grid (heads, batch), kThreads threads ------------
// Every workgroup of sequence b takes an arrival ticket on seq_lens[b], which gives it
// the length before this append; the last of the sequence's `heads` workgroups stores
// the incremented length, so no second kernel is needed to advance the lengths.
template <int SCHEME, int D>
__global__ __launch_bounds__(kThreads) void append_kernel(AppendArgs a) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  append_token<SCHEME, D>(a, b, static_cast<int64_t>(b) * a.heads + h);
}

template <int SCHEME, int D>
hipError_t quantize_t(int batch, int n_blocks, const QuantArgs& a, hipStream_t s) {
  dim3 grid(n_blocks, a.heads, batch * 2);
  hipLaunchKernelGGL((quantize_blocks_kernel<SCHEME, D>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int SCHEME, int D>
hipError_t append_t(const AppendArgs& a, hipStream_t s) {
  dim3 grid(a.heads, a.batch);
  hipLaunchKernelGGL((append_kernel<SCHEME, D>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(int scheme, int head_dim, int batch, int n_blocks,
                           const QuantArgs& a, hipStream_t s) {
  const bool d128 = head_dim == 128;
  switch (scheme) {
    case KVQ_INT4_SYM:
      return d128 ? quantize_t<KVQ_INT4_SYM, 128>(batch, n_blocks, a, s)
                  : quantize_t<KVQ_INT4_SYM, 64>(batch, n_blocks, a, s);
    case KVQ_FP8_E4M3:
      return d128 ? quantize_t<KVQ_FP8_E4M3, 128>(batch, n_blocks, a, s)
                  : quantize_t<KVQ_FP8_E4M3, 64>(batch, n_blocks, a, s);
    default:
      return d128 ? quantize_t<KVQ_UINT8_ASYM, 128>(batch, n_blocks, a, s)
                  : quantize_t<KVQ_UINT8_ASYM, 64>(batch, n_blocks, a, s);
  }
}

hipError_t launch_append(int scheme, int head_dim, const AppendArgs& a, hipStream_t s) {
  const bool d128 = head_dim == 128;
  switch (scheme) {
    case KVQ_INT4_SYM:
      return d128 ? append_t<KVQ_INT4_SYM, 128>(a, s) : append_t<KVQ_INT4_SYM, 64>(a, s);
    case KVQ_FP8_E4M3:
      return d128 ? append_t<KVQ_FP8_E4M3, 128>(a, s) : append_t<KVQ_FP8_E4M3, 64>(a, s);
    default:
      return d128 ? append_t<KVQ_UINT8_ASYM, 128>(a, s) : append_t<KVQ_UINT8_ASYM, 64>(a, s);
  }
}

}  // namespace kvq
