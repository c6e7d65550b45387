// kvq_quant.hip — block quantization of the KV cache (prefill and per-token append).
//
// Formats follow page "DeepSeek-R1推理延迟骤降41.8%？独家披露3类硬件感知调度策略" §2.1
// ("分块量化压缩设计": 4-bit codes, one scale per 64-token block = absmax / 7.5, codes
// rounded and clamped to [-8, 7]) and page "第一章：DeepSeek R1推理模型性能跃迁全景概览"
// §2.2 (INT8 codes with scales from each chunk's extremes; asymmetric min/max reading).
//
// One 256-thread workgroup owns one 64-token block of one (sequence, head, K|V) row.
// Each thread holds 8 channels of one token per 16-byte load, so every wave-wide load
// instruction reads whole token rows (coalesced). The block statistic is reduced with
// DPP inside each wave and through LDS across the 4 waves; every element is divided by
// the scale with the correctly rounded binary32 division and rounded half-to-even.
// uint8 codes are written in natural order ([token][channel]); int4 blocks are staged
// in LDS and written in the matrix-core fragment order described in kvq_device.h, one
// 16-byte store per thread.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

// Maxima of N values over a group of kThreads threads (the workgroup, or one half of a
// two-group workgroup, each half with its own lds); every thread of the group receives
// the results. Contains one workgroup barrier.
template <int N>
__device__ __forceinline__ void block_max(float (&v)[N], float* lds /* [N * kWaves] */) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = wave_max(v[i]);
  const int w = (threadIdx.x % kThreads) / kWave;
  if ((threadIdx.x % kWave) == 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) lds[i * kWaves + w] = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float r = lds[i * kWaves];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) r = fmaxf(r, lds[i * kWaves + k]);
    v[i] = r;
  }
}

template <int SCHEME, int D>
struct QGeo {
  static constexpr int kThreadsPerToken = D / 8;  // 8 channels (16 bytes) per thread
  static constexpr int kTokensPerPass = kThreads / kThreadsPerToken;
  static constexpr int kPasses = kBlock / kTokensPerPass;
  static constexpr int kRowBytes = SCHEME == KVQ_INT4_SYM ? D / 2 : D;
};

template <int SCHEME, int D>
__device__ __forceinline__ void store_codes(uint8_t* token_row, int chunk, const float (&x)[8],
                                            float s, int zpi, bool valid) {
  if constexpr (SCHEME == KVQ_INT4_SYM) {
    const uint32_t w = valid ? pack_int4x8(x, s) : 0u;
    *reinterpret_cast<uint32_t*>(token_row + chunk * 4) = w;
  } else {
    const uint2 w = valid ? pack_uint8x8(x, s, zpi) : make_uint2(0u, 0u);
    *reinterpret_cast<uint2*>(token_row + chunk * 8) = w;
  }
}

// int4: writes one block region (K or V) in fragment order from the block's fp16 values
// staged in LDS (xs[t * D + d], natural order); tokens t >= ntok give zero nibbles.
template <int D>
__device__ __forceinline__ void int4_write_block_from(const _Float16* xs, int ntok, float s,
                                                      bool is_v, uint8_t* out, int tid) {
  constexpr int KS = D / 32;      // 32-channel K steps
  constexpr int kChunks = 2 * D;  // 16-byte chunks per region (32 * D bytes)
  for (int c = tid; c < kChunks; c += kThreads) {
    const int lane = c % kWave, i = c / kWave;
    uint32_t w[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int f = 4 * i + r;
      uint32_t word = 0;
      if (!is_v) {
        const int t = 16 * (f / KS) + lane % 16;
        const int d0 = 32 * (f % KS) + 8 * (lane / 16);
        if (t < ntok) {
#pragma unroll
          for (int q = 0; q < 8; ++q)
            word |= int4_code(static_cast<float>(xs[t * D + d0 + q]), s) << (4 * q);
        }
      } else {
        const int d = 16 * (f / 2) + lane % 16;
        const int t0 = 32 * (f % 2) + 8 * (lane / 16);
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (t0 + q < ntok)
            word |= int4_code(static_cast<float>(xs[(t0 + q) * D + d]), s) << (4 * q);
      }
      w[r] = word;
    }
    *reinterpret_cast<uint4*>(out + c * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

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
  float x[G::kPasses][8];
  float amax = 0.0f, mn = __builtin_inff(), mx = -__builtin_inff();
#pragma unroll
  for (int p = 0; p < G::kPasses; ++p) {
    const int t = p * G::kTokensPerPass + tr;
    const bool valid = t < ntok;
    raw[p] = valid ? *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(t) * a.stride_t)
                   : make_uint4(0u, 0u, 0u, 0u);
    unpack8(raw[p], x[p]);
    if constexpr (SCHEME == KVQ_INT4_SYM)
      *reinterpret_cast<uint4*>(xs + t * D + chunk * 8) = raw[p];
    if (valid) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        amax = fmaxf(amax, fabsf(x[p][i]));
        mn = fminf(mn, x[p][i]);
        mx = fmaxf(mx, x[p][i]);
      }
    }
  }

  float s, zp = 0.0f;
  if constexpr (SCHEME == KVQ_INT4_SYM) {
    float st[1] = {amax};
    block_max<1>(st, red);
    s = int4_scale(st[0]);
  } else {
    float st[2] = {-mn, mx};
    block_max<2>(st, red);
    uint8_scale_zero(-st[0], st[1], s, zp);
  }
  const int zpi = static_cast<int>(zp);

  const int64_t row = static_cast<int64_t>(b) * a.heads + h;
  const int64_t blk = row * a.max_blocks + j;
  uint8_t* codes = (kv ? a.v_codes : a.k_codes) + blk * kBlock * G::kRowBytes;
  if constexpr (SCHEME == KVQ_INT4_SYM) {
    int4_write_block_from<D>(xs, ntok, s, kv != 0, codes, tid);  // block_max synced xs
  } else {
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p) {
      const int t = p * G::kTokensPerPass + tr;
      store_codes<SCHEME, D>(codes + t * G::kRowBytes, chunk, x[p], s, zpi, t < ntok);
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

// ---- append one token per sequence: grid (heads, batch), 2 x 256 threads -------------
// Threads 0..255 handle the row's K, threads 256..511 its V. Every workgroup of sequence
// b first takes an arrival ticket by adding 1 << 24 to seq_lens[b]: the low 24 bits
// give each of them the length before this append, and the last of the sequence's
// `heads` workgroups to arrive stores the incremented length (clearing the count), so
// no second kernel is needed to advance the lengths.
template <int SCHEME, int D>
__global__ __launch_bounds__(2 * kThreads) void append_kernel(AppendArgs a) {
  using G = QGeo<SCHEME, D>;
  __shared__ float red_all[2][4 * kWaves];
  __shared__ __align__(16) _Float16 xs_all[2][SCHEME == KVQ_INT4_SYM ? kBlock * D : 8];
  __shared__ int len_shared;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int kv = threadIdx.x / kThreads;
  const int tid = threadIdx.x % kThreads;
  float* red = red_all[kv];
  _Float16* xs = xs_all[kv];
  const int cap = a.max_blocks * kBlock;
  const int tr = tid / G::kThreadsPerToken;
  const int chunk = tid % G::kThreadsPerToken;
  const int64_t row = static_cast<int64_t>(b) * a.heads + h;
  uint16_t* tail = (kv ? a.v_tail : a.k_tail) + row * kBlock * D + chunk * 8;
  const uint16_t* fresh = (kv ? a.v_new : a.k_new) + row * D + chunk * 8;
  const uint4 fresh_raw = *reinterpret_cast<const uint4*>(fresh);  // independent of the length
  if (threadIdx.x == 0) {
    // system scope: the read-modify-write happens at memory, past the per-XCD L2s
    uint32_t* lens = reinterpret_cast<uint32_t*>(a.seq_lens);
    const uint32_t old = __hip_atomic_fetch_add(lens + b, 1u << 24, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_SYSTEM);
    const int len0 = static_cast<int>(old & 0xFFFFFFu);
    if ((old >> 24) == static_cast<uint32_t>(a.heads - 1))
      __hip_atomic_exchange(lens + b, static_cast<uint32_t>(len0 < cap ? len0 + 1 : len0),
                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    len_shared = len0;
  }
  __syncthreads();
  const int len = len_shared;
  if (len >= cap) return;  // no room: the row is left unchanged (uniform)
  const int slot = len % kBlock;
  const int j = len / kBlock;
  const int64_t blk = row * a.max_blocks + j;
  uint8_t* codes = (kv ? a.v_codes : a.k_codes) + blk * kBlock * G::kRowBytes;

  // int4 V: the dword of each channel that the new token shares with 7 others, read now
  // so that its latency overlaps the tail loads (used only if the block keeps its scale)
  uint32_t v_old[(D + kThreads - 1) / kThreads];
  if constexpr (SCHEME == KVQ_INT4_SYM) {
    if (kv && slot != 0) {
      const int ks = slot / 32, g = (slot % 32) / 8;
#pragma unroll
      for (int i = 0; i < (D + kThreads - 1) / kThreads; ++i) {
        const int d = tid + i * kThreads;
        if (d < D)
          v_old[i] = *reinterpret_cast<const uint32_t*>(
              codes + int4_dword_offset(16 * g + d % 16, 2 * (d / 16) + ks));
      }
    }
  }

  uint4 raw[G::kPasses];
  float x[G::kPasses][8];
  // statistics of the block before (old) and after (new) the token joins it
  float amax_o = 0.0f, mn_o = __builtin_inff(), mx_o = -__builtin_inff();
  float amax_n = 0.0f, mn_n = __builtin_inff(), mx_n = -__builtin_inff();
#pragma unroll
  for (int p = 0; p < G::kPasses; ++p) {
    const int t = p * G::kTokensPerPass + tr;
    if (t < slot)
      raw[p] = *reinterpret_cast<const uint4*>(tail + t * D);
    else if (t == slot)
      raw[p] = fresh_raw;
    else
      raw[p] = make_uint4(0u, 0u, 0u, 0u);
    unpack8(raw[p], x[p]);
    if constexpr (SCHEME == KVQ_INT4_SYM)
      *reinterpret_cast<uint4*>(xs + t * D + chunk * 8) = raw[p];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (t < slot) {
        amax_o = fmaxf(amax_o, fabsf(x[p][i]));
        mn_o = fminf(mn_o, x[p][i]);
        mx_o = fmaxf(mx_o, x[p][i]);
      }
      if (t <= slot) {
        amax_n = fmaxf(amax_n, fabsf(x[p][i]));
        mn_n = fminf(mn_n, x[p][i]);
        mx_n = fmaxf(mx_n, x[p][i]);
      }
    }
  }

  float s, zp = 0.0f;
  bool full;
  if constexpr (SCHEME == KVQ_INT4_SYM) {
    float st[2] = {amax_o, amax_n};
    block_max<2>(st, red);
    full = slot == 0 || st[0] != st[1];
    s = int4_scale(st[1]);
  } else {
    float st[4] = {-mn_o, mx_o, -mn_n, mx_n};
    block_max<4>(st, red);
    full = slot == 0 || st[0] != st[2] || st[1] != st[3];
    uint8_scale_zero(-st[2], st[3], s, zp);
  }
  const int zpi = static_cast<int>(zp);

  if constexpr (SCHEME == KVQ_INT4_SYM) {
    // xs holds tokens 0..slot (block_max synchronised the workgroup after the stores)
    if (full) {
      int4_write_block_from<D>(xs, slot + 1, s, kv != 0, codes, tid);
    } else if (!kv) {
      // K: the new token's D/8 dwords (8 channels each)
      constexpr int KS = D / 32;
      for (int idx = tid; idx < D / 8; idx += kThreads) {
        const int ks = idx / 4, g = idx % 4;
        uint32_t word = 0;
#pragma unroll
        for (int q = 0; q < 8; ++q)
          word |= int4_code(static_cast<float>(xs[slot * D + 32 * ks + 8 * g + q]), s) << (4 * q);
        const int f = (slot / 16) * KS + ks;
        *reinterpret_cast<uint32_t*>(codes + int4_dword_offset(16 * g + slot % 16, f)) = word;
      }
    } else {
      // V: one nibble per channel, merged into the dword it shares with 7 other tokens
      const int ks = slot / 32, g = (slot % 32) / 8, q = slot % 8;
#pragma unroll
      for (int i = 0; i < (D + kThreads - 1) / kThreads; ++i) {
        const int d = tid + i * kThreads;
        if (d < D) {
          const int f = 2 * (d / 16) + ks;
          const uint32_t nib = int4_code(static_cast<float>(xs[slot * D + d]), s);
          *reinterpret_cast<uint32_t*>(codes + int4_dword_offset(16 * g + d % 16, f)) =
              (v_old[i] & ~(0xFu << (4 * q))) | (nib << (4 * q));
        }
      }
    }
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p) {
      const int t = p * G::kTokensPerPass + tr;
      if (t == slot) *reinterpret_cast<uint4*>(tail + t * D) = raw[p];
    }
  } else {
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p) {
      const int t = p * G::kTokensPerPass + tr;
      if (full || t == slot)
        store_codes<SCHEME, D>(codes + t * G::kRowBytes, chunk, x[p], s, zpi, t <= slot);
      if (t == slot) *reinterpret_cast<uint4*>(tail + t * D) = raw[p];
    }
  }
  if (tid == 0 && full) {
    (kv ? a.v_scale : a.k_scale)[blk] = s;
    float* zero = kv ? a.v_zero : a.k_zero;
    if (zero) zero[blk] = zp;
  }
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
  hipLaunchKernelGGL((append_kernel<SCHEME, D>), grid, dim3(2 * kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(int scheme, int head_dim, int batch, int n_blocks,
                           const QuantArgs& a, hipStream_t s) {
  if (scheme == KVQ_INT4_SYM)
    return head_dim == 128 ? quantize_t<KVQ_INT4_SYM, 128>(batch, n_blocks, a, s)
                           : quantize_t<KVQ_INT4_SYM, 64>(batch, n_blocks, a, s);
  return head_dim == 128 ? quantize_t<KVQ_UINT8_ASYM, 128>(batch, n_blocks, a, s)
                         : quantize_t<KVQ_UINT8_ASYM, 64>(batch, n_blocks, a, s);
}

hipError_t launch_append(int scheme, int head_dim, const AppendArgs& a, hipStream_t s) {
  if (scheme == KVQ_INT4_SYM)
    return head_dim == 128 ? append_t<KVQ_INT4_SYM, 128>(a, s) : append_t<KVQ_INT4_SYM, 64>(a, s);
  return head_dim == 128 ? append_t<KVQ_UINT8_ASYM, 128>(a, s)
                         : append_t<KVQ_UINT8_ASYM, 64>(a, s);
}

}  // namespace kvq
