// kvq_append.h — block quantization pieces shared by the prefill quantizer, the
// append kernel and the fused decode step (one workgroup appends a row's token, then
// attends over the row).
//
// Formats follow page "DeepSeek-R1推理延迟骤降41.8%？独家披露3类硬件感知调度策略" §2.1
// ("分块量化压缩设计": 4-bit codes, one scale per 64-token block = absmax / 7.5, codes
// rounded and clamped to [-8, 7]) and page "第一章：DeepSeek R1推理模型性能跃迁全景概览"
// §2.2 (INT8 codes with scales from each chunk's extremes; asymmetric min/max reading).
// Appending into a partly filled block is not described by the pages: the block is
// re-quantized over exactly its valid tokens, so the cache always equals a fresh
// quantization of the whole history.
#pragma once

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

constexpr int kThreads = 256;  // threads of one block's quantizer
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

// ---- append one token to one row (K and V) -----------------------------------------
// Called by all kThreads threads of a workgroup (contains one workgroup barrier).
// len = the row's length before the token (< capacity); fresh[kv] = this thread's 16
// bytes of the new K (kv = 0) or V (kv = 1) token, channels chunk*8 .. +7. The new
// token's fp16 values go to the row's tail staging. A block whose statistic (absmax, or
// min and max) the token leaves unchanged keeps its scale and gets only the new
// token's codes; otherwise (and for a block the token opens) the whole block is
// re-quantized from the staged values and its scale (and zero point) rewritten. Both
// tensors are reduced in one pass so that their loads and barriers overlap.
// xs: 2 * kBlock * D fp16 of LDS, 16-byte aligned (int4 only; unused for uint8);
// red: kAppendStats<SCHEME> * kWaves floats of LDS.
template <int SCHEME>
constexpr int kAppendStats = SCHEME == KVQ_INT4_SYM ? 4 : 8;  // old and new, K and V

template <int SCHEME, int D>
__device__ __forceinline__ void append_row(const AppendArgs& a, int64_t row, int len,
                                           const uint4 (&fresh)[2], _Float16* xs, float* red) {
  using G = QGeo<SCHEME, D>;
  constexpr int NS = kAppendStats<SCHEME> / 2;  // statistics per tensor
  const int tid = threadIdx.x % kThreads;
  const int tr = tid / G::kThreadsPerToken;
  const int chunk = tid % G::kThreadsPerToken;
  const int slot = len % kBlock;
  const int64_t blk = row * a.max_blocks + len / kBlock;

  // The staged tokens 0..slot-1 through buffer resources that end at token `slot`:
  // every lane loads unconditionally and the loads past the end return zeros without
  // touching memory (no divergent branches around the loads).
  uint4 raw[2][G::kPasses];
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (kv ? a.v_tail : a.k_tail) + row * kBlock * D, 0, slot * D * 2, kBufferRsrcWord3);
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p) {
      const int t = p * G::kTokensPerPass + tr;
      const uint4 staged = load_b128<0>(rs, (t * D + chunk * 8) * 2, 0);
      raw[kv][p] = t == slot ? fresh[kv] : staged;
    }
  }

  // statistics of each block before (old) and after (new) the token joins it
  float st[2 * NS];
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    float amax_o = 0.0f, mn_o = __builtin_inff(), mx_o = -__builtin_inff();
    float amax_n = 0.0f, mn_n = __builtin_inff(), mx_n = -__builtin_inff();
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p) {
      const int t = p * G::kTokensPerPass + tr;
      float x[8];
      unpack8(raw[kv][p], x);
      if constexpr (SCHEME == KVQ_INT4_SYM)
        *reinterpret_cast<uint4*>(xs + kv * kBlock * D + t * D + chunk * 8) = raw[kv][p];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (t < slot) {
          amax_o = fmaxf(amax_o, fabsf(x[i]));
          mn_o = fminf(mn_o, x[i]);
          mx_o = fmaxf(mx_o, x[i]);
        }
        if (t <= slot) {
          amax_n = fmaxf(amax_n, fabsf(x[i]));
          mn_n = fminf(mn_n, x[i]);
          mx_n = fmaxf(mx_n, x[i]);
        }
      }
    }
    if constexpr (SCHEME == KVQ_INT4_SYM) {
      st[kv * NS + 0] = amax_o;
      st[kv * NS + 1] = amax_n;
    } else {
      st[kv * NS + 0] = -mn_o;
      st[kv * NS + 1] = mx_o;
      st[kv * NS + 2] = -mn_n;
      st[kv * NS + 3] = mx_n;
    }
  }
  block_max<2 * NS>(st, red);  // also makes the xs stores visible to the workgroup

#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    const bool is_v = kv != 0;
    const float* sv = st + kv * NS;
    float s, zp = 0.0f;
    bool full;
    if constexpr (SCHEME == KVQ_INT4_SYM) {
      full = slot == 0 || sv[0] != sv[1];
      s = int4_scale(sv[1]);
    } else {
      full = slot == 0 || sv[0] != sv[2] || sv[1] != sv[3];
      uint8_scale_zero(-sv[2], sv[3], s, zp);
    }
    uint8_t* codes = (is_v ? a.v_codes : a.k_codes) + blk * kBlock * G::kRowBytes;
    uint16_t* tail = (is_v ? a.v_tail : a.k_tail) + row * kBlock * D + chunk * 8;
    if constexpr (SCHEME == KVQ_INT4_SYM) {
      const _Float16* xt = xs + kv * kBlock * D;  // tokens 0..slot, zeros after
      if (full) {
        int4_write_block_from<D>(xt, slot + 1, s, is_v, codes, tid);
      } else if (!is_v) {
        // K: the new token's D/8 dwords (8 channels each)
        constexpr int KS = D / 32;
        for (int idx = tid; idx < D / 8; idx += kThreads) {
          const int ks = idx / 4, g = idx % 4;
          uint32_t word = 0;
#pragma unroll
          for (int q = 0; q < 8; ++q)
            word |= int4_code(static_cast<float>(xt[slot * D + 32 * ks + 8 * g + q]), s) << (4 * q);
          const int f = (slot / 16) * KS + ks;
          *reinterpret_cast<uint32_t*>(codes + int4_dword_offset(16 * g + slot % 16, f)) = word;
        }
      } else {
        // V: each channel's new nibble shares a dword with 7 other tokens; with the
        // scale unchanged, rebuilding the dword from the staged values reproduces the
        // stored nibbles (and zeros past the token), so the cache is never read back
        const int ks = slot / 32, g = (slot % 32) / 8, t0 = 32 * ks + 8 * g;
        for (int d = tid; d < D; d += kThreads) {
          uint32_t word = 0;
#pragma unroll
          for (int q = 0; q < 8; ++q)
            if (t0 + q <= slot)
              word |= int4_code(static_cast<float>(xt[(t0 + q) * D + d]), s) << (4 * q);
          const int f = 2 * (d / 16) + ks;
          *reinterpret_cast<uint32_t*>(codes + int4_dword_offset(16 * g + d % 16, f)) = word;
        }
      }
#pragma unroll
      for (int p = 0; p < G::kPasses; ++p) {
        const int t = p * G::kTokensPerPass + tr;
        if (t == slot) *reinterpret_cast<uint4*>(tail + t * D) = raw[kv][p];
      }
    } else {
      const int zpi = static_cast<int>(zp);
#pragma unroll
      for (int p = 0; p < G::kPasses; ++p) {
        const int t = p * G::kTokensPerPass + tr;
        if (full || t == slot) {
          float x[8];
          unpack8(raw[kv][p], x);
          store_codes<SCHEME, D>(codes + t * G::kRowBytes, chunk, x, s, zpi, t <= slot);
        }
        if (t == slot) *reinterpret_cast<uint4*>(tail + t * D) = raw[kv][p];
      }
    }
    if (tid == 0 && full) {
      (is_v ? a.v_scale : a.k_scale)[blk] = s;
      float* zero = is_v ? a.v_zero : a.k_zero;
      if (zero) zero[blk] = zp;
    }
  }
}

// The sequence's arrival ticket of an append: adds 1 << 24 to seq_lens[b] and returns
// the length before the append (low 24 bits). The last of the sequence's `arrivals`
// callers stores the incremented length (clearing the count). System scope: the
// read-modify-write happens at memory, past the per-XCD L2s.
__device__ __forceinline__ int append_ticket(int32_t* seq_lens, int b, int arrivals, int cap) {
  uint32_t* lens = reinterpret_cast<uint32_t*>(seq_lens);
  const uint32_t old = __hip_atomic_fetch_add(lens + b, 1u << 24, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_SYSTEM);
  const int len0 = static_cast<int>(old & 0xFFFFFFu);
  if ((old >> 24) == static_cast<uint32_t>(arrivals - 1))
    __hip_atomic_exchange(lens + b, static_cast<uint32_t>(len0 < cap ? len0 + 1 : len0),
                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  return len0;
}

// One decode step's append for row (b, h) = `row`: takes the sequence's arrival ticket
// (`arrivals` = heads workgroups per sequence, one per row) and appends the row's new
// K and V token. Called by all kThreads threads of the workgroup; returns the row's
// length after the append (unchanged when the row is at capacity, which the append
// leaves untouched). On return the new codes, scales and staging are visible to every
// thread of the workgroup (a workgroup barrier follows the stores).
template <int SCHEME, int D>
__device__ __forceinline__ int append_token(const AppendArgs& a, int b, int64_t row) {
  using G = QGeo<SCHEME, D>;
  __shared__ __align__(16) _Float16 xs[SCHEME == KVQ_INT4_SYM ? 2 * kBlock * D : 8];
  __shared__ float red[kAppendStats<SCHEME> * kWaves];
  __shared__ int len_shared;
  const int cap = a.max_blocks * kBlock;
  const int off = (threadIdx.x % G::kThreadsPerToken) * 8;
  const uint4 fresh[2] = {*reinterpret_cast<const uint4*>(a.k_new + row * D + off),
                          *reinterpret_cast<const uint4*>(a.v_new + row * D + off)};
  if (threadIdx.x == 0) len_shared = append_ticket(a.seq_lens, b, a.heads, cap);
  __syncthreads();
  const int len = len_shared;
  if (len >= cap) return len;  // uniform over the workgroup
  append_row<SCHEME, D>(a, row, len, fresh, xs, red);
  __syncthreads();
  return len + 1;
}

}  // namespace kvq
