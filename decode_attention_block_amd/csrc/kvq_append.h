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

// Maxima of N values over a group of NT threads (one wave, or a workgroup of NT
// threads); every thread of the group receives the results. For NT > kWave it contains
// one workgroup barrier (lds: N * NT / kWave floats); a single wave needs no LDS.
template <int N, int NT>
__device__ __forceinline__ void group_max(float (&v)[N], float* lds) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = wave_max(v[i]);
  if constexpr (NT > kWave) {
    constexpr int W = NT / kWave;
    const int w = (threadIdx.x % NT) / kWave;
    if ((threadIdx.x % kWave) == 0) {
#pragma unroll
      for (int i = 0; i < N; ++i) lds[i * W + w] = v[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i) {
      float r = lds[i * W];
#pragma unroll
      for (int k = 1; k < W; ++k) r = fmaxf(r, lds[i * W + k]);
      v[i] = r;
    }
  }
}

// The same over the kThreads threads of a block quantizer workgroup.
template <int N>
__device__ __forceinline__ void block_max(float (&v)[N], float* lds /* [N * kWaves] */) {
  group_max<N, kThreads>(v, lds);
}

template <int SCHEME, int D>
struct QGeo {
  static constexpr int kThreadsPerToken = D / 8;  // 8 channels (16 bytes) per thread
  static constexpr int kTokensPerPass = kThreads / kThreadsPerToken;
  static constexpr int kPasses = kBlock / kTokensPerPass;
  static constexpr int kRowBytes = SCHEME == KVQ_INT4_SYM ? D / 2 : D;
};

template <int SCHEME, int D, class T>
__device__ __forceinline__ void store_codes(uint8_t* token_row, int chunk, const T (&x)[8],
                                            const Divisor& s, int zpi, bool valid) {
  if constexpr (SCHEME == KVQ_INT4_SYM) {
    const uint32_t w = valid ? pack_int4x8(x, s) : 0u;
    *reinterpret_cast<uint32_t*>(token_row + chunk * 4) = w;
  } else if constexpr (SCHEME == KVQ_FP8_E4M3) {
    const uint2 w = valid ? pack_fp8x8(x, s) : make_uint2(0u, 0u);
    *reinterpret_cast<uint2*>(token_row + chunk * 8) = w;
  } else {
    const uint2 w = valid ? pack_uint8x8(x, s, zpi) : make_uint2(0u, 0u);
    *reinterpret_cast<uint2*>(token_row + chunk * 8) = w;
  }
}

// int4: dword f of lane `lane` of a block region in fragment order, coded from the
// block's fp16 values staged in LDS (xs[t * D + d], natural order); nibbles of tokens
// t >= ntok are zero. K: the 8 channels 32 (f % (D/32)) + 8 (lane / 16) .. of token
// 16 (f / (D/32)) + lane % 16 (one 16-byte read); V: tokens 32 (f % 2) + 8 (lane / 16) ..
// of channel 16 (f / 2) + lane % 16.
template <int D>
__device__ __forceinline__ uint32_t int4_fragment_word(const _Float16* xs, int ntok,
                                                       const Divisor& s, bool is_v, int lane,
                                                       int f) {
  constexpr int KS = D / 32;  // 32-channel K steps
  _Float16 x[8];
  uint32_t mask = 0xFFFFFFFFu;
  if (!is_v) {
    const int t = 16 * (f / KS) + lane % 16;
    if (t >= ntok) return 0u;
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    const h8 v = *reinterpret_cast<const h8*>(xs + t * D + 32 * (f % KS) + 8 * (lane / 16));
#pragma unroll
    for (int q = 0; q < 8; ++q) x[q] = v[q];
  } else {
    const int d = 16 * (f / 2) + lane % 16;
    const int t0 = 32 * (f % 2) + 8 * (lane / 16);
    const int n = ntok - t0;  // tokens of the 8 that exist
    if (n <= 0) return 0u;
    if (n < 8) mask = (1u << (4 * n)) - 1u;
#pragma unroll
    for (int q = 0; q < 8; ++q) x[q] = xs[(t0 + q) * D + d];
  }
  return pack_int4x8(x, s) & mask;
}

// uint8 / FP8: 16-byte chunk i of lane `lane` of a block region (bytes
// (i * 64 + lane) * 16 .. +15, i.e. 16 channels of one token), coded from the block's
// fp16 values staged in LDS (xs[t * D + d]) with scale s (and zero point zpi); tokens
// t >= ntok give zero bytes.
template <int SCHEME, int D>
__device__ __forceinline__ uint4 byte_codes_chunk(const _Float16* xs, int ntok, const Divisor& s,
                                                  int zpi, int lane, int i) {
  const int byte = (i * kWave + lane) * 16;
  const int t = byte / D, d0 = byte % D;
  if (t >= ntok) return make_uint4(0u, 0u, 0u, 0u);
  float x0[8], x1[8];
  unpack8(*reinterpret_cast<const uint4*>(xs + t * D + d0), x0);
  unpack8(*reinterpret_cast<const uint4*>(xs + t * D + d0 + 8), x1);
  uint2 c0, c1;
  if constexpr (SCHEME == KVQ_FP8_E4M3) {
    c0 = pack_fp8x8(x0, s);
    c1 = pack_fp8x8(x1, s);
  } else {
    c0 = pack_uint8x8(x0, s, zpi);
    c1 = pack_uint8x8(x1, s, zpi);
  }
  return make_uint4(c0.x, c0.y, c1.x, c1.y);
}

// int4: writes one block region (K or V) in fragment order from the block's fp16 values
// staged in LDS (xs[t * D + d], natural order); tokens t >= ntok give zero nibbles.
// Called by NT threads (tid = 0 .. NT-1).
template <int D, int NT = kThreads>
__device__ __forceinline__ void int4_write_block_from(const _Float16* xs, int ntok, const Divisor& s,
                                                      bool is_v, uint8_t* out, int tid) {
  constexpr int kChunks = 2 * D;  // 16-byte chunks per region (32 * D bytes)
  for (int c = tid; c < kChunks; c += NT) {
    const int lane = c % kWave, i = c / kWave;
    uint32_t w[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) w[r] = int4_fragment_word<D>(xs, ntok, s, is_v, lane, 4 * i + r);
    *reinterpret_cast<uint4*>(out + c * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// ---- append one token to one row (K and V) -----------------------------------------
// The append of one token to row `row` (length len before it, len < capacity) runs in
// three phases, each called by the NT threads (tid = 0 .. NT-1: a whole workgroup of NT
// threads, or one wave) that take part:
//   append_stage:  stages tokens 0..slot of the open block of both tensors in LDS (the
//                  new token from `fresh`, zeros after it) and reduces the block
//                  statistics before and after the token joins;
//   code writes:   a block whose statistic (absmax, or min and max) the token leaves
//                  unchanged keeps its scale and gets only the new token's codes;
//                  otherwise (and for a block the token opens) the whole block is
//                  re-quantized from the staged values (append_write_codes, or the
//                  register-resident variant of the fused decode step);
//   append_finish: the new token's fp16 staging and the changed scales (zero points).
// fresh[kv] = this thread's 16 bytes of the new K (kv = 0) or V (kv = 1) token,
// channels (tid % (D/8)) * 8 .. +7. xs: 2 * kBlock * D fp16 of LDS, 16-byte aligned;
// red: kAppendStats<SCHEME> * NT / kWave floats of LDS (unused for one wave).
template <int SCHEME>
constexpr int kAppendStats = SCHEME != KVQ_UINT8_ASYM ? 4 : 8;  // old and new, K and V

// Index of the block that receives the token of row `row` (= b * heads + h) at position
// len (see block_slot).
__device__ __forceinline__ int64_t append_slot(const AppendArgs& a, int64_t row, int len) {
  return block_slot(a.block_table, a.num_pages, a.heads, a.max_blocks,
                    static_cast<int>(row / a.heads), static_cast<int>(row % a.heads),
                    len / kBlock);
}

struct AppendPlan {  // one tensor's outcome: the block's scale, zero point, re-quantized?
  float s, zp;
  bool full;
};

struct BlockScales {
  float ks, kz, vs, vz;
};

// The staged tokens of the open block as loaded by append_stage_load: pass p of tensor kv
// holds this thread's 16 bytes of token p * (NT / (D/8)) + tid / (D/8).
template <int D, int NT>
struct StagedTokens {
  static constexpr int kPasses = (kBlock + NT / (D / 8) - 1) / (NT / (D / 8));
  uint4 v[2][kPasses];
};

// Requests the staged tokens 0 .. slot-1 of the open block (slot = len % 64). They are
// read through buffer resources that end at token `slot`: every lane loads
// unconditionally and the loads past the end return zeros without touching memory.
template <int D, int NT>
__device__ __forceinline__ void append_stage_load(const AppendArgs& a, int64_t row, int len,
                                                  int tid, StagedTokens<D, NT>& g) {
  constexpr int TPT = D / 8;
  constexpr int TPP = NT / TPT;
  const int tr = tid / TPT;
  const int chunk = tid % TPT;
  const int slot = len % kBlock;
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (kv ? a.v_tail : a.k_tail) + row * kBlock * D, 0, slot * D * 2, kBufferRsrcWord3);
#pragma unroll
    for (int p = 0; p < StagedTokens<D, NT>::kPasses; ++p)
      g.v[kv][p] = load_b128<0>(rs, ((p * TPP + tr) * D + chunk * 8) * 2, 0);
  }
}

// One wave requests the staged tokens 0 .. slot-1 of the open block straight into LDS,
// in xs's layout (tensor kv at xs + kv * 64 * D, token t at t * D): each request moves
// 1 KiB, lane l's 16 bytes to byte 16 l of it, and the lanes past the end of the buffer
// resource (tokens >= slot) write zeros.
template <int D>
__device__ __forceinline__ void append_stage_load_lds(const AppendArgs& a, int64_t row, int len,
                                                      int lane, _Float16* xs) {
  typedef __attribute__((address_space(3))) void* lds_t;
  const int slot = len % kBlock;
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (kv ? a.v_tail : a.k_tail) + row * kBlock * D, 0, slot * D * 2, kBufferRsrcWord3);
#pragma unroll
    for (int p = 0; p < kBlock * D * 2 / 1024; ++p)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_t)(xs + kv * kBlock * D + p * 512), 16,
                                               lane * 16, p * 1024, 0, 0);
  }
}

// The staged tokens and the new one into xs, the statistics, the plan. staged(kv, p, t,
// chunk) gives this thread's 16 bytes of token t of tensor kv (pass p). kInLds: the
// tokens, the new one included, are in xs already (staged reads them there).
template <int SCHEME, int D, int NT, bool kInLds = false, class Staged>
__device__ __forceinline__ void append_stage_reduce(int len, int tid, Staged staged,
                                                    const uint4 (&fresh)[2], _Float16* xs,
                                                    float* red, AppendPlan (&plan)[2]) {
  constexpr int TPT = D / 8;             // threads per token row (16 bytes each)
  constexpr int TPP = NT / TPT;          // tokens per pass
  constexpr int PASSES = (kBlock + TPP - 1) / TPP;  // the last may run past the block
  constexpr int NS = kAppendStats<SCHEME> / 2;  // statistics per tensor
  const int tr = tid / TPT;
  const int chunk = tid % TPT;
  const int slot = len % kBlock;

  float st[2 * NS];
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    float amax_o = 0.0f, mn_o = __builtin_inff(), mx_o = -__builtin_inff();
    float amax_n = 0.0f, mn_n = __builtin_inff(), mx_n = -__builtin_inff();
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int t = p * TPP + tr;
      uint4 raw;  // zeros past the slot
      if constexpr (kInLds) {
        raw = staged(kv, p, t, chunk);
      } else {
        raw = t == slot ? fresh[kv] : staged(kv, p, t, chunk);
        if (PASSES * TPP == kBlock || t < kBlock)
          *reinterpret_cast<uint4*>(xs + kv * kBlock * D + t * D + chunk * 8) = raw;
      }
      float x[8];
      unpack8(raw, x);
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
    if constexpr (SCHEME != KVQ_UINT8_ASYM) {  // absmax schemes
      st[kv * NS + 0] = amax_o;
      st[kv * NS + 1] = amax_n;
    } else {
      st[kv * NS + 0] = -mn_o;
      st[kv * NS + 1] = mx_o;
      st[kv * NS + 2] = -mn_n;
      st[kv * NS + 3] = mx_n;
    }
  }
  // Makes the LDS stores visible to the group: the workgroup barrier inside group_max,
  // or for one wave the in-order execution of its LDS requests (the wave barrier keeps
  // the compiler from moving reads of other lanes' values above the stores).
  if constexpr (NT == kWave) __builtin_amdgcn_wave_barrier();
  group_max<2 * NS, NT>(st, red);
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    const float* sv = st + kv * NS;
    plan[kv].zp = 0.0f;
    if constexpr (SCHEME != KVQ_UINT8_ASYM) {  // absmax schemes
      plan[kv].full = slot == 0 || sv[0] != sv[1];
      plan[kv].s = SCHEME == KVQ_INT4_SYM ? int4_scale(sv[1]) : fp8_scale(sv[1]);
    } else {
      plan[kv].full = slot == 0 || sv[0] != sv[2] || sv[1] != sv[3];
      uint8_scale_zero(-sv[2], sv[3], plan[kv].s, plan[kv].zp);
    }
  }
}

template <int SCHEME, int D, int NT>
__device__ __forceinline__ void append_stage(const AppendArgs& a, int64_t row, int len, int tid,
                                             const uint4 (&fresh)[2], _Float16* xs, float* red,
                                             AppendPlan (&plan)[2]) {
  StagedTokens<D, NT> g;
  append_stage_load<D, NT>(a, row, len, tid, g);
  append_stage_reduce<SCHEME, D, NT>(
      len, tid, [&](int kv, int p, int, int) { return g.v[kv][p]; }, fresh, xs, red, plan);
}

// Code writes through memory (see above): the whole block, or the new token's codes.
template <int SCHEME, int D, int NT>
__device__ __forceinline__ void append_write_codes(const AppendArgs& a, int64_t row, int len,
                                                   int tid, const _Float16* xs,
                                                   const AppendPlan (&plan)[2]) {
  constexpr int TPT = D / 8;
  constexpr int TPP = NT / TPT;
  constexpr int PASSES = kBlock / TPP;
  constexpr int RB = SCHEME == KVQ_INT4_SYM ? D / 2 : D;  // code bytes per token
  const int tr = tid / TPT;
  const int chunk = tid % TPT;
  const int slot = len % kBlock;
  const int64_t blk = append_slot(a, row, len);
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    const bool is_v = kv != 0;
    const Divisor s(plan[kv].s);
    uint8_t* codes = (is_v ? a.v_codes : a.k_codes) + blk * kBlock * RB;
    const _Float16* xt = xs + kv * kBlock * D;  // tokens 0..slot, zeros after
    if constexpr (SCHEME == KVQ_INT4_SYM) {
      if (plan[kv].full) {
        int4_write_block_from<D, NT>(xt, slot + 1, s, is_v, codes, tid);
      } else if (!is_v) {
        // K: the new token's D/8 dwords (8 channels each)
        constexpr int KS = D / 32;
        for (int idx = tid; idx < D / 8; idx += NT) {
          const int ks = idx / 4, g = idx % 4;
          const int lane = 16 * g + slot % 16, f = (slot / 16) * KS + ks;
          *reinterpret_cast<uint32_t*>(codes + int4_dword_offset(lane, f)) =
              int4_fragment_word<D>(xt, slot + 1, s, false, lane, f);
        }
      } else {
        // V: each channel's new nibble shares a dword with 7 other tokens; with the
        // scale unchanged, rebuilding the dword from the staged values reproduces the
        // stored nibbles (and zeros past the token), so the cache is never read back
        const int ks = slot / 32, g = (slot % 32) / 8;
        for (int d = tid; d < D; d += NT) {
          const int lane = 16 * g + d % 16, f = 2 * (d / 16) + ks;
          *reinterpret_cast<uint32_t*>(codes + int4_dword_offset(lane, f)) =
              int4_fragment_word<D>(xt, slot + 1, s, true, lane, f);
        }
      }
    } else {
      // natural order: each thread codes its own staged 8 channels of each token
      const int zpi = static_cast<int>(plan[kv].zp);
#pragma unroll
      for (int p = 0; p < PASSES; ++p) {
        const int t = p * TPP + tr;
        if (plan[kv].full || t == slot) {
          float x[8];
          unpack8(*reinterpret_cast<const uint4*>(xt + t * D + chunk * 8), x);
          store_codes<SCHEME, D>(codes + t * RB, chunk, x, s, zpi, t <= slot);
        }
      }
    }
  }
}

// The new token's fp16 staging and the scales (zero points) of re-quantized blocks.
template <int D, int NT>
__device__ __forceinline__ BlockScales append_finish(const AppendArgs& a, int64_t row, int len,
                                                     int tid, const uint4 (&fresh)[2],
                                                     const AppendPlan (&plan)[2]) {
  constexpr int TPT = D / 8;
  constexpr int TPP = NT / TPT;
  const int slot = len % kBlock;
  const int64_t blk = append_slot(a, row, len);
  if (tid / TPT == slot % TPP) {
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      uint16_t* tail = (kv ? a.v_tail : a.k_tail) + row * kBlock * D;
      *reinterpret_cast<uint4*>(tail + slot * D + (tid % TPT) * 8) = fresh[kv];
    }
  }
  if (tid == 0) {
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      if (!plan[kv].full) continue;
      (kv ? a.v_scale : a.k_scale)[blk] = plan[kv].s;
      float* zero = kv ? a.v_zero : a.k_zero;
      if (zero) zero[blk] = plan[kv].zp;
    }
  }
  return {plan[0].s, plan[0].zp, plan[1].s, plan[1].zp};
}

// ---- int4 tail block kept in registers (fused decode step) ---------------------------
// One wave's view of an int4 block region: lane l holds chunk i (i < D/32) = bytes
// ((i * 64) + l) * 16 .. +15, i.e. its matrix-core fragments.

// The new codes of one int4 tensor's open block, built in registers by one wave: r
// receives chunk i (i < D/32) of the lane, i.e. bytes ((i * 64) + lane) * 16 .. +15 of
// the block's region, coded from the staged values (tokens 0..slot, zeros after) with
// the block's scale after the append. Whether or not the token changed the scale this
// is the block's content: every stored code of the open block is the code of its staged
// value under the block's current scale (prefill, re-quantization and appends all code
// that way), so the block need not be read back. Nothing is written here: the wave
// writes r whole at the end of the decode step, after the stream of the row's other
// blocks (see the step kernel).
template <int D>
__device__ __forceinline__ void int4_tail_fragments(const _Float16* xt, int slot,
                                                    const AppendPlan& pl, bool is_v, int lane,
                                                    uint4 (&r)[D / 32]) {
  constexpr int LOADS = D / 32;  // chunks per lane
  const Divisor s(pl.s);
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    uint32_t w[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) w[c] = int4_fragment_word<D>(xt, slot + 1, s, is_v, lane, 4 * i + c);
    r[i] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// The sequence's arrival ticket of an append, in two parts. append_ticket adds 1 << 24 to
// seq_lens[b], as one request of the whole wave whose lanes past the first fall outside a
// 4-byte buffer resource and so do not touch memory (a branch around a one-lane atomic
// would merge its result with the other lanes' value and make the compiler wait for it
// at once); the result, meaningful in lane 0, is the count and length before the add.
// append_ticket_done then lets the last of the sequence's `arrivals` workgroups store
// the length after the append (the length before it at capacity), clearing the count.
// System scope (cache policy sc1): the read-modify-writes happen at memory, past the
// per-XCD L2s.
constexpr int kTicketPolicy = 16;  // sc1

__device__ __forceinline__ uint32_t append_ticket(int32_t* seq_lens, int b, int lane) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(seq_lens + b, 0, 4, kBufferRsrcWord3);
  return static_cast<uint32_t>(__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(
      1 << 24, rs, lane == 0 ? 0 : 4, 0, kTicketPolicy));
}

__device__ __forceinline__ void append_ticket_done(int32_t* seq_lens, int b, int arrivals,
                                                   int cap, uint32_t old, int lane) {
  if (lane != 0 || (old >> 24) != static_cast<uint32_t>(arrivals - 1)) return;
  const int len0 = static_cast<int>(old & 0xFFFFFFu);
  __hip_atomic_exchange(reinterpret_cast<uint32_t*>(seq_lens) + b,
                        static_cast<uint32_t>(len0 < cap ? len0 + 1 : len0), __ATOMIC_RELAXED,
                        __HIP_MEMORY_SCOPE_SYSTEM);
}

// The append of row (b, h) = `row` by the kThreads threads of a workgroup (`heads`
// workgroups per sequence, one per row): the row's new K and V token (nothing for a row
// at capacity). The length is read first with a plain load (the arrival count in the top
// 8 bits masked off) and the sequence's ticket taken by wave 0 only once the workgroup
// has its staged tokens: the tickets of a sequence's workgroups are performed one after
// another at memory, and taken first they held every workgroup's loads behind the
// queue (8K workload: 8.7 us per call). Every workgroup has read the length before it
// takes its ticket, so the last arrival's store of the new length comes after all the
// reads; the ticket's result is used only once the workgroup's writes are issued.
template <int SCHEME, int D>
__device__ __forceinline__ void append_token(const AppendArgs& a, int b, int64_t row) {
  __shared__ __align__(16) _Float16 xs[2 * kBlock * D];
  __shared__ float red[kAppendStats<SCHEME> * kWaves];
  __shared__ int len_shared;
  const int cap = a.max_blocks * kBlock;
  const int lane = threadIdx.x % kWave;
  const bool ticket_wave = threadIdx.x < kWave;
  const int off = (threadIdx.x % (D / 8)) * 8;
  const uint4 fresh[2] = {*reinterpret_cast<const uint4*>(a.k_new + row * D + off),
                          *reinterpret_cast<const uint4*>(a.v_new + row * D + off)};
  if (threadIdx.x == 0)
    len_shared = static_cast<int>(static_cast<uint32_t>(a.seq_lens[b]) & 0xFFFFFFu);
  __syncthreads();
  const int len = len_shared;
  uint32_t old = 0;
  if (len >= cap) {  // uniform over the workgroup: nothing to append; the arrival counts
    if (ticket_wave) {
      old = append_ticket(a.seq_lens, b, lane);
      append_ticket_done(a.seq_lens, b, a.heads, cap, old, lane);
    }
    return;
  }
  AppendPlan plan[2];
  append_stage<SCHEME, D, kThreads>(a, row, len, threadIdx.x, fresh, xs, red, plan);
  if (ticket_wave) old = append_ticket(a.seq_lens, b, lane);
  append_write_codes<SCHEME, D, kThreads>(a, row, len, threadIdx.x, xs, plan);
  append_finish<D, kThreads>(a, row, len, threadIdx.x, fresh, plan);
  if (ticket_wave) append_ticket_done(a.seq_lens, b, a.heads, cap, old, lane);
}

}  // namespace kvq
