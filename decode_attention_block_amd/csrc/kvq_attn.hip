// kvq_attn.hip — single-token decode attention over the block-quantized cache.
//
// Attention is textbook scaled dot-product attention of one query row over the
// dequantized cache. The context is cut into splits of whole 64-token blocks handled by
// independent workgroups (the schedulable sub-blocks of the chunked attention in page
// "第一章：DeepSeek R1推理模型性能跃迁全景概览" chapter 1), and a second kernel merges
// the splits by their log-sum-exp. Decode attention at long context is bound by reads
// of the cache (that page's §2.3 and page "DeepSeek-R1推理延迟骤降41.8%？…" §2.1), so
// the kernel is written around streaming the packed codes once at full HBM rate:
//
//  * every wave-wide load is a 16-byte-per-lane read of 1 KiB of consecutive codes;
//    lane l holds channel chunk l % LPT of token group l / LPT (LPT = 16-byte chunks
//    per token row), so a 64-token block is LPT loads per tensor per wave;
//  * codes are never converted one by one: a mask turns two stored 4-bit (or 8-bit)
//    codes into a pair of fp16 subnormals u * 2^-24 (or u * 2^-20 for a high nibble),
//    u the unsigned stored code, which v_fma_mix_f32 reads directly (fp16 operand,
//    binary32 product and accumulate, one rounding) against the binary32 query (QK^T)
//    and the binary32 weights (P.V). For QK^T the code offset (8 for int4, the zero
//    point for uint8) is removed once per score; for P.V it is removed from each fp16
//    pair by a packed fp16 add (exact), since a dominant weight on codes equal to the
//    offset would otherwise cancel catastrophically. The power-of-two units are
//    removed once per score / per split. (The
//    fp16 dot-product instruction was measured to round its result far more coarsely
//    than binary32, so it is not used.)
//  * the block scale is folded into the score (K) and into the weight (V), once per
//    token per lane;
//  * online softmax in base 2 with a wave-uniform running max: the rescale of the
//    accumulators happens only when a block raises the max;
//  * at the end of a split the waves' states are merged through LDS into one partial
//    (max, sum, o[D]) per split; in fused mode (decode_attn_qkv) the last workgroup of
//    each row to finish merges the row's partials itself, otherwise the combine kernel
//    does (decode_attn_split + decode_attn_combine).
#include "kvq_append.h"

namespace kvq {
namespace {

constexpr int kSplitWaves = 4;

// Geometry of the vector-ALU kernel over the 8-bit caches (uint8, FP8): one code byte
// per channel, natural order; the int4 cache has its own kernels (matrix cores).
template <int SCHEME, int D>
struct AGeo {
  static_assert(SCHEME != KVQ_INT4_SYM, "the int4 cache has its own kernels");
  static constexpr int kRowBytes = D;               // bytes per token
  static constexpr int kLPT = kRowBytes / 16;       // lanes per token row
  static constexpr int kGroups = kWave / kLPT;      // tokens per wave-wide load
  static constexpr int kTPL = kLPT;                 // tokens per lane per block
  static constexpr int kDPL = 16;                   // channels per lane
};

__device__ __forceinline__ half2_t as_h2(uint32_t w) { return __builtin_bit_cast(half2_t, w); }

// 16-byte load of codes that are read once per call, through a buffer resource
// (voffset per lane, soffset uniform): non-temporal, so the stream does not evict what
// is reused (scales, partials) from the caches.
__device__ __forceinline__ uint4 load_stream(__amdgpu_buffer_rsrc_t rsrc, int voffset, int soffset) {
  return load_b128<2 /* non-temporal */>(rsrc, voffset, soffset);
}

// Partial states cross workgroups (and L2 slices: the eight XCDs do not share an L2)
// through agent-scope atomic stores and agent-coherent loads (merge_row), which go to
// memory instead of a possibly stale L2 line; a full device-scope fence would write
// back and invalidate the whole L2 in every workgroup.
__device__ __forceinline__ void store_shared(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Publication of a workgroup's partial state before its arrival ticket. Every wave
// waits until its own vector memory requests have completed (s_waitcnt vmcnt(0);
// expcnt and lgkmcnt left at their maxima, i.e. not waited for): the agent-scope
// stores above are acknowledged only once they have been written through to memory, so
// after the wait they are visible to every workgroup on any XCD. The workgroup
// barrier that follows then orders all waves' completed stores before thread 0's
// ticket, which is performed at memory. A workgroup-scope release fence would not do
// this: outside thread-group-split mode it compiles to nothing, and the barrier alone
// lets a wave arrive with its stores still in flight. The reader (the last arriver)
// issues its loads only after the ticket's result has returned and a barrier, and every
// one of them carries the agent-coherence bit (merge_row), so none can be served by a
// stale cache line.
__device__ __forceinline__ void wait_own_stores() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0) expcnt(7) lgkmcnt(15) on gfx9-family chips
}

// Log-sum-exp merge of the n partial states of one row into its fp16 output channel d:
// M = max_j m_j, o = sum_j o_j 2^(m_j - M) / sum_j l_j 2^(m_j - M); zeros when n = 0.
// A row of at most kMergeChunk splits is read in one batch (one memory round trip);
// longer rows kMergeChunk splits at a time, all of a chunk's loads issued before any is
// used, in two passes (the max, then the sums): about 2 n / kMergeChunk round trips
// instead of 2 n. The sums run over j in order either way, so the result does not
// depend on the batching. They are buffer loads over exactly the row's partials, every
// offset in the per-lane (VGPR) operand, which the range check covers dword by dword
// (also where the compiler merges neighbouring loads), so loads past the n-th return 0
// without touching memory and are masked out. In the fused merge (kCoherent) they carry
// the agent-scope coherence bit sc1, so that they read what other workgroups stored with
// agent-scope atomic stores rather than a possibly stale L2 line, as an agent-scope
// atomic load would, but without an atomic's ordering, which made every load wait for
// the previous one.
constexpr int kMergeChunk = 8;
constexpr int kCachePolicyAgent = 16;  // sc1

template <int D, bool kCoherent>
__device__ __forceinline__ void merge_row(const AttnArgs& a, int64_t row, int n, int d) {
  _Float16 r = 0;
  if (n > 0) {
    constexpr int aux = kCoherent ? kCachePolicyAgent : 0;
    const __amdgpu_buffer_rsrc_t mlr = __builtin_amdgcn_make_buffer_rsrc(
        a.ws_ml + row * a.n_split * 2, 0, n * 2 * 4, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t por = __builtin_amdgcn_make_buffer_rsrc(
        a.ws_o + row * a.n_split * D, 0, n * D * 4, kBufferRsrcWord3);
    auto ld = [](__amdgpu_buffer_rsrc_t rs, int voff) {
      return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, voff, 0, aux));
    };
    float M = -__builtin_inff();
    float L = 0.0f, acc = 0.0f;
    if (n <= kMergeChunk) {  // one batch: every partial state of the row at once
      float m[kMergeChunk], l[kMergeChunk], o[kMergeChunk];
#pragma unroll
      for (int k = 0; k < kMergeChunk; ++k) {
        m[k] = ld(mlr, k * 8);
        l[k] = ld(mlr, k * 8 + 4);
        o[k] = ld(por, (k * D + d) * 4);
      }
      __builtin_amdgcn_sched_barrier(0);  // every request out before the first use
#pragma unroll
      for (int k = 0; k < kMergeChunk; ++k)
        if (k < n) M = fmaxf(M, m[k]);
#pragma unroll
      for (int k = 0; k < kMergeChunk; ++k) {
        if (k < n) {
          const float w = __builtin_amdgcn_exp2f(m[k] - M);
          L = __builtin_fmaf(w, l[k], L);
          acc = __builtin_fmaf(w, o[k], acc);
        }
      }
      a.out[row * D + d] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(acc / L));
      return;
    }
    for (int j0 = 0; j0 < n; j0 += kMergeChunk) {
      float m[kMergeChunk];
#pragma unroll
      for (int k = 0; k < kMergeChunk; ++k) m[k] = ld(mlr, (j0 + k) * 8);
#pragma unroll
      for (int k = 0; k < kMergeChunk; ++k)
        if (j0 + k < n) M = fmaxf(M, m[k]);
    }
    for (int j0 = 0; j0 < n; j0 += kMergeChunk) {
      float m[kMergeChunk], l[kMergeChunk], o[kMergeChunk];
#pragma unroll
      for (int k = 0; k < kMergeChunk; ++k) {
        m[k] = ld(mlr, (j0 + k) * 8);
        l[k] = ld(mlr, (j0 + k) * 8 + 4);
        o[k] = ld(por, ((j0 + k) * D + d) * 4);
      }
#pragma unroll
      for (int k = 0; k < kMergeChunk; ++k) {
        if (j0 + k < n) {
          const float w = __builtin_amdgcn_exp2f(m[k] - M);
          L = __builtin_fmaf(w, l[k], L);
          acc = __builtin_fmaf(w, o[k], acc);
        }
      }
    }
    r = static_cast<_Float16>(acc / L);
  }
  a.out[row * D + d] = __builtin_bit_cast(uint16_t, r);
}

// The fused merge of R rows (row0 + k * step, k < R) of channel d by one thread, as
// merge_row<D, true> each; with at most kMergeChunk splits the loads of all R rows are
// issued before any is used (one memory round trip for the R rows instead of R).
template <int D, int R>
__device__ __forceinline__ void merge_rows(const AttnArgs& a, int64_t row0, int step, int n,
                                           int d) {
  if (n <= 0 || n > kMergeChunk) {
#pragma unroll
    for (int k = 0; k < R; ++k) merge_row<D, true>(a, row0 + k * step, n, d);
    return;
  }
  auto ld = [](__amdgpu_buffer_rsrc_t rs, int voff) {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_raw_buffer_load_b32(rs, voff, 0, kCachePolicyAgent));
  };
  float m[R][kMergeChunk], l[R][kMergeChunk], o[R][kMergeChunk];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int64_t row = row0 + k * step;
    const __amdgpu_buffer_rsrc_t mlr = __builtin_amdgcn_make_buffer_rsrc(
        a.ws_ml + row * a.n_split * 2, 0, n * 2 * 4, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t por = __builtin_amdgcn_make_buffer_rsrc(
        a.ws_o + row * a.n_split * D, 0, n * D * 4, kBufferRsrcWord3);
#pragma unroll
    for (int j = 0; j < kMergeChunk; ++j) {
      m[k][j] = ld(mlr, j * 8);
      l[k][j] = ld(mlr, j * 8 + 4);
      o[k][j] = ld(por, (j * D + d) * 4);
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // every request out before the first use
#pragma unroll
  for (int k = 0; k < R; ++k) {
    float M = -__builtin_inff(), L = 0.0f, acc = 0.0f;
#pragma unroll
    for (int j = 0; j < kMergeChunk; ++j)
      if (j < n) M = fmaxf(M, m[k][j]);
#pragma unroll
    for (int j = 0; j < kMergeChunk; ++j) {
      if (j < n) {
        const float w = __builtin_amdgcn_exp2f(m[k][j] - M);
        L = __builtin_fmaf(w, l[k][j], L);
        acc = __builtin_fmaf(w, o[k][j], acc);
      }
    }
    a.out[(row0 + k * step) * D + d] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(acc / L));
  }
}

// ---- the split of a row ---------------------------------------------------------------
// Blocks [begin, end) of a row of nb blocks that split `split` streams, and the number of
// splits n of the row (the merge's count). A caller's plan (a.bps > 0) cuts every row
// into a.bps-block pieces. With a.bps == 0 the split is chosen here, from the lengths of
// all rows, so that a batch of unequal lengths is balanced without the host knowing
// them: the whole batch's blocks T = heads * sum_b ceil(len_b / 64) are shared out in
// chunks of about T / plan_target blocks, a row of nb blocks is cut into
// n = ceil(nb / chunk) equal pieces (at most a.n_split), and rows no longer than a chunk
// stay whole. Rows of equal length therefore get the split the host would choose for
// them (one piece per row once the rows fill the GPU), and in a ragged batch the long
// rows are cut so that no workgroup streams much more than a chunk (the chunked,
// schedulable sub-blocks of page "第一章：DeepSeek R1推理模型性能跃迁全景概览" chapter 1).
// Every workgroup of a row, and the combine kernel, compute the same n from the same
// lengths, which no call changes while it runs.
struct SplitRange {
  int begin, end, n;
};

// Sum over all 64 lanes, in the same order in every wave (DPP within rows of 16 lanes,
// then the four rows' sums read out and added in order).
__device__ __forceinline__ float row16_sum_all(float v) {
  v += dpp<kDppQuadXor1>(v);
  v += dpp<kDppQuadXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppRowMirror>(v);
  const int iv = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ int clamp_len(const AttnArgs& a, int len, int cap) {
  return len < 0 ? 0 : min(len, min(a.max_len, cap));
}

// Whether the rows alone reach the automatic plan's workgroup target.
__device__ __forceinline__ bool fills_gpu(const AttnArgs& a) {
  return static_cast<int64_t>(a.batch) * a.heads >= a.plan_target;
}

// The batch's blocks T = sum_b ceil(len_b / 64) for the device plan, wave-uniform.
// Every lane adds up the blocks of sequences lane, lane + 64, ..., then the wave
// (binary32: exact up to 2^24 blocks, and beyond that rounded the same way in every
// workgroup, which is all the plan needs: every workgroup of a row must find the same
// n). The total is made wave-uniform explicitly (readfirstlane): left as a per-lane
// value it would make the split bounds, and with them the streaming loop's trip count,
// divergent for the compiler, which then rebuilds the loop around them (the 8K int4
// attention measured 49.4 us instead of 41.8 us).
__device__ __forceinline__ float batch_blocks(const AttnArgs& a, int cap) {
  float t = 0.0f;
  for (int i = threadIdx.x % kWave; i < a.batch; i += kWave)
    t += static_cast<float>((clamp_len(a, a.seq_lens[i], cap) + kBlock - 1) / kBlock);
  t = row16_sum_all(t);
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, t)));
}

// split_range with the batch's blocks t (batch_blocks; unused for a caller's plan).
__device__ __forceinline__ SplitRange split_range_of(const AttnArgs& a, int nb, int split,
                                                     float t) {
  SplitRange r;
  int piece = a.bps;
  if (a.bps > 0) {
    r.n = (nb + a.bps - 1) / a.bps;
  } else {
    const float work = t * static_cast<float>(a.heads);
    const float chunk = fmaxf(ceilf(work / static_cast<float>(a.plan_target)), 1.0f);
    float pieces = ceilf(static_cast<float>(nb) / chunk);
    // once the rows fill the GPU, a row that is cut at all is cut in pieces of about
    // 1/(1.5 target) of the batch's blocks (up to the grid's three split columns), which
    // the column pairing (paired_sequence) can spread over compute units more evenly
    // than halves; rows of equal length stay whole as before
    if (fills_gpu(a) && pieces > 1.0f)
      pieces = ceilf(static_cast<float>(nb) /
                     fmaxf(ceilf(work / (1.5f * static_cast<float>(a.plan_target))), 1.0f));
    const int n_max = static_cast<int>(fminf(pieces, static_cast<float>(a.n_split)));
    // equal pieces of ceil(nb / n_max) blocks; the count is recomputed from that size,
    // since n_max pieces of it may cover the row with fewer (11 blocks in at most 8
    // pieces: pieces of 2 blocks, 6 of them), and the merge must wait for exactly the
    // splits that hold blocks
    piece = nb > 0 ? (nb + n_max - 1) / n_max : 1;
    r.n = nb > 0 ? (nb + piece - 1) / piece : 0;
  }
  r.begin = split * piece;
  r.end = min(r.begin + piece, nb);
  return r;
}

__device__ __forceinline__ SplitRange split_range(const AttnArgs& a, int nb, int split, int cap) {
  return split_range_of(a, nb, split, a.bps > 0 ? 0.0f : batch_blocks(a, cap));
}

// Which sequence's row a workgroup of split column z >= 1 streams, in the automatic plan
// once the rows fill the GPU (the grid then has three split columns, and the long rows
// of a ragged batch are cut in two or three pieces). The dispatcher sends workgroup i to
// XCD i % 8 and fills each XCD's compute units in turn, and a column of the grid is a
// whole number of such rounds, so workgroup (h, b, z) runs on the compute unit of
// (h, b, 0) (a placement probe on MI355X: all 256 of 256 for z = 1): all pieces of a
// cut row would stream on one CU while the CUs of uncut rows stream one. Column z
// therefore takes piece z of sequence sigma_z(b) of the same head (same XCD): after
// column 0 (each position its own first piece), sigma_z pairs the positions' loads so
// far in ascending order with the sequences' z-th pieces in descending order (ties by
// index; a row of fewer pieces has empty ones), computed from the lengths by every
// wave for batches of at most 64 sequences (larger batches keep sigma_z(b) = b). Each
// sigma_z is a permutation, so every piece is streamed exactly once whatever the
// placement; only the balance depends on it.
constexpr int kPairedColumns = 3;

__device__ __forceinline__ int paired_sequence(const AttnArgs& a, int b, int z, int cap,
                                               float t) {
  if (a.batch > kWave) return b;
  const int c = threadIdx.x % kWave;
  int piece[kPairedColumns] = {0, 0, 0};
  if (c < a.batch) {
    const int nb = (clamp_len(a, a.seq_lens[c], cap) + kBlock - 1) / kBlock;
    const SplitRange r = split_range_of(a, nb, 0, t);
    const int size = r.end - r.begin;
#pragma unroll
    for (int k = 0; k < kPairedColumns; ++k)
      piece[k] = k < r.n ? min(size, nb - k * size) : 0;
  }
  int load = c < a.batch ? piece[0] : 0x7FFFFFFF;
#pragma unroll
  for (int col = 1; col < kPairedColumns; ++col) {
    const int pc = c < a.batch ? piece[col] : -1;
    int rank_load = 0, rank_piece = 0;
    for (int d = 0; d < a.batch; ++d) {
      const int ld = __builtin_amdgcn_readlane(load, d);
      const int pd = __builtin_amdgcn_readlane(pc, d);
      rank_load += ld < load || (ld == load && d < c);
      rank_piece += pd > pc || (pd == pc && d < c);
    }
    if (col == z) {
      const int i = __builtin_amdgcn_readlane(rank_load, b);
      const uint64_t m = __builtin_amdgcn_ballot_w64(c < a.batch && rank_piece == i);
      return __builtin_amdgcn_readfirstlane(static_cast<int>(__builtin_ctzll(m)));
    }
    // position c takes the piece of the sequence whose piece rank equals its load rank
    int add = 0;
    for (int d = 0; d < a.batch; ++d)
      if (__builtin_amdgcn_readlane(rank_piece, d) == rank_load)
        add = __builtin_amdgcn_readlane(pc, d);
    load += add;
  }
  return b;
}

// End of a split: thread d < D holds channel d of the split's merged (unnormalised)
// output, M and L its max and weight sum. A single-split row in fused mode is written
// out directly. Otherwise the partial goes to the workspace; in fused mode the
// workgroup then waits until its stores have reached memory, takes an arrival ticket
// for its row, and the last workgroup to arrive merges all of the row's partials and
// resets the row's counter.
template <int D>
__device__ __forceinline__ void finish_split(const AttnArgs& a, int64_t row, int split, int n_row,
                                             float od, float M, float L) {
  const int tid = threadIdx.x;
  if (a.fused && n_row == 1) {
    if (tid < D) a.out[row * D + tid] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(od / L));
    return;
  }
  float* po = a.ws_o + (row * a.n_split + split) * D;
  float* ml = a.ws_ml + (row * a.n_split + split) * 2;
  if (!a.fused) {
    if (tid < D) po[tid] = od;
    if (tid == 0) {
      ml[0] = M;
      ml[1] = L;
    }
    return;
  }
  if (tid < D) store_shared(po + tid, od);
  if (tid == 0) {
    store_shared(ml, M);
    store_shared(ml + 1, L);
  }
  __shared__ uint32_t ticket;
  wait_own_stores();  // every wave's partial stores have reached memory
  __syncthreads();
  // system scope: the read-modify-write is performed at memory, past the per-XCD L2s
  if (tid == 0)
    ticket = __hip_atomic_fetch_add(a.counters + row, 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_SYSTEM);
  __syncthreads();
  if (ticket == static_cast<uint32_t>(n_row - 1)) {
    if (tid < D) merge_row<D, true>(a, row, n_row, tid);
    if (tid == 0)
      __hip_atomic_store(a.counters + row, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

// Marks the query's raw bits as produced at this point (an empty asm statement that the
// compiler must keep after the memory requests issued before it): the operand built
// from them is then not hoisted above the stream's first requests, and the wait for the
// query's load lands here.
__device__ __forceinline__ uint4 query_ready(uint4 r) {
  asm volatile("" : "+v"(r.x), "+v"(r.y), "+v"(r.z), "+v"(r.w) : : "memory");
  return r;
}

template <int SCHEME, int D>
struct Query {
  using G = AGeo<SCHEME, D>;
  // The lane's query channels as loaded: fp16, two per register (channel 2k in the low
  // half). v_fma_mix_f32 reads either half as an fp16 operand.
  uint32_t qh[G::kDPL / 2];
  float sum;  // sum of the lane's query channels

  static constexpr int kLoads = G::kDPL / 8;
  uint4 raw[kLoads];  // the lane's channels as requested

  // Requests the lane's channels; ready() waits for them and fills qh and sum.
  __device__ __forceinline__ void request(const uint16_t* q) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) raw[i] = *reinterpret_cast<const uint4*>(q + 8 * i);
  }
  __device__ __forceinline__ void ready() {
    sum = 0.0f;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const uint4 r = query_ready(raw[i]);
      qh[4 * i + 0] = r.x;
      qh[4 * i + 1] = r.y;
      qh[4 * i + 2] = r.z;
      qh[4 * i + 3] = r.w;
      float x[8];
      unpack8(r, x);
#pragma unroll
      for (int k = 0; k < 8; ++k) sum += x[k];
    }
  }
  // query channel c (0 <= c < DPL) as an fp16 value
  __device__ __forceinline__ _Float16 at(int c) const {
    const half2_t h = as_h2(qh[c >> 1]);
    return (c & 1) ? h.y : h.x;
  }
};

__device__ __forceinline__ float fma_h(_Float16 a, _Float16 b, float c) {
  return __builtin_fmaf(static_cast<float>(a), static_cast<float>(b), c);
}

// Partial dot product of one 16-byte code chunk (channels c0 .. c0+15) with the lane's
// query, in units of the stored code u (uint8: u = c, the zero point taken out per
// score; FP8: the code's value itself). Code and query are both fp16 operands of
// v_fma_mix_f32 (FP8: binary32 values); the products are exact in binary32.
template <int SCHEME, int D>
__device__ __forceinline__ float chunk_dot(const uint4& raw, const Query<SCHEME, D>& q) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  if constexpr (SCHEME == KVQ_FP8_E4M3) {
    // the hardware decodes E4M3 codes to binary32 exactly, two per instruction
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[j]), false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[j]), true);
      const int c = 4 * j;
      a0 = __builtin_fmaf(lo[0], static_cast<float>(q.at(c + 0)), a0);
      a1 = __builtin_fmaf(lo[1], static_cast<float>(q.at(c + 1)), a1);
      a0 = __builtin_fmaf(hi[0], static_cast<float>(q.at(c + 2)), a0);
      a1 = __builtin_fmaf(hi[1], static_cast<float>(q.at(c + 3)), a1);
    }
    return a0 + a1;
  } else {
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const half2_t e = as_h2(w[j] & 0x00FF00FFu);         // channels 0, 2
      const half2_t f = as_h2((w[j] >> 8) & 0x00FF00FFu);  // channels 1, 3
      const int c = 4 * j;
      a0 = fma_h(e.x, q.at(c + 0), a0);
      a1 = fma_h(f.x, q.at(c + 1), a1);
      a0 = fma_h(e.y, q.at(c + 2), a0);
      a1 = fma_h(f.y, q.at(c + 3), a1);
    }
    return (a0 + a1) * 16777216.0f;
  }
}

// o[k] += p * c_k for the 16-byte code chunk, c = u - offset. The offset (the uint8 zero
// point) is taken out of each fp16 pair with one packed fp16 add before the binary32 FMA,
// so a heavily weighted token whose codes sit at the offset adds (almost) nothing
// instead of two large terms that cancel later. off: the pair (-zp * 2^-24) (exact while
// |u - zp| < 2048, else rounded to fp16, a 2^-11 relative error on a term that then
// dominates).
template <int SCHEME>
__device__ __forceinline__ void chunk_axpy(const uint4& raw, float p, half2_t off, float* o) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  if constexpr (SCHEME == KVQ_FP8_E4M3) {
    // FP8 codes carry no offset and decode exactly to binary32
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[j]), false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[j]), true);
      float* oj = o + 4 * j;
      oj[0] = __builtin_fmaf(lo[0], p, oj[0]);
      oj[1] = __builtin_fmaf(lo[1], p, oj[1]);
      oj[2] = __builtin_fmaf(hi[0], p, oj[2]);
      oj[3] = __builtin_fmaf(hi[1], p, oj[3]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const half2_t e = as_h2(w[j] & 0x00FF00FFu) + off;         // channels 0, 2
      const half2_t f = as_h2((w[j] >> 8) & 0x00FF00FFu) + off;  // channels 1, 3
      float* oj = o + 4 * j;
      oj[0] = __builtin_fmaf(static_cast<float>(e.x), p, oj[0]);
      oj[2] = __builtin_fmaf(static_cast<float>(e.y), p, oj[2]);
      oj[1] = __builtin_fmaf(static_cast<float>(f.x), p, oj[1]);
      oj[3] = __builtin_fmaf(static_cast<float>(f.y), p, oj[3]);
    }
  }
}

// ---- the load pipeline shared by the split kernels -----------------------------------
// Streams one wave's share of a split [blk_begin, blk_end) of n blocks: the blocks
// blk_begin + (wave + 4i + rot) mod n, i = 0, 1, ..., where rot is a per-row offset so
// that workgroups streaming different rows are not in step across memory (rows a
// power-of-two-ish stride apart measured up to 20% slower in lock step). Each block's K
// codes, then its V codes, pass through two buffers: block i's V codes are requested
// before its K codes are consumed, block i+1's K codes before its V codes are; the last
// block of a chunk is peeled off the loop, so the loop body's loads are unconditional,
// every path issues the same loads and the compiler's wait counts stay exact (a
// conditional load makes it drain the whole pipeline instead). Per-block
// parameters (scales, zero points) are loaded one block per lane, 64 blocks at a time,
// and handed out by readlane: a vector load per block would sit behind the prefetched
// codes, and waiting for it would drain the pipeline too.
__device__ __forceinline__ float lane_value(float v, int i) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), i));
}

// `start()` runs once, after the wave's first code load has been issued and before
// anything waits for it: work that waits for the query's own load goes there, so the
// stream's first requests are not held behind it.
template <int LOADS, class LoadParams, class Load, class OnK, class OnV, class Start>
__device__ __forceinline__ void stream_wave_blocks(int blk_begin, int blk_end, int wave, int lane,
                                                   int64_t row, LoadParams load_params, Load load,
                                                   OnK on_k, OnV on_v, Start start) {
  const int n = blk_end - blk_begin;
  if (n <= 0) {  // uniform (a decode step's streaming waves may have no block)
    start();
    return;
  }
  const int rot = static_cast<int>((static_cast<uint32_t>(row) * 2654435761u) >> 8) % n;
  const int n_wave = wave < n ? (n - wave + kSplitWaves - 1) / kSplitWaves : 0;
  auto blk_of = [&](int i) {
    const int b = wave + kSplitWaves * i + rot;
    return blk_begin + (b >= n ? b - n : b);
  };
  uint4 kbuf[LOADS], vbuf[LOADS];
  for (int i0 = 0; i0 < n_wave; i0 += kWave) {
    const int i1 = min(n_wave, i0 + kWave);
    const auto params = load_params(blk_of(min(i0 + lane, i1 - 1)));
    load(false, blk_of(i0), params, 0, kbuf);
    if (i0 == 0) {
      __builtin_amdgcn_sched_barrier(0);
      start();
    }
    for (int i = i0; i < i1 - 1; ++i) {
      const int blk = blk_of(i);
      load(true, blk, params, i - i0, vbuf);
      // keep each request where it is: the scheduler would otherwise sink it below the
      // work it is meant to overlap, to shorten its registers' lifetime
      __builtin_amdgcn_sched_barrier(0);
      const auto pb = params.at(i - i0);
      on_k(blk, pb, kbuf);
      load(false, blk_of(i + 1), params, i + 1 - i0, kbuf);
      __builtin_amdgcn_sched_barrier(0);
      on_v(blk, pb, vbuf);
    }
    {  // the chunk's last block: nothing further to request
      const int blk = blk_of(i1 - 1);
      load(true, blk, params, i1 - 1 - i0, vbuf);
      __builtin_amdgcn_sched_barrier(0);
      const auto pb = params.at(i1 - 1 - i0);
      on_k(blk, pb, kbuf);
      on_v(blk, pb, vbuf);
    }
  }
}

__device__ __forceinline__ int lane_int(int v, int i) { return __builtin_amdgcn_readlane(v, i); }

// Per-block values a lane preloads for the pipeline: block scales (and zero points) of K
// and V, and, in the paged layout, the block's index in the pools (block_slot).
struct ScaleParams {
  float ks, vs;
  int slot;
  __device__ __forceinline__ ScaleParams at(int j) const {
    return {lane_value(ks, j), lane_value(vs, j), lane_int(slot, j)};
  }
};
struct ScaleZeroParams {
  float ks, kz, vs, vz;
  int slot;
  __device__ __forceinline__ ScaleZeroParams at(int j) const {
    return {lane_value(ks, j), lane_value(kz, j), lane_value(vs, j), lane_value(vz, j),
            lane_int(slot, j)};
  }
};

// A buffer resource over one block region (the paged layout gives every block its own
// base; offsets inside a region stay small).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t region_rsrc(const uint8_t* pool, int64_t slot,
                                                              int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(pool + slot * bytes), 0, bytes,
                                           kBufferRsrcWord3);
}

// ---- fused decode step ----------------------------------------------------------------
// In a decode step (kAppend) the workgroup of row (b, h) has one wave more than the
// attention. The row's length is read once, before anything else. The last wave (the
// append wave) then requests the row's staged tokens (straight into LDS) and the new
// token while waves 0 .. kSplitWaves-1 start streaming the blocks the append leaves
// untouched. (Holding the streaming waves at a barrier until the append wave's requests
// were out, so that they would enter the memory pipeline first, measured slower: 8K
// steps int4 45.5 against 46.0 us, uint8 85.1 against 86.4 us, FP8 84.4 against 85.9
// us, 32K unchanged.) The append wave reduces the block statistics before and after
// the token, codes the block (the
// whole block if its statistic changed, else the token), writes the token's staging and
// the scales, and attends the block that holds the token. The block's new codes stay in
// the append wave's registers (coded from the staged values) and are written at the end
// of the kernel: int4 the whole block, uint8 and FP8 the token's row (the whole block if
// it was re-quantized).
// The append wave takes the sequence's arrival ticket (in two levels, see step_ticket)
// once its own loads have completed, and the last of the sequence's `heads` workgroups
// stores the new length once its append wave has done its work. Every workgroup of the
// sequence reads the length before it takes its ticket, and the length changes only
// after the last ticket, so none can see the new length.
constexpr int kStepWaves = kSplitWaves + 1;

struct StepLens {
  int len0;          // the row's length before the append
  int len;           // attended length: after the append, within max_len and capacity
  int tail_blk;      // the block the append wave attends (holding the new token), or -1
  int len_streamed;  // tokens in the blocks the other waves attend
};

// The length is read with a plain load, which most workgroups find in their XCD's L2
// (a system-scope atomic load goes to memory every time): within the kernel the low 24
// bits of seq_lens[b] change only at the sequence's last ticket, which comes after every
// workgroup of the sequence has read them, and the top 8 bits (the arrival count that
// other workgroups are adding to) are masked off. The barrier orders the read before
// this workgroup's own ticket.
__device__ __forceinline__ StepLens step_lengths(const AttnArgs& a, int b, int cap) {
  __shared__ int len_shared;
  if (threadIdx.x == 0)
    len_shared = static_cast<int>(static_cast<uint32_t>(a.ap.seq_lens[b]) & 0xFFFFFFu);
  __syncthreads();
  StepLens r;
  r.len0 = len_shared;
  r.len = min(r.len0 < cap ? r.len0 + 1 : r.len0, min(a.max_len, cap));
  const int j = r.len0 / kBlock;
  r.tail_blk = r.len0 < cap && r.len > j * kBlock ? j : -1;
  r.len_streamed = r.tail_blk >= 0 ? j * kBlock : r.len;
  return r;
}

// The append wave's view of the open block: `fresh` is the lane's 16 bytes of the new K
// and V token (channels (lane % (D/8)) * 8 ..), `plan` the outcome per tensor. The new
// token is held as plain vector values (u32x4) until the wave has waited for its loads.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Requests the row's staged tokens (into xs) and the new token (append wave, row below
// capacity).
template <int D>
__device__ __forceinline__ void step_stage_load(const AttnArgs& a, const StepLens& sl,
                                                int64_t row, int lane, _Float16* xs,
                                                u32x4& fresh_k, u32x4& fresh_v) {
  append_stage_load_lds<D>(a.ap, row, sl.len0, lane, xs);
  const int off = (lane % (D / 8)) * 8;
  fresh_k = *reinterpret_cast<const u32x4*>(a.ap.k_new + row * D + off);
  fresh_v = *reinterpret_cast<const u32x4*>(a.ap.v_new + row * D + off);
}

// Waits for the staged tokens, puts the new token in its row of xs
// and reduces the block (append wave).
template <int SCHEME, int D>
__device__ __forceinline__ void step_stage_reduce(const StepLens& sl, int lane, _Float16* xs,
                                                  const uint4 (&fresh)[2],
                                                  AppendPlan (&plan)[2]) {
  constexpr int TPT = D / 8;  // lanes per token row
  const int slot = sl.len0 % kBlock;
  __builtin_amdgcn_s_waitcnt(0);  // the loads into LDS have landed
  if (lane / TPT == slot % (kWave / TPT)) {
    _Float16* row_k = xs + slot * D + (lane % TPT) * 8;
    *reinterpret_cast<u32x4*>(row_k) = u32x4{fresh[0].x, fresh[0].y, fresh[0].z, fresh[0].w};
    *reinterpret_cast<u32x4*>(row_k + kBlock * D) =
        u32x4{fresh[1].x, fresh[1].y, fresh[1].z, fresh[1].w};
  }
  __builtin_amdgcn_wave_barrier();
  append_stage_reduce<SCHEME, D, kWave, true>(
      sl.len0, lane,
      [&](int kv, int, int t, int chunk) {
        return *reinterpret_cast<const uint4*>(xs + kv * kBlock * D + t * D + chunk * 8);
      },
      fresh, xs, nullptr, plan);
}

// The sequence's arrival ticket, taken by the append wave after the length was read, in
// two levels. The `heads` workgroups of a sequence arrive in groups of kTicketGroup
// heads, each group on its own counter (the workspace's arrival counter of the group's
// first row, which the one-launch step, one split per row, does not otherwise use); the
// last arrival of a group then arrives, alone for its group, on the sequence's ticket in
// the top 8 bits of seq_lens[b], and the last group's last arrival stores the new
// length. Atomics on one address are performed one after another at memory: with one
// counter per sequence, the 32 heads of the 8K workload queued 32 deep and the wait for
// the ticket cost 1.8 us of the step (a timing-only build without it); in two levels
// they queue at most kTicketGroup + ceil(heads / kTicketGroup) deep.
// The group ticket's latency must overlap the wave's work, so nothing waits for it
// before step_ticket_done: it is issued after the wave's loads have been waited for
// (vector memory requests complete in order, so a later wait would include it), and as
// one request of the whole wave whose lanes past the first fall outside a 4-byte buffer
// resource and so do not touch memory; a branch around a one-lane atomic would merge
// its result with the other lanes' value and make the compiler wait for it at once.
// System scope (cache policy sc1): every add is performed at memory, past the per-XCD
// L2s. The result is meaningful in lane 0.
// Every workgroup of the sequence read the length before its group ticket; a group's
// last arrival has seen all of its group's tickets, and the sequence's last one all the
// groups', so the length changes only after every workgroup of the sequence has read it,
// and no other workgroup reads seq_lens[b]. The new length is stored as soon as the
// append wave has attended its block rather than at the kernel's end (0.1 us faster on
// the 8K int4 step); the group counter is left at zero for the next call.
constexpr int kCachePolicySystem = 16;  // sc1
constexpr int kTicketGroup = 8;

__device__ __forceinline__ uint32_t* step_group_counter(const AttnArgs& a, int b, int h) {
  return a.counters + static_cast<int64_t>(b) * a.heads + (h - h % kTicketGroup);
}

__device__ __forceinline__ uint32_t step_ticket(const AttnArgs& a, int b, int h, int lane) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(step_group_counter(a, b, h), 0, 4, kBufferRsrcWord3);
  return static_cast<uint32_t>(__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(
      1, rs, lane == 0 ? 0 : 4, 0, kCachePolicySystem));
}

__device__ __forceinline__ void step_ticket_done(const AttnArgs& a, const StepLens& sl, int b,
                                                 int h, int cap, uint32_t ticket, int lane) {
  const int in_group = min(kTicketGroup, a.heads - (h - h % kTicketGroup));
  if (lane != 0 || ticket != static_cast<uint32_t>(in_group - 1)) return;
  __hip_atomic_store(step_group_counter(a, b, h), 0u, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_SYSTEM);
  const uint32_t groups = static_cast<uint32_t>((a.heads + kTicketGroup - 1) / kTicketGroup);
  uint32_t* len = reinterpret_cast<uint32_t*>(a.ap.seq_lens) + b;
  const uint32_t old =
      __hip_atomic_fetch_add(len, 1u << 24, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  if ((old >> 24) == groups - 1)
    __hip_atomic_exchange(len, static_cast<uint32_t>(sl.len0 < cap ? sl.len0 + 1 : sl.len0),
                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// The append wave's work after the stage: write_codes(plan) builds the block's new codes
// in registers (written at the end of the kernel), then the token's fp16 staging and the
// changed scales are written. Returns the scales (and zero points) of
// the block holding the new token.
template <int D, class WriteCodes>
__device__ __forceinline__ BlockScales step_append(const AttnArgs& a, const StepLens& sl,
                                                   int64_t row, int cap, int lane,
                                                   const uint4 (&fresh)[2],
                                                   const AppendPlan (&plan)[2],
                                                   WriteCodes write_codes) {
  if (sl.len0 >= cap) return {0.0f, 0.0f, 0.0f, 0.0f};
  write_codes(plan);
  return append_finish<D, kWave>(a.ap, row, sl.len0, lane, fresh, plan);
}

// ---- split kernel: grid (heads, batch, n_split), kSplitWaves waves ------------------
template <int SCHEME, int D, bool kAppend, bool kPaged>
__global__ __launch_bounds__((kAppend ? kStepWaves : kSplitWaves) * kWave) void attn_split_kernel(
    AttnArgs a) {
  using G = AGeo<SCHEME, D>;
  constexpr int TPL = G::kTPL, DPL = G::kDPL, LPT = G::kLPT, GROUPS = G::kGroups;
  constexpr int kStates = kAppend ? kStepWaves : kSplitWaves;  // waves' partial states
  __shared__ float red_o[kStates][kWave][DPL + 1];
  __shared__ float red_l[kStates][kWave];
  __shared__ float red_m[kStates];
  __shared__ __align__(16) _Float16 xs[kAppend ? 2 * kBlock * D : 8];  // append staging

  const int h = blockIdx.x;
  int b = blockIdx.y;
  const int split = blockIdx.z;
  const int cap = a.max_blocks * kBlock;
  StepLens sl = {0, 0, -1, 0};
  int len;
  float plan_t = 0.0f;  // the batch's blocks (automatic plan)
  if constexpr (kAppend) {
    sl = step_lengths(a, b, cap);
    len = sl.len;
  } else {
    if (a.bps == 0) plan_t = batch_blocks(a, cap);
    if (a.bps == 0 && a.n_split == kPairedColumns && fills_gpu(a) && split >= 1)
      b = paired_sequence(a, b, split, cap, plan_t);
    len = clamp_len(a, a.seq_lens[b], cap);
    sl.len_streamed = len;
  }
  const int nb = (len + kBlock - 1) / kBlock;
  const SplitRange sr =
      kAppend ? split_range(a, nb, split, cap) : split_range_of(a, nb, split, plan_t);
  const int blk_begin = sr.begin;
  if (!kAppend && blk_begin >= nb) {  // uniform over the workgroup
    // an empty row has no split to merge: in fused mode split 0 writes its zeros
    if (a.fused && nb == 0 && split == 0 && threadIdx.x < D)
      a.out[(static_cast<int64_t>(b) * a.heads + h) * D + threadIdx.x] = 0;
    return;
  }
  // the blocks this split streams (in a decode step, all but the new token's block)
  const int blk_end = min(sr.end, (sl.len_streamed + kBlock - 1) / kBlock);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int chunk = lane % LPT;
  const int group = lane / LPT;
  const int64_t row = static_cast<int64_t>(b) * a.heads + h;

  // The query is requested here and made ready (make_query) once the wave's first code
  // requests are out (stream_wave_blocks' start), so they do not wait behind its load.
  Query<SCHEME, D> q;
  q.request(a.q + row * D + chunk * DPL);
  float qsum_row = 0.0f;
  auto make_query = [&]() {
    q.ready();
    qsum_row = group_sum<LPT>(q.sum);
  };

  // Dense layout: the row's code regions as buffer resources (uniform base and block
  // offset, the lane's 16-byte slot as the only per-lane address; the host keeps the row
  // below 2^31 bytes). Paged layout: one resource per block at its page.
  constexpr int kRegionBytes = kBlock * G::kRowBytes;
  const int row_bytes = kPaged ? kRegionBytes : a.max_blocks * kRegionBytes;
  const int64_t row_base = kPaged ? 0 : row * row_bytes;
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.k_codes + row_base), 0, row_bytes, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.v_codes + row_base), 0, row_bytes, kBufferRsrcWord3);
  const int lane_off = lane * 16;
  const int64_t sbase = kPaged ? 0 : row * a.max_blocks;  // dense: the row's blocks
  const float* ks = a.k_scale + sbase;
  const float* vs = a.v_scale + sbase;
  // zero points exist for uint8 only (FP8 caches may have none)
  constexpr bool kZero = SCHEME == KVQ_UINT8_ASYM;
  const float* kz = kZero ? a.k_zero + sbase : nullptr;
  const float* vz = kZero ? a.v_zero + sbase : nullptr;

  float o[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) o[k] = 0.0f;
  float m = -__builtin_inff();  // running max of the base-2 scores (wave-uniform)
  float l = 0.0f;               // sum of weights over this lane's tokens

  // Block blk's codes; in the paged layout `slot` locates the block.
  auto load_codes = [&](bool is_v, int blk, int slot, uint4 (&r)[TPL]) {
    if constexpr (kPaged) {
      const __amdgpu_buffer_rsrc_t rs =
          region_rsrc(is_v ? a.v_codes : a.k_codes, slot, kRegionBytes);
#pragma unroll
      for (int i = 0; i < TPL; ++i) r[i] = load_stream(rs, lane_off, i * kWave * 16);
    } else {
#pragma unroll
      for (int i = 0; i < TPL; ++i)
        r[i] = load_stream(is_v ? vrsrc : krsrc, lane_off, blk * kRegionBytes + i * kWave * 16);
    }
  };
  // the index of block blk in the per-block arrays (block_slot)
  auto slot_of = [&](int blk) {
    return kPaged ? static_cast<int>(block_slot(a.block_table, a.num_pages, a.heads,
                                                a.max_blocks, b, h, blk))
                  : blk;
  };

  // Scores of the lane's TPL tokens of block blk (base-2 logits), then the online
  // softmax update; returns the weights p (relative to the running max m).
  auto block_weights = [&](int blk, float kscale, float kzero, const uint4 (&kr)[TPL],
                           float (&p)[TPL]) {
    const float sk = kscale * a.qk_scale;
    const float offset = SCHEME == KVQ_UINT8_ASYM ? kzero : 0.0f;
    const float bias_k = offset * qsum_row;
    float s[TPL];
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      const float part = chunk_dot<SCHEME, D>(kr[i], q);
      s[i] = (group_sum<LPT>(part) - bias_k) * sk;
    }
    if (blk == nb - 1) {  // tokens past the length in the last block weigh nothing
      const int valid = len - blk * kBlock;
#pragma unroll
      for (int i = 0; i < TPL; ++i)
        if (i * GROUPS + group >= valid) s[i] = -__builtin_inff();
    }
    float mb = s[0];
#pragma unroll
    for (int i = 1; i < TPL; ++i) mb = fmaxf(mb, s[i]);
    mb = wave_max(mb);
    if (mb > m) {  // wave-uniform
      const float alpha = __builtin_amdgcn_exp2f(m - mb);
      l *= alpha;
#pragma unroll
      for (int k = 0; k < DPL; ++k) o[k] *= alpha;
      m = mb;
    }
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      p[i] = __builtin_amdgcn_exp2f(s[i] - m);
      l += p[i];
    }
  };

  // o += sum_i p_i * sv * (V code - offset) over the lane's TPL tokens of block blk.
  // Tokens past the length weigh 0; their (padding) codes only matter for FP8, where a
  // byte may decode to NaN and 0 * NaN is NaN: there they are replaced by code 0.
  auto block_accumulate = [&](int blk, float vscale, float vzero, const uint4 (&vr_in)[TPL],
                              const float (&p)[TPL]) {
    uint4 vr[TPL];
#pragma unroll
    for (int i = 0; i < TPL; ++i) vr[i] = vr_in[i];
    if constexpr (SCHEME == KVQ_FP8_E4M3) {
      if (blk == nb - 1) {  // wave-uniform
        const int valid = len - blk * kBlock;
#pragma unroll
        for (int i = 0; i < TPL; ++i)
          if (i * GROUPS + group >= valid) vr[i] = uint4{0u, 0u, 0u, 0u};
      }
    }
    const float sv = vscale;
    const _Float16 zh = static_cast<_Float16>(vzero * -5.9604644775390625e-08f);
    const half2_t off = half2_t{zh, zh};
#pragma unroll
    for (int i = 0; i < TPL; ++i) chunk_axpy<SCHEME>(vr[i], p[i] * sv, off, o);
  };

  float p[TPL];
  bool streaming = true;
  uint32_t ticket = 0;          // the append wave's arrival ticket (lane 0)
  uint4 kr[TPL], vr[TPL];       // the append wave: the open block's new codes
  AppendPlan plan[2];           // the append wave: the open block's outcome
  int64_t tblk = 0;             // the append wave: the open block's index (block_slot)
  if constexpr (kAppend) {
    tblk = block_slot(a.block_table, a.num_pages, a.heads, a.max_blocks, b, h,
                      min(sl.len0, cap - 1) / kBlock);
    u32x4 fresh_k = {0u, 0u, 0u, 0u}, fresh_v = {0u, 0u, 0u, 0u};
    if (wave == kSplitWaves && sl.len0 < cap)
      step_stage_load<D>(a, sl, row, lane, xs, fresh_k, fresh_v);
    if (wave == kSplitWaves) {  // the append wave
      streaming = false;
      const uint4 fresh[2] = {make_uint4(fresh_k.x, fresh_k.y, fresh_k.z, fresh_k.w),
                              make_uint4(fresh_v.x, fresh_v.y, fresh_v.z, fresh_v.w)};
      if (sl.len0 < cap) step_stage_reduce<SCHEME, D>(sl, lane, xs, fresh, plan);
      ticket = step_ticket(a, b, h, lane);
      // The block's new codes, in registers until the end of the kernel, coded from the
      // staged values with the block's scale after the append: every stored code of an
      // open block is the code of its staged value under the block's current scale, so
      // this is the block's content whether or not the scale changed.
      const BlockScales sc = step_append<D>(
          a, sl, row, cap, lane, fresh, plan, [&](const AppendPlan (&plan)[2]) {
            const int ntok = sl.len0 % kBlock + 1;
#pragma unroll
            for (int kv = 0; kv < 2; ++kv) {
              const Divisor d(plan[kv].s);
              const int zpi = static_cast<int>(plan[kv].zp);
              const _Float16* xt = xs + kv * kBlock * D;
#pragma unroll
              for (int i = 0; i < TPL; ++i)
                (kv ? vr : kr)[i] = byte_codes_chunk<SCHEME, D>(xt, ntok, d, zpi, lane, i);
            }
          });
      if (sl.tail_blk >= 0) {
        make_query();
        block_weights(sl.tail_blk, sc.ks, sc.kz, kr, p);
        block_accumulate(sl.tail_blk, sc.vs, sc.vz, vr, p);
      }
      step_ticket_done(a, sl, b, h, cap, ticket, lane);
    }
  }
  if (streaming)
    stream_wave_blocks<TPL>(
        blk_begin, blk_end, wave, lane, row,
        [&](int blk) {
          const int j = slot_of(blk);
          if constexpr (kZero) return ScaleZeroParams{ks[j], kz[j], vs[j], vz[j], j};
          else return ScaleZeroParams{ks[j], 0.0f, vs[j], 0.0f, j};
        },
        [&](bool is_v, int blk, const ScaleZeroParams& ps, int j, uint4 (&r)[TPL]) {
          load_codes(is_v, blk, kPaged ? lane_int(ps.slot, j) : 0, r);
        },
        [&](int blk, const ScaleZeroParams& pb, const uint4 (&kr)[TPL]) {
          block_weights(blk, pb.ks, pb.kz, kr, p);
        },
        [&](int blk, const ScaleZeroParams& pb, const uint4 (&vr)[TPL]) {
          block_accumulate(blk, pb.vs, pb.vz, vr, p);
        },
        make_query);

  // Per-lane result in true units: o_true[k] = o[k] * unit(k).
#pragma unroll
  for (int k = 0; k < DPL; ++k) {
    const float unit = SCHEME == KVQ_FP8_E4M3 ? 1.0f : 16777216.0f;
    red_o[wave][lane][k] = o[k] * unit;
  }
  red_l[wave][lane] = l;
  if (lane == 0) red_m[wave] = m;
  __syncthreads();

  float M = red_m[0];
#pragma unroll
  for (int w = 1; w < kStates; ++w) M = fmaxf(M, red_m[w]);
  float alpha[kStates];
#pragma unroll
  for (int w = 0; w < kStates; ++w) alpha[w] = __builtin_amdgcn_exp2f(red_m[w] - M);

  float od = 0.0f;
  if (threadIdx.x < D) {
    const int d = threadIdx.x, c = d / DPL, k = d % DPL;
#pragma unroll
    for (int w = 0; w < kStates; ++w) {
      float sw = 0.0f;
#pragma unroll
      for (int g = 0; g < GROUPS; ++g) sw += red_o[w][g * LPT + c][k];
      od = __builtin_fmaf(alpha[w], sw, od);
    }
  }
  float L = 0.0f;
#pragma unroll
  for (int w = 0; w < kStates; ++w) {
    float sw = 0.0f;
    for (int g = 0; g < GROUPS; ++g) sw += red_l[w][g * LPT];
    L = __builtin_fmaf(alpha[w], sw, L);
  }
  finish_split<D>(a, row, split, sr.n, od, M, L);
  if constexpr (kAppend) {
    if (wave == kSplitWaves) {
      // The new codes, written once the row's other blocks have been streamed (stores
      // into the code buffer during the stream slow it by more than their size): the
      // whole block if it was re-quantized, else the token's row (whole 64-byte lines).
      if (sl.len0 < cap) {
        const int slot = sl.len0 % kBlock;
#pragma unroll
        for (int kv = 0; kv < 2; ++kv) {
          uint8_t* codes = (kv ? a.ap.v_codes : a.ap.k_codes) + tblk * kRegionBytes;
#pragma unroll
          for (int i = 0; i < TPL; ++i) {
            const int t = (i * kWave + lane) * 16 / D;
            if (plan[kv].full || t == slot)
              store_b128(codes + (i * kWave + lane) * 16, (kv ? vr : kr)[i]);
          }
        }
      }
    }
  }
}

// ---- int4 split kernel on the matrix cores --------------------------------------------
// The int4 cache is stored in the operand order of v_mfma_f32_16x16x32_f16 (see
// kvq_device.h): a lane's 16-byte loads are its B fragments. One dword of 8 nibbles
// becomes 8 fp16 operands with a mask, an OR with the fp16 exponent of 1024 and one
// packed fp16 subtract per pair (exact), so the matrix cores see normal fp16 integers
// (they round fp16 subnormal inputs too coarsely for scores). QK^T: A = the query in
// row 0 (other rows zero), N = 16 tokens per tile. P.V: A = the weights split into an
// fp16 high part (row 0) and low part (row 1), K = 32 tokens per step, N = 16 channels
// per tile; the weights reach the A layout through a 2 KiB per-wave LDS image. The
// weights p <= 1 (relative to the running max) are scaled by 2^14 before the split so
// that the low part of small weights is still a normal fp16 (a subnormal low part
// would leave weights of 1e-4 with only ~11 significant bits).

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

typedef float float4_t __attribute__((ext_vector_type(4)));

// Nibble of a dword held by operand slot j (0, 4, 1, 5, 2, 6, 3, 7 for j = 0..7), and
// the slot of nibble q (the inverse). Arithmetic rather than a table: a table indexed by
// lane would be read from memory.
__device__ __forceinline__ constexpr int slot_nibble(int j) { return (j >> 1) | ((j & 1) << 2); }

// Element k (0..7) of 8 fp16 values held in a uint4 (k a compile-time constant after
// unrolling, so this stays in registers).
__device__ __forceinline__ _Float16 half_of(const uint4& r, int k) {
  const uint32_t w = k < 2 ? r.x : (k < 4 ? r.y : (k < 6 ? r.z : r.w));
  return __builtin_bit_cast(_Float16, static_cast<uint16_t>((k & 1) ? w >> 16 : w & 0xFFFFu));
}
__device__ __forceinline__ constexpr int nibble_slot(int q) { return ((q & 3) << 1) | (q >> 2); }

// 8 stored nibbles -> fp16 operands in slot order: slots 2, 3, 6, 7 hold 16*c * 2^-10,
// the others c * 2^-10 (c = nibble - 8). A mask leaves each nibble pair as fp16
// subnormals u * 2^-24 (or 16u * 2^-24); one packed fp16 FMA scales them by 2^14 and
// removes the offset, which is exact and lands on normal fp16 values (or zero).
__device__ __forceinline__ half8_t int4_operand(uint32_t w) {
  const uint32_t w8 = w >> 8;
  const half2_t scale = as_h2(0x74007400u);    // 2^14
  const half2_t lo_bias = as_h2(0xA000A000u);  // -8 * 2^-10
  const half2_t hi_bias = as_h2(0xB000B000u);  // -128 * 2^-10
  const half2_t a = as_h2(w & 0x000F000Fu) * scale + lo_bias;   // nibbles 0, 4
  const half2_t b = as_h2(w & 0x00F000F0u) * scale + hi_bias;   // nibbles 1, 5
  const half2_t c = as_h2(w8 & 0x000F000Fu) * scale + lo_bias;  // nibbles 2, 6
  const half2_t d = as_h2(w8 & 0x00F000F0u) * scale + hi_bias;  // nibbles 3, 7
  return half8_t{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

template <int N>
__device__ __forceinline__ uint32_t dword_of(const uint4 (&r)[N], int f) {
  const uint4 v = r[f >> 2];
  switch (f & 3) {
    case 0: return v.x;
    case 1: return v.y;
    case 2: return v.z;
    default: return v.w;
  }
}

// Maximum over lanes 0..15 (row 0 of the MFMA output), returned uniformly.
__device__ __forceinline__ float row0_max(float v) {
  v = dpp_max<kDppQuadXor1>(v);
  v = dpp_max<kDppQuadXor2>(v);
  v = dpp_max<kDppHalfMirror>(v);
  v = dpp_max<kDppRowMirror>(v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
}

__device__ __forceinline__ float row0_sum(float v) {
  v += dpp<kDppQuadXor1>(v);
  v += dpp<kDppQuadXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppRowMirror>(v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
}

template <int D, bool kAppend, bool kPaged>
__global__ __launch_bounds__((kAppend ? kStepWaves : kSplitWaves) * kWave) void
attn_split_int4_kernel(AttnArgs a) {
  constexpr int KS = D / 32;               // 32-channel K steps of QK^T
  constexpr int NTV = D / 16;              // 16-channel N tiles of P.V
  constexpr int LOADS = D / 32;            // 16-byte loads per lane per region
  constexpr int kRegionBytes = 32 * D;     // one tensor's codes of one block
  constexpr int kStates = kAppend ? kStepWaves : kSplitWaves;  // waves' partial states
  __shared__ __align__(16) _Float16 pimg[kStates][2][4][16][8];
  __shared__ float red_o[kStates][D];
  __shared__ float red_l[kStates];
  __shared__ float red_m[kStates];
  __shared__ __align__(16) _Float16 xs[kAppend ? 2 * kBlock * D : 8];  // append staging

  const int h = blockIdx.x;
  int b = blockIdx.y;
  const int split = blockIdx.z;
  const int cap = a.max_blocks * kBlock;
  StepLens sl = {0, 0, -1, 0};
  int len;
  float plan_t = 0.0f;  // the batch's blocks (automatic plan)
  if constexpr (kAppend) {
    sl = step_lengths(a, b, cap);
    len = sl.len;
  } else {
    if (a.bps == 0) plan_t = batch_blocks(a, cap);
    if (a.bps == 0 && a.n_split == kPairedColumns && fills_gpu(a) && split >= 1)
      b = paired_sequence(a, b, split, cap, plan_t);
    len = clamp_len(a, a.seq_lens[b], cap);
    sl.len_streamed = len;
  }
  const int nb = (len + kBlock - 1) / kBlock;
  const SplitRange sr =
      kAppend ? split_range(a, nb, split, cap) : split_range_of(a, nb, split, plan_t);
  const int blk_begin = sr.begin;
  if (!kAppend && blk_begin >= nb) {  // uniform over the workgroup
    // an empty row has no split to merge: in fused mode split 0 writes its zeros
    if (a.fused && nb == 0 && split == 0 && threadIdx.x < D)
      a.out[(static_cast<int64_t>(b) * a.heads + h) * D + threadIdx.x] = 0;
    return;
  }
  // the blocks this split streams (in a decode step, all but the new token's block)
  const int blk_end = min(sr.end, (sl.len_streamed + kBlock - 1) / kBlock);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int r16 = lane % 16;  // A row / output column of this lane
  const int grp = lane / 16;  // 8-element K group of this lane's fragments
  const int64_t row = static_cast<int64_t>(b) * a.heads + h;

  // This wave's P image: rows 2..15 stay zero, rows 0 and 1 are rewritten per block.
  {
    uint4* img = reinterpret_cast<uint4*>(&pimg[wave][0][0][0][0]);
    img[lane] = make_uint4(0u, 0u, 0u, 0u);
    img[lane + kWave] = make_uint4(0u, 0u, 0u, 0u);
  }

  // Query operand: row 0 holds q in slot order, x16 slots pre-divided by 16. The query's
  // bits are requested here; make_query builds the operand once the wave's first code
  // requests are out (stream_wave_blocks' start), so they do not wait behind this load.
  uint4 qraw[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qraw[ks] = *reinterpret_cast<const uint4*>(a.q + row * D + 32 * ks + 8 * grp);
  half8_t aq[KS];
  auto make_query = [&]() {
    const float keep = r16 == 0 ? 1.0f : 0.0f;
    uint4 qr[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qr[ks] = query_ready(qraw[ks]);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float x = static_cast<float>(half_of(qr[ks], slot_nibble(j))) * keep;
        if (j & 2) x *= 0.0625f;
        aq[ks][j] = static_cast<_Float16>(x);
      }
  };

  // Dense layout: the row's code regions as buffer resources, so a load's address is
  // the uniform block offset (a scalar register) plus the lane's 16-byte slot, with no
  // per-lane 64-bit address arithmetic (the host keeps max_blocks * 32 * D below 2^31).
  // Paged layout: one resource per block at its page.
  const int row_bytes = kPaged ? kRegionBytes : a.max_blocks * kRegionBytes;
  const int64_t row_base = kPaged ? 0 : row * row_bytes;
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.k_codes + row_base), 0, row_bytes, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.v_codes + row_base), 0, row_bytes, kBufferRsrcWord3);
  const int lane_off = lane * 16;
  const int64_t sbase = kPaged ? 0 : row * a.max_blocks;  // dense: the row's blocks
  const float* ks_ptr = a.k_scale + sbase;
  const float* vs_ptr = a.v_scale + sbase;

  float o[NTV];
#pragma unroll
  for (int n = 0; n < NTV; ++n) o[n] = 0.0f;
  float m = -__builtin_inff();  // running max of the base-2 scores (wave-uniform)
  float l = 0.0f;               // lanes 0..15: sum of their tokens' weights

  // Block blk's codes; in the paged layout `slot` locates the block.
  auto load_codes = [&](bool is_v, int blk, int slot, uint4 (&r)[LOADS]) {
    if constexpr (kPaged) {
      const __amdgpu_buffer_rsrc_t rs =
          region_rsrc(is_v ? a.v_codes : a.k_codes, slot, kRegionBytes);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) r[i] = load_stream(rs, lane_off, i * kWave * 16);
    } else {
#pragma unroll
      for (int i = 0; i < LOADS; ++i)
        r[i] = load_stream(is_v ? vrsrc : krsrc, lane_off, blk * kRegionBytes + i * kWave * 16);
    }
  };
  // the index of block blk in the per-block arrays (block_slot)
  auto slot_of = [&](int blk) {
    return kPaged ? static_cast<int>(block_slot(a.block_table, a.num_pages, a.heads,
                                                a.max_blocks, b, h, blk))
                  : blk;
  };


  // Scores of the block's 64 tokens (lanes 0..15 hold tokens 16*nt + lane), the
  // online-softmax update, and the weights p (relative to the running max).
  auto block_weights = [&](int blk, float kscale, const uint4 (&kr)[LOADS], float (&p)[4]) {
    const float sk = kscale * a.qk_scale * 1024.0f;  // operands carry 2^-10
    float4_t acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[nt] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            aq[ks], int4_operand(dword_of(kr, nt * KS + ks)), acc[nt], 0, 0, 0);
    float s[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) s[nt] = acc[nt][0] * sk;
    if (blk == nb - 1) {  // tokens past the length in the last block weigh nothing
      const int valid = len - blk * kBlock;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        if (16 * nt + r16 >= valid) s[nt] = -__builtin_inff();
    }
    float mb = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mb = row0_max(mb);
    if (mb > m) {  // wave-uniform
      const float alpha = __builtin_amdgcn_exp2f(m - mb);
      l *= alpha;
#pragma unroll
      for (int n = 0; n < NTV; ++n) o[n] *= alpha;
      m = mb;
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      p[nt] = __builtin_amdgcn_exp2f(s[nt] - m);
      l += p[nt];
    }
  };

  // o[n] += sv * sum_t p_t * c(t, 16n + lane) for the block (lanes 0..15).
  const int p_slot = nibble_slot(lane & 7);                    // this lane's weights' slot
  const float p_unit = (p_slot & 2) ? 1024.0f : 16384.0f;      // x16 slots: 2^14 / 16
  auto block_accumulate = [&](float vscale, const uint4 (&vr)[LOADS], const float (&p)[4]) {
    // Operands carry 2^-10 (codes) and 2^14 (weights): p <= 1 is split as p * 2^14 into
    // fp16 high and low parts so that the low part of small weights stays a normal fp16.
    const float sv = vscale * (1024.0f / 16384.0f);
    if (lane < 16) {
      const int slot = p_slot;
      const float scale = p_unit;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const float x = p[nt] * scale;
        const _Float16 hi = static_cast<_Float16>(x);
        const _Float16 lo = static_cast<_Float16>(x - static_cast<float>(hi));
        const int kstep = nt >> 1, kgrp = (nt & 1) * 2 + (lane >> 3);
        pimg[wave][kstep][kgrp][0][slot] = hi;
        pimg[wave][kstep][kgrp][1][slot] = lo;
      }
    }
    __builtin_amdgcn_wave_barrier();
    const half8_t ap0 = *reinterpret_cast<const half8_t*>(&pimg[wave][0][grp][r16][0]);
    const half8_t ap1 = *reinterpret_cast<const half8_t*>(&pimg[wave][1][grp][r16][0]);
#pragma unroll
    for (int n = 0; n < NTV; ++n) {
      float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap0, int4_operand(dword_of(vr, 2 * n)), acc, 0,
                                                   0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap1, int4_operand(dword_of(vr, 2 * n + 1)), acc,
                                                   0, 0, 0);
      o[n] = __builtin_fmaf(sv, acc[0] + acc[1], o[n]);
    }
    __builtin_amdgcn_wave_barrier();
  };

  float p[4];
  bool streaming = true;
  uint32_t ticket = 0;  // the append wave's arrival ticket (lane 0)
  uint4 kr[LOADS], vr[LOADS];  // the append wave: the open block's new codes
  AppendPlan plan[2];          // the append wave: the open block's outcome
  int64_t tblk = 0;            // the append wave: the open block's index (block_slot)
  if constexpr (kAppend) {
    // the append wave requests the staged tokens and the new token
    tblk = block_slot(a.block_table, a.num_pages, a.heads, a.max_blocks, b, h,
                      min(sl.len0, cap - 1) / kBlock);
    u32x4 fresh_k = {0u, 0u, 0u, 0u}, fresh_v = {0u, 0u, 0u, 0u};
    if (wave == kSplitWaves && sl.len0 < cap)
      step_stage_load<D>(a, sl, row, lane, xs, fresh_k, fresh_v);
    if (wave == kSplitWaves) {  // the append wave
      streaming = false;
      const uint4 fresh[2] = {make_uint4(fresh_k.x, fresh_k.y, fresh_k.z, fresh_k.w),
                              make_uint4(fresh_v.x, fresh_v.y, fresh_v.z, fresh_v.w)};
      if (sl.len0 < cap) step_stage_reduce<KVQ_INT4_SYM, D>(sl, lane, xs, fresh, plan);
      ticket = step_ticket(a, b, h, lane);
      // the block's new codes, in registers until the end of the kernel
      const BlockScales sc = step_append<D>(
          a, sl, row, cap, lane, fresh, plan, [&](const AppendPlan (&plan)[2]) {
            const int slot = sl.len0 % kBlock;
            int4_tail_fragments<D>(xs, slot, plan[0], false, lane, kr);
            int4_tail_fragments<D>(xs + kBlock * D, slot, plan[1], true, lane, vr);
          });
      if (sl.tail_blk >= 0) {
        make_query();
        block_weights(sl.tail_blk, sc.ks, kr, p);
        block_accumulate(sc.vs, vr, p);
      }
      step_ticket_done(a, sl, b, h, cap, ticket, lane);
    }
  }
  if (streaming)
    stream_wave_blocks<LOADS>(
        blk_begin, blk_end, wave, lane, row,
        [&](int blk) {
          const int j = slot_of(blk);
          return ScaleParams{ks_ptr[j], vs_ptr[j], j};
        },
        [&](bool is_v, int blk, const ScaleParams& ps, int j, uint4 (&r)[LOADS]) {
          load_codes(is_v, blk, kPaged ? lane_int(ps.slot, j) : 0, r);
        },
        [&](int blk, const ScaleParams& pb, const uint4 (&kr)[LOADS]) {
          block_weights(blk, pb.ks, kr, p);
        },
        [&](int, const ScaleParams& pb, const uint4 (&vr)[LOADS]) {
          block_accumulate(pb.vs, vr, p);
        },
        make_query);

  const float lw = row0_sum(lane < 16 ? l : 0.0f);
  if (lane < 16) {
#pragma unroll
    for (int n = 0; n < NTV; ++n) red_o[wave][16 * n + lane] = o[n];
  }
  if (lane == 0) {
    red_l[wave] = lw;
    red_m[wave] = m;
  }
  __syncthreads();

  float M = red_m[0];
#pragma unroll
  for (int w = 1; w < kStates; ++w) M = fmaxf(M, red_m[w]);
  float alpha[kStates];
#pragma unroll
  for (int w = 0; w < kStates; ++w) alpha[w] = __builtin_amdgcn_exp2f(red_m[w] - M);
  float od = 0.0f;
  if (threadIdx.x < D) {
#pragma unroll
    for (int w = 0; w < kStates; ++w) od = __builtin_fmaf(alpha[w], red_o[w][threadIdx.x], od);
  }
  float L = 0.0f;
#pragma unroll
  for (int w = 0; w < kStates; ++w) L = __builtin_fmaf(alpha[w], red_l[w], L);
  finish_split<D>(a, row, split, sr.n, od, M, L);
  if constexpr (kAppend) {
    if (wave == kSplitWaves) {
      // The open block's new codes, written once the row's other blocks have been
      // streamed: stores into the code buffer during the stream slow it by more than
      // their size (measured on the 8K int4 step: token-sized stores at once 47.8 us,
      // whole block at once 49.0 us, whole block at the end 46.5 us, no stores 45.6
      // us). Whole 64-byte lines: the block if it was re-quantized, else the lines that
      // hold the token's nibbles.
      if (sl.len0 < cap) {
        uint8_t* kc = a.ap.k_codes + tblk * kRegionBytes;
        uint8_t* vc = a.ap.v_codes + tblk * kRegionBytes;
        const int slot = sl.len0 % kBlock;
        // the 64-byte lines (4 lanes' chunks) that hold the token's nibbles: K dwords
        // (slot / 16) * KS .. + KS - 1 (chunk (slot / 16) * KS / 4) of lanes 16 g + slot %
        // 16; V every chunk of lanes 16 g', g' = (slot % 32) / 8
        const bool k_line = (lane % 16) / 4 == (slot % 16) / 4;
        const bool v_line = lane / 16 == (slot % 32) / 8;
        const int k_chunk = (slot / 16) * KS / 4;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
          if (plan[0].full || (k_line && i == k_chunk))
            store_b128(kc + (i * kWave + lane) * 16, kr[i]);
          if (plan[1].full || v_line) store_b128(vc + (i * kWave + lane) * 16, vr[i]);
        }
      }
    }
  }
}

// ---- grouped-query attention: G query heads per cached head ---------------------------
// Query head h * G + g reads cache row (b, h), so the codes of a block are converted to
// matrix-core operands once for all G queries. Rows 0..G-1 of the QK^T A tile hold the
// G queries and rows G..2G-1 hold them again (the one-query kernel above leaves rows
// 1..15 zero; the tile costs the same either way). Output element i of lane l is row
// 4 * (l / 16) + i, column l % 16, so each 16-lane group holds four rows and each row
// keeps its own running max (the accumulators are rescaled when any row's max rises);
// a repeated row computes exactly what its original does. P.V: the weights reach the A
// layout through a per-wave LDS image, split as above into fp16 high and low parts (of
// p * 2^14): row g < G of the image takes the high part of query g's weights, row G + g
// (the repeat) the low part, so one A operand carries both and a 16-channel tile takes
// two MFMAs (one per 32-token K step) instead of four. Output row g then holds the
// high parts' sum and row G + g the low parts'; the two are added once per split, in
// the merge of the waves through LDS.

// Maximum / sum over the 16 lanes of each DPP row; every lane of the row gets it.
__device__ __forceinline__ float row16_max(float v) {
  v = dpp_max<kDppQuadXor1>(v);
  v = dpp_max<kDppQuadXor2>(v);
  v = dpp_max<kDppHalfMirror>(v);
  return dpp_max<kDppRowMirror>(v);
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<kDppQuadXor1>(v);
  v += dpp<kDppQuadXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  return v + dpp<kDppRowMirror>(v);
}

// The fp16 part of the scaled weight x = p * unit that a row of the P.V image holds:
// the high part (x rounded to fp16) on rows g < G, the low part x - high on rows
// G <= g < 2G. Both are x - h rounded to fp16, with h = high on the low-part rows
// (cut = unit) and h = 0 on the others (cut = 0): two mixed-precision FMAs and no
// select. x - high is exact in binary32, so the parts are those of the plain split.
__device__ __forceinline__ _Float16 weight_part(float p, float unit, float cut) {
  const _Float16 h = static_cast<_Float16>(p * cut);
  return static_cast<_Float16>(__builtin_fmaf(p, unit, -static_cast<float>(h)));
}

template <int D, int G, bool kPaged>
__global__ __launch_bounds__(kSplitWaves * kWave) void attn_split_int4_gqa_kernel(AttnArgs a) {
  constexpr int KS = D / 32;            // 32-channel K steps of QK^T
  constexpr int NTV = D / 16;           // 16-channel N tiles of P.V
  constexpr int LOADS = D / 32;         // 16-byte loads per lane per region
  constexpr int kRegionBytes = 32 * D;  // one tensor's codes of one block
  // per wave: [k step][8-token group][row][slot]; rows < G high parts, G..2G-1 low parts
  __shared__ __align__(16) _Float16 pimg[kSplitWaves][2][4][16][8];
  __shared__ float red_o[kSplitWaves][2 * G][D];  // rows G..2G-1: the low parts' sums
  __shared__ float red_l[kSplitWaves][G];
  __shared__ float red_m[kSplitWaves][G];

  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int split = blockIdx.z;
  const int cap = a.max_blocks * kBlock;
  const int64_t row = static_cast<int64_t>(b) * a.heads + h;  // the cache row
  const int len = clamp_len(a, a.seq_lens[b], cap);
  const int nb = (len + kBlock - 1) / kBlock;
  const SplitRange sr = split_range(a, nb, split, cap);
  const int blk_begin = sr.begin;
  if (blk_begin >= nb) {  // uniform over the workgroup
    // an empty row has no split to merge: in fused mode split 0 writes its zeros
    if (a.fused && nb == 0 && split == 0)
      for (int t = threadIdx.x; t < G * D; t += kSplitWaves * kWave) a.out[row * G * D + t] = 0;
    return;
  }
  const int blk_end = sr.end;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int r16 = lane % 16;  // A row / output column of this lane
  const int grp = lane / 16;  // 8-element K group of this lane's fragments; its output rows / 4

  {  // this wave's P image: rows 2G..15 stay zero
    uint4* img = reinterpret_cast<uint4*>(&pimg[wave][0][0][0][0]);
#pragma unroll
    for (int k = 0; k < 2; ++k) img[lane + k * kWave] = make_uint4(0u, 0u, 0u, 0u);
  }

  // Query operand: rows g and G + g (g < G) hold query g in slot order, x16 slots
  // pre-divided by 16, built by make_query once the wave's first code requests are out
  // (as above).
  uint4 qraw[KS];
  {
    const uint16_t* qrow = a.q + (row * G + (r16 < 2 * G ? r16 % G : 0)) * D + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qraw[ks] = *reinterpret_cast<const uint4*>(qrow + 32 * ks);
  }
  half8_t aq[KS];
  auto make_query = [&]() {
    const float keep = r16 < 2 * G ? 1.0f : 0.0f;
    uint4 qr[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qr[ks] = query_ready(qraw[ks]);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float x = static_cast<float>(half_of(qr[ks], slot_nibble(j))) * keep;
        if (j & 2) x *= 0.0625f;
        aq[ks][j] = static_cast<_Float16>(x);
      }
  };

  const int row_bytes = kPaged ? kRegionBytes : a.max_blocks * kRegionBytes;
  const int64_t row_base = kPaged ? 0 : row * row_bytes;
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.k_codes + row_base), 0, row_bytes, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.v_codes + row_base), 0, row_bytes, kBufferRsrcWord3);
  const int lane_off = lane * 16;
  const int64_t sbase = kPaged ? 0 : row * a.max_blocks;
  const float* ks_ptr = a.k_scale + sbase;
  const float* vs_ptr = a.v_scale + sbase;

  float o[NTV][4];
#pragma unroll
  for (int n = 0; n < NTV; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) o[n][i] = 0.0f;
  float m[4], l[4];  // per output row 4 * grp + i: running max (base 2), lane's weight sum
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = -__builtin_inff();
    l[i] = 0.0f;
  }

  auto load_codes = [&](bool is_v, int blk, int slot, uint4 (&r)[LOADS]) {
    if constexpr (kPaged) {
      const __amdgpu_buffer_rsrc_t rs =
          region_rsrc(is_v ? a.v_codes : a.k_codes, slot, kRegionBytes);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) r[i] = load_stream(rs, lane_off, i * kWave * 16);
    } else {
#pragma unroll
      for (int i = 0; i < LOADS; ++i)
        r[i] = load_stream(is_v ? vrsrc : krsrc, lane_off, blk * kRegionBytes + i * kWave * 16);
    }
  };
  auto slot_of = [&](int blk) {
    return kPaged ? static_cast<int>(block_slot(a.block_table, a.num_pages, a.heads,
                                                a.max_blocks, b, h, blk))
                  : blk;
  };

  // Scores of the block's 64 tokens for the lane's rows, the per-row online-softmax
  // update, and the weights p[nt][i] (token 16 nt + r16, row 4 grp + i).
  auto block_weights = [&](int blk, float kscale, const uint4 (&kr)[LOADS], float (&p)[4][4]) {
    const float sk = kscale * a.qk_scale * 1024.0f;  // operands carry 2^-10
    float4_t acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[nt] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            aq[ks], int4_operand(dword_of(kr, nt * KS + ks)), acc[nt], 0, 0, 0);
    float s[4][4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) s[nt][i] = acc[nt][i] * sk;
    if (blk == nb - 1) {  // tokens past the length in the last block weigh nothing
      const int valid = len - blk * kBlock;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        if (16 * nt + r16 >= valid) {
#pragma unroll
          for (int i = 0; i < 4; ++i) s[nt][i] = -__builtin_inff();
        }
    }
    float mb[4];
    bool raise = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mb[i] = row16_max(fmaxf(fmaxf(s[0][i], s[1][i]), fmaxf(s[2][i], s[3][i])));
      raise |= mb[i] > m[i];
    }
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {  // some row's max rose
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float mn = fmaxf(m[i], mb[i]);
        const float alpha = __builtin_amdgcn_exp2f(m[i] - mn);
        l[i] *= alpha;
#pragma unroll
        for (int n = 0; n < NTV; ++n) o[n][i] *= alpha;
        m[i] = mn;
      }
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[nt][i] = __builtin_amdgcn_exp2f(s[nt][i] - m[i]);
        l[i] += p[nt][i];
      }
  };

  // o[n][i] += sv * sum_t w_t * c(t, 16 n + r16) for row r = 4 grp + i, where w is the
  // high part of the weights of query r (r < G) or the low part of those of query r - G
  // (G <= r < 2G).
  const int p_slot = nibble_slot(r16 & 7);                 // this lane's tokens' slot
  const float p_unit = (p_slot & 2) ? 1024.0f : 16384.0f;  // x16 slots: 2^14 / 16
  auto block_accumulate = [&](float vscale, const uint4 (&vr)[LOADS], const float (&p)[4][4]) {
    const float sv = vscale * (1024.0f / 16384.0f);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int kstep = nt >> 1, kgrp = (nt & 1) * 2 + (r16 >> 3);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * grp + i;
        if (r < 2 * G)
          pimg[wave][kstep][kgrp][r][p_slot] =
              weight_part(p[nt][i], p_unit, r < G ? 0.0f : p_unit);
      }
    }
    __builtin_amdgcn_wave_barrier();
    const half8_t ap0 = *reinterpret_cast<const half8_t*>(&pimg[wave][0][grp][r16][0]);
    const half8_t ap1 = *reinterpret_cast<const half8_t*>(&pimg[wave][1][grp][r16][0]);
#pragma unroll
    for (int n = 0; n < NTV; ++n) {
      float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap0, int4_operand(dword_of(vr, 2 * n)), acc,
                                                   0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap1, int4_operand(dword_of(vr, 2 * n + 1)),
                                                   acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) o[n][i] = __builtin_fmaf(sv, acc[i], o[n][i]);
    }
    __builtin_amdgcn_wave_barrier();
  };

  float p[4][4];
  stream_wave_blocks<LOADS>(
      blk_begin, blk_end, wave, lane, row,
      [&](int blk) {
        const int j = slot_of(blk);
        return ScaleParams{ks_ptr[j], vs_ptr[j], j};
      },
      [&](bool is_v, int blk, const ScaleParams& ps, int j, uint4 (&r)[LOADS]) {
        load_codes(is_v, blk, kPaged ? lane_int(ps.slot, j) : 0, r);
      },
      [&](int blk, const ScaleParams& pb, const uint4 (&kr)[LOADS]) {
        block_weights(blk, pb.ks, kr, p);
      },
      [&](int, const ScaleParams& pb, const uint4 (&vr)[LOADS]) {
        block_accumulate(pb.vs, vr, p);
      },
      make_query);

  // The waves' states per row through LDS (a wave with no block has m = -inf, l = o = 0):
  // o of rows 0..2G-1 (high and low parts), max and weight sum of rows 0..G-1 (a
  // repeated row's are the same).
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * grp + i;
    const float lr = row16_sum(l[i]);
    if (r < G && r16 == 0) {
      red_l[wave][r] = lr;
      red_m[wave][r] = m[i];
    }
    if (r < 2 * G) {
#pragma unroll
      for (int n = 0; n < NTV; ++n) red_o[wave][r][16 * n + r16] = o[n][i];
    }
  }
  __syncthreads();

  // Merge the waves per (row, channel), then finish as the one-query kernel does, for all
  // G output rows of the cache row (one arrival ticket per cache row).
  const int n_row = sr.n;
  const int64_t qrow0 = row * G;  // first output row
  constexpr int kThreadsWg = kSplitWaves * kWave;
  auto merged = [&](int g, int d, float& M, float& L) {
    M = red_m[0][g];
#pragma unroll
    for (int w = 1; w < kSplitWaves; ++w) M = fmaxf(M, red_m[w][g]);
    float od = 0.0f;
    L = 0.0f;
#pragma unroll
    for (int w = 0; w < kSplitWaves; ++w) {
      const float alpha = __builtin_amdgcn_exp2f(red_m[w][g] - M);
      od = __builtin_fmaf(alpha, red_o[w][g][d] + red_o[w][G + g][d], od);
      L = __builtin_fmaf(alpha, red_l[w][g], L);
    }
    return od;
  };
  if (a.fused && n_row == 1) {
    for (int t = threadIdx.x; t < G * D; t += kThreadsWg) {
      float M, L;
      const float od = merged(t / D, t % D, M, L);
      a.out[qrow0 * D + t] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(od / L));
    }
    return;
  }
  for (int t = threadIdx.x; t < G * D; t += kThreadsWg) {
    const int g = t / D, d = t % D;
    float M, L;
    const float od = merged(g, d, M, L);
    float* po = a.ws_o + ((qrow0 + g) * a.n_split + split) * D;
    float* ml = a.ws_ml + ((qrow0 + g) * a.n_split + split) * 2;
    if (a.fused) {
      store_shared(po + d, od);
      if (d == 0) {
        store_shared(ml, M);
        store_shared(ml + 1, L);
      }
    } else {
      po[d] = od;
      if (d == 0) {
        ml[0] = M;
        ml[1] = L;
      }
    }
  }
  if (!a.fused) return;
  __shared__ uint32_t ticket;
  wait_own_stores();  // every wave's partial stores have reached memory
  __syncthreads();
  // system scope: the read-modify-write is performed at memory, past the per-XCD L2s
  if (threadIdx.x == 0)
    ticket = __hip_atomic_fetch_add(a.counters + row, 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_SYSTEM);
  __syncthreads();
  if (ticket == static_cast<uint32_t>(n_row - 1)) {
    // thread t merges rows t / D + k * (threads / D) of channel t % D; a wave's 64 threads
    // share t / D (D is a multiple of the wave size): uniform rows
    constexpr int kRowsPerPass = kThreadsWg / D;
    constexpr int R = (G * D + kThreadsWg - 1) / kThreadsWg;
    const int t = threadIdx.x;
    if (t < G * D)
      merge_rows<D, R>(a, qrow0 + __builtin_amdgcn_readfirstlane(t / D), kRowsPerPass, n_row,
                       t % D);
    if (threadIdx.x == 0)
      __hip_atomic_store(a.counters + row, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

// ---- grouped-query attention over the 8-bit caches on the matrix cores ---------------
// The schedule of the int4 grouped-query kernel (queries in rows 0..G-1 of the A tile and
// again in rows G..2G-1; P.V with the weights' fp16 high parts in rows g < G and low
// parts in rows G + g of one A operand), over caches in natural token order:
// - QK^T: B operand lane l holds 8 channels of token l % 16 of a 16-token tile. Lane
//   (n, g) = (l % 16, l / 16) loads the D/4 bytes g * D/4 .. of token n (16-byte loads,
//   a tile's 16 tokens x D bytes shared by the 64 lanes); K step s uses its bytes 8s ..
//   8s + 7. The contraction runs over the channels in that order, so the query operand
//   takes the same order (lane (r, g), step s: channels g * D/4 + 8s .. + 7 of query r).
// - P.V: the B operand needs 8 tokens of one channel per lane, across the natural rows.
//   Each wave stages its block of V codes in LDS (rows of D + 16 bytes: the 16 rows a
//   transposing read gathers then fall in distinct banks) and reads it back with
//   ds_read_b64_tr_b8, which gives lane l of each 16-lane group byte l % 8 of the 8-byte
//   pieces pointed to by lanes 2j + l / 8 of the group (j = 0..7, measured on gfx950):
//   with lane r of group g pointing at token 32 ks + 8 g + r / 2, channels 16 n + 8 (r %
//   2) .., lane (n', g) receives tokens 32 ks + 8 g .. + 7 of channel 16 n + n', which is
//   the B operand of K step ks and N tile n.
// - Operands: FP8 codes convert exactly to fp16 (v_cvt_scalef32_pk_f16_fp8 with scale 1,
//   two codes per instruction, every E4M3 value a normal fp16); uint8 codes become
//   1024 + c by a byte permute with the bits of 1024, and one packed fp16 add of
//   -(1024 + z) leaves c - z exactly (|c - z| <= 255). The scales apply to the fp32
//   results. Tokens past the length in the last block are masked in the scores, and for
//   FP8 their V bytes are replaced by 0 (a padding byte may be NaN, and 0 * NaN is NaN).
template <int SCHEME>
__device__ __forceinline__ half8_t byte_operand(uint32_t w0, uint32_t w1, half2_t neg_off) {
  half2_t h[4];
  if constexpr (SCHEME == KVQ_FP8_E4M3) {
    h[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(w0), 1.0f, false);
    h[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(w0), 1.0f, true);
    h[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(w1), 1.0f, false);
    h[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(w1), 1.0f, true);
  } else {
    constexpr uint32_t kBits1024 = 0x64646464u;  // high byte of fp16 1024 in every byte
    h[0] = as_h2(__builtin_amdgcn_perm(kBits1024, w0, 0x04010400u)) + neg_off;  // bytes 0, 1
    h[1] = as_h2(__builtin_amdgcn_perm(kBits1024, w0, 0x04030402u)) + neg_off;  // bytes 2, 3
    h[2] = as_h2(__builtin_amdgcn_perm(kBits1024, w1, 0x04010400u)) + neg_off;
    h[3] = as_h2(__builtin_amdgcn_perm(kBits1024, w1, 0x04030402u)) + neg_off;
  }
  return half8_t{h[0].x, h[0].y, h[1].x, h[1].y, h[2].x, h[2].y, h[3].x, h[3].y};
}

typedef int int2_t __attribute__((ext_vector_type(2)));

template <int SCHEME, int D, int G, bool kPaged>
__global__ __launch_bounds__(kSplitWaves * kWave) void attn_split_gqa8_kernel(AttnArgs a) {
  constexpr int KS = D / 32;             // 32-channel K steps of QK^T
  constexpr int NTV = D / 16;            // 16-channel N tiles of P.V
  constexpr int LPT = D / 64;            // 16-byte loads per lane per 16-token tile
  constexpr int LOADS = 4 * LPT;         // 16-byte loads per lane per region
  constexpr int kRegionBytes = kBlock * D;
  constexpr int kRow = D + 16;           // LDS row stride of a staged V block
  constexpr int kTile = kBlock * kRow;   // one wave's staged V block
  __shared__ __align__(16) _Float16 pimg[kSplitWaves][2][4][16][8];
  // the waves' staged V blocks while streaming; afterwards the waves' partial outputs
  __shared__ __align__(16) uint8_t vstage[kSplitWaves * kTile];
  __shared__ float red_l[kSplitWaves][G];
  __shared__ float red_m[kSplitWaves][G];
  static_assert(sizeof(float) * kSplitWaves * 2 * G * D <= sizeof(vstage), "red_o in vstage");
  float(*red_o)[2 * G][D] = reinterpret_cast<float(*)[2 * G][D]>(vstage);

  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int split = blockIdx.z;
  const int cap = a.max_blocks * kBlock;
  const int64_t row = static_cast<int64_t>(b) * a.heads + h;  // the cache row
  const int len = clamp_len(a, a.seq_lens[b], cap);
  const int nb = (len + kBlock - 1) / kBlock;
  const SplitRange sr = split_range(a, nb, split, cap);
  if (sr.begin >= nb) {  // uniform over the workgroup
    // an empty row has no split to merge: in fused mode split 0 writes its zeros
    if (a.fused && nb == 0 && split == 0)
      for (int t = threadIdx.x; t < G * D; t += kSplitWaves * kWave) a.out[row * G * D + t] = 0;
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int r16 = lane % 16;  // A row / output column / B column of this lane
  const int grp = lane / 16;  // K group of this lane's fragments; its output rows / 4

  {  // this wave's P image: rows 2G..15 stay zero
    uint4* img = reinterpret_cast<uint4*>(&pimg[wave][0][0][0][0]);
#pragma unroll
    for (int k = 0; k < 2; ++k) img[lane + k * kWave] = make_uint4(0u, 0u, 0u, 0u);
  }

  // Query operand: rows g and G + g (g < G) hold query g, K step s the channels
  // grp * D/4 + 8s .. + 7; built by make_query once the first code requests are out.
  uint4 qraw[KS];
  {
    const uint16_t* qrow = a.q + (row * G + (r16 < 2 * G ? r16 % G : 0)) * D + grp * (D / 4);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qraw[ks] = *reinterpret_cast<const uint4*>(qrow + 8 * ks);
  }
  half8_t aq[KS];
  auto make_query = [&]() {
    const bool keep = r16 < 2 * G;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 qr = query_ready(qraw[ks]);
#pragma unroll
      for (int j = 0; j < 8; ++j) aq[ks][j] = keep ? half_of(qr, j) : static_cast<_Float16>(0.0f);
    }
  };

  const int row_bytes = kPaged ? kRegionBytes : a.max_blocks * kRegionBytes;
  const int64_t row_base = kPaged ? 0 : row * row_bytes;
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.k_codes + row_base), 0, row_bytes, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.v_codes + row_base), 0, row_bytes, kBufferRsrcWord3);
  // lane (n, g): token n of each tile, bytes g * D/4 ..
  const int lane_off = r16 * D + grp * (D / 4);
  const int64_t sbase = kPaged ? 0 : row * a.max_blocks;
  const float* ks_ptr = a.k_scale + sbase;
  const float* vs_ptr = a.v_scale + sbase;
  constexpr bool kZero = SCHEME == KVQ_UINT8_ASYM;
  const float* kz_ptr = kZero ? a.k_zero + sbase : nullptr;
  const float* vz_ptr = kZero ? a.v_zero + sbase : nullptr;

  float o[NTV][4];
#pragma unroll
  for (int n = 0; n < NTV; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) o[n][i] = 0.0f;
  float m[4], l[4];  // per output row 4 * grp + i: running max (base 2), lane's weight sum
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = -__builtin_inff();
    l[i] = 0.0f;
  }

  // load i = tile * LPT + half: token 16 tile + n, bytes g * D/4 + 16 half ..
  auto load_codes = [&](bool is_v, int blk, int slot, uint4 (&r)[LOADS]) {
    if constexpr (kPaged) {
      const __amdgpu_buffer_rsrc_t rs =
          region_rsrc(is_v ? a.v_codes : a.k_codes, slot, kRegionBytes);
#pragma unroll
      for (int i = 0; i < LOADS; ++i)
        r[i] = load_stream(rs, lane_off, (i / LPT) * 16 * D + (i % LPT) * 16);
    } else {
#pragma unroll
      for (int i = 0; i < LOADS; ++i)
        r[i] = load_stream(is_v ? vrsrc : krsrc, lane_off,
                           blk * kRegionBytes + (i / LPT) * 16 * D + (i % LPT) * 16);
    }
  };
  auto slot_of = [&](int blk) {
    return kPaged ? static_cast<int>(block_slot(a.block_table, a.num_pages, a.heads,
                                                a.max_blocks, b, h, blk))
                  : blk;
  };
  auto neg_offset = [](float zero) {  // -(1024 + z) in both halves (uint8)
    const _Float16 v = static_cast<_Float16>(-(1024.0f + zero));
    return half2_t{v, v};
  };

  // Scores of the block's 64 tokens for the lane's rows, the per-row online-softmax
  // update, and the weights p[nt][i] (token 16 nt + r16, row 4 grp + i).
  auto block_weights = [&](int blk, float kscale, float kzero, const uint4 (&kr)[LOADS],
                           float (&p)[4][4]) {
    const float sk = kscale * a.qk_scale;
    const half2_t off = neg_offset(kzero);
    float4_t acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[nt] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        // bytes 8 ks .. 8 ks + 7 of the lane's slice of token 16 nt + r16
        const int f = nt * 4 * LPT + 2 * ks;  // dword index over the loads
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            aq[ks], byte_operand<SCHEME>(dword_of(kr, f), dword_of(kr, f + 1), off), acc[nt],
            0, 0, 0);
      }
    float s[4][4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) s[nt][i] = acc[nt][i] * sk;
    if (blk == nb - 1) {  // tokens past the length in the last block weigh nothing
      const int valid = len - blk * kBlock;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        if (16 * nt + r16 >= valid) {
#pragma unroll
          for (int i = 0; i < 4; ++i) s[nt][i] = -__builtin_inff();
        }
    }
    float mb[4];
    bool raise = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mb[i] = row16_max(fmaxf(fmaxf(s[0][i], s[1][i]), fmaxf(s[2][i], s[3][i])));
      raise |= mb[i] > m[i];
    }
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {  // some row's max rose
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float mn = fmaxf(m[i], mb[i]);
        const float alpha = __builtin_amdgcn_exp2f(m[i] - mn);
        l[i] *= alpha;
#pragma unroll
        for (int n = 0; n < NTV; ++n) o[n][i] *= alpha;
        m[i] = mn;
      }
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[nt][i] = __builtin_amdgcn_exp2f(s[nt][i] - m[i]);
        l[i] += p[nt][i];
      }
  };

  // o[n][i] += sv * sum_t w_t * v(t, 16 n + r16) for row r = 4 grp + i, where w is the
  // high part of the weights of query r (r < G) or the low part of those of query r - G.
  uint8_t* vt = vstage + wave * kTile;
  // the transposing read: lane r16 of group grp points at token 8 grp + r16 / 2 of the K
  // step, channels 8 (r16 % 2) .. of the N tile
  const int tr_off = (8 * grp + r16 / 2) * kRow + 8 * (r16 % 2);
  auto block_accumulate = [&](int blk, float vscale, float vzero, const uint4 (&vr)[LOADS],
                              const float (&p)[4][4]) {
    const float sv = vscale * (1.0f / 16384.0f);
    const half2_t off = neg_offset(vzero);
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      *reinterpret_cast<uint4*>(vt + (16 * (i / LPT) + r16) * kRow + grp * (D / 4) +
                                16 * (i % LPT)) = vr[i];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int kstep = nt >> 1, kgrp = (nt & 1) * 2 + (r16 >> 3);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * grp + i;
        if (r < 2 * G)
          pimg[wave][kstep][kgrp][r][r16 & 7] =
              weight_part(p[nt][i], 16384.0f, r < G ? 0.0f : 16384.0f);
      }
    }
    __builtin_amdgcn_wave_barrier();
    const half8_t ap0 = *reinterpret_cast<const half8_t*>(&pimg[wave][0][grp][r16][0]);
    const half8_t ap1 = *reinterpret_cast<const half8_t*>(&pimg[wave][1][grp][r16][0]);
    // FP8: tokens past the length get code 0 (their bytes j of the K step's read are
    // tokens 32 ks + 8 grp + j)
    const int valid = blk == nb - 1 ? len - blk * kBlock : kBlock;
#pragma unroll
    for (int n = 0; n < NTV; ++n) {
      float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        int2_t w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) int2_t*)(vt + 32 * ks * kRow + 16 * n + tr_off));
        if constexpr (SCHEME == KVQ_FP8_E4M3) {
          if (valid < kBlock) {  // uniform: the row's last block only
            const int t0 = 32 * ks + 8 * grp;
            uint64_t v = (static_cast<uint64_t>(static_cast<uint32_t>(w.y)) << 32) |
                         static_cast<uint32_t>(w.x);
            const int keep = min(max(valid - t0, 0), 8);  // leading tokens kept
            v = keep >= 8 ? v : (v & ((uint64_t{1} << (8 * keep)) - 1));
            w.x = static_cast<int>(static_cast<uint32_t>(v));
            w.y = static_cast<int>(static_cast<uint32_t>(v >> 32));
          }
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            ks == 0 ? ap0 : ap1,
            byte_operand<SCHEME>(static_cast<uint32_t>(w.x), static_cast<uint32_t>(w.y), off),
            acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) o[n][i] = __builtin_fmaf(sv, acc[i], o[n][i]);
    }
    __builtin_amdgcn_wave_barrier();
  };

  float p[4][4];
  stream_wave_blocks<LOADS>(
      sr.begin, sr.end, wave, lane, row,
      [&](int blk) {
        const int j = slot_of(blk);
        if constexpr (kZero) return ScaleZeroParams{ks_ptr[j], kz_ptr[j], vs_ptr[j], vz_ptr[j], j};
        else return ScaleZeroParams{ks_ptr[j], 0.0f, vs_ptr[j], 0.0f, j};
      },
      [&](bool is_v, int blk, const ScaleZeroParams& ps, int j, uint4 (&r)[LOADS]) {
        load_codes(is_v, blk, kPaged ? lane_int(ps.slot, j) : 0, r);
      },
      [&](int blk, const ScaleZeroParams& pb, const uint4 (&kr)[LOADS]) {
        block_weights(blk, pb.ks, pb.kz, kr, p);
      },
      [&](int blk, const ScaleZeroParams& pb, const uint4 (&vr)[LOADS]) {
        block_accumulate(blk, pb.vs, pb.vz, vr, p);
      },
      make_query);

  // The waves' states per row through LDS, after every wave is done with its staged V
  // block (red_o reuses that memory).
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * grp + i;
    const float lr = row16_sum(l[i]);
    if (r < G && r16 == 0) {
      red_l[wave][r] = lr;
      red_m[wave][r] = m[i];
    }
    if (r < 2 * G) {
#pragma unroll
      for (int n = 0; n < NTV; ++n) red_o[wave][r][16 * n + r16] = o[n][i];
    }
  }
  __syncthreads();

  const int n_row = sr.n;
  const int64_t qrow0 = row * G;  // first output row
  constexpr int kThreadsWg = kSplitWaves * kWave;
  auto merged = [&](int g, int d, float& M, float& L) {
    M = red_m[0][g];
#pragma unroll
    for (int w = 1; w < kSplitWaves; ++w) M = fmaxf(M, red_m[w][g]);
    float od = 0.0f;
    L = 0.0f;
#pragma unroll
    for (int w = 0; w < kSplitWaves; ++w) {
      const float alpha = __builtin_amdgcn_exp2f(red_m[w][g] - M);
      od = __builtin_fmaf(alpha, red_o[w][g][d] + red_o[w][G + g][d], od);
      L = __builtin_fmaf(alpha, red_l[w][g], L);
    }
    return od;
  };
  if (a.fused && n_row == 1) {
    for (int t = threadIdx.x; t < G * D; t += kThreadsWg) {
      float M, L;
      const float od = merged(t / D, t % D, M, L);
      a.out[qrow0 * D + t] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(od / L));
    }
    return;
  }
  for (int t = threadIdx.x; t < G * D; t += kThreadsWg) {
    const int g = t / D, d = t % D;
    float M, L;
    const float od = merged(g, d, M, L);
    float* po = a.ws_o + ((qrow0 + g) * a.n_split + split) * D;
    float* ml = a.ws_ml + ((qrow0 + g) * a.n_split + split) * 2;
    if (a.fused) {
      store_shared(po + d, od);
      if (d == 0) {
        store_shared(ml, M);
        store_shared(ml + 1, L);
      }
    } else {
      po[d] = od;
      if (d == 0) {
        ml[0] = M;
        ml[1] = L;
      }
    }
  }
  if (!a.fused) return;
  __shared__ uint32_t ticket;
  wait_own_stores();  // every wave's partial stores have reached memory
  __syncthreads();
  // system scope: the read-modify-write is performed at memory, past the per-XCD L2s
  if (threadIdx.x == 0)
    ticket = __hip_atomic_fetch_add(a.counters + row, 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_SYSTEM);
  __syncthreads();
  if (ticket == static_cast<uint32_t>(n_row - 1)) {
    // thread t merges rows t / D + k * (threads / D) of channel t % D; a wave's 64 threads
    // share t / D (D is a multiple of the wave size): uniform rows
    constexpr int R = (G * D + kThreadsWg - 1) / kThreadsWg;
    const int t = threadIdx.x;
    if (t < G * D)
      merge_rows<D, R>(a, qrow0 + __builtin_amdgcn_readfirstlane(t / D), kThreadsWg / D, n_row,
                       t % D);
    if (threadIdx.x == 0)
      __hip_atomic_store(a.counters + row, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

// ---- combine kernel: grid (heads, batch), D threads ---------------------------------
template <int D>
__global__ __launch_bounds__(D) void attn_combine_kernel(AttnArgs a) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int d = threadIdx.x;
  const int cap = a.max_blocks * kBlock;
  const int nb = (clamp_len(a, a.seq_lens[b], cap) + kBlock - 1) / kBlock;
  const int n = split_range(a, nb, 0, cap).n;
  const int64_t row = static_cast<int64_t>(b) * a.heads + h;
  merge_row<D, false>(a, row, n, d);
}

template <int SCHEME, int D, bool kAppend, bool kPaged>
hipError_t split_t(int batch, const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.heads, batch, a.n_split);  // splits last: every row's first split comes first
  dim3 block((kAppend ? kStepWaves : kSplitWaves) * kWave);
  if constexpr (SCHEME == KVQ_INT4_SYM)
    hipLaunchKernelGGL((attn_split_int4_kernel<D, kAppend, kPaged>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((attn_split_kernel<SCHEME, D, kAppend, kPaged>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int SCHEME, int D, bool kAppend>
hipError_t layout_t(int batch, const AttnArgs& a, hipStream_t s) {
  return a.block_table ? split_t<SCHEME, D, kAppend, true>(batch, a, s)
                       : split_t<SCHEME, D, kAppend, false>(batch, a, s);
}

template <bool kAppend>
hipError_t launch(int scheme, int head_dim, int batch, const AttnArgs& a, hipStream_t s) {
  const bool d128 = head_dim == 128;
  switch (scheme) {
    case KVQ_INT4_SYM:
      return d128 ? layout_t<KVQ_INT4_SYM, 128, kAppend>(batch, a, s)
                  : layout_t<KVQ_INT4_SYM, 64, kAppend>(batch, a, s);
    case KVQ_FP8_E4M3:
      return d128 ? layout_t<KVQ_FP8_E4M3, 128, kAppend>(batch, a, s)
                  : layout_t<KVQ_FP8_E4M3, 64, kAppend>(batch, a, s);
    default:
      return d128 ? layout_t<KVQ_UINT8_ASYM, 128, kAppend>(batch, a, s)
                  : layout_t<KVQ_UINT8_ASYM, 64, kAppend>(batch, a, s);
  }
}

}  // namespace

hipError_t launch_attn_split(int scheme, int head_dim, int batch, const AttnArgs& a,
                             hipStream_t s) {
  return launch<false>(scheme, head_dim, batch, a, s);
}

hipError_t launch_decode_step(int scheme, int head_dim, int batch, const AttnArgs& a,
                              hipStream_t s) {
  return launch<true>(scheme, head_dim, batch, a, s);
}

namespace {
template <int SCHEME, int D, int G>
hipError_t gqa_t(int batch, const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.heads, batch, a.n_split);
  dim3 block(kSplitWaves * kWave);
  const bool paged = a.block_table != nullptr;
  if constexpr (SCHEME == KVQ_INT4_SYM) {
    if (paged)
      hipLaunchKernelGGL((attn_split_int4_gqa_kernel<D, G, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((attn_split_int4_gqa_kernel<D, G, false>), grid, block, 0, s, a);
  } else {
    if (paged)
      hipLaunchKernelGGL((attn_split_gqa8_kernel<SCHEME, D, G, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((attn_split_gqa8_kernel<SCHEME, D, G, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}
template <int SCHEME, int D>
hipError_t gqa_d(int group, int batch, const AttnArgs& a, hipStream_t s) {
  switch (group) {
    case 2: return gqa_t<SCHEME, D, 2>(batch, a, s);
    case 4: return gqa_t<SCHEME, D, 4>(batch, a, s);
    default: return gqa_t<SCHEME, D, 8>(batch, a, s);
  }
}
template <int SCHEME>
hipError_t gqa_s(int head_dim, int group, int batch, const AttnArgs& a, hipStream_t s) {
  return head_dim == 128 ? gqa_d<SCHEME, 128>(group, batch, a, s)
                         : gqa_d<SCHEME, 64>(group, batch, a, s);
}
}  // namespace

hipError_t launch_attn_gqa(int scheme, int head_dim, int group, int batch, const AttnArgs& a,
                           hipStream_t s) {
  switch (scheme) {
    case KVQ_INT4_SYM: return gqa_s<KVQ_INT4_SYM>(head_dim, group, batch, a, s);
    case KVQ_FP8_E4M3: return gqa_s<KVQ_FP8_E4M3>(head_dim, group, batch, a, s);
    default: return gqa_s<KVQ_UINT8_ASYM>(head_dim, group, batch, a, s);
  }
}

hipError_t launch_attn_combine(int head_dim, int batch, const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.heads, batch);
  if (head_dim == 128)
    hipLaunchKernelGGL((attn_combine_kernel<128>), grid, dim3(128), 0, s, a);
  else
    hipLaunchKernelGGL((attn_combine_kernel<64>), grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq
