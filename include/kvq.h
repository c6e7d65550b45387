/*
 * kvq.h — C ABI of libkvq: a block-quantized KV cache and single-token decode
 * attention that reads it, for AMD Instinct MI355X (gfx950).
 *
 * Method sources (web pages on DeepSeek-R1 inference optimisation):
 *   [Pg1] "第一章：DeepSeek R1推理模型性能跃迁全景概览" (aicoding.csdn.net)
 *         §2.2 — INT8 KV codes whose scales come from each chunk's extreme values;
 *         §2.3 and chapter 1 — decode attention at long context is bound by reads of
 *         the cache; attention is split into schedulable sub-blocks.
 *   [Pg2] "DeepSeek-R1推理延迟骤降41.8%？独家披露3类硬件感知调度策略" (jsqmd.com)
 *         §2.1 "基于A100显存带宽瓶颈的KV Cache分块压缩策略", sub-section
 *         "分块量化压缩设计" — 4-bit codes with one scale per 64-token block,
 *         scale = block absmax / 7.5, codes rounded and clamped to [-8, 7].
 *
 * Conventions shared by every call:
 *   * Ownership: the caller allocates every buffer (device memory unless stated) and
 *     keeps it alive until the work queued on `stream` has finished. The library
 *     allocates nothing and keeps no state of its own between calls; calls on different
 *     streams that touch different buffers may run concurrently, calls that share a
 *     buffer must be ordered by the caller (one stream).
 *   * Execution: every call validates its arguments on the host, then queues its
 *     kernels on `stream` (a hipStream_t; NULL means the null stream) and returns
 *     without waiting. Faults inside kernels surface at the caller's next
 *     synchronisation.
 *   * Errors: a negative KVQ_E* code means nothing was queued, except KVQ_EHIP, which
 *     means a launch failed (earlier launches of the same call may have been queued).
 *   * Block: 64 tokens of one (sequence, head) row, all head_dim channels — one scale
 *     (and, for uint8, one zero point) per block.
 *   * Rounding: codes use round-half-to-even of the IEEE binary32 quotient x / s, the
 *     division correctly rounded: the kernels take the code from a reciprocal multiply
 *     only where it provably decides the same code, and divide otherwise.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_BLOCK_TOKENS 64
#define KVQ_VERSION 5
/* Size of the static device array decode_attn_qkv_noalloc works in (per GPU). */
#define KVQ_NOALLOC_SCRATCH_BYTES (4u << 20)

/* Cache formats. */
enum kvq_scheme {
  /* [Pg2] §2.1: s = RN(absmax / 7.5f) (s = 0 for an all-zero block);
   * code = clamp(rint(RN(x / s)), -8, 7) (0 when s = 0), stored as the offset-binary
   * nibble code + 8 (order: see k_codes below). Zero points (if the buffers are given)
   * are written +0.0f. */
  KVQ_INT4_SYM = 0,
  /* [Pg1] §2.2, asymmetric per-chunk reading: s = RN(RN(max - min) / 255f),
   * zp = rint(RN(-min / s)) + 0.0f, code = clamp(rint(RN(x / s)) + (int)zp, 0, 255).
   * A chunk whose elements all equal c: c == 0 gives s = 0, zp = 0, codes 0;
   * otherwise the range is widened to [min(c,0), max(c,0)]. */
  KVQ_UINT8_ASYM = 1,
  /* [Pg3] §一 (FP8 KV cache; its scaling is not given there, this mirrors the 4-bit
   * scheme): s = RN(absmax / 448f) (448 = the largest finite E4M3 magnitude; s = 0 for
   * an all-zero block); code = the FP8 E4M3 (OCP "fn" variant: bias 7, no
   * infinities) value nearest to RN(x / s), ties to even, sign kept, saturating at
   * +-448; 0 when s = 0. One byte per channel, stored like KVQ_UINT8_ASYM codes. Zero
   * points (if the buffers are given) are written +0.0f. */
  KVQ_FP8_E4M3 = 2
};

/* Status codes. */
enum kvq_status {
  KVQ_OK = 0,
  KVQ_EINVAL = -1,     /* null pointer, bad scheme/shape/count, negative length */
  KVQ_ENOTSUP = -2,    /* head_dim other than 64 or 128; size or scheme limits of a call */
  KVQ_ECAPACITY = -3,  /* a length bound exceeds max_blocks * 64 */
  KVQ_EALIGN = -4,     /* a pointer or stride breaks the 16-byte alignment rule */
  KVQ_EWORKSPACE = -5, /* workspace missing or smaller than decode_attn_workspace_bytes */
  KVQ_EHIP = -6        /* a kernel launch failed */
};

/* Cache descriptor. Plain data; every pointer is device memory owned by the caller.
 * B = batch, H = heads, D = head_dim, MB = max_blocks (capacity MB * 64 tokens/row).
 *   k_codes, v_codes : uint8 [B][H][MB][64][D/2 (int4) | D (uint8, fp8)], 16-byte aligned;
 *                      each block of a row is one contiguous 32*D (int4) or 64*D
 *                      (uint8, fp8) byte region, uint8 and fp8 codes [token][channel].
 *                      int4 codes are stored in matrix-core operand order: the region
 *                      is 64 lanes x F = D/8 dwords, dword f of lane l at byte
 *                      ((f/4)*64 + l)*16 + (f%4)*4, nibble q (bits 4q..4q+3) =
 *                      K: channel 32*ks + 8*(l/16) + q of token 16*nt + l%16, f = nt*D/32 + ks;
 *                      V: token 32*ks + 8*(l/16) + q of channel 16*nt + l%16, f = 2*nt + ks.
 *                      kvq_int4_to_natural / kvq_int4_from_natural convert (host).
 *                      Codes of tokens at or past a row's length inside its last block
 *                      are written as zero nibbles / bytes by the quantizing calls.
 *   k_scale, v_scale : float [B][H][MB].
 *   k_zero,  v_zero  : float [B][H][MB]; required for KVQ_UINT8_ASYM, may be NULL for
 *                      KVQ_INT4_SYM and KVQ_FP8_E4M3.
 *   k_tail,  v_tail  : fp16 [B][H][64][D], 16-byte aligned: the original fp16 values
 *                      of each row's open (partially filled) block, which kv_append
 *                      needs to re-quantize that block. May be NULL if kv_append is
 *                      never called.
 *   seq_lens         : int32 [B], the number of valid tokens of each sequence (device
 *                      memory). Entries are clamped to [0, MB*64] by every kernel.
 *   block_table      : NULL for the dense layout above. Otherwise the cache is paged
 *                      ([Pg3] §四: PagedAttention against KV-cache fragmentation; [Pg1]
 *                      §3.1: a cache sized to the current length from a memory pool):
 *                      int32 [B][MB] device memory, entry (b, j) = the page that holds
 *                      block j of sequence b, and the per-block arrays become pools of
 *                      num_pages pages, a page being one 64-token block of one sequence
 *                      for all H heads:
 *                        k_codes, v_codes : [num_pages][H][64][D/2 | D] (same block
 *                                           regions and order as above),
 *                        k_scale .. v_zero: [num_pages][H].
 *                      Tail staging and seq_lens stay per sequence. Entries for blocks
 *                      a call reads or writes must be set before the call (an append
 *                      that opens block j writes page (b, j)); entries outside
 *                      [0, num_pages) are clamped into it. Every call gives bitwise the
 *                      results of the dense layout with the same contents.
 *   num_pages        : pages in the pools (>= 1 when block_table is set, else ignored). */
typedef struct kvq_cache {
  int32_t scheme;
  int32_t batch;
  int32_t heads;
  int32_t head_dim;
  int32_t max_blocks;
  void* k_codes;
  void* v_codes;
  float* k_scale;
  float* v_scale;
  float* k_zero;
  float* v_zero;
  void* k_tail;
  void* v_tail;
  int32_t* seq_lens;
  const int32_t* block_table;
  int32_t num_pages;
} kvq_cache;

/* Quantizes the prefill: for every row (b, h), blocks [0, ceil(n_b / 64)) of K and V,
 * where n_b = min(seq_lens[b], max_len), and stages the fp16 values of a partially
 * filled last block into k_tail/v_tail (when those are non-NULL). Blocks past
 * ceil(n_b / 64) are not touched. [Pg2] §2.1 (int4), [Pg1] §2.2 (uint8).
 *   k, v      : fp16 device tensors; element (b, t, h, d) at base[b*stride_b +
 *               t*stride_t + h*stride_h + d] (strides in elements, channels
 *               contiguous). Pointers 16-byte aligned, strides multiples of 8.
 *               [B][S][H][D] contiguous means stride_b = S*H*D, stride_t = H*D,
 *               stride_h = D. Only tokens t < n_b are read.
 *   max_len   : host-side bound on seq_lens, sizes the launch; 0 <= max_len <= MB*64.
 * Returns KVQ_OK or a negative kvq_status. */
int kv_quantize_blocks(const kvq_cache* cache, const void* k, const void* v,
                       int64_t stride_b, int64_t stride_t, int64_t stride_h,
                       int32_t max_len, void* stream);

/* Appends one decoded token per sequence: for every row, the token is written at
 * position n_b = seq_lens[b] (its fp16 value staged in the tail buffer), the row's
 * tail block is brought to exactly what kv_quantize_blocks would produce for the first
 * n_b + 1 tokens, and then seq_lens[b] is incremented. (Codes of positions past the
 * length are zero as kv_quantize_blocks leaves them; a caller that shortens seq_lens
 * and appends again may find stale codes there, which nothing reads.) When the new token leaves the
 * block's statistic (absmax, or min and max) unchanged only its own codes are written;
 * otherwise the whole tail block is re-quantized from the staged fp16 values.
 * Sequences with seq_lens[b] >= MB*64 are left unchanged. The tail staging (written
 * by kv_quantize_blocks or earlier appends) must be present. One kernel does all of
 * it: the workgroups of a sequence count their arrivals in the top 8 bits of
 * seq_lens[b] while it runs, and the last one stores the new length; hence
 * heads <= 255 and MB*64 < 2^24 (KVQ_ENOTSUP otherwise), entries of seq_lens must lie
 * in [0, MB*64], and nothing else may read seq_lens while the append runs.
 *   k_new, v_new  : fp16 [B][H][D] contiguous, 16-byte aligned.
 *   max_len_after : host-side bound on the lengths after the append; must be
 *                   <= MB*64 (KVQ_ECAPACITY otherwise).
 * Returns KVQ_OK or a negative kvq_status. */
int kv_append(const kvq_cache* cache, const void* k_new, const void* v_new,
              int32_t max_len_after, void* stream);

/* Work split of decode_attn_qkv: the context of each row is cut into splits of
 * `blocks_per_split` 64-token blocks, each handled by one workgroup, then merged by
 * their log-sum-exp. blocks_per_split = 0 lets the kernels choose each row's split on
 * the device from the rows' actual lengths (the host does not know them): the batch's
 * blocks are shared out in chunks of about 1/256 of them (1/512 for int4 grouped-query rows),
 * and a row is cut into ceil(its blocks / chunk) equal pieces, so equal rows that fill
 * the GPU stay whole and the long rows of a ragged batch are cut ([Pg1] chapter 1:
 * chunked attention as schedulable sub-blocks); once the rows fill the GPU, a row that
 * is cut takes pieces of about 1/384 of the blocks instead, at most three. Writes blocks_per_split_out (0 for the
 * device's choice) and splits_per_row_out, the most splits a row may take for this
 * max_len (the workspace is sized for it): ceil(blocks / blocks_per_split), or for the
 * device's choice 3 once batch * heads reaches 256 (2 once grouped-query rows reach 512
 * over int4, 256 over 8-bit caches), else one more than 256 / (batch * heads)
 * (512 / ... for int4 grouped-query rows), never more than
 * the blocks. Host only. */
int decode_attn_plan(const kvq_cache* cache, int32_t max_len, int32_t blocks_per_split,
                     int32_t* blocks_per_split_out, int32_t* splits_per_row_out);

/* Kernel launches decode_step_qkv queues for these arguments: 1 when every row is one
 * piece (blocks_per_split = 0 with batch * heads >= 256, or a blocks_per_split covering
 * max_len_after), else 2 (kv_append's kernel, then the attention). Negative kvq_status
 * on invalid arguments. Host only. */
int decode_step_launches(const kvq_cache* cache, int32_t max_len_after,
                         int32_t blocks_per_split);

/* Bytes of device workspace decode_attn_qkv needs for these arguments (0 on invalid
 * arguments). The workspace holds, first, one uint32 arrival counter per row (B*H,
 * padded to 256 bytes), then the per-split partial softmax states. The counters must
 * be zero before the first call that uses the workspace (allocate it zero-filled);
 * every call leaves them zero again. The partial states need no initialisation. */
size_t decode_attn_workspace_bytes(const kvq_cache* cache, int32_t max_len,
                                   int32_t blocks_per_split);

/* Decode attention of one query token per row against the quantized cache:
 *   out[b][h][:] = sum_t softmax_t(softmax_scale * q . K^_t) * V^_t,  t < n_b,
 * with K^, V^ the dequantized cache (c*s, or (c - zp)*s), n_b = min(seq_lens[b],
 * max_len). Codes are dequantized in registers; QK^T, an online softmax (base 2,
 * softmax_scale*log2(e) folded into the scores) and the weighted sum of V accumulate
 * in binary32 per split of the context; the splits are merged by their log-sum-exp
 * and rounded to fp16. One kernel launch: the last workgroup of each row to finish
 * (counted with the workspace's arrival counters) merges that row. Rows with n_b = 0
 * get zeros. (Attention is the textbook scaled dot product; splitting it into
 * schedulable pieces follows [Pg1] chapter 1's chunked attention.)
 *   q               : fp16 [B][H][D] contiguous, 16-byte aligned.
 *   out             : fp16 [B][H][D] contiguous, 16-byte aligned.
 *   workspace       : device buffer of >= decode_attn_workspace_bytes(...) bytes,
 *                     16-byte aligned; must not be shared by concurrent calls.
 *   max_len         : host-side bound on seq_lens, sizes the launch; <= MB*64.
 *   blocks_per_split: 0 = chosen per row on the device (decode_attn_plan), else the
 *                     split size in blocks.
 * A row's codes must stay below 2^31 bytes (MB*64*D/2 for int4, MB*64*D for uint8):
 * they are addressed with 32-bit offsets, and a row may take at most 65,535 splits
 * (KVQ_ENOTSUP otherwise, also from decode_attn_split / decode_attn_combine).
 * Returns KVQ_OK or a negative kvq_status. */
int decode_attn_qkv(const kvq_cache* cache, const void* q, float softmax_scale, void* out,
                    void* workspace, size_t workspace_bytes, int32_t max_len,
                    int32_t blocks_per_split, void* stream);

/* decode_attn_qkv without a workspace argument and without any allocation, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, plan, kernels and result as
 * decode_attn_qkv (bitwise). The arrival counters and partial softmax states live in a
 * static device array of KVQ_NOALLOC_SCRATCH_BYTES that the library holds on every GPU
 * it runs on until the process ends: 256 KiB of counters for up to 65,536 rows
 * (batch * heads), then the partial states, rows * splits_per_row * (head_dim + 2) * 4
 * bytes. Its device address is looked up once per GPU (first call with that GPU
 * current), when the counters are also cleared; every call leaves them zero.
 * Calls that overlap on one GPU (concurrent streams, or threads) share the array and
 * race: the caller must order them.
 * Returns decode_attn_qkv's status codes; KVQ_EWORKSPACE when batch * heads exceeds
 * 65,536 or the partial states of the plan do not fit (use decode_attn_qkv then), and
 * KVQ_EHIP when the array's address cannot be obtained. */
int decode_attn_qkv_noalloc(const kvq_cache* cache, const void* q, float softmax_scale,
                            void* out, int32_t max_len, int32_t blocks_per_split,
                            void* stream);

/* The same attention as two kernels, queued separately (same arguments, same plan):
 * decode_attn_split writes every split's partial state to the workspace (it does not
 * touch the counters), decode_attn_combine merges them into `out` with the same
 * arithmetic in the same order. Running split then combine on one stream gives
 * bitwise the result of decode_attn_qkv. */
int decode_attn_split(const kvq_cache* cache, const void* q, float softmax_scale,
                      void* workspace, size_t workspace_bytes, int32_t max_len,
                      int32_t blocks_per_split, void* stream);
int decode_attn_combine(const kvq_cache* cache, void* out, void* workspace,
                        size_t workspace_bytes, int32_t max_len, int32_t blocks_per_split,
                        void* stream);

/* One decode step of every row: kv_append of (k_new, v_new) followed by
 * decode_attn_qkv of q over the lengths after the append. The cache and seq_lens end
 * bitwise as after those two calls made in that order on one stream, and so does out
 * when they are what runs: unless every row is one piece, the two kernels are queued
 * (decode_step_launches). With one piece per row (blocks_per_split = 0 whenever
 * B*H >= 256) the step is one kernel launch: each row's workgroup has one
 * wave more than the attention, which appends the row's token and then attends the
 * block holding it while the other waves attend the rest of the row, so the append
 * costs no launch. out then equals the two calls'
 * up to the order of the binary32 sums (the new token's block is merged last), i.e. to
 * the last place of the fp16 result. Arguments and limits are
 * those of kv_append and decode_attn_qkv (max_len_after bounds the lengths after the
 * append and sizes the plan; the workspace is sized by
 * decode_attn_workspace_bytes(cache, max_len_after, blocks_per_split), and its arrival
 * counters, which the one-launch step uses to count the rows' appends, start at zero and
 * are left zero); the same status codes. (The step is one iteration of the decode phase, one token generated
 * per sequence, [Pg1] §3.1; each such token reads the whole cache, [Pg2] §2.1.)
 * Returns KVQ_OK or a negative kvq_status. */
int decode_step_qkv(const kvq_cache* cache, const void* k_new, const void* v_new, const void* q,
                    float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                    int32_t max_len_after, int32_t blocks_per_split, void* stream);

/* Grouped-query decode attention (several query heads share each cached head, as in
 * multi-query and grouped-query attention): query head hq = h * group + g of sequence b
 * attends over cache row (b, h), for g < group. The result is decode_attn_qkv's for
 * each query head against its cache row (same definition, splits and merge for the
 * same blocks_per_split); the codes of a block are turned into matrix-core operands
 * once for all `group` queries (uint8 and FP8 V codes reach the operand layout through a
 * transposing LDS read). The automatic plan (blocks_per_split = 0) aims at about two
 * workgroups per compute unit for group > 1 over an int4 cache and one over the 8-bit
 * caches (decode_attn_gqa_plan).
 * (Decode attention as in decode_attn_qkv with cached heads shared between query
 * heads: MLA with its projections absorbed decodes as multi-query attention, [Pg3] §二.)
 *   q, out    : fp16 [B][H * group][D] contiguous, 16-byte aligned.
 *   group     : 1 (exactly decode_attn_qkv), 2, 4 or 8 (KVQ_EINVAL otherwise); every
 *               scheme.
 *   workspace : >= decode_attn_gqa_workspace_bytes(cache, group, max_len,
 *               blocks_per_split) bytes (one arrival counter per cache row, partial
 *               states per query row); zero counters before first use, left zero.
 * Other arguments as decode_attn_qkv. Returns KVQ_OK or a negative kvq_status. */
int decode_attn_gqa(const kvq_cache* cache, const void* q, int32_t group, float softmax_scale,
                    void* out, void* workspace, size_t workspace_bytes, int32_t max_len,
                    int32_t blocks_per_split, void* stream);

/* Bytes of device workspace decode_attn_gqa needs (0 on invalid arguments). */
size_t decode_attn_gqa_workspace_bytes(const kvq_cache* cache, int32_t group, int32_t max_len,
                                       int32_t blocks_per_split);

/* Work split of decode_attn_gqa, as decode_attn_plan: writes the effective blocks per
 * split and splits per cache row for this group and max_len (group 1 gives
 * decode_attn_plan's). Host only. Returns KVQ_OK, KVQ_EINVAL for group < 1, or
 * decode_attn_plan's errors. */
int decode_attn_gqa_plan(const kvq_cache* cache, int32_t group, int32_t max_len,
                         int32_t blocks_per_split, int32_t* blocks_per_split_out,
                         int32_t* splits_per_row_out);

/* Host-side layout converters (host memory, no GPU work): n_regions consecutive int4
 * block regions of 32 * head_dim bytes (the K or V codes of one block of one row, as in
 * k_codes / v_codes; is_v selects the V order) from the stored matrix-core order to
 * natural order [64 tokens][head_dim / 2] (channel 2k in the low nibble of byte k), and
 * back. src and dst must not overlap. Returns KVQ_OK, KVQ_EINVAL (null pointer,
 * n_regions < 0) or KVQ_ENOTSUP (head_dim other than 64 or 128). */
int kvq_int4_to_natural(const uint8_t* stored, uint8_t* natural, int32_t head_dim,
                        int32_t is_v, int64_t n_regions);
int kvq_int4_from_natural(const uint8_t* natural, uint8_t* stored, int32_t head_dim,
                          int32_t is_v, int64_t n_regions);

/* Measurement aid (not part of the method): reads `bytes` bytes of device memory at
 * `buf` once, the way the attention kernels read a row's codes (each of at most
 * `workgroups` 256-thread workgroups streams one contiguous slab, 16-byte non-temporal
 * loads), and stores one folded word per thread to `sink` (device memory, at least
 * workgroups * 256 uint32). Its rate is the practical streaming-read ceiling of the
 * GPU that the decode kernels' HBM rates are set against. Asynchronous on `stream`.
 *   buf        : device memory, 16-byte aligned, bytes > 0.
 *   workgroups : > 0; slabs are whole 4 KiB units below 2^31 bytes (KVQ_ENOTSUP when
 *                bytes / workgroups does not fit).
 * Returns KVQ_OK, KVQ_EINVAL, KVQ_EALIGN, KVQ_ENOTSUP or KVQ_EHIP. */
int kvq_probe_stream_read(const void* buf, size_t bytes, int32_t workgroups, uint32_t* sink,
                          void* stream);

/* Measurement aid (not part of the method): launches one wave on `stream` that sleeps
 * until `microseconds` of the GPU's 100 MHz real-time counter have passed (bounded also
 * by a fixed number of sleeps), touching no memory. Work and timing events queued behind
 * it on the same stream start when it ends, so a timing event recorded right after it
 * marks the moment the GPU reaches the following work rather than the moment the host
 * queued it.
 *   microseconds : 1 .. 100000 (KVQ_EINVAL otherwise).
 * Returns KVQ_OK, KVQ_EINVAL or KVQ_EHIP. */
int kvq_probe_hold(uint32_t microseconds, void* stream);

/* Human-readable text of a kvq_status (static storage). */
const char* kvq_strerror(int status);

/* KVQ_VERSION of the built library. */
int kvq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
