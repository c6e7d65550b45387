// kvq_api.hip — the C ABI of libkvq (declared in include/kvq.h): argument validation,
// the split plan and kernel launches. No allocation. Nothing is kept between calls except
// what lives in caller-owned buffers (the workspace's arrival counters), and, for
// decode_attn_qkv_noalloc only, a static device array per GPU with its address.
#include <stdint.h>

#include <mutex>

#include "kvq.h"
#include "kvq_internal.h"

namespace {

constexpr int kBlockTokens = KVQ_BLOCK_TOKENS;
constexpr int64_t kTargetWorkgroups = 256;  // automatic plan: one workgroup per MI355X CU

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_cache(const kvq_cache* c) {
  if (!c) return KVQ_EINVAL;
  if (c->scheme != KVQ_INT4_SYM && c->scheme != KVQ_UINT8_ASYM && c->scheme != KVQ_FP8_E4M3)
    return KVQ_EINVAL;
  if (c->batch <= 0 || c->heads <= 0 || c->max_blocks <= 0) return KVQ_EINVAL;
  if (c->batch > 32767 || c->heads > 65535) return KVQ_EINVAL;  // launch-grid limits
  if (static_cast<int64_t>(c->max_blocks) * kBlockTokens > INT32_MAX) return KVQ_EINVAL;
  if (c->head_dim != 64 && c->head_dim != 128) return KVQ_ENOTSUP;
  if (!c->k_codes || !c->v_codes || !c->k_scale || !c->v_scale || !c->seq_lens)
    return KVQ_EINVAL;
  if (c->scheme == KVQ_UINT8_ASYM && (!c->k_zero || !c->v_zero)) return KVQ_EINVAL;
  if (!aligned16(c->k_codes) || !aligned16(c->v_codes)) return KVQ_EALIGN;
  if ((c->k_tail && !aligned16(c->k_tail)) || (c->v_tail && !aligned16(c->v_tail)))
    return KVQ_EALIGN;
  // paged layout: block indices (page * heads + head) are 32-bit in the kernels
  if (c->block_table && (c->num_pages <= 0 ||
                         static_cast<int64_t>(c->num_pages) * c->heads > INT32_MAX))
    return KVQ_EINVAL;
  return KVQ_OK;
}

int check_len(const kvq_cache* c, int32_t max_len) {
  if (max_len < 0) return KVQ_EINVAL;
  if (static_cast<int64_t>(max_len) > static_cast<int64_t>(c->max_blocks) * kBlockTokens)
    return KVQ_ECAPACITY;
  return KVQ_OK;
}

int n_blocks_for(int32_t len) { return (len + kBlockTokens - 1) / kBlockTokens; }

// The split plan. A caller's blocks_per_split cuts every row into pieces of that many
// blocks. With blocks_per_split = 0 the pieces are chosen on the device from the rows'
// actual lengths (split_range in kvq_attn.hip): the batch's blocks are shared out in
// chunks of about 1/target of them, one chunk per workgroup, where target is one
// workgroup per CU, and two for int4 grouped-query rows (that kernel is bound by its
// per-block work on one wave per SIMD, and a second workgroup on the CU overlaps its
// latencies: measured on the 8K grouped-query workload, 8 queries per cached head,
// 24.7 us with one workgroup per CU, 23.2 us with two, 33.8 us with four). The 8-bit
// grouped-query kernel streams twice the bytes per block for the same operand work and
// keeps one workgroup per CU (the same workload over FP8 and uint8 caches: 29.7 us
// with one, 30.7 us with two). Long unbroken
// runs of one row's codes stream from HBM faster than many short ones, and every extra
// split costs a merge, so rows of equal length stay whole once they fill the GPU; the
// host only bounds the pieces a row may take (the grid's split dimension): once the rows
// alone reach the target, three (a ragged batch cuts its long rows in two or three, and
// the device pairs the pieces of different rows on each compute unit) or two for
// grouped-query rows, else one more than the splits that equal rows take (the target
// over the rows). Every column of the
// grid that no row uses still runs as workgroups that exit at once, which costs little
// while they fit on the CUs beside the working ones and about 1 us where they wait for
// them (8K grouped-query workload with twice the columns: 21.3 against 20.2 us).
constexpr int64_t kMaxGridSplits = 65535;  // the grid's split dimension (z)

int64_t plan_target(int group, int scheme) {
  return group > 1 && scheme == KVQ_INT4_SYM ? 2 * kTargetWorkgroups : kTargetWorkgroups;
}

int device_plan_splits(const kvq_cache* c, int nb, int group) {
  const int64_t rows = static_cast<int64_t>(c->batch) * c->heads;
  const int64_t target = plan_target(group, c->scheme);
  const int64_t s = rows >= target ? (group > 1 ? 2 : 3) : (target + rows - 1) / rows + 1;
  return static_cast<int>(s < nb ? s : nb);
}

int plan(const kvq_cache* c, int32_t max_len, int32_t bps_req, int* bps, int* n_split,
         int group = 1) {
  int rc = check_cache(c);
  if (rc != KVQ_OK) return rc;
  rc = check_len(c, max_len);
  if (rc != KVQ_OK) return rc;
  if (bps_req < 0) return KVQ_EINVAL;
  const int nb = n_blocks_for(max_len);
  *bps = bps_req;  // 0: chosen per row on the device
  *n_split = nb == 0 ? 0 : bps_req > 0 ? (nb + bps_req - 1) / bps_req
                                       : device_plan_splits(c, nb, group);
  return KVQ_OK;
}

// decode_step_qkv is one launch (each row's workgroup appends, then attends the whole
// row) when every row is one piece: the automatic plan once the rows alone fill the GPU,
// or a caller's blocks_per_split that covers max_len_after.
bool step_is_one_launch(const kvq_cache* c, int32_t max_len_after, int32_t bps_req) {
  const int nb = n_blocks_for(max_len_after);
  if (bps_req > 0) return nb <= bps_req;
  return static_cast<int64_t>(c->batch) * c->heads >= kTargetWorkgroups;
}

// Workspace layout: [rows] uint32 arrival counters (padded to 256 bytes), then the
// partial outputs [rows][n_split][D] and partial (max, sum) [rows][n_split][2] floats.
size_t counter_bytes(const kvq_cache* c) {
  const size_t rows = static_cast<size_t>(c->batch) * c->heads;
  return (rows * sizeof(uint32_t) + 255) / 256 * 256;
}

size_t workspace_bytes(const kvq_cache* c, int n_split, int group = 1) {
  const size_t parts = static_cast<size_t>(c->batch) * c->heads * group * n_split;
  return counter_bytes(c) + parts * (static_cast<size_t>(c->head_dim) + 2) * sizeof(float);
}

// Fills the attention launch descriptor after validating the workspace.
int attn_args(const kvq_cache* c, const void* q, float softmax_scale, void* out,
              void* workspace, size_t workspace_bytes_given, int32_t max_len, int32_t bps_req,
              int fused, kvq::AttnArgs* a, int group = 1) {
  int bps, n_split;
  int rc = plan(c, max_len, bps_req, &bps, &n_split, group);
  if (rc != KVQ_OK) return rc;
  // the split kernels address a row's codes with 32-bit buffer offsets (dense layout;
  // the paged layout addresses each block separately)
  const int64_t row_code_bytes = static_cast<int64_t>(c->max_blocks) * kBlockTokens *
                                 (c->scheme == KVQ_INT4_SYM ? c->head_dim / 2 : c->head_dim);
  if (!c->block_table && row_code_bytes > INT32_MAX) return KVQ_ENOTSUP;
  if (n_split > kMaxGridSplits) return KVQ_ENOTSUP;
  if (n_split > 0) {
    if (!workspace || workspace_bytes_given < workspace_bytes(c, n_split, group))
      return KVQ_EWORKSPACE;
    if (!aligned16(workspace)) return KVQ_EALIGN;
  }
  const size_t parts = static_cast<size_t>(c->batch) * c->heads * group * n_split;
  a->k_codes = static_cast<const uint8_t*>(c->k_codes);
  a->v_codes = static_cast<const uint8_t*>(c->v_codes);
  a->k_scale = c->k_scale;
  a->v_scale = c->v_scale;
  a->k_zero = c->k_zero;
  a->v_zero = c->v_zero;
  a->seq_lens = c->seq_lens;
  a->q = static_cast<const uint16_t*>(q);
  a->out = static_cast<uint16_t*>(out);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  a->counters = n_split > 0 ? reinterpret_cast<uint32_t*>(ws) : nullptr;
  a->ws_o = n_split > 0 ? reinterpret_cast<float*>(ws + counter_bytes(c)) : nullptr;
  a->ws_ml = n_split > 0 ? a->ws_o + parts * c->head_dim : nullptr;
  a->fused = fused;
  a->heads = c->heads;
  a->max_blocks = c->max_blocks;
  a->max_len = max_len;
  a->bps = bps;
  a->n_split = n_split;
  a->batch = c->batch;
  a->plan_target = static_cast<int>(plan_target(group, c->scheme));
  a->qk_scale = softmax_scale * 1.44269504088896340736f;  // log2(e)
  a->block_table = c->block_table;
  a->num_pages = c->num_pages;
  return KVQ_OK;
}

// Validates an append and fills its launch descriptor.
int append_args(const kvq_cache* c, const void* k_new, const void* v_new, int32_t max_len_after,
                kvq::AppendArgs* a) {
  int rc = check_cache(c);
  if (rc != KVQ_OK) return rc;
  if (max_len_after < 1) return KVQ_EINVAL;
  rc = check_len(c, max_len_after);
  if (rc != KVQ_OK) return rc;
  if (!c->k_tail || !c->v_tail || !k_new || !v_new) return KVQ_EINVAL;
  if (!aligned16(k_new) || !aligned16(v_new)) return KVQ_EALIGN;
  // the arrival ticket lives in the top 8 bits of each length
  if (c->heads > 255 || static_cast<int64_t>(c->max_blocks) * kBlockTokens >= (1 << 24))
    return KVQ_ENOTSUP;
  a->k_new = static_cast<const uint16_t*>(k_new);
  a->v_new = static_cast<const uint16_t*>(v_new);
  a->k_codes = static_cast<uint8_t*>(c->k_codes);
  a->v_codes = static_cast<uint8_t*>(c->v_codes);
  a->k_scale = c->k_scale;
  a->v_scale = c->v_scale;
  a->k_zero = c->k_zero;
  a->v_zero = c->v_zero;
  a->k_tail = static_cast<uint16_t*>(c->k_tail);
  a->v_tail = static_cast<uint16_t*>(c->v_tail);
  a->seq_lens = c->seq_lens;
  a->batch = c->batch;
  a->heads = c->heads;
  a->max_blocks = c->max_blocks;
  a->block_table = c->block_table;
  a->num_pages = c->num_pages;
  return KVQ_OK;
}

// ---- the no-allocation variant of decode_attn_qkv -----------------------------------
// Its arrival counters and partial states live in `scratch`, a device array of static
// storage (one copy per GPU, zero when the code object is loaded). Layout: the first
// kScratchRows uint32 are the rows' arrival counters, always at the same place, so that
// calls of any shape find them zero (every call leaves the counters it used at zero);
// the partial states of one call follow them. Host code never passes `scratch` itself
// to a kernel: its name is a host-side stand-in, and the device address of each GPU's
// copy comes from hipGetSymbolAddress.
constexpr int64_t kScratchRows = 65536;
constexpr size_t kScratchCounterBytes = kScratchRows * sizeof(uint32_t);
static __device__ __align__(256) uint8_t scratch[KVQ_NOALLOC_SCRATCH_BYTES];

__global__ void clear_counters_kernel(uint32_t* c, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) c[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
uint8_t* g_scratch_ptr[kMaxDevices] = {};

// This GPU's copy of `scratch` (device address), looked up once per device with that
// device current; the first lookup also clears the counter region on `stream` (unless
// the stream is being captured, where the kernel would only be recorded: the array is
// zero from the code object's load). Returns nullptr on a HIP error.
uint8_t* scratch_for_current_device(hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev]) return g_scratch_ptr[dev];
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return nullptr;
  if (cs == hipStreamCaptureStatusNone) {
    hipLaunchKernelGGL(clear_counters_kernel, dim3((kScratchRows + 255) / 256), dim3(256), 0,
                       stream, static_cast<uint32_t*>(p), kScratchRows);
    if (hipGetLastError() != hipSuccess) return nullptr;
  }
  g_scratch_ptr[dev] = static_cast<uint8_t*>(p);
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int kv_quantize_blocks(const kvq_cache* cache, const void* k, const void* v,
                       int64_t stride_b, int64_t stride_t, int64_t stride_h, int32_t max_len,
                       void* stream) {
  int rc = check_cache(cache);
  if (rc != KVQ_OK) return rc;
  rc = check_len(cache, max_len);
  if (rc != KVQ_OK) return rc;
  if (!k || !v) return KVQ_EINVAL;
  if (stride_b < 0 || stride_t < 0 || stride_h < 0) return KVQ_EINVAL;
  if (!aligned16(k) || !aligned16(v) || stride_b % 8 || stride_t % 8 || stride_h % 8)
    return KVQ_EALIGN;
  const int nb = n_blocks_for(max_len);
  if (nb == 0) return KVQ_OK;
  kvq::QuantArgs a = {};
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.stride_b = stride_b;
  a.stride_t = stride_t;
  a.stride_h = stride_h;
  a.k_codes = static_cast<uint8_t*>(cache->k_codes);
  a.v_codes = static_cast<uint8_t*>(cache->v_codes);
  a.k_scale = cache->k_scale;
  a.v_scale = cache->v_scale;
  a.k_zero = cache->k_zero;
  a.v_zero = cache->v_zero;
  a.k_tail = static_cast<uint16_t*>(cache->k_tail);
  a.v_tail = static_cast<uint16_t*>(cache->v_tail);
  a.seq_lens = cache->seq_lens;
  a.heads = cache->heads;
  a.max_blocks = cache->max_blocks;
  a.max_len = max_len;
  a.block_table = cache->block_table;
  a.num_pages = cache->num_pages;
  const hipError_t e = kvq::launch_quantize(cache->scheme, cache->head_dim, cache->batch, nb, a,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_EHIP;
}

int kv_append(const kvq_cache* cache, const void* k_new, const void* v_new,
              int32_t max_len_after, void* stream) {
  kvq::AppendArgs a = {};
  const int rc = append_args(cache, k_new, v_new, max_len_after, &a);
  if (rc != KVQ_OK) return rc;
  const hipError_t e = kvq::launch_append(cache->scheme, cache->head_dim, a,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_EHIP;
}

int decode_attn_plan(const kvq_cache* cache, int32_t max_len, int32_t blocks_per_split,
                     int32_t* blocks_per_split_out, int32_t* splits_per_row_out) {
  int bps, n_split;
  const int rc = plan(cache, max_len, blocks_per_split, &bps, &n_split);
  if (rc != KVQ_OK) return rc;
  if (blocks_per_split_out) *blocks_per_split_out = bps;
  if (splits_per_row_out) *splits_per_row_out = n_split;
  return KVQ_OK;
}

int decode_step_launches(const kvq_cache* cache, int32_t max_len_after,
                         int32_t blocks_per_split) {
  int bps, n_split;
  const int rc = plan(cache, max_len_after, blocks_per_split, &bps, &n_split);
  if (rc != KVQ_OK) return rc;
  return step_is_one_launch(cache, max_len_after, blocks_per_split) ? 1 : 2;
}

size_t decode_attn_workspace_bytes(const kvq_cache* cache, int32_t max_len,
                                   int32_t blocks_per_split) {
  int bps, n_split;
  if (plan(cache, max_len, blocks_per_split, &bps, &n_split) != KVQ_OK) return 0;
  return workspace_bytes(cache, n_split);
}

int decode_attn_split(const kvq_cache* cache, const void* q, float softmax_scale,
                      void* workspace, size_t workspace_bytes_given, int32_t max_len,
                      int32_t blocks_per_split, void* stream) {
  if (!q) return KVQ_EINVAL;
  if (!aligned16(q)) return KVQ_EALIGN;
  kvq::AttnArgs a = {};
  const int rc = attn_args(cache, q, softmax_scale, nullptr, workspace, workspace_bytes_given,
                           max_len, blocks_per_split, 0, &a);
  if (rc != KVQ_OK) return rc;
  if (a.n_split == 0) return KVQ_OK;
  const hipError_t e = kvq::launch_attn_split(cache->scheme, cache->head_dim, cache->batch, a,
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_EHIP;
}

int decode_attn_combine(const kvq_cache* cache, void* out, void* workspace,
                        size_t workspace_bytes_given, int32_t max_len, int32_t blocks_per_split,
                        void* stream) {
  if (!out) return KVQ_EINVAL;
  if (!aligned16(out)) return KVQ_EALIGN;
  kvq::AttnArgs a = {};
  const int rc = attn_args(cache, nullptr, 1.0f, out, workspace, workspace_bytes_given, max_len,
                           blocks_per_split, 0, &a);
  if (rc != KVQ_OK) return rc;
  const hipError_t e = kvq::launch_attn_combine(cache->head_dim, cache->batch, a,
                                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_EHIP;
}

int decode_attn_qkv(const kvq_cache* cache, const void* q, float softmax_scale, void* out,
                    void* workspace, size_t workspace_bytes_given, int32_t max_len,
                    int32_t blocks_per_split, void* stream) {
  if (!q || !out) return KVQ_EINVAL;
  if (!aligned16(q) || !aligned16(out)) return KVQ_EALIGN;
  kvq::AttnArgs a = {};
  const int rc = attn_args(cache, q, softmax_scale, out, workspace, workspace_bytes_given,
                           max_len, blocks_per_split, 1, &a);
  if (rc != KVQ_OK) return rc;
  // One launch: the last workgroup of each row merges its splits. With no context at all
  // a single split column still runs so that every row's zeros are written.
  if (a.n_split == 0) a.n_split = 1;
  return kvq::launch_attn_split(cache->scheme, cache->head_dim, cache->batch, a,
                                static_cast<hipStream_t>(stream)) == hipSuccess ? KVQ_OK
                                                                                : KVQ_EHIP;
}

int decode_attn_qkv_noalloc(const kvq_cache* cache, const void* q, float softmax_scale,
                            void* out, int32_t max_len, int32_t blocks_per_split, void* stream) {
  if (!q || !out) return KVQ_EINVAL;
  if (!aligned16(q) || !aligned16(out)) return KVQ_EALIGN;
  int rc = check_cache(cache);
  if (rc != KVQ_OK) return rc;
  int bps, n_split;
  rc = plan(cache, max_len, blocks_per_split, &bps, &n_split);
  if (rc != KVQ_OK) return rc;
  // the partial states must fit behind the fixed counter region, the rows into it
  const int64_t rows = static_cast<int64_t>(cache->batch) * cache->heads;
  const size_t parts = static_cast<size_t>(rows) * static_cast<size_t>(n_split);
  const size_t need = parts * (static_cast<size_t>(cache->head_dim) + 2) * sizeof(float);
  if (rows > kScratchRows || need > KVQ_NOALLOC_SCRATCH_BYTES - kScratchCounterBytes)
    return KVQ_EWORKSPACE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* base = scratch_for_current_device(s);
  if (!base) return KVQ_EHIP;
  kvq::AttnArgs a = {};
  // the descriptor's workspace fields are set below, from the scratch layout
  rc = attn_args(cache, q, softmax_scale, out, base, workspace_bytes(cache, n_split), max_len,
                 blocks_per_split, 1, &a);
  if (rc != KVQ_OK) return rc;
  a.counters = reinterpret_cast<uint32_t*>(base);
  a.ws_o = reinterpret_cast<float*>(base + kScratchCounterBytes);
  a.ws_ml = a.ws_o + parts * cache->head_dim;
  if (a.n_split == 0) a.n_split = 1;  // every row's zeros are still written
  return kvq::launch_attn_split(cache->scheme, cache->head_dim, cache->batch, a, s) ==
                 hipSuccess ? KVQ_OK : KVQ_EHIP;
}

int decode_step_qkv(const kvq_cache* cache, const void* k_new, const void* v_new, const void* q,
                    float softmax_scale, void* out, void* workspace,
                    size_t workspace_bytes_given, int32_t max_len_after,
                    int32_t blocks_per_split, void* stream) {
  if (!q || !out) return KVQ_EINVAL;
  if (!aligned16(q) || !aligned16(out)) return KVQ_EALIGN;
  kvq::AttnArgs a = {};
  int rc = append_args(cache, k_new, v_new, max_len_after, &a.ap);
  if (rc != KVQ_OK) return rc;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (step_is_one_launch(cache, max_len_after, blocks_per_split)) {
    // one workgroup per row: it appends, then attends the whole row
    const int32_t whole = n_blocks_for(max_len_after) > 0 ? n_blocks_for(max_len_after) : 1;
    rc = attn_args(cache, q, softmax_scale, out, workspace, workspace_bytes_given,
                   max_len_after, whole, 1, &a);
    if (rc != KVQ_OK) return rc;
    return kvq::launch_decode_step(cache->scheme, cache->head_dim, cache->batch, a, s) ==
                   hipSuccess ? KVQ_OK : KVQ_EHIP;
  }
  rc = attn_args(cache, q, softmax_scale, out, workspace, workspace_bytes_given, max_len_after,
                 blocks_per_split, 1, &a);
  if (rc != KVQ_OK) return rc;
  // several splits per row: the splits must all see the appended token
  if (kvq::launch_append(cache->scheme, cache->head_dim, a.ap, s) != hipSuccess) return KVQ_EHIP;
  return kvq::launch_attn_split(cache->scheme, cache->head_dim, cache->batch, a, s) == hipSuccess
             ? KVQ_OK
             : KVQ_EHIP;
}

size_t decode_attn_gqa_workspace_bytes(const kvq_cache* cache, int32_t group, int32_t max_len,
                                       int32_t blocks_per_split) {
  int bps, n_split;
  if (group < 1 || plan(cache, max_len, blocks_per_split, &bps, &n_split, group) != KVQ_OK)
    return 0;
  return workspace_bytes(cache, n_split, group);
}

int decode_attn_gqa_plan(const kvq_cache* cache, int32_t group, int32_t max_len,
                         int32_t blocks_per_split, int32_t* blocks_per_split_out,
                         int32_t* splits_per_row_out) {
  if (group < 1) return KVQ_EINVAL;
  int bps, n_split;
  const int rc = plan(cache, max_len, blocks_per_split, &bps, &n_split, group);
  if (rc != KVQ_OK) return rc;
  if (blocks_per_split_out) *blocks_per_split_out = bps;
  if (splits_per_row_out) *splits_per_row_out = n_split;
  return KVQ_OK;
}

int decode_attn_gqa(const kvq_cache* cache, const void* q, int32_t group, float softmax_scale,
                    void* out, void* workspace, size_t workspace_bytes_given, int32_t max_len,
                    int32_t blocks_per_split, void* stream) {
  if (group == 1)
    return decode_attn_qkv(cache, q, softmax_scale, out, workspace, workspace_bytes_given,
                           max_len, blocks_per_split, stream);
  if (group != 2 && group != 4 && group != 8) return KVQ_EINVAL;
  if (!q || !out) return KVQ_EINVAL;
  if (!aligned16(q) || !aligned16(out)) return KVQ_EALIGN;
  int rc = check_cache(cache);
  if (rc != KVQ_OK) return rc;
  kvq::AttnArgs a = {};
  rc = attn_args(cache, q, softmax_scale, out, workspace, workspace_bytes_given, max_len,
                 blocks_per_split, 1, &a, group);
  if (rc != KVQ_OK) return rc;
  if (a.n_split == 0) a.n_split = 1;  // every row's zeros are still written
  return kvq::launch_attn_gqa(cache->scheme, cache->head_dim, group, cache->batch, a,
                              static_cast<hipStream_t>(stream)) == hipSuccess ? KVQ_OK
                                                                              : KVQ_EHIP;
}

const char* kvq_strerror(int status) {
  switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_EINVAL: return "invalid argument (null pointer, bad scheme, shape, count or length)";
    case KVQ_ENOTSUP:
      return "unsupported configuration (head_dim other than 64 or 128, or a size or scheme "
             "limit of the call)";
    case KVQ_ECAPACITY: return "length bound exceeds the cache capacity (max_blocks * 64)";
    case KVQ_EALIGN: return "pointer or stride breaks the 16-byte alignment rule";
    case KVQ_EWORKSPACE: return "workspace missing or too small";
    case KVQ_EHIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

int kvq_version(void) { return KVQ_VERSION; }

}  // extern "C"
