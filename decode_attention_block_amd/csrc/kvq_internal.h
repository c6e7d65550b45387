// kvq_internal.h — host-side launch descriptors shared by the libkvq sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

struct QuantArgs {
  const uint16_t* k;
  const uint16_t* v;
  int64_t stride_b, stride_t, stride_h;
  uint8_t* k_codes;
  uint8_t* v_codes;
  float* k_scale;
  float* v_scale;
  float* k_zero;
  float* v_zero;
  uint16_t* k_tail;
  uint16_t* v_tail;
  const int32_t* seq_lens;
  int heads, max_blocks, max_len;
  const int32_t* block_table;  // paged layout, else nullptr
  int num_pages;
};

struct AppendArgs {
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint8_t* k_codes;
  uint8_t* v_codes;
  float* k_scale;
  float* v_scale;
  float* k_zero;
  float* v_zero;
  uint16_t* k_tail;
  uint16_t* v_tail;
  int32_t* seq_lens;
  int batch, heads, max_blocks;
  const int32_t* block_table;  // paged layout, else nullptr
  int num_pages;
};

struct AttnArgs {
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const float* k_scale;
  const float* v_scale;
  const float* k_zero;
  const float* v_zero;
  const int32_t* seq_lens;
  const uint16_t* q;
  uint16_t* out;
  uint32_t* counters;  // [rows] arrival counters of the fused combine (zero between calls)
  float* ws_o;         // [rows][n_split][D] unnormalised partial outputs
  float* ws_ml;        // [rows][n_split][2]  (running max in log2 units, sum of weights)
  int heads, max_blocks, max_len, bps, n_split;
  // bps == 0: the split of every row is chosen on the device from all the rows' lengths
  // (split_plan in kvq_attn.hip), aiming at plan_target workgroups; n_split is then the
  // most splits a row may take (the grid's split dimension)
  int batch, plan_target;
  int fused;           // 1: the last workgroup of each row merges the splits and writes out
  float qk_scale;      // softmax_scale * log2(e)
  const int32_t* block_table;  // paged layout, else nullptr
  int num_pages;
  AppendArgs ap;       // fused decode step: the token each row's workgroup appends first
};

// Launchers (return hipError_t of the launch).
hipError_t launch_quantize(int scheme, int head_dim, int batch, int n_blocks,
                           const QuantArgs& a, hipStream_t s);
hipError_t launch_append(int scheme, int head_dim, const AppendArgs& a, hipStream_t s);
hipError_t launch_attn_split(int scheme, int head_dim, int batch, const AttnArgs& a,
                             hipStream_t s);
// Fused decode step (one split per row): each workgroup appends its row's token (a.ap),
// then attends over the row including it.
hipError_t launch_decode_step(int scheme, int head_dim, int batch, const AttnArgs& a,
                              hipStream_t s);
hipError_t launch_attn_combine(int head_dim, int batch, const AttnArgs& a, hipStream_t s);
// Grouped-query attention: `group` (2, 4 or 8) query rows per cache row, in one launch,
// on the matrix cores for every scheme; out and the partial states are indexed by query
// row (cache row * group + g).
hipError_t launch_attn_gqa(int scheme, int head_dim, int group, int batch, const AttnArgs& a,
                           hipStream_t s);

}  // namespace kvq
