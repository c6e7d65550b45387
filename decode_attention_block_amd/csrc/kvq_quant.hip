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
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

// Maxima of N values over the workgroup; every thread receives the results.
template <int N>
__device__ __forceinline__ void block_max(float (&v)[N], float* lds /* [N * kWaves] */) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = wave_max(v[i]);
  const int w = threadIdx.x / kWave;
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

// ---- prefill: grid (blocks, heads, batch * 2) ---------------------------------------
template <int SCHEME, int D>
__global__ __launch_bounds__(kThreads) void quantize_blocks_kernel(QuantArgs a) {
  using G = QGeo<SCHEME, D>;
  __shared__ float red[2 * kWaves];
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
#pragma unroll
  for (int p = 0; p < G::kPasses; ++p) {
    const int t = p * G::kTokensPerPass + tr;
    store_codes<SCHEME, D>(codes + t * G::kRowBytes, chunk, x[p], s, zpi, t < ntok);
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

// ---- append one token per sequence: grid (heads, batch, 2) --------------------------
template <int SCHEME, int D>
__global__ __launch_bounds__(kThreads) void append_kernel(AppendArgs a) {
  using G = QGeo<SCHEME, D>;
  __shared__ float red[4 * kWaves];
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int kv = blockIdx.z;
  const int cap = a.max_blocks * kBlock;
  const int len = a.seq_lens[b];
  if (len < 0 || len >= cap) return;  // no room: the row is left unchanged
  const int slot = len % kBlock;
  const int j = len / kBlock;

  const int tid = threadIdx.x;
  const int tr = tid / G::kThreadsPerToken;
  const int chunk = tid % G::kThreadsPerToken;
  const int64_t row = static_cast<int64_t>(b) * a.heads + h;
  uint16_t* tail = (kv ? a.v_tail : a.k_tail) + row * kBlock * D + chunk * 8;
  const uint16_t* fresh = (kv ? a.v_new : a.k_new) + row * D + chunk * 8;

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
      raw[p] = *reinterpret_cast<const uint4*>(fresh);
    else
      raw[p] = make_uint4(0u, 0u, 0u, 0u);
    unpack8(raw[p], x[p]);
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

  const int64_t blk = row * a.max_blocks + j;
  uint8_t* codes = (kv ? a.v_codes : a.k_codes) + blk * kBlock * G::kRowBytes;
#pragma unroll
  for (int p = 0; p < G::kPasses; ++p) {
    const int t = p * G::kTokensPerPass + tr;
    if (full || t == slot)
      store_codes<SCHEME, D>(codes + t * G::kRowBytes, chunk, x[p], s, zpi, t <= slot);
    if (t == slot) *reinterpret_cast<uint4*>(tail + t * D) = raw[p];
  }
  if (tid == 0 && full) {
    (kv ? a.v_scale : a.k_scale)[blk] = s;
    float* zero = kv ? a.v_zero : a.k_zero;
    if (zero) zero[blk] = zp;
  }
}

__global__ void bump_lens_kernel(int32_t* seq_lens, int batch, int cap) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch) {
    const int len = seq_lens[b];
    if (len >= 0 && len < cap) seq_lens[b] = len + 1;
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
  dim3 grid(a.heads, a.batch, 2);
  hipLaunchKernelGGL((append_kernel<SCHEME, D>), grid, dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int threads = 256;
  hipLaunchKernelGGL(bump_lens_kernel, dim3((a.batch + threads - 1) / threads), dim3(threads),
                     0, s, a.seq_lens, a.batch, a.max_blocks * kBlock);
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
