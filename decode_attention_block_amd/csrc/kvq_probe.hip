// kvq_probe.hip — measurement aids, not part of the method: a plain streaming read of
// a device buffer at the access pattern of the attention kernels, whose rate is the
// practical read ceiling those kernels are compared with (HBM peak being the spec), and
// a kernel that holds a stream for a set time (so that timing events recorded behind it
// bracket only the GPU's execution of the work queued after them).
//
// Each 256-thread workgroup reads one contiguous slab of the buffer (as an attention
// workgroup reads one row's codes) with 16-byte non-temporal buffer loads, every lane
// with kUnroll loads in flight, and folds what it read into one word per thread (so the
// loads cannot be dropped) that it stores to `sink`.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"
#include "kvq_device.h"

namespace kvq {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kUnroll = 8;
constexpr int kStride = kProbeThreads * 16;  // bytes one load instruction of the group covers

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint8_t* buf, int64_t bytes,
                                                                   int slab, uint32_t* sink) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * slab;
  const int len = static_cast<int>(min(static_cast<int64_t>(slab), bytes - base));
  // loads past `len` return zeros and touch no memory
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(buf + base), 0, len, kBufferRsrcWord3);
  // The whole offset is the per-lane operand, which the range check covers, so the
  // loads of the last slab past `len` return zeros instead of reading past the buffer.
  const int voff = threadIdx.x * 16;
  uint32_t acc = 0;
  for (int off = 0; off < len; off += kStride * kUnroll) {
    uint4 r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) r[u] = load_b128<2>(rs, off + u * kStride + voff, 0);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= r[u].x ^ r[u].y ^ r[u].z ^ r[u].w;
  }
  sink[static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x] = acc;
}

// Holds its stream for `ticks` of the 100 MHz real-time counter: one wave sleeping in a
// loop, no memory traffic. Bounded twice: by the counter and by kMaxSpins sleeps.
constexpr uint32_t kMaxSpins = 1u << 22;

__global__ __launch_bounds__(64) void hold_kernel(uint64_t ticks) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (uint32_t spins = 0; spins < kMaxSpins; ++spins) {
    if (__builtin_amdgcn_s_memrealtime() - t0 >= ticks) break;
    __builtin_amdgcn_s_sleep(8);
  }
}

}  // namespace
}  // namespace kvq

extern "C" int kvq_probe_hold(uint32_t microseconds, void* stream) {
  if (microseconds == 0 || microseconds > 100000) return KVQ_EINVAL;
  hipLaunchKernelGGL(kvq::hold_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint64_t>(microseconds) * 100u);
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_EHIP;
}

extern "C" int kvq_probe_stream_read(const void* buf, size_t bytes, int32_t workgroups,
                                     uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes == 0 || workgroups <= 0) return KVQ_EINVAL;
  if (reinterpret_cast<uintptr_t>(buf) & 15u) return KVQ_EALIGN;
  // slabs are whole multiples of one group-wide load (4 KiB) and stay below 2^31 bytes
  const int64_t b = static_cast<int64_t>(bytes);
  const int64_t unit = kvq::kStride;
  const int64_t slab = (b + static_cast<int64_t>(workgroups) * unit - 1) /
                       (static_cast<int64_t>(workgroups) * unit) * unit;
  if (slab > INT32_MAX - kvq::kStride * kvq::kUnroll) return KVQ_ENOTSUP;
  const int64_t n = (b + slab - 1) / slab;  // <= workgroups, every slab non-empty
  hipLaunchKernelGGL(kvq::read_probe_kernel, dim3(static_cast<uint32_t>(n)),
                     dim3(kvq::kProbeThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint8_t*>(buf), b, static_cast<int>(slab), sink);
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_EHIP;
}
