// stream_read.hip -- a plain streaming read of device memory: what one kernel
// pulls from HBM on this GPU with the same 16-byte nontemporal loads the
// attention kernel uses, the reference next to the nominal 8 TB/s peak.
//
// Each workgroup reads kUnroll consecutive 4 KiB runs per round (every lane
// 16 bytes of each, coalesced), with all of them in flight before the first
// is used; the grid strides over the buffer.  The loaded words are folded
// into one value per lane, stored only if it equals a constant no real
// buffer is expected to produce, so the loads cannot be dropped while
// nothing is written in practice.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace pkv {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kUnroll = 8;

__global__ __launch_bounds__(kBlockThreads) void stream_read_kernel(
    const u32x4_t* __restrict__ src, int64_t n16, uint32_t* __restrict__ sink) {
  const int64_t per_round = (int64_t)kBlockThreads * kUnroll;
  const int64_t stride = (int64_t)gridDim.x * per_round;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (int64_t base = blockIdx.x * per_round + threadIdx.x; base < n16; base += stride) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + (int64_t)u * kBlockThreads;
      v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  const uint32_t h = acc[0] ^ (acc[1] * 3u) ^ (acc[2] * 5u) ^ (acc[3] * 7u);
  if (h == 0x9e3779b9u) sink[threadIdx.x] = h;
}

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int n_groups,
                              hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)n_groups), dim3(kBlockThreads), 0, stream,
                     static_cast<const u32x4_t*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace pkv
