// blocks.hip -- whole-block copies inside the KV pool (copy on write).
//
// A block that several sequences share (a common prefix, "Lesson 13.17
// TensorRT-LLM: NVIDIA's Optimized Inference Engine", section "The paged KV
// cache, in-flight batching and CUDA graphs") is copied to a fresh block
// before one of them appends to it; the host allocator names the pairs.  The
// copy moves a block's K and V bytes for every head and slot as they are
// stored, so the layout inside a block does not matter here.  It is a plain
// HBM-bound copy: one workgroup per (pair, K or V) streams 16-byte words.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace pkv {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kBlockThreads) void copy_blocks_kernel(
    const int32_t* __restrict__ pairs, int64_t block_words, int32_t num_blocks,
    char* __restrict__ k_pool, char* __restrict__ v_pool, uint32_t* __restrict__ err) {
  const int32_t src = pairs[2 * (int64_t)blockIdx.x];
  const int32_t dst = pairs[2 * (int64_t)blockIdx.x + 1];
  if ((unsigned)src >= (unsigned)num_blocks || (unsigned)dst >= (unsigned)num_blocks) {
    if (threadIdx.x == 0) err[0] = 1u;
    return;
  }
  if (src == dst) return;
  char* base = blockIdx.y == 0 ? k_pool : v_pool;
  const u32x4_t* s = reinterpret_cast<const u32x4_t*>(base + (int64_t)src * block_words * 16);
  u32x4_t* d = reinterpret_cast<u32x4_t*>(base + (int64_t)dst * block_words * 16);
  for (int64_t i = threadIdx.x; i < block_words; i += kBlockThreads) d[i] = s[i];
}

}  // namespace

hipError_t launch_copy_blocks(const int32_t* pairs, int32_t n, int64_t block_bytes,
                              int32_t num_blocks, void* k_pool, void* v_pool, uint32_t* err,
                              hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)n, 2), dim3(kBlockThreads), 0, stream,
                     pairs, block_bytes / 16, num_blocks, static_cast<char*>(k_pool),
                     static_cast<char*>(v_pool), err);
  return hipGetLastError();
}

}  // namespace pkv
