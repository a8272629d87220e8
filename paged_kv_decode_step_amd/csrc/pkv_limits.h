// pkv_limits.h -- sizes the kernels are built for, shared by the launch code and
// the host-only checks (no HIP headers, so plain C++ can use them too).
#pragma once

namespace pkv {

constexpr int kGroupMax = 16;      // query heads per KV head the kernel serves
constexpr int kMaxBatch = 4096;    // requests per step (LDS prefix array)
constexpr int kWaveThreads = 64;
constexpr int kBlockThreads = 256; // 4 wavefronts per workgroup
constexpr int kTileTokens = 16;    // tokens per KV tile (the unit of work)
constexpr int kMaxPieceCost = 64;  // work units a sequence start may cost
constexpr int kWeightMinShare = 256;  // units per wavefront for uneven weights

}  // namespace pkv
