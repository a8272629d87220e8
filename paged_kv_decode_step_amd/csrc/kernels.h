// kernels.h -- launch interface between the host library and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_limits.h"

namespace pkv {

enum KvKind : int { KV_F32 = 0, KV_BF16 = 1, KV_FP8 = 2 };

struct DecodeParams {
  const void* q;             // [B][Hq][D] io dtype
  const void* k_new;         // [B][Hkv][D]
  const void* v_new;
  void* out;                 // [B][Hq][D]
  const int32_t* positions;  // [B]
  const int32_t* block_tables;  // [B][max_blocks]
  const int32_t* context_lens;  // [B]
  void* k_pool;
  void* v_pool;
  const float* rope_cos;     // [max_pos][D/2]
  const float* rope_sin;
  const float* fp8_scales;   // [4][Hkv]: k_scale, v_scale, 1/k_scale, 1/v_scale
  float* partials;           // [n_waves][2][partial_floats(D)]
  int4* headers;             // [n_waves] {split, request * Hkv + head, pieces, slot} of the
                             // split sequence whose first piece the wavefront holds
  const void* dummy;         // >= 8 KiB of readable device memory (tail loads)
  uint64_t* timeline;        // [n_waves][8] per-wavefront phase stamps (timeline builds; else null)
  uint32_t* err;             // [4] range flags
  int32_t num_blocks;        // < 2^31 (checked at pool creation)
  int32_t batch;
  int32_t n_kv_heads;
  int32_t group;
  int32_t max_blocks;        // block-table row length
  int32_t max_pos;
  int32_t n_waves;           // wavefronts launched (multiple of 4)
  int32_t min_units;         // fewest work units a wavefront is given (> piece_cost)
  int32_t piece_cost;        // work units a sequence costs on top of its tiles
  int32_t n_first;           // wavefronts of the first workgroup on each compute unit
  int32_t weight_first;      // their share weight ...
  int32_t weight_rest;       // ... and that of the others (weight_first >= weight_rest >= 1)
  int32_t weight_odd;        // parity weight of odd workgroups, percent of even ones' (1..100)
  int32_t weight_min_share;  // units per wavefront below which the weights are even
  float sm_scale_log2;       // log2(e) / sqrt(D)
  int32_t window;            // attention window in tokens (0 = the whole context)
  int32_t n_qtok;            // new tokens per request (1, or up to 16 / group)
};

// Floats of one partial softmax state: the accumulator of all 64 lanes
// (lane-major, D/4 floats each) and a (max, sum) pair per query head.
constexpr int partial_floats(int head_dim) { return 16 * head_dim + 2 * kGroupMax; }

// Launch the fused append+attention kernel and the split-merge kernel on
// `stream`; with `events` (4 of them), the start and stop of each kernel.
hipError_t launch_decode(int kv_kind, int head_dim, int block_size, const DecodeParams& p,
                         hipStream_t stream, hipEvent_t* events);

// The kernels of one cache type (each built in an object of its own): with
// p, launch a step; without, the occupancy of the attention kernel in
// *blocks.  And the tiles each wavefront keeps in flight.
template <int KV>
hipError_t decode_dispatch(int head_dim, int block_size, const DecodeParams* p, hipStream_t stream,
                           hipEvent_t* events, int* blocks);
template <> hipError_t decode_dispatch<KV_F32>(int, int, const DecodeParams*, hipStream_t,
                                               hipEvent_t*, int*);
template <> hipError_t decode_dispatch<KV_BF16>(int, int, const DecodeParams*, hipStream_t,
                                                hipEvent_t*, int*);
template <> hipError_t decode_dispatch<KV_FP8>(int, int, const DecodeParams*, hipStream_t,
                                               hipEvent_t*, int*);
template <int KV>
int decode_ring_tiles_of(int head_dim);
template <> int decode_ring_tiles_of<KV_F32>(int);
template <> int decode_ring_tiles_of<KV_BF16>(int);
template <> int decode_ring_tiles_of<KV_FP8>(int);

// Tiles the attention kernel keeps in flight per wavefront (its load ring).
int decode_ring_tiles(int kv_kind, int head_dim);

// Resident 256-thread workgroups per compute unit for the attention kernel.
hipError_t decode_occupancy(int kv_kind, int head_dim, int block_size, int* blocks_per_cu);

// Copy n whole blocks of the pool, K and V, from pairs[2i] to pairs[2i + 1]
// (device int32 pairs; block_bytes per block of K, a multiple of 16).  Ids
// outside [0, num_blocks) set err[0] and are skipped.
hipError_t launch_copy_blocks(const int32_t* pairs, int32_t n, int64_t block_bytes,
                              int32_t num_blocks, void* k_pool, void* v_pool, uint32_t* err,
                              hipStream_t stream);

// Read `bytes` (a multiple of 16) at `src` with n_groups workgroups of
// nontemporal 16-byte loads; sink (256 words) is written only if the folded
// data equals a fixed constant.
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int n_groups,
                              hipStream_t stream);

// Bytes of workspace the kernels need for n_waves wavefronts (partials).
constexpr size_t partials_bytes(int n_waves, int head_dim) {
  return (size_t)n_waves * 2 * partial_floats(head_dim) * sizeof(float);
}

// Bytes of a whole split-K workspace: the partial states, then (at the next
// 256-byte boundary) one header per wavefront.
constexpr size_t headers_offset(int n_waves, int head_dim) {
  return (partials_bytes(n_waves, head_dim) + 255) / 256 * 256;
}
constexpr size_t workspace_bytes(int n_waves, int head_dim) {
  return headers_offset(n_waves, head_dim) + (size_t)n_waves * 16;
}

// The fixed per-device workspace of decode_step_noalloc: room for 2048
// wavefronts (8 per compute unit on 256 compute units) at head_dim <= 128,
// about 32.5 MiB.
constexpr int kScratchMaxWaves = 2048;
constexpr int kScratchMaxHeadDim = 128;
constexpr size_t kScratchBytes = workspace_bytes(kScratchMaxWaves, kScratchMaxHeadDim);

// Device address of the fixed workspace on `device` (looked up once per
// device, with that device current, then kept).
hipError_t scratch_address(int device, void** addr);

constexpr size_t kDummyBytes = 16384;

}  // namespace pkv
