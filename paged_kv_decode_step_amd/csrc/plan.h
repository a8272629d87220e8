// plan.h -- work partition of one decode step, shared by the device kernel and
// the host replay used in tests.
//
// Ragged batches are the throughput problem the pages keep returning to: a
// static batch pads every request to the longest one ("TensorRT-LLM Guide:
// High-Throughput GPU Inference Engine", section "2. The Failure of Static
// Batching") and in-flight batching computes no padding at all (same page,
// "1. In-Flight Batching: Continuous Iteration Scheduling").  Here no padding
// is computed and the work is spread evenly over the GPU's wavefronts:
//
//  * a sequence is one (request b, KV head h) pair; it is cut into tiles of
//    16 tokens (the last one partial), at least one tile each;
//  * sequences are concatenated in (b, h) order: N tiles in all;
//  * wavefront w of W active ones takes tiles [w*N/W, (w+1)*N/W), so any two
//    wavefronts differ by at most one tile whatever the length mix;
//  * a sequence cut between wavefronts ("split") leaves one partial softmax
//    state per piece; the wavefront that finishes the last of its pieces
//    merges them.
//
// A split sequence starts in exactly one wavefront (as that wavefront's last
// piece), so the arrival counter and the merge of a split sequence are keyed
// by that first wavefront.  A wavefront keeps at most two partial states:
// slot 0 for its first piece, slot 1 for its last piece.
#pragma once

#include <stdint.h>

#ifndef PKV_HD
#if defined(__HIPCC__)
#define PKV_HD __host__ __device__
#else
#define PKV_HD
#endif
#endif

namespace pkv {

enum : int {
  PIECE_SPLIT = 1,      // the piece's sequence spans more than one wavefront
  PIECE_FIRST = 2,      // the piece is its wavefront's first
  PIECE_LAST = 4,       // the piece ends its sequence
};

// Tiles of one sequence with context length L (clamped to [0, cap]).
PKV_HD inline int tiles_of(int L, int cap) {
  if (L < 0) L = 0;
  if (L > cap) L = cap;
  int n = (L + 15) >> 4;
  return n < 1 ? 1 : n;
}

// Active wavefronts: all of them, unless that leaves fewer than min_tiles
// tiles each.  Never more than N, so every active wavefront has work.
PKV_HD inline int64_t active_waves(int64_t n_tiles, int64_t n_waves, int64_t min_tiles) {
  int64_t by_min = (n_tiles + min_tiles - 1) / min_tiles;
  if (by_min < 1) by_min = 1;
  return n_waves < by_min ? n_waves : by_min;
}

PKV_HD inline int64_t wave_start(int64_t w, int64_t n_tiles, int64_t n_active) {
  return (w * n_tiles) / n_active;
}

// The wavefront whose range holds global tile g: the largest w with
// wave_start(w) <= g.
PKV_HD inline int64_t wave_of_tile(int64_t g, int64_t n_tiles, int64_t n_active) {
  return ((g + 1) * n_active - 1) / n_tiles;
}

// Largest b in [0, B) with hkv * P[b] <= pos, for a strictly increasing
// prefix array P (P[0] = 0) of tiles per request.
PKV_HD inline int find_request(const int* P, int B, int64_t pos, int hkv) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if ((int64_t)hkv * P[mid] <= pos) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Where the partial state of a split sequence's piece k lives, given the
// sequence's first global tile `seq_begin` and first wavefront wf: piece k
// is held by wavefront wf + k; pieces k > 0 are their wavefront's first
// piece (slot 0); piece 0 is wavefront wf's last piece, which is also its
// first (slot 0) only if wf starts exactly at the sequence.
PKV_HD inline int first_piece_slot(int64_t seq_begin, int64_t wf, int64_t n_tiles,
                                   int64_t n_active) {
  return wave_start(wf, n_tiles, n_active) == seq_begin ? 0 : 1;
}

}  // namespace pkv
