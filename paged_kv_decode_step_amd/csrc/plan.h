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
//  * a sequence is one (request b, KV head h) pair; it is cut into steps of
//    STEP tokens (the last one partial), at least one step each;
//  * sequences are concatenated in (b, h) order: N steps in all;
//  * wavefront w of We active ones takes steps [w*N/We, (w+1)*N/We), so any
//    two wavefronts differ by at most one step whatever the length mix;
//  * a sequence cut between wavefronts ("split") leaves one partial softmax
//    state per piece; the reduce kernel merges them.
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
  HDR_TRIGGER = 1,      // header: this wavefront's first piece closes a split
                        // sequence, so the reduce kernel merges it here
};

// Steps of one sequence with context length L (clamped to [0, cap]).
PKV_HD inline int steps_of(int L, int cap, int step_tokens) {
  if (L < 0) L = 0;
  if (L > cap) L = cap;
  int n = (L + step_tokens - 1) / step_tokens;
  return n < 1 ? 1 : n;
}

// Active wavefronts: all of them, unless that leaves fewer than min_steps
// steps each.  Never more than N, so every active wavefront has work.
PKV_HD inline int64_t active_waves(int64_t n_steps, int64_t n_waves,
                                   int64_t min_steps) {
  int64_t by_min = (n_steps + min_steps - 1) / min_steps;
  if (by_min < 1) by_min = 1;
  return n_waves < by_min ? n_waves : by_min;
}

PKV_HD inline int64_t wave_start(int64_t w, int64_t n_steps, int64_t n_active) {
  return (w * n_steps) / n_active;
}

// The wavefront whose range holds global step s: the largest w with
// wave_start(w) <= s.
PKV_HD inline int64_t wave_of_step(int64_t s, int64_t n_steps, int64_t n_active) {
  return ((s + 1) * n_active - 1) / n_steps;
}

// Largest b in [0, B) with hkv * P[b] <= pos, for a strictly increasing
// prefix array P (P[0] = 0) of steps per request.
PKV_HD inline int find_request(const int* P, int B, int64_t pos, int hkv) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if ((int64_t)hkv * P[mid] <= pos) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace pkv
