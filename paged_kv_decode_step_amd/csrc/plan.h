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
//  * a sequence of n tiles costs n + A work units: one per tile, plus A for
//    starting it (the query rotation and, at its end, the append; a
//    wavefront pays these with its loads stalled), and its first tile owns
//    the A + 1 units [s, s + A], tile j >= 1 the unit s + A + j;
//  * sequences are concatenated in (b, h) order: C units in all;
//  * wavefront w of W active ones takes the units [w*C/W, (w+1)*C/W), i.e.
//    the tiles whose first unit falls there, so wavefronts that start many
//    short sequences get fewer tiles and all of them finish together;
//  * a sequence cut between wavefronts ("split") leaves one partial softmax
//    state per piece; a second kernel merges them.
//
// A split sequence starts in exactly one wavefront (as that wavefront's last
// piece) and its pieces sit in consecutive wavefronts (every wavefront owns
// at least one tile when W <= C / (A + 1)).  A wavefront keeps at most two
// partial states: slot 0 for its first piece, slot 1 for its last piece.
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

// Active wavefronts: all of them, unless that leaves fewer than min_units
// work units each.  Never more than C, so every active wavefront has work.
PKV_HD inline int64_t active_waves(int64_t n_units, int64_t n_waves, int64_t min_units) {
  int64_t by_min = (n_units + min_units - 1) / min_units;
  if (by_min < 1) by_min = 1;
  return n_waves < by_min ? n_waves : by_min;
}

PKV_HD inline int64_t wave_start(int64_t w, int64_t n_units, int64_t n_active) {
  return (w * n_units) / n_active;
}

// The wavefront whose unit range holds unit u: the largest w with
// wave_start(w) <= u.
PKV_HD inline int64_t wave_of_unit(int64_t u, int64_t n_units, int64_t n_active) {
  return ((u + 1) * n_active - 1) / n_units;
}

// Largest b in [0, B) with P[b] <= pos, for a non-decreasing prefix array
// P (P[0] = 0) of work units per request (P[b + 1] > P[b]).
PKV_HD inline int find_request(const int* P, int B, int64_t pos) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if ((int64_t)P[mid] <= pos) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Units of request b (hkv sequences of n tiles) and its tiles per sequence,
// from the unit prefix array.
PKV_HD inline int tiles_per_seq(const int* P, int b, int hkv, int cost) {
  return (P[b + 1] - P[b]) / hkv - cost;
}

// First unit of tile j of sequence (b, h) with n tiles.
PKV_HD inline int64_t first_unit(const int* P, int b, int h, int j, int n, int cost) {
  return (int64_t)P[b] + (int64_t)h * (n + cost) + (j == 0 ? 0 : cost + j);
}

// The first tile whose first unit is >= x (x < total units), as
// (request, head, tile), with the tile possibly == n (then it is tile 0 of
// the next sequence).
struct TilePos { int b, h, j, n; };
PKV_HD inline TilePos tile_at_unit(const int* P, int B, int hkv, int cost, int64_t x) {
  TilePos t;
  t.b = find_request(P, B, x);
  t.n = tiles_per_seq(P, t.b, hkv, cost);
  const int64_t r = x - P[t.b];
  const int per = t.n + cost;
  t.h = (int)(r / per);
  const int c = (int)(r - (int64_t)t.h * per);
  t.j = c == 0 ? 0 : (c - cost > 1 ? c - cost : 1);
  return t;
}

// Global tile index (tiles of all sequences concatenated) of tile (b, h, j)
// of a sequence with n tiles.
PKV_HD inline int64_t global_tile(const int* P, int b, int h, int j, int n, int hkv, int cost) {
  return ((int64_t)P[b] - (int64_t)hkv * cost * b) + (int64_t)h * n + j;
}

}  // namespace pkv
