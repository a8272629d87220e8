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
//  * sequences are concatenated in (b, h) order: U units in all;
//  * wavefront w has a weight: the first n_first wavefronts (the first
//    workgroup that lands on each compute unit) weigh wa, the others wb.
//    Two wavefronts that share a SIMD do not progress alike: the older one
//    wins most issue slots and streams 1.6-1.9x faster while both run, so
//    equal shares leave the younger ones finishing long after.  The
//    weights apply only with at least min_share units per wavefront;
//    below that, start-up dominates and the weights are even;  With
//    Omega(w) the summed weight of wavefronts [0, w), wavefront w of W
//    active ones takes the units [U Omega(w) / Omega(W), U Omega(w+1) /
//    Omega(W)), i.e. the tiles whose first unit falls there;
//  * W is the most wavefronts (at most n_waves) that still give the
//    lightest one min_units units, and min_units > A: every window of A + 1
//    consecutive units holds the first unit of some tile, so every active
//    wavefront owns at least one tile;
//  * a sequence cut between wavefronts ("split") leaves one partial softmax
//    state per piece; a second kernel merges them.
//
// A split sequence starts in exactly one wavefront (as that wavefront's last
// piece) and its pieces sit in consecutive wavefronts.  A wavefront keeps at
// most two partial states: slot 0 for its first piece, slot 1 for its last
// piece.
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

// Weights of the wavefronts: [0, n_first) weigh wa, the rest wb (wa >= wb >= 1).
struct WaveWeights {
  int64_t wa, wb, n_first;
};

// The weights in force for a step of n_units units: the given ones when
// there are at least min_share units per launched wavefront, else even
// weights (with a few tiles per wavefront the start-up dominates and the
// older wavefront has no time to pull ahead).
PKV_HD inline WaveWeights weights_for(int64_t n_units, int64_t n_waves, int64_t min_share,
                                      const WaveWeights& k) {
  if (n_units >= min_share * n_waves) return k;
  return WaveWeights{1, 1, k.n_first};
}

// Omega(w): summed weight of wavefronts [0, w).
PKV_HD inline int64_t cum_weight(int64_t w, const WaveWeights& k) {
  return w <= k.n_first ? k.wa * w : k.wa * k.n_first + k.wb * (w - k.n_first);
}

// Largest w >= 0 with Omega(w) <= x, for x >= 0.
PKV_HD inline int64_t weight_index(int64_t x, const WaveWeights& k) {
  const int64_t f = k.wa * k.n_first;
  return x < f ? x / k.wa : k.n_first + (x - f) / k.wb;
}

// Active wavefronts: the most (at most n_waves, at least 1) whose lightest
// member still gets min_units units, U * weight / Omega(W) >= min_units.
PKV_HD inline int64_t active_waves(int64_t n_units, int64_t n_waves, int64_t min_units,
                                   const WaveWeights& k) {
  int64_t W = n_units / min_units;                 // all of weight wa
  if (W > k.n_first) W = weight_index(n_units * k.wb / min_units, k);
  if (W < k.n_first && n_units / min_units >= k.n_first) W = k.n_first;
  if (W > n_waves) W = n_waves;
  return W < 1 ? 1 : W;
}

PKV_HD inline int64_t wave_start(int64_t w, int64_t n_units, int64_t n_active,
                                 const WaveWeights& k) {
  return n_units * cum_weight(w, k) / cum_weight(n_active, k);
}

// The wavefront whose unit range holds unit u: the largest w < n_active
// with wave_start(w) <= u.
PKV_HD inline int64_t wave_of_unit(int64_t u, int64_t n_units, int64_t n_active,
                                   const WaveWeights& k) {
  const int64_t w = weight_index(((u + 1) * cum_weight(n_active, k) - 1) / n_units, k);
  return w < n_active - 1 ? w : n_active - 1;
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
