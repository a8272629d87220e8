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
//  * wavefront w has a weight, the product of an age weight and a parity
//    weight.  Age: the first n_first wavefronts (the first workgroup that
//    lands on each compute unit) weigh wa, the others wb.  Two wavefronts
//    that share a SIMD do not progress alike: the older one wins most issue
//    slots and streams 1.6-1.9x faster while both run, so equal shares leave
//    the younger ones finishing long after.  The age weights apply only with
//    at least min_share units per wavefront; below that, start-up dominates
//    and they are even.  Parity: wavefronts of odd workgroups, which run on
//    the odd XCDs, weigh po percent of the others.  With Omega(w) the summed
//    weight of wavefronts [0, w), wavefront w of W active ones takes the
//    units [U Omega(w) / Omega(W), U Omega(w+1) / Omega(W)), i.e. the tiles
//    whose first unit falls there;
//  * W is the most wavefronts (at most n_waves) that would still give a
//    wavefront of the lightest weight min_units units, and min_units > A:
//    every window of A + 1 consecutive units holds the first unit of some
//    tile, so every active wavefront owns at least one tile.  A step too
//    small to give the first workgroup of every compute unit that much is
//    spread over up to those wavefronts with smaller shares, still > A
//    (active_waves);
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

// floor(a / b) for 0 <= a < 2^62 and b >= 1 with a quotient below 2^50.
// The double quotient is within one of the exact one at these sizes, and
// the two integer products settle it; on the GPU this costs a few VALU
// operations where a 64-bit integer division is a long scalar routine run
// by every wavefront before its first load.
PKV_HD inline int64_t floor_div(int64_t a, int64_t b) {
  int64_t q = (int64_t)((double)a / (double)b);
  if (q * b > a) --q;
  else if ((q + 1) * b <= a) ++q;
  return q;
}

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

// First tile a sequence of context length L (clamped to [0, cap]) reads: with
// an attention window of `window` >= 1 tokens the step attends to the tokens
// [L - window, L), so the whole tiles before token L - window are skipped;
// without one (window 0) it is tile 0.  A sequence then reads
// tiles_of(L, cap) - window_first_tile(L, cap, window) >= 1 tiles.
PKV_HD inline int window_first_tile(int L, int cap, int window) {
  if (L < 0) L = 0;
  if (L > cap) L = cap;
  return (window > 0 && L > window) ? (L - window) >> 4 : 0;
}

// Weights of the wavefronts.  Wavefront w belongs to workgroup w / 4; its
// weight is its age weight (wa for the first n_first wavefronts, the first
// workgroup that lands on each compute unit, wb for the others, wa >= wb >= 1)
// times its parity weight: 100 in even workgroups, po in odd ones
// (1 <= po <= 100).  Workgroups are dealt to the GPU's eight XCDs in turn,
// so odd workgroups run on odd XCDs, which were measured to stream about a
// tenth slower than the even ones.
struct WaveWeights {
  int32_t wa, wb, n_first, po;
};

// The weights in force for a step of n_units units: the given ones when
// there are at least min_share units per launched wavefront, else even age
// weights (with a few tiles per wavefront the start-up dominates and the
// older wavefront has no time to pull ahead); the parity weight stays.
PKV_HD inline WaveWeights weights_for(int64_t n_units, int64_t n_waves, int64_t min_share,
                                      const WaveWeights& k) {
  if (n_units >= min_share * n_waves) return k;
  return WaveWeights{1, 1, k.n_first, k.po};
}

// Summed parity weight of wavefronts [0, w): 100 per wavefront of an even
// workgroup, po per wavefront of an odd one.
PKV_HD inline int64_t parity_sum(int64_t w, int64_t po) {
  const int64_t g = w >> 2, r = w & 3;
  const int64_t odd = 4 * (g >> 1) + ((g & 1) ? r : 0);
  return 100 * (w - odd) + po * odd;
}

// Largest w >= 0 with parity_sum(w) <= y, for y >= 0: whole pairs of an
// even and an odd workgroup (400 + 4 po), then the wavefronts of the pair.
PKV_HD inline int64_t parity_index(int64_t y, int64_t po) {
  const int64_t per = 400 + 4 * po;
  const int64_t n = floor_div(y, per);
  const int rem = (int)(y - n * per);
  return 8 * n + (rem < 400 ? rem / 100 : 4 + (rem - 400) / (int)po);
}

// Omega(w): summed weight of wavefronts [0, w).
PKV_HD inline int64_t cum_weight(int64_t w, const WaveWeights& k) {
  if (w <= k.n_first) return k.wa * parity_sum(w, k.po);
  const int64_t sf = parity_sum(k.n_first, k.po);
  return k.wa * sf + k.wb * (parity_sum(w, k.po) - sf);
}

// Largest w >= 0 with Omega(w) <= x, for x >= 0.
PKV_HD inline int64_t weight_index(int64_t x, const WaveWeights& k) {
  const int64_t sf = parity_sum(k.n_first, k.po);
  const int64_t f = k.wa * sf;
  return x < f ? parity_index(floor_div(x, k.wa), k.po)
               : parity_index(sf + floor_div(x - f, k.wb), k.po);
}

// Smallest share a small step's wavefronts are given (see active_waves):
// min_units / 4, and never less than cost + 1 units, which still gives every
// active wavefront a tile.
PKV_HD inline int64_t small_share(int64_t min_units, int64_t cost) {
  const int64_t q = min_units / 4;
  return q > cost + 1 ? q : cost + 1;
}

// Active wavefronts: the most (at most n_waves, at least 1) with
// Omega(W) <= U * w_min / m, w_min the lightest weight any of the n_waves
// wavefronts has; then every active one gets at least m units,
// U * weight / Omega(W) >= m.  m is min_units, except for a step so small
// that min_units each would leave some of the first n_first wavefronts (the
// first workgroup on each compute unit) idle.  Such a step is latency-bound:
// each wavefront's chain of a few tiles sets its time, not the memory.  It
// is spread further, with m = small_share(min_units, cost), over at most
// n_first wavefronts, which run one to a SIMD.  Measured on the
// Llama-3-8B-shaped batch with a 256-token window (665 wavefronts at 16
// units each, 11 tiles apiece) and on 3 requests of 84-1012 tokens
// (24 wavefronts), attention us at m = 16 / 12 / 10 / 8 / 7: 27.0 / 25.4 /
// 28.3 / 28.0 / 25.8 (the dips where the second workgroups join) and
// 23.4 / 20.5 / 19.3 / 16.7 / 15.8.
PKV_HD inline int64_t active_waves(int64_t n_units, int64_t n_waves, int64_t min_units,
                                   int64_t cost, const WaveWeights& k) {
  const int64_t age = n_waves > k.n_first ? k.wb : k.wa;
  const int64_t par = n_waves > 4 && k.po < 100 ? k.po : 100;
  int64_t W = weight_index(floor_div(n_units * age * par, min_units), k);
  if (W > n_waves) W = n_waves;
  const int64_t cap = k.n_first < n_waves ? k.n_first : n_waves;
  const int64_t ms = small_share(min_units, cost);
  if (W < cap && ms < min_units) {
    const int64_t Ws = weight_index(floor_div(n_units * age * par, ms), k);
    W = Ws < cap ? Ws : cap;          // Ws >= W, as ms < min_units
  }
  return W < 1 ? 1 : W;
}

PKV_HD inline int64_t wave_start(int64_t w, int64_t n_units, int64_t n_active,
                                 const WaveWeights& k) {
  return floor_div(n_units * cum_weight(w, k), cum_weight(n_active, k));
}

// The wavefront whose unit range holds unit u: the largest w < n_active
// with wave_start(w) <= u.
PKV_HD inline int64_t wave_of_unit(int64_t u, int64_t n_units, int64_t n_active,
                                   const WaveWeights& k) {
  const int64_t w = weight_index(floor_div((u + 1) * cum_weight(n_active, k) - 1, n_units), k);
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
// The same inside request b, which holds unit x (P[b] <= x < P[b + 1]).
PKV_HD inline TilePos tile_in_request(const int* P, int b, int hkv, int cost, int64_t x) {
  TilePos t;
  t.b = b;
  t.n = tiles_per_seq(P, b, hkv, cost);
  const int r = (int)(x - P[b]);          // < units of one request < 2^31
  const int per = t.n + cost;
  t.h = (int)floor_div(r, per);
  const int c = r - t.h * per;
  t.j = c == 0 ? 0 : (c - cost > 1 ? c - cost : 1);
  return t;
}
PKV_HD inline TilePos tile_at_unit(const int* P, int B, int hkv, int cost, int64_t x) {
  return tile_in_request(P, find_request(P, B, x), hkv, cost, x);
}

// Global tile index (tiles of all sequences concatenated) of tile (b, h, j)
// of a sequence with n tiles.
PKV_HD inline int64_t global_tile(const int* P, int b, int h, int j, int n, int hkv, int cost) {
  return ((int64_t)P[b] - (int64_t)hkv * cost * b) + (int64_t)h * n + j;
}

}  // namespace pkv
