// host_api.cpp -- the library's host-only entry points: the error message,
// the RoPE table build, the argument checks of a decode step and the host
// replay of the kernel's work partition.  Plain C++ without HIP, so the same
// source builds into the library and into a sanitizer-instrumented host
// build for the CPU tests.
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>
#include <vector>

#include "../../include/pkv.h"
#include "host_errors.h"
#include "pkv_limits.h"
#include "plan.h"

namespace {
thread_local std::string g_last_error;
}  // namespace

namespace pkv {

pkv_status fail(pkv_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

pkv_status set_error(pkv_status s, const char* msg) {
  g_last_error = msg;
  return s;
}

}  // namespace pkv

using pkv::fail;

extern "C" {

const char* pkv_last_error(void) { return g_last_error.c_str(); }

int32_t pkv_tile_tokens(void) { return pkv::kTileTokens; }

pkv_status pkv_rope_table_host(double theta, int32_t head_dim, int32_t max_position,
                               float* cos_out, float* sin_out) {
  if (!(theta > 0.0) || !std::isfinite(theta))
    return fail(PKV_ERR_INVALID, "rope theta must be finite and > 0");
  if (head_dim < 2 || head_dim % 2) return fail(PKV_ERR_INVALID, "head_dim must be even");
  if (max_position < 1) return fail(PKV_ERR_INVALID, "max_position must be >= 1");
  if (!cos_out || !sin_out) return fail(PKV_ERR_INVALID, "null output");
  const int half = head_dim / 2;
  std::vector<double> inv(half);
  for (int i = 0; i < half; ++i) inv[i] = std::pow(theta, -(2.0 * i) / head_dim);
  for (int64_t p = 0; p < max_position; ++p) {
    for (int i = 0; i < half; ++i) {
      const double ang = (double)p * inv[i];
      cos_out[p * half + i] = (float)std::cos(ang);
      sin_out[p * half + i] = (float)std::sin(ang);
    }
  }
  return PKV_OK;
}

pkv_status pkv_check_decode_args(int64_t num_blocks, int32_t block_size, int32_t n_kv_heads,
                                 int32_t head_dim, pkv_dtype kv_dtype, pkv_dtype io_dtype,
                                 const void* q, const void* k_new, const void* v_new,
                                 const int32_t* positions, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 int32_t batch, int32_t n_q_heads, const void* out) {
  if (batch < 0) return fail(PKV_ERR_INVALID, "batch must be >= 0");
  if (batch > pkv::kMaxBatch)
    return fail(PKV_ERR_UNSUPPORTED, "batch %d above %d", batch, pkv::kMaxBatch);
  if (io_dtype != PKV_F32 && io_dtype != PKV_BF16 && io_dtype != PKV_FP8_E4M3)
    return fail(PKV_ERR_INVALID, "unknown io_dtype %d", (int)io_dtype);
  const bool pair_ok = (io_dtype == PKV_F32 && kv_dtype == PKV_F32) ||
                       (io_dtype == PKV_BF16 && kv_dtype == PKV_BF16) ||
                       (io_dtype == PKV_BF16 && kv_dtype == PKV_FP8_E4M3);
  if (!pair_ok)
    return fail(PKV_ERR_UNSUPPORTED, "io/kv dtype pair (%d, %d) not supported", (int)io_dtype,
                (int)kv_dtype);
  if (n_kv_heads < 1) return fail(PKV_ERR_INVALID, "n_kv_heads must be >= 1");
  if (n_q_heads < 1 || n_q_heads % n_kv_heads)
    return fail(PKV_ERR_INVALID, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)",
                n_q_heads, n_kv_heads);
  const int g = n_q_heads / n_kv_heads;
  if (g > pkv::kGroupMax)
    return fail(PKV_ERR_UNSUPPORTED, "group size %d above %d", g, pkv::kGroupMax);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d not supported", head_dim);
  if (block_size != 16 && block_size != 32 && block_size != 64)
    return fail(PKV_ERR_UNSUPPORTED, "block_size %d not supported", block_size);
  if (num_blocks < 1) return fail(PKV_ERR_INVALID, "num_blocks must be >= 1");
  if (max_blocks_per_seq < 1) return fail(PKV_ERR_INVALID, "max_blocks_per_seq must be >= 1");
  const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
  if (cap > ((int64_t)1 << 24))
    return fail(PKV_ERR_UNSUPPORTED, "max_blocks_per_seq * block_size above 2^24 tokens");
  const int64_t tile = pkv::kTileTokens;
  if ((int64_t)batch * n_kv_heads * ((cap + tile - 1) / tile + pkv::kMaxPieceCost) >
      ((int64_t)1 << 31) - 1)
    return fail(PKV_ERR_UNSUPPORTED, "batch * n_kv_heads * (tiles + piece cost) above 2^31");
  if (batch == 0) return PKV_OK;
  if (!q || !k_new || !v_new || !positions || !block_tables || !context_lens || !out)
    return fail(PKV_ERR_INVALID, "null device pointer");
  if (((uintptr_t)q | (uintptr_t)out | (uintptr_t)k_new | (uintptr_t)v_new) % 16)
    return fail(PKV_ERR_INVALID, "q, k_new, v_new and out must be 16-byte aligned");
  if (((uintptr_t)positions | (uintptr_t)block_tables | (uintptr_t)context_lens) % 4)
    return fail(PKV_ERR_INVALID, "int32 arrays must be 4-byte aligned");
  return PKV_OK;
}

pkv_status pkv_plan_host(const int32_t* context_lens, int32_t batch, int32_t n_kv_heads,
                         int32_t max_tokens, int32_t n_waves, int32_t min_units,
                         int32_t piece_cost, int32_t n_first, int32_t weight_first,
                         int32_t weight_rest, int32_t weight_odd, int32_t weight_min_share,
                         int32_t window, int32_t max_pieces, int32_t* pieces,
                         int32_t* n_pieces, int32_t* splits) {
  if (!context_lens || !n_pieces || !splits || (max_pieces > 0 && !pieces))
    return fail(PKV_ERR_INVALID, "null argument");
  if (batch < 1 || n_kv_heads < 1 || n_waves < 1 || min_units < 1 || max_tokens < 1)
    return fail(PKV_ERR_INVALID, "sizes must be positive");
  if (piece_cost < 0 || piece_cost > pkv::kMaxPieceCost)
    return fail(PKV_ERR_INVALID, "piece_cost must be in [0, %d]", pkv::kMaxPieceCost);
  if (n_first < 0 || weight_rest < 1 || weight_first < weight_rest || weight_first > 1000)
    return fail(PKV_ERR_INVALID, "need n_first >= 0 and 1 <= weight_rest <= weight_first <= 1000");
  if (weight_odd < 1 || weight_odd > 100) return fail(PKV_ERR_INVALID, "weight_odd must be in [1, 100]");
  if (window < 0) return fail(PKV_ERR_INVALID, "window must be >= 0");
  if (weight_min_share < 0) return fail(PKV_ERR_INVALID, "weight_min_share must be >= 0");
  const int hkv = n_kv_heads, cost = piece_cost;
  std::vector<int> P(batch + 1, 0);
  for (int b = 0; b < batch; ++b)
    P[b + 1] = P[b] + hkv * (pkv::tiles_of(context_lens[b], max_tokens) -
                              pkv::window_first_tile(context_lens[b], max_tokens, window) + cost);
  const int64_t C = P[batch];
  const pkv::WaveWeights ww = pkv::weights_for(
      C, n_waves, weight_min_share, pkv::WaveWeights{weight_first, weight_rest, n_first, weight_odd});
  const int64_t W = pkv::active_waves(C, n_waves, std::max(min_units, cost + 1), cost, ww);
  const int64_t n_tiles = (int64_t)P[batch] - (int64_t)hkv * cost * batch;
  for (int64_t w = 0; w < n_waves; ++w) {
    int32_t* row = splits + 4 * w;
    row[0] = row[1] = row[2] = row[3] = 0;
  }
  int64_t count = 0;
  for (int64_t w = 0; w < W; ++w) {
    pkv::TilePos t = pkv::tile_at_unit(P.data(), batch, hkv, cost, pkv::wave_start(w, C, W, ww));
    const int64_t g0 = pkv::global_tile(P.data(), t.b, t.h, t.j, t.n, hkv, cost);
    int64_t g1 = n_tiles;
    const int64_t x1 = pkv::wave_start(w + 1, C, W, ww);
    if (x1 < C) {
      const pkv::TilePos t1 = pkv::tile_at_unit(P.data(), batch, hkv, cost, x1);
      g1 = pkv::global_tile(P.data(), t1.b, t1.h, t1.j, t1.n, hkv, cost);
    }
    int64_t left = g1 - g0;
    if (left > 0 && t.j == t.n) {
      t.j = 0;
      if (++t.h == hkv) {
        t.h = 0;
        ++t.b;
        t.n = pkv::tiles_per_seq(P.data(), t.b, hkv, cost);
      }
    }
    bool first = true;
    while (left > 0) {
      const int j0 = t.j;
      const int64_t take = std::min<int64_t>(left, t.n - j0);
      const int pe = j0 + (int)take;
      const bool split = j0 > 0 || pe < t.n;
      if (count < max_pieces) {
        int32_t* r = pieces + 6 * count;
        r[0] = (int32_t)w;
        r[1] = t.b;
        r[2] = t.h;
        r[3] = j0;
        r[4] = pe;
        r[5] = (split ? pkv::PIECE_SPLIT : 0) | (first ? pkv::PIECE_FIRST : 0) |
               (pe == t.n ? pkv::PIECE_LAST : 0);
      }
      ++count;
      if (split && j0 == 0) {     // the sequence starts here: wave w is its first
        int32_t* row = splits + 4 * w;
        const int64_t last = pkv::first_unit(P.data(), t.b, t.h, t.n - 1, t.n, cost);
        row[0] = 1;
        row[1] = t.b * hkv + t.h;
        row[2] = (int32_t)(pkv::wave_of_unit(last, C, W, ww) - w + 1);
        row[3] = first ? 0 : 1;
      }
      first = false;
      left -= take;
      t.j = pe;
      if (t.j == t.n) {
        t.j = 0;
        if (++t.h == hkv) {
          t.h = 0;
          if (++t.b < batch) t.n = pkv::tiles_per_seq(P.data(), t.b, hkv, cost);
        }
      }
    }
  }
  *n_pieces = (int32_t)std::min<int64_t>(count, INT32_MAX);
  return PKV_OK;
}

}  // extern "C"
