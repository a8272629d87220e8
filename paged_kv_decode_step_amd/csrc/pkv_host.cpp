// pkv_host.cpp -- the C ABI of include/pkv.h: pool ownership, RoPE table, FP8
// scales, argument checks, the host replay of the work partition, launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/pkv.h"
#include "host_errors.h"
#include "kernels.h"
#include "plan.h"

namespace {

using pkv::fail;

pkv_status hip_fail(hipError_t e, const char* what) {
  return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int elem_bytes(pkv_dtype t) {
  switch (t) {
    case PKV_F32: return 4;
    case PKV_BF16: return 2;
    case PKV_FP8_E4M3: return 1;
    case PKV_DTYPE_MAX_ENUM: break;
  }
  return 0;
}

int kv_kind(pkv_dtype t) {
  return t == PKV_F32 ? pkv::KV_F32 : (t == PKV_BF16 ? pkv::KV_BF16 : pkv::KV_FP8);
}

int env_int(const char* name, int dflt) {
  const char* s = std::getenv(name);
  if (!s || !*s) return dflt;
  return std::atoi(s);
}

// Work units charged for starting a sequence.  Its query loads queue behind
// every tile load the wavefront has in flight, so a start stalls the
// wavefront for about its ring of tiles plus one more round trip (the query
// and the append); -1 asks for that estimate, ring + 2.
int resolve_piece_cost(int requested, int ring_tiles) {
  const int c = requested < 0 ? ring_tiles + 2 : requested;
  return std::max(0, std::min(c, pkv::kMaxPieceCost));
}

// Share weight of the wavefronts of later workgroups on a compute unit, in
// percent of the first workgroup's.  Two wavefronts on one SIMD do not
// stream alike: the older wins most issue slots and, while both run, moves
// 1.6-1.9x the younger's bytes; -1 asks for 65%.
int resolve_young_pct(int requested) {
  const int v = requested < 0 ? 65 : requested;
  return std::max(1, std::min(v, 100));
}

// Share weight of the wavefronts of odd workgroups, in percent of the even
// ones'.  Workgroups are dealt to the eight XCDs in turn, and the odd XCDs
// were measured to stream about a tenth slower; -1 asks for 90%.
int resolve_odd_pct(int requested) {
  const int v = requested < 0 ? 90 : requested;
  return std::max(1, std::min(v, 100));
}

}  // namespace

struct pkv_pool {
  int device = 0;
  int64_t num_blocks = 0;
  int32_t block_size = 0, n_kv_heads = 0, head_dim = 0;
  pkv_dtype kv_dtype = PKV_BF16;
  void* k = nullptr;
  void* v = nullptr;
  int64_t kv_bytes = 0;
  float* rope_cos = nullptr;
  float* rope_sin = nullptr;
  size_t rope_cap = 0;             // floats each table buffer holds
  int32_t rope_max_pos = 0;
  double rope_theta = 0.0;
  float* fp8_scales = nullptr;     // [4][Hkv]
  bool has_scales = false;
  float* partials = nullptr;
  int4* headers = nullptr;         // per-wave split records (attention -> merge)
  uint64_t* timeline = nullptr;    // [ws_waves][8] phase stamps (timeline builds only)
  void* dummy = nullptr;           // zeroed buffer read by loads past a wave's range
  uint32_t* err = nullptr;
  int64_t ws_bytes = 0;
  int cus = 0;
  int occ_blocks = 0;              // resident workgroups per CU (occupancy)
  int waves_per_cu = 0;
  int n_waves = 0;
  int ws_waves = 0;                // wavefronts the workspace has room for
  int min_units = 16;
  int piece_cost = 0;       // resolved (never the automatic -1)
  int ring_tiles = 0;
  int young_pct = 100;      // share weight of later workgroups, % of the first's
  int odd_pct = 100;        // share weight of odd workgroups, % of the even ones'
  int window = 0;           // attention window in tokens (0 = the whole context)
  // Buffers replaced by a larger one (RoPE table, workspace).  A graph
  // captured before the replacement still points at them, so they are freed
  // only with the pool.
  std::vector<void*> retired;
  // measurement: per call, start and stop events of each of the two kernels
  bool timing = false;
  std::vector<hipEvent_t> events;
  int timed_calls = 0;
};

static constexpr int kMaxTimedCalls = 65536;

// Makes `device` current for its lifetime and restores the caller's device.
struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int device) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    (void)hipSetDevice(device);
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
  DeviceGuard(const DeviceGuard&) = delete;
  DeviceGuard& operator=(const DeviceGuard&) = delete;
};

static void free_pool(pkv_pool* p) {
  if (!p) return;
  for (hipEvent_t e : p->events) (void)hipEventDestroy(e);
  for (void* r : p->retired) (void)hipFree(r);
  (void)hipFree(p->k);
  (void)hipFree(p->v);
  (void)hipFree(p->rope_cos);
  (void)hipFree(p->rope_sin);
  (void)hipFree(p->fp8_scales);
  (void)hipFree(p->partials);
  (void)hipFree(p->headers);
  (void)hipFree(p->timeline);
  (void)hipFree(p->dummy);
  (void)hipFree(p->err);
  delete p;
}

static pkv_status size_workspace(pkv_pool* p, int waves_per_cu) {
  int wpc = waves_per_cu > 0 ? waves_per_cu : p->occ_blocks * 4;
  wpc = std::max(4, std::min(wpc, 32));
  wpc = (wpc + 3) / 4 * 4;
  const int n_waves = p->cus * wpc;
  if (p->partials && n_waves <= p->ws_waves) {     // the workspace holds them
    p->n_waves = n_waves;
    p->waves_per_cu = wpc;
    return PKV_OK;
  }
  // a larger workspace; the old one is kept until the pool is destroyed
  const size_t pb = pkv::partials_bytes(n_waves, p->head_dim);
  float* partials = nullptr;
  int4* headers = nullptr;
  hipError_t e = hipMalloc(&partials, pb);
  if (e != hipSuccess) return fail(PKV_ERR_OOM, "workspace (%zu bytes): %s", pb, hipGetErrorString(e));
  e = hipMalloc(&headers, sizeof(int4) * n_waves);
  if (e != hipSuccess) {
    (void)hipFree(partials);
    return fail(PKV_ERR_OOM, "headers: %s", hipGetErrorString(e));
  }
#ifdef PKV_TIMELINE
  uint64_t* timeline = nullptr;
  e = hipMalloc(&timeline, sizeof(uint64_t) * 8 * n_waves);
  if (e == hipSuccess) e = hipMemset(timeline, 0, sizeof(uint64_t) * 8 * n_waves);
  if (e != hipSuccess) {
    (void)hipFree(partials);
    (void)hipFree(headers);
    (void)hipFree(timeline);
    return fail(PKV_ERR_OOM, "timeline: %s", hipGetErrorString(e));
  }
  if (p->timeline) p->retired.push_back(p->timeline);
  p->timeline = timeline;
#endif
  if (p->partials) p->retired.push_back(p->partials);
  if (p->headers) p->retired.push_back(p->headers);
  p->partials = partials;
  p->headers = headers;
  p->ws_waves = n_waves;
  p->n_waves = n_waves;
  p->waves_per_cu = wpc;
  p->ws_bytes = (int64_t)pb + (int64_t)sizeof(int4) * n_waves + (int64_t)pkv::kDummyBytes;
  return PKV_OK;
}

extern "C" {

pkv_status kv_pool_create(int64_t num_blocks, int32_t block_size, int32_t n_kv_heads,
                          int32_t head_dim, pkv_dtype kv_dtype, pkv_pool** out_pool) {
  if (!out_pool) return fail(PKV_ERR_INVALID, "out_pool is null");
  *out_pool = nullptr;
  if (kv_dtype != PKV_F32 && kv_dtype != PKV_BF16 && kv_dtype != PKV_FP8_E4M3)
    return fail(PKV_ERR_INVALID, "unknown kv_dtype %d", (int)kv_dtype);
  if (num_blocks < 1 || num_blocks > INT32_MAX)
    return fail(PKV_ERR_INVALID, "num_blocks must be in [1, 2^31)");
  if (n_kv_heads < 1 || n_kv_heads > 256)
    return fail(PKV_ERR_INVALID, "n_kv_heads must be in [1, 256]");
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d not supported (64, 128)", head_dim);
  if (block_size != 16 && block_size != 32 && block_size != 64)
    return fail(PKV_ERR_UNSUPPORTED, "block_size %d not supported (16, 32, 64)", block_size);
  const int64_t per_block = (int64_t)n_kv_heads * block_size * head_dim * elem_bytes(kv_dtype);
  if (num_blocks > ((int64_t)1 << 40) / per_block)
    return fail(PKV_ERR_INVALID, "pool larger than 2^40 bytes");

  pkv_pool* p = new pkv_pool();
  hipError_t e = hipGetDevice(&p->device);
  if (e != hipSuccess) { delete p; return hip_fail(e, "hipGetDevice"); }
  e = hipDeviceGetAttribute(&p->cus, hipDeviceAttributeMultiprocessorCount, p->device);
  if (e != hipSuccess) { delete p; return hip_fail(e, "hipDeviceGetAttribute"); }
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->n_kv_heads = n_kv_heads;
  p->head_dim = head_dim;
  p->kv_dtype = kv_dtype;
  p->kv_bytes = num_blocks * per_block;
  e = hipMalloc(&p->k, p->kv_bytes);
  if (e != hipSuccess) { free_pool(p); return fail(PKV_ERR_OOM, "K pool (%lld bytes): %s", (long long)per_block * num_blocks, hipGetErrorString(e)); }
  e = hipMalloc(&p->v, p->kv_bytes);
  if (e != hipSuccess) { free_pool(p); return fail(PKV_ERR_OOM, "V pool: %s", hipGetErrorString(e)); }
  e = hipMalloc(&p->err, 4 * sizeof(uint32_t));
  if (e != hipSuccess) { free_pool(p); return fail(PKV_ERR_OOM, "flags: %s", hipGetErrorString(e)); }
  e = hipMemset(p->err, 0, 4 * sizeof(uint32_t));
  if (e != hipSuccess) { free_pool(p); return hip_fail(e, "hipMemset"); }
  e = hipMalloc(&p->fp8_scales, 4 * sizeof(float) * n_kv_heads);
  if (e != hipSuccess) { free_pool(p); return fail(PKV_ERR_OOM, "scales: %s", hipGetErrorString(e)); }
  e = hipMalloc(&p->dummy, pkv::kDummyBytes);
  if (e != hipSuccess) { free_pool(p); return fail(PKV_ERR_OOM, "dummy buffer: %s", hipGetErrorString(e)); }
  e = hipMemset(p->dummy, 0, pkv::kDummyBytes);
  if (e != hipSuccess) { free_pool(p); return hip_fail(e, "hipMemset"); }
  e = pkv::decode_occupancy(kv_kind(kv_dtype), head_dim, block_size, &p->occ_blocks);
  if (e != hipSuccess) { free_pool(p); return hip_fail(e, "occupancy query"); }
  p->occ_blocks = std::max(1, p->occ_blocks);
  p->min_units = std::max(1, env_int("PKV_MIN_UNITS", 16));
  p->ring_tiles = pkv::decode_ring_tiles(kv_kind(kv_dtype), head_dim);
  p->piece_cost = resolve_piece_cost(env_int("PKV_PIECE_COST", -1), p->ring_tiles);
  p->young_pct = resolve_young_pct(env_int("PKV_YOUNG_WEIGHT", -1));
  p->odd_pct = resolve_odd_pct(env_int("PKV_ODD_WEIGHT", -1));
  pkv_status s = size_workspace(p, env_int("PKV_WAVES_PER_CU", 0));
  if (s != PKV_OK) { free_pool(p); return s; }
  *out_pool = p;
  return PKV_OK;
}

pkv_status kv_pool_destroy(pkv_pool* pool) {
  if (!pool) return PKV_OK;
  DeviceGuard g(pool->device);
  (void)hipDeviceSynchronize();
  free_pool(pool);
  return PKV_OK;
}

pkv_status kv_pool_set_rope(pkv_pool* pool, double theta, int32_t max_position) {
  if (!pool) return fail(PKV_ERR_INVALID, "pool is null");
  if (max_position < 1 || max_position > (1 << 24))
    return fail(PKV_ERR_INVALID, "max_position must be in [1, 2^24]");
  const size_t n = (size_t)max_position * (pool->head_dim / 2);
  std::vector<float> c(n), s(n);
  pkv_status st = pkv_rope_table_host(theta, pool->head_dim, max_position, c.data(), s.data());
  if (st != PKV_OK) return st;
  DeviceGuard g(pool->device);
  hipError_t e;
  if (n > pool->rope_cap) {
    // a larger table: new buffers, the old ones kept until the pool is
    // destroyed (a graph captured earlier still reads them)
    float *cs = nullptr, *sn = nullptr;
    e = hipMalloc(&cs, n * sizeof(float));
    if (e != hipSuccess) return fail(PKV_ERR_OOM, "rope table: %s", hipGetErrorString(e));
    e = hipMalloc(&sn, n * sizeof(float));
    if (e != hipSuccess) {
      (void)hipFree(cs);
      return fail(PKV_ERR_OOM, "rope table: %s", hipGetErrorString(e));
    }
    if (pool->rope_cos) pool->retired.push_back(pool->rope_cos);
    if (pool->rope_sin) pool->retired.push_back(pool->rope_sin);
    pool->rope_cos = cs;
    pool->rope_sin = sn;
    pool->rope_cap = n;
  } else {
    // rewritten in place: wait for any step that may still read the table
    e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
  }
  pool->rope_max_pos = 0;
  e = hipMemcpy(pool->rope_cos, c.data(), n * sizeof(float), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy rope");
  e = hipMemcpy(pool->rope_sin, s.data(), n * sizeof(float), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy rope");
  pool->rope_max_pos = max_position;
  pool->rope_theta = theta;
  return PKV_OK;
}

pkv_status kv_pool_set_fp8_scales(pkv_pool* pool, const float* k_scale, const float* v_scale) {
  if (!pool) return fail(PKV_ERR_INVALID, "pool is null");
  if (pool->kv_dtype != PKV_FP8_E4M3) return fail(PKV_ERR_INVALID, "pool is not fp8");
  if (!k_scale || !v_scale) return fail(PKV_ERR_INVALID, "null scale array");
  const int h = pool->n_kv_heads;
  std::vector<float> all(4 * h);
  for (int i = 0; i < h; ++i) {
    if (!(k_scale[i] > 0.f) || !std::isfinite(k_scale[i]) || !(v_scale[i] > 0.f) ||
        !std::isfinite(v_scale[i]))
      return fail(PKV_ERR_INVALID, "scale of head %d must be finite and > 0", i);
    all[i] = k_scale[i];
    all[h + i] = v_scale[i];
    all[2 * h + i] = 1.0f / k_scale[i];
    all[3 * h + i] = 1.0f / v_scale[i];
  }
  hipError_t e = hipMemcpy(pool->fp8_scales, all.data(), all.size() * sizeof(float),
                           hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy scales");
  pool->has_scales = true;
  return PKV_OK;
}

pkv_status kv_pool_get_info(const pkv_pool* pool, pkv_pool_info* info) {
  if (!pool || !info) return fail(PKV_ERR_INVALID, "null argument");
  std::memset(info, 0, sizeof *info);
  info->num_blocks = pool->num_blocks;
  info->block_size = pool->block_size;
  info->n_kv_heads = pool->n_kv_heads;
  info->head_dim = pool->head_dim;
  info->kv_dtype = pool->kv_dtype;
  info->kv_elem_bytes = elem_bytes(pool->kv_dtype);
  info->tile_bytes = 16 * pool->head_dim * info->kv_elem_bytes;
  info->k_base = pool->k;
  info->v_base = pool->v;
  info->k_bytes = pool->kv_bytes;
  info->v_bytes = pool->kv_bytes;
  info->rope_cos = pool->rope_cos;
  info->rope_sin = pool->rope_sin;
  info->rope_max_position = pool->rope_max_pos;
  info->rope_theta = pool->rope_theta;
  info->has_fp8_scales = pool->has_scales ? 1 : 0;
  info->device = pool->device;
  info->n_waves = pool->n_waves;
  info->workspace_bytes = pool->ws_bytes;
  info->ring_tiles = pool->ring_tiles;
  info->min_units = pool->min_units;
  info->piece_cost = pool->piece_cost;
  info->young_weight_pct = pool->young_pct;
  info->odd_weight_pct = pool->odd_pct;
  info->window = pool->window;
  info->n_first = std::min(pool->n_waves, 4 * pool->cus);
  return PKV_OK;
}

pkv_status kv_pool_layout(const pkv_pool* pool, void** k_base, void** v_base,
                          int64_t byte_strides[3], int32_t* tile_bytes) {
  if (!pool || !k_base || !v_base || !byte_strides || !tile_bytes)
    return fail(PKV_ERR_INVALID, "null argument");
  const int64_t t = (int64_t)pkv::kTileTokens * pool->head_dim * elem_bytes(pool->kv_dtype);
  const int64_t tpb = pool->block_size / pkv::kTileTokens;
  *k_base = pool->k;
  *v_base = pool->v;
  byte_strides[0] = (int64_t)pool->n_kv_heads * tpb * t;   // block
  byte_strides[1] = tpb * t;                               // KV head
  byte_strides[2] = t;                                     // 16-token tile
  *tile_bytes = (int32_t)t;
  return PKV_OK;
}

pkv_status kv_pool_rope_table(const pkv_pool* pool, const float** cos_dev, const float** sin_dev,
                              int32_t* max_position) {
  if (!pool || !cos_dev || !sin_dev || !max_position)
    return fail(PKV_ERR_INVALID, "null argument");
  *cos_dev = pool->rope_cos;
  *sin_dev = pool->rope_sin;
  *max_position = pool->rope_max_pos;
  if (pool->rope_max_pos < 1) return fail(PKV_ERR_STATE, "kv_pool_set_rope was not called");
  return PKV_OK;
}

pkv_status kv_pool_set_tuning(pkv_pool* pool, int32_t waves_per_cu, int32_t min_units,
                              int32_t piece_cost, int32_t young_weight_pct,
                              int32_t odd_weight_pct) {
  if (!pool) return fail(PKV_ERR_INVALID, "pool is null");
  if (min_units < 1) return fail(PKV_ERR_INVALID, "min_units must be >= 1");
  if (piece_cost < -1 || piece_cost > pkv::kMaxPieceCost)
    return fail(PKV_ERR_INVALID, "piece_cost must be -1 (automatic) or in [0, %d]",
                pkv::kMaxPieceCost);
  if (young_weight_pct < -1 || young_weight_pct == 0 || young_weight_pct > 100)
    return fail(PKV_ERR_INVALID, "young_weight_pct must be -1 (automatic) or in [1, 100]");
  if (odd_weight_pct < -1 || odd_weight_pct == 0 || odd_weight_pct > 100)
    return fail(PKV_ERR_INVALID, "odd_weight_pct must be -1 (automatic) or in [1, 100]");
  if (waves_per_cu < 0 || waves_per_cu > 32)
    return fail(PKV_ERR_INVALID, "waves_per_cu must be in [0, 32]");
  pkv_status s;
  {
    DeviceGuard g(pool->device);
    (void)hipDeviceSynchronize();
    s = size_workspace(pool, waves_per_cu);
  }
  if (s != PKV_OK) return s;
  pool->min_units = min_units;
  pool->piece_cost = resolve_piece_cost(piece_cost, pool->ring_tiles);
  pool->young_pct = resolve_young_pct(young_weight_pct);
  pool->odd_pct = resolve_odd_pct(odd_weight_pct);
  return PKV_OK;
}

static pkv_status debug_validate(const pkv_pool* pool, const int32_t* positions,
                                 const int32_t* block_tables, int32_t max_blocks,
                                 const int32_t* context_lens, int32_t batch, int32_t n_new,
                                 hipStream_t stream) {
  std::vector<int32_t> lens(batch), pos(batch), tab((size_t)batch * max_blocks);
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  e = hipMemcpy(lens.data(), context_lens, batch * 4, hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpy(pos.data(), positions, batch * 4, hipMemcpyDeviceToHost);
  if (e == hipSuccess)
    e = hipMemcpy(tab.data(), block_tables, tab.size() * 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy (debug validation)");
  const int64_t cap = (int64_t)max_blocks * pool->block_size;
  std::vector<int32_t> last_owner(pool->num_blocks, -1);
  for (int b = 0; b < batch; ++b) {
    if (lens[b] < n_new || lens[b] > cap)
      return fail(PKV_ERR_DEVICE_DATA, "context_lens[%d] = %d outside [%d, %lld]", b, lens[b],
                  n_new, (long long)cap);
    if (pos[b] < 0 || pos[b] + n_new - 1 >= pool->rope_max_pos)
      return fail(PKV_ERR_DEVICE_DATA, "positions[%d] = %d: new tokens outside [0, %d)", b,
                  pos[b], pool->rope_max_pos);
    const int nb = (lens[b] + pool->block_size - 1) / pool->block_size;
    for (int j = 0; j < nb; ++j) {
      const int32_t id = tab[(size_t)b * max_blocks + j];
      if (id < 0 || id >= pool->num_blocks)
        return fail(PKV_ERR_DEVICE_DATA, "block_tables[%d][%d] = %d outside [0, %lld)", b, j, id,
                    (long long)pool->num_blocks);
    }
    // every block that receives one of the request's new tokens
    const int j0 = (lens[b] - n_new) / pool->block_size;
    for (int j = j0; j < nb; ++j) {
      const int32_t lb = tab[(size_t)b * max_blocks + j];
      if (last_owner[lb] >= 0 && last_owner[lb] != b)
        return fail(PKV_ERR_DEVICE_DATA,
                    "block %d receives new tokens of requests %d and %d", lb, last_owner[lb], b);
      last_owner[lb] = b;
    }
  }
  for (int b = 0; b < batch; ++b) {   // the appended block must not be read by others
    const int nb = (lens[b] + pool->block_size - 1) / pool->block_size;
    for (int j = 0; j < nb; ++j) {
      const int32_t id = tab[(size_t)b * max_blocks + j];
      if (last_owner[id] >= 0 && last_owner[id] != b)
        return fail(PKV_ERR_DEVICE_DATA,
                    "block %d is appended to by request %d and read by request %d", id,
                    last_owner[id], b);
    }
  }
  return PKV_OK;
}

// Work for a pool goes on a stream of the pool's device (NULL: the current
// device's default stream); a kernel on another device would read this
// device's memory from there.
static pkv_status check_stream_device(const pkv_pool* pool, hipStream_t st) {
  int dev = -1;
  const hipError_t e = hipStreamGetDevice(st, &dev);
  if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
  if (dev != pool->device)
    return fail(PKV_ERR_INVALID, "stream is on device %d, the pool on device %d", dev,
                pool->device);
  return PKV_OK;
}

// A split-K workspace: the pool's own, or the fixed per-device one.
struct Workspace {
  float* partials;
  int4* headers;
};

static pkv_status launch_step(pkv_pool* pool, const void* q, const void* k_new,
                              const void* v_new, pkv_dtype io_dtype, int32_t n_new,
                              const int32_t* positions, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* context_lens,
                              int32_t batch, int32_t n_q_heads, void* out, void* stream,
                              const Workspace* fixed = nullptr);

pkv_status decode_step(pkv_pool* pool, const void* q, const void* k_new, const void* v_new,
                       pkv_dtype io_dtype, const int32_t* positions, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t batch,
                       int32_t n_q_heads, void* out, void* stream) {
  return launch_step(pool, q, k_new, v_new, io_dtype, 1, positions, block_tables,
                     max_blocks_per_seq, context_lens, batch, n_q_heads, out, stream);
}

pkv_status decode_step_multi(pkv_pool* pool, const void* q, const void* k_new, const void* v_new,
                             pkv_dtype io_dtype, int32_t n_new, const int32_t* positions,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t batch, int32_t n_q_heads,
                             void* out, void* stream) {
  if (!pool) return fail(PKV_ERR_INVALID, "pool is null");
  if (n_new < 1) return fail(PKV_ERR_INVALID, "n_new must be >= 1");
  if (n_new > 1) {
    if (pool->kv_dtype == PKV_F32)
      return fail(PKV_ERR_UNSUPPORTED, "several new tokens need a bf16 or fp8 cache");
    if (pool->window > 0)
      return fail(PKV_ERR_UNSUPPORTED, "several new tokens with an attention window");
    if (n_q_heads >= pool->n_kv_heads && n_q_heads % pool->n_kv_heads == 0 &&
        (int64_t)(n_q_heads / pool->n_kv_heads) * n_new > pkv::kGroupMax)
      return fail(PKV_ERR_UNSUPPORTED, "group (%d) x new tokens (%d) above %d",
                  n_q_heads / pool->n_kv_heads, n_new, pkv::kGroupMax);
    if (pool->rope_max_pos >= 1 && pool->rope_max_pos < n_new)
      return fail(PKV_ERR_INVALID, "RoPE table of %d positions for %d new tokens",
                  pool->rope_max_pos, n_new);
  }
  return launch_step(pool, q, k_new, v_new, io_dtype, n_new, positions, block_tables,
                     max_blocks_per_seq, context_lens, batch, n_q_heads, out, stream);
}

pkv_status decode_step_noalloc(pkv_pool* pool, const void* q, const void* k_new,
                               const void* v_new, pkv_dtype io_dtype, const int32_t* positions,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t batch, int32_t n_q_heads,
                               void* out, void* stream) {
  if (!pool) return fail(PKV_ERR_INVALID, "pool is null");
  if (pool->n_waves > pkv::kScratchMaxWaves)
    return fail(PKV_ERR_UNSUPPORTED,
                "decode_step_noalloc: the pool runs %d wavefronts, the fixed workspace holds %d",
                pool->n_waves, pkv::kScratchMaxWaves);
  if (pool->head_dim > pkv::kScratchMaxHeadDim)
    return fail(PKV_ERR_UNSUPPORTED, "decode_step_noalloc: head_dim above %d",
                pkv::kScratchMaxHeadDim);
  void* base = nullptr;
  const hipError_t e = pkv::scratch_address(pool->device, &base);
  if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress (fixed workspace)");
  Workspace ws;
  ws.partials = static_cast<float*>(base);
  ws.headers = reinterpret_cast<int4*>(static_cast<char*>(base) +
                                       pkv::headers_offset(pool->n_waves, pool->head_dim));
  return launch_step(pool, q, k_new, v_new, io_dtype, 1, positions, block_tables,
                     max_blocks_per_seq, context_lens, batch, n_q_heads, out, stream, &ws);
}

static pkv_status launch_step(pkv_pool* pool, const void* q, const void* k_new,
                              const void* v_new, pkv_dtype io_dtype, int32_t n_new,
                              const int32_t* positions, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* context_lens,
                              int32_t batch, int32_t n_q_heads, void* out, void* stream,
                              const Workspace* fixed) {
  if (!pool) return fail(PKV_ERR_INVALID, "pool is null");
  pkv_status s = pkv_check_decode_args(pool->num_blocks, pool->block_size, pool->n_kv_heads,
                                       pool->head_dim, pool->kv_dtype, io_dtype, q, k_new, v_new,
                                       positions, block_tables, max_blocks_per_seq, context_lens,
                                       batch, n_q_heads, out);
  if (s != PKV_OK) return s;
  if (batch == 0) return PKV_OK;
  if (pool->rope_max_pos < 1) return fail(PKV_ERR_STATE, "kv_pool_set_rope was not called");
  if (pool->kv_dtype == PKV_FP8_E4M3 && !pool->has_scales)
    return fail(PKV_ERR_STATE, "kv_pool_set_fp8_scales was not called");
  hipStream_t st = static_cast<hipStream_t>(stream);
  s = check_stream_device(pool, st);
  if (s != PKV_OK) return s;
  if (!fixed && env_int("PKV_DEBUG", 0) == 1) {
    s = debug_validate(pool, positions, block_tables, max_blocks_per_seq, context_lens, batch,
                       n_new, st);
    if (s != PKV_OK) return s;
  }
  pkv::DecodeParams p;
  p.q = q;
  p.k_new = k_new;
  p.v_new = v_new;
  p.out = out;
  p.positions = positions;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.k_pool = pool->k;
  p.v_pool = pool->v;
  p.rope_cos = pool->rope_cos;
  p.rope_sin = pool->rope_sin;
  p.fp8_scales = pool->fp8_scales;
  p.partials = fixed ? fixed->partials : pool->partials;
  p.headers = fixed ? fixed->headers : pool->headers;
  p.dummy = pool->dummy;
  p.timeline = fixed ? nullptr : pool->timeline;
  p.err = pool->err;
  p.num_blocks = (int32_t)pool->num_blocks;
  p.batch = batch;
  p.n_kv_heads = pool->n_kv_heads;
  p.group = n_q_heads / pool->n_kv_heads;
  p.max_blocks = max_blocks_per_seq;
  p.max_pos = pool->rope_max_pos;
  p.n_waves = pool->n_waves;
  p.piece_cost = pool->piece_cost;
  p.min_units = std::max(pool->min_units, pool->piece_cost + 1);
  // the first workgroup dispatched to each compute unit: 4 wavefronts per CU
  p.n_first = std::min(pool->n_waves, 4 * pool->cus);
  p.weight_first = 100;
  p.weight_rest = pool->young_pct;
  p.weight_odd = pool->odd_pct;
  p.weight_min_share = pkv::kWeightMinShare;
  p.sm_scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)pool->head_dim));
  p.window = pool->window;
  p.n_qtok = n_new;
  hipEvent_t* ev = nullptr;
  if (!fixed && pool->timing && pool->timed_calls < kMaxTimedCalls) {
    const size_t need = 4 * (size_t)(pool->timed_calls + 1);
    DeviceGuard g(pool->device);
    while (pool->events.size() < need) {
      hipEvent_t e;
      hipError_t he = hipEventCreate(&e);
      if (he != hipSuccess) return hip_fail(he, "hipEventCreate");
      pool->events.push_back(e);
    }
    ev = &pool->events[4 * (size_t)pool->timed_calls];
    ++pool->timed_calls;
  }
  hipError_t e = pkv::launch_decode(kv_kind(pool->kv_dtype), pool->head_dim, pool->block_size, p,
                                    st, ev);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return PKV_OK;
}

pkv_status kv_pool_set_window(pkv_pool* pool, int32_t window) {
  if (!pool) return fail(PKV_ERR_INVALID, "pool is null");
  if (window < 0) return fail(PKV_ERR_INVALID, "window must be >= 0 (0 = none)");
  pool->window = window;
  return PKV_OK;
}

pkv_status kv_pool_copy_blocks(pkv_pool* pool, const int32_t* pairs, int32_t n_pairs,
                               void* stream) {
  if (!pool) return fail(PKV_ERR_INVALID, "pool is null");
  if (n_pairs < 0) return fail(PKV_ERR_INVALID, "n_pairs must be >= 0");
  if (n_pairs == 0) return PKV_OK;
  if (!pairs) return fail(PKV_ERR_INVALID, "pairs is null");
  const pkv_status s = check_stream_device(pool, static_cast<hipStream_t>(stream));
  if (s != PKV_OK) return s;
  const hipError_t e = pkv::launch_copy_blocks(pairs, n_pairs, pool->kv_bytes / pool->num_blocks,
                                               (int32_t)pool->num_blocks, pool->k, pool->v,
                                               pool->err, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "block copy launch");
  return PKV_OK;
}

pkv_status pkv_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink) return fail(PKV_ERR_INVALID, "null pointer");
  if (bytes <= 0 || bytes % 16) return fail(PKV_ERR_INVALID, "bytes must be a positive multiple of 16");
  if ((uintptr_t)src % 16 || (uintptr_t)sink % 4)
    return fail(PKV_ERR_INVALID, "src must be 16-byte aligned, sink 4-byte aligned");
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "device query");
  // 16 workgroups of 256 threads per compute unit, as many as fit at once
  e = pkv::launch_stream_read(src, bytes, sink, 16 * std::max(cus, 1),
                              static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "stream read launch");
  return PKV_OK;
}

pkv_status kv_pool_enable_timing(pkv_pool* pool, int32_t enable) {
  if (!pool) return fail(PKV_ERR_INVALID, "pool is null");
  pool->timing = enable != 0;
  pool->timed_calls = 0;
  return PKV_OK;
}

pkv_status kv_pool_read_timing(pkv_pool* pool, double* attn_ms, double* merge_ms,
                               int32_t* calls) {
  if (!pool || !attn_ms || !merge_ms || !calls) return fail(PKV_ERR_INVALID, "null argument");
  double a = 0.0, m = 0.0;
  for (int i = 0; i < pool->timed_calls; ++i) {
    hipEvent_t* ev = &pool->events[4 * (size_t)i];
    hipError_t e = hipEventSynchronize(ev[3]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float t0 = 0.f, t1 = 0.f;
    e = hipEventElapsedTime(&t0, ev[0], ev[1]);
    if (e == hipSuccess) e = hipEventElapsedTime(&t1, ev[2], ev[3]);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    a += t0;
    m += t1;
  }
  *attn_ms = a;
  *merge_ms = m;
  *calls = pool->timed_calls;
  pool->timed_calls = 0;
  return PKV_OK;
}

pkv_status kv_pool_read_timeline(pkv_pool* pool, uint64_t* records, int32_t capacity,
                                 int32_t* n_waves) {
  if (!pool || !records || !n_waves) return fail(PKV_ERR_INVALID, "null argument");
  if (capacity < 0) return fail(PKV_ERR_INVALID, "capacity must be >= 0");
  if (!pool->timeline)
    return fail(PKV_ERR_UNSUPPORTED, "not a timeline build (libpkv_timeline.so records the timeline)");
  DeviceGuard g(pool->device);
  hipError_t e = hipDeviceSynchronize();
  const int32_t n = std::min(capacity, pool->n_waves);
  if (e == hipSuccess && n > 0)
    e = hipMemcpy(records, pool->timeline, sizeof(uint64_t) * 8 * n, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "reading the timeline");
  *n_waves = pool->n_waves;
  return PKV_OK;
}

pkv_status kv_pool_device_errors(pkv_pool* pool, uint32_t* flags) {
  if (!pool || !flags) return fail(PKV_ERR_INVALID, "null argument");
  uint32_t f[4] = {0, 0, 0, 0};
  DeviceGuard g(pool->device);
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(f, pool->err, sizeof f, hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemset(pool->err, 0, sizeof f);
  if (e != hipSuccess) return hip_fail(e, "reading device flags");
  *flags = (f[0] ? 1u : 0u) | (f[1] ? 2u : 0u) | (f[2] ? 4u : 0u);
  return PKV_OK;
}

}  // extern "C"
