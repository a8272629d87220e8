/*
 * pkv.h -- C ABI of the paged-KV decode step for AMD Instinct MI355X (gfx950).
 *
 * One decode step of an LLM server: every in-flight request of a ragged batch
 * brings one new query token.  The step rotates the new query and key with
 * RoPE, appends the new key/value into a pool of fixed-size KV blocks through
 * the request's block table, and computes softmax(q K^T / sqrt(D)) V over the
 * request's whole context, with query heads sharing KV heads (GQA) and a
 * bf16, fp32 or FP8 (E4M3) cache.
 *
 * Where the operation is defined:
 *   - fixed-size token blocks with per-request block tables, resolved inside
 *     the attention kernel: "Scaling TensorRT-LLM: Kernel Fusion and Inflight
 *     Batching in Production", section "The Paged KV-Cache: vLLM Borrowed by
 *     TensorRT-LLM"; the scheduler, not the kernel, hands out blocks and
 *     updates the tables (same page, "What the Scheduler Actually Does");
 *   - RoPE applied inside the attention kernel and attention intermediates
 *     kept on chip: same page, "What Gets Fused";
 *   - KV-cache update fused with attention: "TensorRT-LLM" glossary
 *     (inferensys.com), paragraph on the KV cache;
 *   - KV heads shared by groups of query heads: "TensorRT-LLM Guide:
 *     High-Throughput GPU Inference Engine", section "3. Custom Fused
 *     Attention Kernels: FMHA and XQA";
 *   - E4M3 cache with precomputed per-tensor scales: same page, section
 *     "4. Native FP8 Quantization on NVIDIA Hopper & Blackwell" (here one
 *     fp32 scale per KV head for K and one for V).
 *
 * Around the step: several new tokens per request (decode_step_multi), a
 * sliding attention window (kv_pool_set_window), whole-block copies for copy
 * on write (kv_pool_copy_blocks) and a host block allocator (pkv_alloc_*,
 * pkv_seq_*); each declaration below cites the passage it follows.
 *
 * Conventions.  All sizes are element counts unless named *_bytes.  Device
 * pointers are HIP device addresses on the pool's device.  Every function
 * returns a pkv_status and never throws; on failure pkv_last_error() returns a
 * thread-local message.  Host-visible arguments are checked before any HIP
 * call.  Calls that take a stream refuse (PKV_ERR_INVALID) one that is not on
 * the pool's device; NULL is the current device's default stream.  Calls
 * that allocate do so on the pool's device, whichever device is current.
 *
 * HIP graphs.  decode_step and decode_step_multi launch their kernels with
 * the pool's settings (window, tuning, RoPE table and workspace addresses)
 * as kernel arguments, and (with timing off and PKV_DEBUG unset) never
 * allocate, synchronise or memset, so they can be captured.  A captured graph keeps replaying the settings of capture
 * time: re-capture after kv_pool_set_window, kv_pool_set_tuning or a
 * kv_pool_set_rope that enlarges the table.  Every buffer such a graph
 * points to stays allocated until kv_pool_destroy (a larger table or
 * workspace is a new buffer; the old one is kept).
 */
#ifndef PKV_H_
#define PKV_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_INVALID = -1,      /* bad argument (null, out of range, mismatch) */
  PKV_ERR_UNSUPPORTED = -2,  /* valid but not built (dtype/size combination) */
  PKV_ERR_OOM = -3,          /* device allocation failed, or the block
                                allocator is out of blocks or sequence ids */
  PKV_ERR_HIP = -4,          /* a HIP runtime call or kernel launch failed */
  PKV_ERR_STATE = -5,        /* call order (e.g. no RoPE table set yet) */
  PKV_ERR_DEVICE_DATA = -6   /* device-resident arguments out of range */
} pkv_status;

typedef enum pkv_dtype {
  PKV_F32 = 0,               /* IEEE binary32 */
  PKV_BF16 = 1,              /* bfloat16 */
  PKV_FP8_E4M3 = 2,          /* OCP E4M3FN: bias 7, max 448, no inf */
  /* Not a dtype: makes every int32 value a valid pkv_dtype, so that an
   * unknown value from a C caller is refused (PKV_ERR_INVALID) rather than
   * undefined behaviour in the C++ implementation. */
  PKV_DTYPE_MAX_ENUM = 0x7fffffff
} pkv_dtype;

/* Opaque pool: owns the K and V block storage, the RoPE table, the FP8
 * scales and the split-K workspace, all on one device (the current HIP
 * device at kv_pool_create). */
typedef struct pkv_pool pkv_pool;

/* Physical layout of the pool, for callers that fill or inspect it.
 *
 * A block of block_size tokens is cut into block_size / 16 tiles of 16
 * tokens; for each (block n, KV head h, tile s) the tile's K and its V each
 * fill T = 16 * head_dim * kv_elem_bytes contiguous bytes, a whole number of
 * 1 KiB chunks.  With tpb = block_size / 16, the tile of (n, h, s) starts at
 * byte ((n * n_kv_heads + h) * tpb + s) * T of k_base (K) and of v_base (V).
 * Inside a tile, token t (0..15), dim d, element size E, x = 16 / E:
 *   K: byte ((d / x) * 16 + t) * 16 + (d % x) * E
 *      i.e. the tile is [head_dim / x][16 tokens][x]: 16-byte rows of x
 *      consecutive dims of one token;
 *   V: with g = 4 / E 16-dim groups per 16-byte row, nt = d / 16,
 *      c = nt / g, k = nt % g:
 *      byte ((c * 64 + (t / 4) * 16 + d % 16) * 16 + (4 * k + t % 4) * E
 *      i.e. each 16-byte row holds tokens 4*(t/4) .. +3 of one dim in each of
 *      g dim groups.
 * These are the orders in which the matrix-core operands are read: each
 * 16-byte row is one lane's share of one chunk.  Keys are stored after RoPE.
 * FP8 codes hold value / scale.
 */
typedef struct pkv_pool_info {
  int64_t num_blocks;
  int32_t block_size;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t kv_dtype;          /* pkv_dtype */
  int32_t kv_elem_bytes;
  int32_t tile_bytes;        /* T above */
  void* k_base;              /* device */
  void* v_base;              /* device */
  int64_t k_bytes;           /* bytes of K storage (equal for V) */
  int64_t v_bytes;
  const float* rope_cos;     /* device [rope_max_position][head_dim/2], or NULL */
  const float* rope_sin;
  int32_t rope_max_position; /* 0 until kv_pool_set_rope */
  double rope_theta;
  int32_t has_fp8_scales;
  int32_t device;            /* HIP device ordinal */
  int32_t n_waves;           /* wavefronts one decode_step launch runs */
  int64_t workspace_bytes;
  int32_t ring_tiles;        /* tiles each wavefront keeps in flight */
  int32_t min_units;         /* tuning in effect (kv_pool_set_tuning) */
  int32_t piece_cost;
  int32_t young_weight_pct;
  int32_t n_first;           /* wavefronts of the first workgroup on each CU */
  int32_t odd_weight_pct;
  int32_t window;            /* attention window in tokens, 0 = none */
} pkv_pool_info;

/* Create a pool of num_blocks blocks of block_size token slots for n_kv_heads
 * heads of head_dim dimensions in kv_dtype, on the current HIP device: the
 * KV cache kept in fixed-size token blocks that requests reach through
 * their block tables ("Scaling TensorRT-LLM: Kernel Fusion and Inflight
 * Batching in Production", section "The Paged KV-Cache: vLLM Borrowed by
 * TensorRT-LLM"; "TensorRT-LLM Guide: High-Throughput GPU Inference
 * Engine", section "2. Paged KV Cache & Memory Virtualization").  Block ids
 * are the caller's to hand out (the scheduler's job, same first page,
 * "What the Scheduler Actually Does").
 * Supported: head_dim in {64, 128}; block_size in {16, 32, 64};
 * 1 <= n_kv_heads <= 256; 1 <= num_blocks < 2^31 and the pool at most 2^40
 * bytes.
 * Contents are left uninitialised.  On success *out_pool owns device memory
 * until kv_pool_destroy.  Errors: INVALID (null/out of range), UNSUPPORTED,
 * OOM, HIP. */
pkv_status kv_pool_create(int64_t num_blocks, int32_t block_size,
                          int32_t n_kv_heads, int32_t head_dim,
                          pkv_dtype kv_dtype, pkv_pool** out_pool);

/* Free every device buffer of the pool (after synchronising its device).
 * NULL is accepted and ignored. */
pkv_status kv_pool_destroy(pkv_pool* pool);

/* Build the RoPE table for positions [0, max_position): for i < head_dim/2,
 * angle = p * theta^(-2i/head_dim) in double precision, cos and sin each
 * rounded once to fp32 (rotate-half pairing (i, i + head_dim/2), as in
 * "What Gets Fused" of "Scaling TensorRT-LLM: ...").  Synchronous.
 * Errors: INVALID (theta <= 0, max_position < 1), OOM, HIP. */
pkv_status kv_pool_set_rope(pkv_pool* pool, double theta, int32_t max_position);

/* Set the FP8 scales of an E4M3 cache with precomputed ("delayed") scale
 * factors ("TensorRT-LLM Guide: High-Throughput GPU Inference Engine",
 * section "4. Native FP8 Quantization on NVIDIA Hopper & Blackwell"; here one
 * fp32 scale per KV head for K and one for V, host arrays of n_kv_heads
 * values, all > 0 and finite): a cached code c of head h means
 * c * k_scale[h] (K) or c * v_scale[h] (V).  New tokens are encoded as
 * E4M3(y * fp32(1/scale)) with round-to-nearest-even and saturation to
 * +-448; a NaN is stored as the NaN code S.1111.111 with its sign.  The NaN
 * codes read back as NaN, so a NaN in the cache makes the rows that attend
 * to it NaN, as with a bf16 or fp32 cache.  Synchronous.  Only for
 * PKV_FP8_E4M3 pools (else INVALID). */
pkv_status kv_pool_set_fp8_scales(pkv_pool* pool, const float* k_scale,
                                  const float* v_scale);

/* Describe the pool (layout, device pointers). */
pkv_status kv_pool_get_info(const pkv_pool* pool, pkv_pool_info* info);

/* The pool's storage, for callers that fill or read it in place (zero
 * copy).  The blocks of the paged cache ("Scaling TensorRT-LLM: Kernel
 * Fusion and Inflight Batching in Production", section "The Paged
 * KV-Cache: vLLM Borrowed by TensorRT-LLM") are addressed by three byte
 * strides: byte_strides[0] per block, [1] per KV head, [2] per 16-token
 * tile, from k_base (K) and v_base (V), device pointers the pool owns.
 * Inside a tile of *tile_bytes bytes the elements are not strided: they sit
 * in the matrix-core operand order given above pkv_pool_info (K as 16-byte
 * rows of x consecutive dims of one token, V as 16-byte rows of four
 * consecutive tokens of one dim), which no (slot, dim) stride pair can
 * express.  Errors: INVALID (null argument). */
pkv_status kv_pool_layout(const pkv_pool* pool, void** k_base, void** v_base,
                          int64_t byte_strides[3], int32_t* tile_bytes);

/* The RoPE table the kernels read (built by kv_pool_set_rope; RoPE applied
 * inside the attention kernel, "Scaling TensorRT-LLM: ...", section "What
 * Gets Fused"): device arrays of *max_position rows of head_dim/2 fp32
 * values, cos and sin of p * theta^(-2i/head_dim), owned by the pool.
 * Errors: INVALID (null argument), STATE (no table yet; the pointers are
 * then NULL and *max_position 0). */
pkv_status kv_pool_rope_table(const pkv_pool* pool, const float** cos_dev,
                              const float** sin_dev, int32_t* max_position);

/* One decode step for `batch` requests: the cache update and the attention
 * fused in one pass ("TensorRT-LLM" glossary, inferensys.com, paragraph on
 * the KV cache), RoPE applied inside the attention kernel and its
 * intermediates kept on chip ("Scaling TensorRT-LLM: Kernel Fusion and
 * Inflight Batching in Production", section "What Gets Fused"), launched
 * once per iteration after the scheduler has updated the block tables (same
 * page, "What the Scheduler Actually Does").  Asynchronous on `stream`, a
 * hipStream_t; NULL = the default stream; no host synchronisation unless the
 * environment variable PKV_DEBUG=1 asks for device-argument validation.
 *
 * Arguments (device pointers, contiguous, row-major; q, k_new, v_new and out
 * 16-byte aligned, the int32 arrays 4-byte aligned):
 *   q            [batch][n_q_heads][head_dim]   io_dtype, not rotated
 *   k_new, v_new [batch][n_kv_heads][head_dim]  io_dtype, k_new not rotated
 *   positions    [batch] int32   RoPE position of the new token
 *   block_tables [batch][max_blocks_per_seq] int32 physical block ids
 *   context_lens [batch] int32   L_b: tokens of request b counting the new one
 *   out          [batch][n_q_heads][head_dim]   io_dtype (written)
 * Effect: for each request b and KV head h, the rotated k_new and v_new are
 * cast to kv_dtype and stored in slot L_b - 1 (block
 * block_tables[b][(L_b-1)/block_size], offset (L_b-1) % block_size); then
 * out[b][hq] = softmax over t < L_b of (rope(q[b][hq]) . K[t]) / sqrt(D),
 * applied to V[t], with K/V read from head hq / (n_q_heads / n_kv_heads).
 * Nothing else in the pool is written.
 * Supported io/kv pairs: (F32, F32), (BF16, BF16), (BF16, FP8_E4M3);
 * n_q_heads = G * n_kv_heads with 1 <= G <= 16; batch <= 4096.
 * Two kernels are launched: the fused append + attention kernel, and a small
 * kernel that merges the partial softmax states of sequences split between
 * wavefronts.
 * Caller guarantees (checked only under PKV_DEBUG=1; otherwise the kernel
 * clamps out-of-range values, computes garbage for that request, and raises a
 * flag readable with kv_pool_device_errors):
 *   1 <= L_b <= max_blocks_per_seq * block_size;
 *   entries 0 .. ceil(L_b/block_size)-1 of row b are ids in [0, num_blocks);
 *   the block holding slot L_b-1 belongs to request b alone (other blocks may
 *   be shared read-only between requests);
 *   0 <= positions[b] < the RoPE max_position.
 * The pool's workspace is shared: one decode_step at a time per pool.
 * Every pointer must stay valid until the stream work completes.
 * batch == 0 is a no-op.  Errors: INVALID, UNSUPPORTED, STATE (RoPE table or
 * FP8 scales missing), HIP, DEVICE_DATA (debug validation). */
pkv_status decode_step(pkv_pool* pool, const void* q, const void* k_new,
                       const void* v_new, pkv_dtype io_dtype,
                       const int32_t* positions, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* context_lens,
                       int32_t batch, int32_t n_q_heads, void* out,
                       void* stream);

/* decode_step for callers that cannot allocate device memory at step time:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same kernels, arguments and results as decode_step, with
 * the split-K workspace (partial softmax states and per-wavefront headers)
 * in a fixed per-device array that the library holds from the moment its
 * code object loads until the process ends, instead of the pool's: 32.5 MiB
 * per GPU, room for 2048 wavefronts at head_dim <= 128.  It allocates
 * nothing, synchronises nothing, and neither reads PKV_DEBUG nor records
 * timing events.  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (on different streams, or from different pools) race
 * and give wrong outputs, so serialise them.  The array keeps the last
 * call's partial states; none of it needs clearing, since every launch
 * writes all of it that it later reads.  Errors as decode_step, plus
 * UNSUPPORTED when the pool runs more than 2048 wavefronts
 * (kv_pool_set_tuning above 8 per compute unit on 256 compute units). */
pkv_status decode_step_noalloc(pkv_pool* pool, const void* q, const void* k_new,
                               const void* v_new, pkv_dtype io_dtype,
                               const int32_t* positions, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* context_lens,
                               int32_t batch, int32_t n_q_heads, void* out, void* stream);

/* A step that brings n_new >= 1 new tokens per request: a chunk of a long
 * prompt processed beside decoding requests ("Lesson 13.17 TensorRT-LLM:
 * NVIDIA's Optimized Inference Engine", section "The paged KV cache, in-flight
 * batching and CUDA graphs"), or draft tokens verified in one pass (same page,
 * section "Speculative decoding and running one model across many GPUs";
 * "Scaling TensorRT-LLM: Kernel Fusion and Inflight Batching in Production",
 * section "3. Speculative Decoding for Tail Latency").  Layouts as
 * decode_step with a token axis: q and out [B][n_new][n_q_heads][head_dim],
 * k_new and v_new [B][n_new][n_kv_heads][head_dim]; positions[b] is the RoPE
 * position of the first new token (new token i is at positions[b] + i);
 * context_lens[b] counts all n_new new tokens, which go to slots
 * L - n_new .. L - 1.  Query i attends to the tokens [0, L - n_new + i]
 * (causal inside the new tokens).  n_new = 1 is decode_step.  For n_new > 1:
 * a bf16 or fp8 cache, no attention window, (n_q_heads / n_kv_heads) x n_new
 * <= 16 (PKV_ERR_UNSUPPORTED otherwise), a RoPE table of >= n_new positions;
 * the new tokens are appended by a separate launch before the attention
 * kernel.  The blocks holding the new tokens must be the request's own. */
pkv_status decode_step_multi(pkv_pool* pool, const void* q, const void* k_new,
                             const void* v_new, pkv_dtype io_dtype, int32_t n_new,
                             const int32_t* positions, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* context_lens,
                             int32_t batch, int32_t n_q_heads, void* out, void* stream);

/* Read and clear the device-side range flags raised by earlier decode_step
 * calls (synchronises the device).  Bit 0: a block id outside
 * [0, num_blocks); bit 1: a position outside [0, max_position); bit 2: a
 * context length outside [1, max_blocks_per_seq * block_size]. */
pkv_status kv_pool_device_errors(pkv_pool* pool, uint32_t* flags);

/* Tuning knobs (also read from PKV_WAVES_PER_CU, PKV_MIN_UNITS,
 * PKV_PIECE_COST, PKV_YOUNG_WEIGHT and PKV_ODD_WEIGHT at pool creation).  The step's work is
 * measured in units: one per 16-token tile, plus piece_cost for starting
 * each (request, KV head) sequence (its query rotation and append stall the
 * wavefront's loads), and split over the wavefronts in proportion to their
 * weights (pkv_plan_host states the rule).
 *  - waves_per_cu: wavefronts per compute unit (0 = as many as are resident
 *    at once, 8 on gfx950).
 *  - min_units: fewest units the lightest wavefront is given before fewer
 *    wavefronts are used (>= 1; raised to piece_cost + 1; default 16); a step
 *    too small to fill the first workgroup of every compute unit that way
 *    goes down to a quarter of it, never below piece_cost + 1, on at most
 *    those wavefronts (pkv_plan_host states the rule).
 *  - piece_cost: in [0, 64], or -1 (the default) for ring_tiles + 2.  A
 *    sequence start waits for the wavefront's whole ring of in-flight tile
 *    loads and then for its own query loads.
 *  - young_weight_pct: share weight of the wavefronts of the later
 *    workgroups on each compute unit, in percent of the first workgroup's
 *    ([1, 100], or -1 for the default 65).  Two wavefronts on one SIMD
 *    share its issue slots unevenly: the older streams 1.6-1.9x faster
 *    while both run.  100 splits evenly.  The weights apply only to steps
 *    with at least 256 units per launched wavefront (below that start-up
 *    dominates and the split is even).
 *  - odd_weight_pct: share weight of the wavefronts of odd workgroups, in
 *    percent of the even ones' ([1, 100], or -1 for the default 90), on
 *    top of the age weight and at every step size.  Workgroups are dealt to
 *    the eight XCDs in turn, so odd workgroups run on odd XCDs, which stream
 *    about a tenth slower on MI355X.  100 splits evenly.
 * Synchronises the device. */
pkv_status kv_pool_set_tuning(pkv_pool* pool, int32_t waves_per_cu,
                              int32_t min_units, int32_t piece_cost,
                              int32_t young_weight_pct, int32_t odd_weight_pct);

/* Sliding-window attention for the pool's layer ("TensorRT-LLM" glossary
 * entry, inferensys.com, which names Sliding Window Attention among the
 * architecture patterns the kernels exploit): with window >= 1, each request
 * of a later decode_step attends to its last `window` tokens only, the new
 * one included, i.e. the tokens [max(0, L - window), L); whole blocks before
 * the window are not read.  0 (the default) attends to the whole context.
 * The append is unchanged.  PKV_ERR_INVALID for window < 0. */
pkv_status kv_pool_set_window(pkv_pool* pool, int32_t window);

/* Copy whole blocks inside the pool: for i < n_pairs, block pairs[2i + 1]
 * gets the K and V contents (every head and slot) of block pairs[2i].  This
 * is the copy on write of a shared prefix block, done before a step appends
 * to it (pkv_alloc_prepare_step names the pairs); blocks reused across
 * requests that share a prefix: "Lesson 13.17 TensorRT-LLM: NVIDIA's
 * Optimized Inference Engine", section "The paged KV cache, in-flight
 * batching and CUDA graphs".  pairs: device int32 [n_pairs][2], owned by the
 * caller, valid until the copy has run on `stream`; no destination may also
 * be a source or appear twice (the copies run in any order).  Asynchronous on
 * `stream` (a hipStream_t; NULL = the default stream).  Ids outside [0, num_blocks) are skipped and reported as flag 1
 * of kv_pool_device_errors; a pair with equal ids does nothing. */
pkv_status kv_pool_copy_blocks(pkv_pool* pool, const int32_t* pairs, int32_t n_pairs,
                               void* stream);

/* Measurement.  While enabled, decode_step launches its two kernels (the
 * fused attention kernel and the split-merge kernel) with HIP start/stop
 * events that the dispatches themselves stamp.  kv_pool_read_timing waits
 * for the recorded events, returns the summed kernel milliseconds of each
 * kind and the number of decode_step calls since the last read (or enable),
 * and starts over.  At most 65536 calls are recorded between reads (later
 * ones are not timed). */
pkv_status kv_pool_enable_timing(pkv_pool* pool, int32_t enable);
pkv_status kv_pool_read_timing(pkv_pool* pool, double* attn_ms, double* merge_ms,
                               int32_t* calls);

/* Per-wavefront timeline of the last decode_step on this pool, from a
 * timeline build of the library (libpkv_timeline.so, built with
 * -DPKV_TIMELINE; the kernels are otherwise the same): where each attention
 * wavefront's time went, the measurement that splits a step's duration into
 * start-up, streaming and tail.  Synchronises the device, then copies
 * min(capacity, n_waves) records of 8 uint64 to `records` (host memory):
 * stamps of the GPU's constant 100 MHz clock at 0 entry, 1 request table
 * built, 2 tile range found, 3 load ring filled, 4 tile loop done, 5 exit;
 * 6 the wavefront's tiles; 7 HW_ID in the low word (bits 3:0 wave slot, 5:4
 * SIMD, 11:8 compute unit, 15:13 shader engine) and XCC_ID in the high word.
 * A wavefront without tiles records its entry in 0-5 and 0 tiles.
 * *n_waves = wavefronts of the pool's launch.  decode_step_noalloc records
 * nothing.  Errors: INVALID (null argument, capacity < 0), UNSUPPORTED (not
 * a timeline build), HIP. */
pkv_status kv_pool_read_timeline(pkv_pool* pool, uint64_t* records, int32_t capacity,
                                 int32_t* n_waves);

/* Read `bytes` of device memory at `src` once with the attention kernel's
 * 16-byte nontemporal loads, on the current device, asynchronously on
 * `stream` (NULL = the default stream): the bandwidth a plain streaming read
 * reaches, the reference next to the nominal HBM peak when a step is judged
 * by its HBM bandwidth (decode waits on memory transfers: "TensorRT-LLM
 * Guide: High-Throughput GPU Inference Engine", section "The Problem: The
 * Memory-Bandwidth Wall and Static Batching Inefficiencies").  src: device,
 * 16-byte aligned; bytes: a positive multiple of 16; sink: device, 1 KiB,
 * written only in the unlikely case that the folded data equals a fixed
 * constant.  Errors: INVALID, HIP. */
pkv_status pkv_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);

/* Thread-local message of the last failing call on this thread ("" if none). */
const char* pkv_last_error(void);

/* ---- block allocator (host only, no GPU needed) --------------------------
 *
 * The cache lives in fixed-size blocks handed out on demand as tokens are
 * generated, with waste bounded by each sequence's last, partly filled block
 * ("TensorRT-LLM Guide: High-Throughput GPU Inference Engine", section
 * "2. Paged KV Cache & Memory Virtualization"); the scheduler updates the
 * block tables every iteration ("Scaling TensorRT-LLM: Kernel Fusion and
 * Inflight Batching in Production", section "What the Scheduler Actually
 * Does"); blocks are reused across requests that share a prefix ("Lesson
 * 13.17 TensorRT-LLM: NVIDIA's Optimized Inference Engine", section "The
 * paged KV cache, in-flight batching and CUDA graphs").
 *
 * A sequence holds a list of block ids and a length in tokens.  A block
 * carries a reference count: the number of sequences holding it.  Free blocks
 * sit on a stack: a new allocator hands out 0, 1, 2, ..., and the most
 * recently freed block is the next one handed out.  Sequence ids are the
 * lowest free id.  Not thread-safe; it never touches the GPU.  Every call
 * that fails leaves the allocator unchanged. */
typedef struct pkv_block_alloc pkv_block_alloc;

/* An allocator over num_blocks blocks of block_size tokens and at most
 * max_seqs live sequences.  PKV_ERR_INVALID for sizes < 1. */
pkv_status pkv_alloc_create(int64_t num_blocks, int32_t block_size, int32_t max_seqs,
                            pkv_block_alloc** out);
pkv_status pkv_alloc_destroy(pkv_block_alloc* alloc);

/* Free blocks and live sequences (either pointer may be NULL). */
pkv_status pkv_alloc_stats(const pkv_block_alloc* alloc, int64_t* free_blocks,
                           int32_t* live_seqs);

/* Reference count of one block (0 = free). */
pkv_status pkv_alloc_refcount(const pkv_block_alloc* alloc, int32_t block, int32_t* count);

/* A new sequence already holding `length` tokens (a prompt whose K/V the
 * caller writes into its blocks): ceil(length / block_size) fresh blocks.
 * PKV_ERR_OOM if the blocks or a sequence id are not available. */
pkv_status pkv_seq_add(pkv_block_alloc* alloc, int32_t length, int32_t* seq);

/* A new sequence sharing every block of `parent` (prefix sharing: parallel
 * samples, beams, a common system prompt); same length; each shared block's
 * count goes up by one. */
pkv_status pkv_seq_fork(pkv_block_alloc* alloc, int32_t parent, int32_t* child);

/* End a sequence: each of its blocks' counts goes down by one, and blocks
 * that reach zero are freed (its last block first). */
pkv_status pkv_seq_release(pkv_block_alloc* alloc, int32_t seq);

/* Length, block count and the first min(max_blocks, count) block ids. */
pkv_status pkv_seq_info(const pkv_block_alloc* alloc, int32_t seq, int32_t* length,
                        int32_t* n_blocks, int32_t* blocks, int32_t max_blocks);

/* The host side of one decode step for the batch seq_ids[0 .. batch): each
 * sequence (distinct ids) grows by the step's new token, at slot = its old
 * length.  If the slot starts a block, a fresh block is appended; if the
 * block holding the slot is shared, the sequence gets a fresh block in its
 * place and the pair {shared, fresh} goes to `copies` (copy on write; when
 * every holder of a shared block appends in the same step, the last of them
 * in batch order keeps it).  Writes, in host memory the caller owns, the
 * arguments decode_step takes: block_tables [batch][max_blocks_per_seq]
 * (ids, then -1), context_lens [batch] (the new lengths, counting the new
 * token) and positions [batch] (new length - 1), plus up to max_copies pairs
 * to copies [max_copies][2] and their number to *n_copies.  The caller runs
 * kv_pool_copy_blocks on the pairs before decode_step.  PKV_ERR_INVALID for a
 * dead or repeated id, a sequence outgrowing max_blocks_per_seq blocks or more
 * copies than max_copies; PKV_ERR_OOM if the free blocks do not cover the
 * fresh blocks and copies. */
pkv_status pkv_alloc_prepare_step(pkv_block_alloc* alloc, const int32_t* seq_ids, int32_t batch,
                                  int32_t max_blocks_per_seq, int32_t* block_tables,
                                  int32_t* context_lens, int32_t* positions, int32_t* copies,
                                  int32_t max_copies, int32_t* n_copies);

/* ---- host-only helpers (no GPU needed) --------------------------------- */

/* Check decode_step's host-visible arguments against a pool description,
 * exactly as decode_step does before touching the GPU. */
pkv_status pkv_check_decode_args(int64_t num_blocks, int32_t block_size,
                                 int32_t n_kv_heads, int32_t head_dim,
                                 pkv_dtype kv_dtype, pkv_dtype io_dtype,
                                 const void* q, const void* k_new,
                                 const void* v_new, const int32_t* positions,
                                 const int32_t* block_tables,
                                 int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t batch,
                                 int32_t n_q_heads, const void* out);

/* The RoPE table kv_pool_set_rope uploads, computed into host arrays of
 * max_position * head_dim/2 floats each. */
pkv_status pkv_rope_table_host(double theta, int32_t head_dim,
                               int32_t max_position, float* cos_out,
                               float* sin_out);

/* The work partition decode_step's kernel computes on the device, replayed
 * on the host from host copies of context_lens, for testing.  Each
 * (request, KV head) sequence is cut into 16-token tiles (at least one;
 * lengths clamped to [0, max_tokens]) and costs its tiles plus piece_cost
 * units; its tile 0 owns the units [s, s + piece_cost], tile j >= 1 the unit
 * s + piece_cost + j.  The sequences' units are concatenated in (request,
 * head) order, U in all.  Wavefront w weighs a * p: its age weight a is
 * weight_first if w < n_first, else weight_rest (1 <= weight_rest <=
 * weight_first <= 1000), when U >= weight_min_share * n_waves, and 1
 * otherwise; its parity weight p is weight_odd (in [1, 100]) if its
 * workgroup w / 4 is odd, else 100.  With Omega(w) the summed weight of
 * wavefronts [0, w), W active wavefronts split the units at
 * floor(U * Omega(w) / Omega(W)), and W is the largest value <= n_waves (and
 * >= 1) with U * a_min * p_min >= m * Omega(W), where m = max(min_units,
 * piece_cost + 1) and a_min * p_min is the lightest weight any of the
 * n_waves wavefronts has: every active wavefront gets at least m units.  If
 * that W is below min(n_first, n_waves) (a step too small to fill the first
 * workgroup of every compute unit), W is instead the largest value with the
 * same inequality for m' = max(m / 4, piece_cost + 1), capped at
 * min(n_first, n_waves): small steps are latency-bound, and more wavefronts
 * with fewer tiles each finish sooner.  A wavefront takes the tiles whose
 * first unit falls in its range.
 * With window >= 1 a sequence of context L costs only the tiles from its
 * window's first one, floor(max(L - window, 0) / 16), on.
 * decode_step uses n_first = the first workgroup on each compute unit (4
 * wavefronts per CU), weight_first = 100, weight_rest = young_weight_pct,
 * weight_odd = odd_weight_pct, weight_min_share = 256 and the pool's
 * window.  Writes up to
 * max_pieces rows of 6 int32 to pieces:
 * {wave, request, kv_head, first_tile, end_tile, flags} with flags bit 0 =
 * the piece is part of a split sequence, bit 1 = it is the wave's first
 * piece, bit 2 = it is the last piece of its sequence; and n_waves rows of
 * 4 int32 to splits: row w describes the split sequence whose first piece
 * wave w holds, {1, request * n_kv_heads + kv_head, pieces, partial slot of
 * the first piece}, or zeros.  *n_pieces receives the total count. */
pkv_status pkv_plan_host(const int32_t* context_lens, int32_t batch,
                         int32_t n_kv_heads, int32_t max_tokens, int32_t n_waves,
                         int32_t min_units, int32_t piece_cost, int32_t n_first,
                         int32_t weight_first, int32_t weight_rest, int32_t weight_odd,
                         int32_t weight_min_share, int32_t window, int32_t max_pieces,
                         int32_t* pieces, int32_t* n_pieces,
                         int32_t* splits);

/* Tokens per tile, the kernel's unit of work (16). */
int32_t pkv_tile_tokens(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
