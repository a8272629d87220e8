// decode.hip -- fused paged-KV decode step for gfx950 (MI355X).
//
// One kernel does the whole step for its share of the batch: RoPE of the new
// query and key, the append of the new K/V into the block pool, the gather of
// the cached K/V through the block table, and softmax(q K^T / sqrt(D)) V with
// an online softmax.  A second, small kernel merges the partial softmax
// states of the sequences that were cut between wavefronts (split-K).
//
// The pages ask for: the block-table lookup done inside the attention kernel
// ("Scaling TensorRT-LLM: Kernel Fusion and Inflight Batching in Production",
// section "The Paged KV-Cache: vLLM Borrowed by TensorRT-LLM"); RoPE inside the
// attention kernel and intermediates kept on chip (same page, "What Gets
// Fused"); KV blocks read once and reused by every query head of the group
// ("TensorRT-LLM Guide: High-Throughput GPU Inference Engine", section
// "3. Custom Fused Attention Kernels: FMHA and XQA"); an E4M3 cache with
// precomputed scales (same page, section "4. Native FP8 Quantization on NVIDIA
// Hopper & Blackwell"); attention and KV-cache update fused ("TensorRT-LLM"
// glossary, inferensys.com, paragraph on the KV cache).
//
// Mapping onto CDNA4.  The step streams the KV cache from HBM once per KV
// head, so it is bound by HBM bandwidth.  The unit of work is a tile: 16
// tokens of one (request, KV head) sequence.  A tile's K and its V are each a
// whole number of contiguous 1 KiB chunks inside one block, laid out so that
// one 16-byte load per lane per chunk (all lanes of a wavefront at one
// wave-uniform base) lands every element in the register the matrix cores
// read it from: no LDS round trip and no shuffles on the data path.
//
// Each wavefront owns a contiguous range of tiles (plan.h) and keeps RING
// tiles in flight in registers, refilling a slot as soon as it has been used;
// the ring runs on across sequence boundaries.  Block ids come from the block
// table through the scalar cache, one tile ahead of the loads that need
// them, so the vector memory counter only ever tracks the KV stream.
//
// Arithmetic.  Scores are a 16-token x G-head product over D, values a
// D x G product over 16 tokens, G <= 16: both go to 16x16 MFMA tiles with the
// group padded to 16 columns (the matrix cores have far more throughput than
// the KV stream needs; the VALU would be busy with the FMAs at G = 8).
// Lane = 16 * lq + lr with lr in [0, 16), lq in [0, 4):
//  * scores: A = K rows (row lr = token lr of the tile), B = rotated queries
//    (column lr = head lr, zero past G); the contraction over the head
//    dimension is order-free, so lane (lr, lq) supplies the X dims
//    [X*(4c + lq), X*(4c + lq) + X) of chunk c, X = 16 bytes / element size;
//    the result gives lane (lr, lq) S[tokens 4lq .. 4lq+3][head lr];
//  * values: A = V^T (16 dims x 4 tokens per lane), B = P^T; lane (lr, lq)
//    supplies tokens 4lq .. 4lq+3 of dim lr of each 16-dim group, exactly the
//    probabilities it already holds; the result gives it
//    O[head lr][dims 16*nt + 4lq .. 16*nt + 4lq + 3].
// The four lanes of a head (lq = 0..3) combine maxima and sums with the
// gfx950 permlane16/permlane32 swaps.
//
// Split merge.  The partial states are plain stores and are merged by a
// second launch: the kernel boundary makes them visible across the eight
// XCDs' L2 caches with one write-back, where a device-scope release inside
// the kernel would write back an XCD's whole L2 once per wavefront.
#include <hip/hip_ext.h>

#include <utility>

#include "kernels.h"
#include "plan.h"

// One object per cache type: the build compiles this file once for each of
// KV_F32, KV_BF16 and KV_FP8 (-DPKV_KV=0, 1, 2), in parallel.
#ifndef PKV_KV
#error "decode.hip is compiled once per cache type, with -DPKV_KV=<KvKind>"
#endif

// K+V bytes each wavefront keeps in flight (fp8 needs registers for the code
// conversions, so it keeps a little less).
#ifndef PKV_RING_BYTES
#define PKV_RING_BYTES 32768
#endif
#ifndef PKV_RING_BYTES_FP8
#define PKV_RING_BYTES_FP8 16384
#endif
// Bytes of LDS per wavefront that hold the global writes of the tile loop
// (output rows, appended rows, the first partial state) until the loop ends.
#ifndef PKV_QUEUE_BYTES
#define PKV_QUEUE_BYTES 10240
#endif
// Resident wavefronts per SIMD the attention kernel is compiled for (its
// register budget is 512 / this).
#ifndef PKV_WAVES_PER_EU
#define PKV_WAVES_PER_EU 2
#endif

// Timeline builds (-DPKV_TIMELINE, a separate library): every attention
// wavefront records when it reached each phase of its work, from the GPU's
// constant 100 MHz clock, into p.timeline[wave][8]: 0 entry, 1 request table
// built in LDS, 2 tile range found, 3 load ring filled, 4 tile loop done,
// 5 exit (after the queued writes), 6 its tiles, 7 HW_ID (low word: wave
// slot, SIMD, CU, shader engine) and XCC_ID (high word).  A wavefront with
// no tiles records its entry in slots 0-5 and 0 tiles.  Normal builds
// compile none of this.
#ifdef PKV_TIMELINE
#define PKV_STAMP(i) const uint64_t stamp##i = __builtin_amdgcn_s_memrealtime()
#else
#define PKV_STAMP(i)
#endif

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <class F, int... Is>
__device__ __forceinline__ void static_for(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}

// ---------------------------------------------------------------- scalars
__device__ __forceinline__ float exp2_fast(float x) {
  return __builtin_amdgcn_exp2f(x);   // v_exp_f32; -inf -> 0
}

// Combine a value over the four lanes lr, lr+16, lr+32, lr+48 (the lanes of
// one query head).  Every lane gets the same bits.
__device__ __forceinline__ float max_over_lq(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float sum_over_lq(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// The value of lane (lr + 8) mod 16 of the same row of 16 lanes (DPP
// row_ror:8): pairs the MFMA columns g and g + 8.
__device__ __forceinline__ float swap_half_row(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false));
}

// Wait for every vector memory operation of the wavefront (vmcnt 0; the
// other counters untouched).  Ends a rarely taken branch that stores inside
// the tile loop: the stores are then complete where the branch rejoins, and
// the waits for tile loads that follow keep their exact in-order counts
// instead of degrading to full drains on every path.
__device__ __forceinline__ void wait_vector_memory() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// Issue priority of the wavefront (0..3, uniform argument).  Two
// wavefronts on one SIMD otherwise share its issue slots oldest-first, and
// the older one streams its tiles much faster while both run.  Each
// wavefront lowers its priority as it gets through its tiles (3 until half
// done, 2 until 3/4, 1 until 7/8, then 0), so the one that is behind wins
// the issue slots until it catches up: the two meet at each of those marks
// and finish within about 1/8 of their tiles of each other.
__device__ __forceinline__ void set_priority(int level) {
  if (level >= 3) __builtin_amdgcn_s_setprio(3);
  else if (level == 2) __builtin_amdgcn_s_setprio(2);
  else if (level == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// float32 -> bfloat16 bits, round to nearest even (finite), quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// float32 -> E4M3FN code: saturating round-to-nearest-even, sign copied.
__device__ __forceinline__ uint32_t fp8_encode(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  if (!(a == a)) return sign | 0x7fu;
  if (a >= 448.0f) return sign | 0x7eu;
  if (a < 0.015625f) {                       // subnormal grid: 2^-9 steps
    return sign | (uint32_t)__builtin_rintf(a * 512.0f);   // 8 -> 0x08 = 2^-6
  }
  int e;
  (void)__builtin_frexpf(a, &e);             // a = f * 2^e, f in [0.5, 1)
  e -= 1;                                    // a in [2^e, 2^(e+1))
  const float mant = __builtin_ldexpf(a, -e) - 1.0f;    // exact, in [0, 1)
  uint32_t m = (uint32_t)__builtin_rintf(mant * 8.0f);
  if (m == 8u) { m = 0u; e += 1; }
  return sign | ((uint32_t)(e + 7) << 3) | m;
}

// Four E4M3 codes (bytes of w, lowest first) -> four f16 holding the same
// values: gfx950's OCP FP8 conversion, two codes per instruction, with a
// scale of 1.  Every E4M3 value (subnormals included) is an f16 value, so
// the conversion is exact, and the NaN codes S.1111.111 give NaN.
__device__ __forceinline__ f16x4_t fp8x4_to_f16x4(uint32_t w) {
  u32x2_t r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
  return __builtin_bit_cast(f16x4_t, r);
}

__device__ __forceinline__ void fp8x16_to_f16(u32x4_t c, f16x8_t& lo, f16x8_t& hi) {
  u32x4_t a, b;
  const f16x4_t a0 = fp8x4_to_f16x4(c[0]), a1 = fp8x4_to_f16x4(c[1]);
  const f16x4_t b0 = fp8x4_to_f16x4(c[2]), b1 = fp8x4_to_f16x4(c[3]);
  const u32x2_t wa0 = __builtin_bit_cast(u32x2_t, a0), wa1 = __builtin_bit_cast(u32x2_t, a1);
  const u32x2_t wb0 = __builtin_bit_cast(u32x2_t, b0), wb1 = __builtin_bit_cast(u32x2_t, b1);
  a[0] = wa0[0]; a[1] = wa0[1]; a[2] = wa1[0]; a[3] = wa1[1];
  b[0] = wb0[0]; b[1] = wb0[1]; b[2] = wb1[0]; b[3] = wb1[1];
  lo = __builtin_bit_cast(f16x8_t, a);
  hi = __builtin_bit_cast(f16x8_t, b);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const _Float16 ha = (_Float16)a, hb = (_Float16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) |
         ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// ---------------------------------------------------------------- io access
template <bool IO_BF16>
__device__ __forceinline__ float load_io(const void* base, int64_t idx) {
  if constexpr (IO_BF16) {
    const uint16_t h = static_cast<const uint16_t*>(base)[idx];
    return __uint_as_float((uint32_t)h << 16);
  } else {
    return static_cast<const float*>(base)[idx];
  }
}

// N consecutive io-dtype elements starting at element `off` -> float.
template <bool IO_BF16, int N>
__device__ __forceinline__ void load_row_f32(const void* base, int64_t off, float (&out)[N]) {
  if constexpr (IO_BF16) {
    static_assert(N % 8 == 0, "bf16 rows are read 16 bytes at a time");
    const u32x4_t* ptr = reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int i = 0; i < N / 8; ++i) {
      const u32x4_t w = ptr[i];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        out[8 * i + 2 * k] = __uint_as_float(w[k] << 16);
        out[8 * i + 2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
      }
    }
  } else {
    static_assert(N % 4 == 0, "f32 rows are read 16 bytes at a time");
    const f32x4_t* ptr = reinterpret_cast<const f32x4_t*>(static_cast<const float*>(base) + off);
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const f32x4_t w = ptr[i];
#pragma unroll
      for (int k = 0; k < 4; ++k) out[4 * i + k] = w[k];
    }
  }
}

template <int N>
__device__ __forceinline__ void load_f32(const float* ptr, float (&out)[N]) {
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {
    const f32x4_t w = reinterpret_cast<const f32x4_t*>(ptr)[i];
#pragma unroll
    for (int k = 0; k < 4; ++k) out[4 * i + k] = w[k];
  }
}

// Encode one float into the cache storage type (bit pattern in the low bits).
template <int KV>
__device__ __forceinline__ uint32_t encode_kv(float y, float inv_scale) {
  if constexpr (KV == KV_F32) return __float_as_uint(y);
  else if constexpr (KV == KV_BF16) return bf16_rne(y);
  else return fp8_encode(y * inv_scale);
}

// ---------------------------------------------------------------- layout
template <int KV, int D, int BS>
struct Cfg {
  static constexpr int ELEM = KV == KV_F32 ? 4 : (KV == KV_BF16 ? 2 : 1);
  static constexpr int X = 16 / ELEM;          // elements per 16-byte row
  static constexpr int KCH = D * ELEM / 64;    // 1 KiB chunks of K (and of V) per tile
  static constexpr int NGR = 4 / ELEM;         // 16-dim groups per 16-byte V row
  static constexpr int NT = D / 16;            // 16-dim groups of the output
  static constexpr int HALF = D / 2;
  static constexpr int KROWS = D / X;          // 16-byte rows of one token's key
  static constexpr int TILE_BYTES = KCH * 1024;
  static constexpr int TPB = BS / kTileTokens; // tiles per block
  static constexpr int LOG2TPB = TPB == 1 ? 0 : (TPB == 2 ? 1 : 2);
  static constexpr int RING0 = (KV == KV_FP8 ? PKV_RING_BYTES_FP8 : PKV_RING_BYTES) / (2 * TILE_BYTES);
  static constexpr int RING = RING0 < 2 ? 2 : (RING0 > 16 ? 16 : RING0);
  static constexpr bool IO_BF16 = KV != KV_F32;
  static_assert(KCH >= 1 && KCH * 64 == D * ELEM, "tile must be whole 1 KiB chunks");
  static_assert(TPB >= 1 && TPB <= 4, "block_size must be 16, 32 or 64");
  static_assert((2 * RING - 1) * KCH <= 63, "in-flight loads must fit the vmcnt counter");
};

// Byte offset of K element (token t of the tile, dim d) inside the tile:
// the tile is [D/X][16 tokens][X], i.e. chunk c, lane 16*lq + t holds dims
// X*(4c + lq) .. + X - 1 of token t.
// Byte offset of V element (t, d): with nt = d / 16, c = nt / NGR,
// k = nt % NGR, lr = d % 16, lq = t / 4, e = t % 4, it is
// (c*64 + lq*16 + lr)*16 + (4k + e)*ELEM, i.e. chunk c, lane 16*lq + lr holds
// tokens 4lq .. 4lq+3 of dims 16*(NGR*c + k) + lr for k < NGR.
template <int KV, int D, int BS>
__device__ __forceinline__ int v_elem_offset(int t, int d) {
  using C = Cfg<KV, D, BS>;
  const int nt = d >> 4, c = nt / C::NGR, k = nt % C::NGR;
  return ((c * 64 + (t >> 2) * 16 + (d & 15)) * 16) + (4 * k + (t & 3)) * C::ELEM;
}

// Store one appended value code of `ELEM` bytes (a piece of a 16-byte row)
// into the pool.  The appended rows go out as nontemporal stores: within a
// step no other wavefront reads the new slot (the appending one patches it
// into its own registers).  Measured against plain stores (same box, two runs
// each, attention us): the mixed B=512 workload 2324 -> 2281, the
// Llama-3-8B-shaped B=64 one 50.1 -> 49.4, the 70B-shaped and fp8 workloads
// unchanged.
template <int ELEM>
__device__ __forceinline__ void store_pool(char* dst, uint32_t code) {
  if constexpr (ELEM == 4) __builtin_nontemporal_store(code, reinterpret_cast<uint32_t*>(dst));
  else if constexpr (ELEM == 2) __builtin_nontemporal_store((uint16_t)code, reinterpret_cast<uint16_t*>(dst));
  else __builtin_nontemporal_store((uint8_t)code, reinterpret_cast<uint8_t*>(dst));
}

template <int KCH>
struct TileRegs {
  u32x4_t k[KCH];
  u32x4_t v[KCH];
};

// Query operand of the score MFMA: the rotated query of head lr (zero if
// lr >= G) at the dims lane (lr, lq) contracts over in chunk c.
template <int KV, int KCH> struct QOp;
template <int KCH> struct QOp<KV_BF16, KCH> { bf16x8_t v[KCH]; };
template <int KCH> struct QOp<KV_FP8, KCH>  { f16x8_t v[KCH][2]; };
template <int KCH> struct QOp<KV_F32, KCH>  { float v[KCH][4]; };

// Position in the concatenation of the wave's sequences (wave-uniform).
// Tiles are counted from the first one the sequence reads (lo, the first
// tile of its attention window, 0 without one): tile j of the walk is tile
// lo + j of the request's context.
struct Walk {
  int b, h, j, n;   // request, KV head, tile in the sequence, tiles of the sequence
  int lo;           // first tile of the request's context that is read
};

__device__ __forceinline__ void walk_next(Walk& w, const int* sP, const int* sLo, int B, int hkv,
                                          int cost) {
  if (++w.j == w.n) {
    w.j = 0;
    if (++w.h == hkv) {
      w.h = 0;
      if (++w.b < B) {
        w.n = uniform(tiles_per_seq(sP, w.b, hkv, cost));
        w.lo = uniform(sLo[w.b]);
      }
    }
  }
}

// ---------------------------------------------------------------- kernel
// MQ: every request brings n_qtok > 1 new tokens (appended beforehand by
// decode_append_kernel); MFMA column lr = qi * G + g holds query head g of new
// token qi, which attends causally to the tokens [0, L - n_qtok + qi].
// LO: a bf16 cache, one new token, G <= 8: the MFMA columns g + 8 carry the
// bf16 low parts of column g's query and probabilities (see lo_cols).
template <int KV, int D, int BS, bool MQ, bool LO>
__global__ __launch_bounds__(kBlockThreads)
__attribute__((amdgpu_waves_per_eu(PKV_WAVES_PER_EU, PKV_WAVES_PER_EU)))
void decode_attn_kernel(DecodeParams p, const int32_t* __restrict__ tables,
                        const int32_t* __restrict__ lens, const int32_t* __restrict__ poss,
                        char* __restrict__ kpool, char* __restrict__ vpool) {
  using C = Cfg<KV, D, BS>;
  constexpr int R = C::RING;
  constexpr int PF = partial_floats(D);
  __shared__ int sP[kMaxBatch + 1];
  __shared__ int sLo[kMaxBatch];       // first tile each request reads (its window's)
  __shared__ int sWsum[kBlockThreads / 64];
  __shared__ u32x4_t sKrow[kBlockThreads / 64][C::KROWS];   // appended key row
  __shared__ uint32_t sVrow[kBlockThreads / 64][D];          // appended value codes
  // Per-wavefront queue of deferred global writes.  On gfx950 stores and
  // loads share one completion counter and may complete out of order with
  // respect to each other, so the first wait for a tile load after any store
  // has to drain every load in flight.  Writes made inside the tile loop are
  // therefore parked here and issued once the wavefront's tiles are done; a
  // write that does not fit is made at once.  Items: a 16-byte header
  // {type | words << 4, request * Hkv + head, block, slot of the new token}
  // and `words` 16-byte payload words.
  constexpr int QW = PKV_QUEUE_BYTES / 16;
  __shared__ u32x4_t sQ[kBlockThreads / 64][QW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  PKV_STAMP(0);
  const int B = p.batch, hkv = p.n_kv_heads, G = p.group;
  const int TQ = MQ ? p.n_qtok : 1;           // new tokens per request
  const int NC = G * TQ;                      // MFMA columns in use (<= 16)
  // Low parts.  With a bf16 cache the rotated query and the probabilities
  // enter the matrix cores rounded to bf16, which costs as much accuracy as
  // the final rounding of the output.  When the used columns fit in the
  // first half (NC <= 8), column g + 8 carries the bf16 remainders
  // x - bf16(x) of column g: the score MFMA then gives both lanes of a pair
  // the two halves of the score, one row rotation adds them, both lanes run
  // the same softmax, and the P V MFMA accumulates the high parts of the
  // probabilities in column g and the low parts in column g + 8, which are
  // added once at the end of the piece.
  static_assert(!LO || (KV == KV_BF16 && !MQ), "low parts: bf16 cache, one new token");
  constexpr bool lo_cols = LO;                     // the host launches LO only for G <= 8
  const int qcol = lr < NC ? lr : ((lo_cols && lr >= 8 && lr < 8 + NC) ? lr - 8 : -1);
  const bool lo_lane = lo_cols && qcol >= 0 && lr >= 8;   // carries the low parts of column qcol
  const int lane_qi = MQ ? (qcol < 0 ? 0 : qcol) / G : 0;   // new token of this lane's column
  const int cap = p.max_blocks * BS;

  const int cost = p.piece_cost;
  // ---- work units per request (hkv sequences of tiles + cost each),
  // prefix-summed into LDS (every workgroup).  Up to 64 requests, every
  // wavefront builds the whole table itself, one request per lane with a
  // wave-wide prefix sum, and reads back only what it wrote itself, so no
  // workgroup barrier holds it back (the four write the same values).
  int lane_p = 0;                      // with B <= 64: P[lane], the first unit of request lane
  if (B <= 64) {
    int u = 0;
    if (lane < B) {
      const int Li = lens[lane];
      const int lo = window_first_tile(Li, cap, p.window);
      u = hkv * (tiles_of(Li, cap) - lo + cost);
      sLo[lane] = lo;
    }
    int incl = u;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    lane_p = incl - u;
    if (lane < B) sP[lane] = lane_p;
    if (lane == B - 1) sP[B] = incl;
  } else {
    for (int i = tid; i < B; i += kBlockThreads) {
      const int Li = lens[i];
      const int lo = window_first_tile(Li, cap, p.window);
      sLo[i] = lo;
      sP[i] = hkv * (tiles_of(Li, cap) - lo + cost);
    }
    __syncthreads();
    const int per = (B + kBlockThreads - 1) / kBlockThreads;
    const int i0 = tid * per;
    int sum = 0;
    for (int i = 0; i < per; ++i)
      if (i0 + i < B) sum += sP[i0 + i];
    int incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    if (lane == 63) sWsum[wid] = incl;
    __syncthreads();
    int run = incl - sum;
    for (int w = 0; w < wid; ++w) run += sWsum[w];
    for (int i = 0; i < per; ++i) {
      if (i0 + i < B) {
        const int v = sP[i0 + i];
        sP[i0 + i] = run;
        run += v;
      }
    }
    if (tid == kBlockThreads - 1) sP[B] = run;
    __syncthreads();
  }
  PKV_STAMP(1);

  // work units (< 2^31, checked on the host); U and W live in scalar
  // registers through the tile loop
  const int64_t U = uniform(sP[B]);
  const WaveWeights ww = weights_for(U, p.n_waves, p.weight_min_share,
                                     WaveWeights{p.weight_first, p.weight_rest, p.n_first, p.weight_odd});
  const int64_t W = uniform((int)active_waves(U, p.n_waves, p.min_units, cost, ww));
  const int wave = uniform(blockIdx.x * (kBlockThreads / 64) + wid);
#ifdef PKV_TIMELINE
  auto record = [&](uint64_t s1, uint64_t s2, uint64_t s3, uint64_t s4, uint64_t s5, int tiles)
      __attribute__((always_inline)) {
    if (lane == 0 && p.timeline) {
      uint64_t* r = p.timeline + (int64_t)wave * 8;
      r[0] = stamp0; r[1] = s1; r[2] = s2; r[3] = s3; r[4] = s4; r[5] = s5;
      r[6] = (uint64_t)tiles;
      r[7] = (uint64_t)(uint32_t)__builtin_amdgcn_s_getreg((31 << 11) | 4) |      // HW_ID
             ((uint64_t)(uint32_t)__builtin_amdgcn_s_getreg((31 << 11) | 20) << 32);   // XCC_ID
    }
  };
#define PKV_RECORD_IDLE() record(stamp0, stamp0, stamp0, stamp0, stamp0, 0)
#else
#define PKV_RECORD_IDLE()
#endif
  if (wave >= W) {
    if (lane == 0) p.headers[wave] = make_int4(0, 0, 0, 0);
    PKV_RECORD_IDLE();
    return;
  }
  // The wave's tiles: those whose first unit lies in its unit range.
  Walk w0;
  int T;
  {
    // Even lanes work out where the range starts and odd lanes where it ends
    // (the next wavefront's start), side by side in one instruction stream.
    const int end = lane & 1;
    const int64_t x = wave_start(wave + end, U, W, ww);
    int64_t g = (int64_t)sP[B] - (int64_t)hkv * cost * B;        // all tiles
    // With B <= 64 the request holding unit x is found with one ballot per
    // end over the lanes' P[lane] (the units are below 2^31): the number of
    // requests whose first unit is <= x, less one.  Else a binary search.
    int rq = 0;
    if (B <= 64) {
      const int x0 = __builtin_amdgcn_readlane((int)x, 0), x1 = __builtin_amdgcn_readlane((int)x, 1);
      const int n0 = __popcll(__ballot(lane < B && lane_p <= x0));
      const int n1 = __popcll(__ballot(lane < B && lane_p <= x1));
      rq = (end ? n1 : n0) - 1;
    }
    TilePos t = {0, 0, 0, 1};
    if (x < U) {
      t = B <= 64 ? tile_in_request(sP, rq, hkv, cost, x) : tile_at_unit(sP, B, hkv, cost, x);
      g = global_tile(sP, t.b, t.h, t.j, t.n, hkv, cost);
    }
    const int g0 = __builtin_amdgcn_readlane((int)g, 0);     // tile counts < 2^31
    const int g1 = __builtin_amdgcn_readlane((int)g, 1);
    T = g1 - g0;
    w0.b = __builtin_amdgcn_readlane(t.b, 0);
    w0.h = __builtin_amdgcn_readlane(t.h, 0);
    w0.j = __builtin_amdgcn_readlane(t.j, 0);
    w0.n = __builtin_amdgcn_readlane(t.n, 0);
    if (T > 0 && w0.j == w0.n) {        // the range begins at the next sequence
      w0.j = 0;
      if (++w0.h == hkv) {
        w0.h = 0;
        ++w0.b;
        w0.n = uniform(tiles_per_seq(sP, w0.b, hkv, cost));
      }
    }
    w0.lo = w0.b < B ? uniform(sLo[w0.b]) : 0;
  }
  if (T <= 0) {
    if (lane == 0) p.headers[wave] = make_int4(0, 0, 0, 0);
    PKV_RECORD_IDLE();
    return;
  }
  PKV_STAMP(2);

  const int lane16 = lane * 16;
  const char* dummy = static_cast<const char*>(p.dummy);
  uint32_t bad_block = 0;

  // ---- prefetch side: RING tiles in flight
  TileRegs<C::KCH> ring[R];
  Walk pw = w0;
  int p_left = T;
  auto load_blk = [&](const Walk& w) __attribute__((always_inline)) -> int {
    return tables[(int64_t)w.b * p.max_blocks + ((w.j + w.lo) >> C::LOG2TPB)];
  };
  int pf_blk = load_blk(pw);
  int64_t pf_off = 0;
  bool pf_live = false;

  auto issue_k = [&](TileRegs<C::KCH>& t) __attribute__((always_inline)) {
    pf_live = p_left > 0;
    int blk = pf_blk;
    if ((unsigned)blk >= (unsigned)p.num_blocks) {
      bad_block |= pf_live ? 1u : 0u;
      blk = 0;
    }
    pf_off = (((int64_t)blk * hkv + pw.h) * C::TPB + ((pw.j + pw.lo) & (C::TPB - 1))) * C::TILE_BYTES;
    const char* base = pf_live ? kpool + pf_off : dummy;
#pragma unroll
    for (int c = 0; c < C::KCH; ++c)
      t.k[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(base + c * 1024 + lane16));
  };
  auto issue_v = [&](TileRegs<C::KCH>& t) __attribute__((always_inline)) {
    const char* base = pf_live ? vpool + pf_off : dummy;
#pragma unroll
    for (int c = 0; c < C::KCH; ++c)
      t.v[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(base + c * 1024 + lane16));
    if (pf_live) {
      --p_left;
      if (p_left > 0) {
        walk_next(pw, sP, sLo, B, hkv, cost);
        pf_blk = load_blk(pw);
      }
    }
  };

  static_for([&](auto U) __attribute__((always_inline)) {
    issue_k(ring[decltype(U)::value]);
    issue_v(ring[decltype(U)::value]);
  }, std::make_integer_sequence<int, R>{});

  // ---- consumer side
  Walk cw = w0;
  QOp<KV, C::KCH> qop;
  f32x4_t acc[C::NT];
  float m_run = -INFINITY, l_run = 0.f;
  float sscale = p.sm_scale_log2, vsc = 1.0f;
  int L = 1, pend = 1, slot = 0;
  int lo_tok = 0;      // first token of the attention window
  bool split = false, app = false;
  int r0 = 0;
  uint32_t bad_len = 0, bad_pos = 0;
  int j0 = 0;
  // the split sequence whose first piece this wavefront holds (its last piece)
  // (request, KV head, tiles, partial slot): its piece count is worked out
  // after the tile loop, where its divisions cost no registers
  int4 split_seq = make_int4(-1, 0, 0, 0);

  const int64_t out_row_stride = (int64_t)hkv * G;   // query heads per request

  enum : uint32_t { Q_OUT = 0, Q_APPEND = 1, Q_PART = 2 };
  constexpr int IO_BYTES = C::IO_BF16 ? 2 : 4;
  const int out_words = NC * D * IO_BYTES / 16;           // G output rows per new token
  constexpr int app_words = C::KROWS + D / 4;             // key row + value codes (u32)
  const int part_words = NC * D / 4 + (NC + 1) / 2;       // [column][dim] accumulators + (m, l)
  int q_used = 0;      // words of sQ[wid] in use
  uint32_t* const sQw = reinterpret_cast<uint32_t*>(&sQ[wid][0]);

  // Room for an item of `words` payload words: the word index of its
  // header, or -1 (the write is then made at once).
  auto q_reserve = [&](int words) __attribute__((always_inline)) -> int {
    if (q_used + 1 + words > QW) return -1;
    const int at = q_used;
    q_used += 1 + words;
    return at;
  };
  auto q_header = [&](int at, uint32_t type, int words, int seq, int blk, int r) __attribute__((always_inline)) {
    if (lane == 0) {
      u32x4_t hd;
      hd[0] = type | ((uint32_t)words << 4);
      hd[1] = (uint32_t)seq;
      hd[2] = (uint32_t)blk;
      hd[3] = (uint32_t)r;
      sQ[wid][at] = hd;
    }
  };
  // Global writes of the appended rows (codes as u32 per value dim), as
  // nontemporal stores (store_pool).
  auto write_append = [&](int h, int blk, int r, const u32x4_t* krow, const uint32_t* vcodes)
      __attribute__((always_inline)) {
    const int64_t toff = (((int64_t)blk * hkv + h) * C::TPB + ((r / kTileTokens) & (C::TPB - 1))) *
                         C::TILE_BYTES;
    const int r16 = r & 15;
    if (lane < C::KROWS)
      __builtin_nontemporal_store(krow[lane], reinterpret_cast<u32x4_t*>(kpool + toff + (lane * 16 + r16) * 16));
#pragma unroll
    for (int k = 0; k < D / 64; ++k) {
      const int d = lane + 64 * k;
      store_pool<C::ELEM>(vpool + toff + v_elem_offset<KV, D, BS>(r16, d), vcodes[d]);
    }
  };

  auto begin_piece = [&](int i) __attribute__((always_inline)) {
    const int b = cw.b, h = cw.h;
    const int Lraw = lens[b];
    int posn = poss[b];
    const bool len_ok = Lraw >= 1 && Lraw <= cap;
    const bool pos_ok = posn >= 0 && posn + TQ - 1 < p.max_pos;
    bad_len |= len_ok ? 0u : 1u;
    bad_pos |= pos_ok ? 0u : 1u;
    posn = posn < 0 ? 0 : (posn + TQ - 1 >= p.max_pos ? p.max_pos - TQ : posn);
    L = Lraw < 0 ? 0 : (Lraw > cap ? cap : Lraw);
    lo_tok = (p.window > 0 && L > p.window) ? L - p.window : 0;
    j0 = cw.j;
    pend = min(cw.n, j0 + (T - i));
    split = j0 > 0 || pend < cw.n;
    slot = i == 0 ? 0 : 1;
    app = !MQ && len_ok && pend == cw.n;

    // Rotated query of column lr at this lane's dims (fp32 RoPE from the
    // table): head g of new token qi (lr = qi * G + g) at position posn + qi.
    // Columns past the last load column 0 and are zeroed.
    const int col = qcol < 0 ? 0 : qcol;
    const int hq = h * G + (col - lane_qi * G);
    const bool hvalid = qcol >= 0;
    const int64_t qrow = (((int64_t)b * TQ + lane_qi) * out_row_stride + hq) * D;
    const float* crow = p.rope_cos + (int64_t)(posn + lane_qi) * C::HALF;
    const float* srow = p.rope_sin + (int64_t)(posn + lane_qi) * C::HALF;
    // Chunks c and c + KCH/2 hold the two halves of the rotate-half pairs
    // (dims d and d + D/2) and share one row of the cos/sin table; with a
    // single chunk, lanes lq < 2 hold the lower half and lq >= 2 the upper.
    constexpr int NPAIR = C::KCH >= 2 ? C::KCH / 2 : 1;
    auto rotate_pair = [&](int c, float (&y0)[C::X], float (&y1)[C::X]) __attribute__((always_inline)) {
      float x[C::X], xp[C::X], cs[C::X], sn[C::X];
      if constexpr (C::KCH >= 2) {
        const int d0 = C::X * (4 * c + lq);
        load_row_f32<C::IO_BF16, C::X>(p.q, qrow + d0, x);
        load_row_f32<C::IO_BF16, C::X>(p.q, qrow + d0 + C::HALF, xp);
        load_f32<C::X>(crow + d0, cs);
        load_f32<C::X>(srow + d0, sn);
#pragma unroll
        for (int e = 0; e < C::X; ++e) {
          y0[e] = hvalid ? x[e] * cs[e] - xp[e] * sn[e] : 0.0f;
          y1[e] = hvalid ? xp[e] * cs[e] + x[e] * sn[e] : 0.0f;
        }
      } else {
        const int d0 = C::X * lq;
        const bool lo = d0 < C::HALF;
        const int pd0 = lo ? d0 + C::HALF : d0 - C::HALF;
        const int i0 = lo ? d0 : pd0;
        load_row_f32<C::IO_BF16, C::X>(p.q, qrow + d0, x);
        load_row_f32<C::IO_BF16, C::X>(p.q, qrow + pd0, xp);
        load_f32<C::X>(crow + i0, cs);
        load_f32<C::X>(srow + i0, sn);
#pragma unroll
        for (int e = 0; e < C::X; ++e) {
          const float y = lo ? (x[e] * cs[e] - xp[e] * sn[e]) : (x[e] * cs[e] + xp[e] * sn[e]);
          y0[e] = hvalid ? y : 0.0f;
          y1[e] = 0.0f;
        }
      }
    };
    sscale = p.sm_scale_log2;
    vsc = 1.0f;
    if constexpr (KV == KV_BF16) {
#pragma unroll
      for (int c = 0; c < NPAIR; ++c) {
        float y0[C::X], y1[C::X];
        rotate_pair(c, y0, y1);
        u32x4_t w0, w1;
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          w0[i2] = pack_bf16x2(y0[2 * i2], y0[2 * i2 + 1]);
          w1[i2] = pack_bf16x2(y1[2 * i2], y1[2 * i2 + 1]);
          if (lo_cols && lo_lane) {   // the remainders (exact in fp32), rounded to bf16
            w0[i2] = pack_bf16x2(y0[2 * i2] - __uint_as_float(w0[i2] << 16),
                                 y0[2 * i2 + 1] - __uint_as_float(w0[i2] & 0xffff0000u));
            w1[i2] = pack_bf16x2(y1[2 * i2] - __uint_as_float(w1[i2] << 16),
                                 y1[2 * i2 + 1] - __uint_as_float(w1[i2] & 0xffff0000u));
          }
        }
        qop.v[c] = __builtin_bit_cast(bf16x8_t, w0);
        if constexpr (C::KCH >= 2) qop.v[c + NPAIR] = __builtin_bit_cast(bf16x8_t, w1);
      }
    } else if constexpr (KV == KV_FP8) {
      // The query is scaled by a power of two so that it fits f16 with room
      // to spare; the factor goes back into the score scale, with the K
      // scale.  A rotation keeps each pair's norm, so
      // |rotated| <= sqrt(2) * max |raw| bounds the scale from the raw row
      // before anything is rotated.
      float amax = 0.f;
      {
        const int d0 = C::X * lq;
#pragma unroll
        for (int c = 0; c < C::KCH; ++c) {
          float x[C::X];
          load_row_f32<C::IO_BF16, C::X>(p.q, qrow + d0 + 4 * C::X * c, x);
#pragma unroll
          for (int e = 0; e < C::X; ++e) amax = fmaxf(amax, fabsf(x[e]));
        }
      }
      amax = max_over_lq(amax) * 1.4142137f;
      int ex = 0;
      if (amax > 0.f) {
        (void)__builtin_frexpf(amax, &ex);   // amax < 2^ex
        ex = ex > 15 ? ex - 15 : 0;
      }
      const float qs = __builtin_ldexpf(1.0f, -ex);
      sscale = p.sm_scale_log2 * p.fp8_scales[h] * __builtin_ldexpf(1.0f, ex);
      vsc = p.fp8_scales[hkv + h];
#pragma unroll
      for (int c = 0; c < NPAIR; ++c) {
        float y0[C::X], y1[C::X];
        rotate_pair(c, y0, y1);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          u32x4_t w0, w1;
#pragma unroll
          for (int i2 = 0; i2 < 4; ++i2) {
            w0[i2] = pack_f16x2(y0[8 * hh + 2 * i2] * qs, y0[8 * hh + 2 * i2 + 1] * qs);
            w1[i2] = pack_f16x2(y1[8 * hh + 2 * i2] * qs, y1[8 * hh + 2 * i2 + 1] * qs);
          }
          qop.v[c][hh] = __builtin_bit_cast(f16x8_t, w0);
          if constexpr (C::KCH >= 2) qop.v[c + NPAIR][hh] = __builtin_bit_cast(f16x8_t, w1);
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < NPAIR; ++c) {
        float y0[C::X], y1[C::X];
        rotate_pair(c, y0, y1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qop.v[c][e] = y0[e];
          if constexpr (C::KCH >= 2) qop.v[c + NPAIR][e] = y1[e];
        }
      }
    }

    // Append of the new token (slot L-1), when this piece ends the sequence.
    // The rotated key uses the pinned fp32 arithmetic: two separate
    // multiplies and one add or subtract, no contraction.  Both rows go to
    // the pool and to LDS; the tile registers get them at the last tile, so
    // it does not matter whether that tile's loads left before or after
    // these stores.
    // An out-of-range block id for the new token's slot raises the flag and
    // skips the append: nothing is written to another block, and the
    // request's output is garbage (its last tile was read from block 0).
    int blk = 0;
    if (app) {
      blk = tables[(int64_t)b * p.max_blocks + (L - 1) / BS];
      if ((unsigned)blk >= (unsigned)p.num_blocks) {
        bad_block |= 1u;
        app = false;
      }
    }
    if (app) {
      r0 = (L - 1) & 15;
      const int64_t nrow = ((int64_t)b * hkv + h) * D;
      float inv_k = 1.0f, inv_v = 1.0f;
      if constexpr (KV == KV_FP8) {
        inv_k = p.fp8_scales[2 * hkv + h];
        inv_v = p.fp8_scales[3 * hkv + h];
      }
      if (lane < C::KROWS) {
        const int d0 = C::X * lane;
        const bool lo = d0 < C::HALF;
        const int pd0 = lo ? d0 + C::HALF : d0 - C::HALF;
        const int i0 = lo ? d0 : pd0;
        float x[C::X], xp[C::X], cs[C::X], sn[C::X];
        load_row_f32<C::IO_BF16, C::X>(p.k_new, nrow + d0, x);
        load_row_f32<C::IO_BF16, C::X>(p.k_new, nrow + pd0, xp);
        load_f32<C::X>(crow + i0, cs);
        load_f32<C::X>(srow + i0, sn);
        uint32_t enc[C::X];
#pragma unroll
        for (int e = 0; e < C::X; ++e) {
          const float a = x[e] * cs[e];
          const float bb = xp[e] * sn[e];
          const float y = lo ? a - bb : a + bb;
          enc[e] = encode_kv<KV>(y, inv_k);
        }
        u32x4_t row;
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          uint32_t w = 0;
#pragma unroll
          for (int k = 0; k < 4 / C::ELEM; ++k) w |= enc[i2 * (4 / C::ELEM) + k] << (k * C::ELEM * 8);
          row[i2] = w;
        }
        sKrow[wid][lane] = row;
      }
#pragma unroll
      for (int k = 0; k < D / 64; ++k) {
        const int d = lane + 64 * k;
        const uint32_t code = encode_kv<KV>(load_io<C::IO_BF16>(p.v_new, nrow + d), inv_v);
        sVrow[wid][d] = code;
      }
      // the global write of the rows: queued (a copy), or made now
      const int at = q_reserve(app_words);
      const int r = (L - 1) & (BS - 1);
      if (at >= 0) {
        q_header(at, Q_APPEND, app_words, b * hkv + h, blk, r);
        if (lane < C::KROWS) sQ[wid][at + 1 + lane] = sKrow[wid][lane];
#pragma unroll
        for (int k = 0; k < D / 64; ++k) sQw[(at + 1 + C::KROWS) * 4 + lane + 64 * k] = sVrow[wid][lane + 64 * k];
      } else {
        write_append(h, blk, r, &sKrow[wid][0], &sVrow[wid][0]);
        wait_vector_memory();
      }
    }
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  };

  // Put the appended token into the registers of the sequence's last tile.
  auto patch = [&](TileRegs<C::KCH>& t) __attribute__((always_inline)) {
    if (lr == r0) {
#pragma unroll
      for (int c = 0; c < C::KCH; ++c) t.k[c] = sKrow[wid][4 * c + lq];
    }
    if (lq == (r0 >> 2)) {
      const int e0 = r0 & 3;
#pragma unroll
      for (int c = 0; c < C::KCH; ++c)
#pragma unroll
        for (int k = 0; k < C::NGR; ++k) {
          const uint32_t code = sVrow[wid][16 * (C::NGR * c + k) + lr];
          const int byte = (4 * k + e0) * C::ELEM;
          const int word = byte >> 2, sh = (byte & 3) * 8;
          const uint32_t m = C::ELEM == 4 ? 0xffffffffu : ((1u << (8 * C::ELEM)) - 1u) << sh;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (q == word) t.v[c][q] = (t.v[c][q] & ~m) | ((code << sh) & m);
        }
    }
  };

  auto scores = [&](const TileRegs<C::KCH>& t) __attribute__((always_inline)) -> f32x4_t {
    f32x4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < C::KCH; ++c) {
      if constexpr (KV == KV_BF16) {
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, t.k[c]),
                                                    qop.v[c], a, 0, 0, 0);
      } else if constexpr (KV == KV_FP8) {
        f16x8_t lo, hi;
        fp8x16_to_f16(t.k[c], lo, hi);
        a = __builtin_amdgcn_mfma_f32_16x16x32_f16(lo, qop.v[c][0], a, 0, 0, 0);
        a = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi, qop.v[c][1], a, 0, 0, 0);
      } else {
        const f32x4_t kf = __builtin_bit_cast(f32x4_t, t.k[c]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          a = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[e], qop.v[c][e], a, 0, 0, 0);
      }
    }
    return a;
  };

  // Online softmax over the tile (log2 domain) and P V.  On the sequence's
  // last tile, tokens at or past L, and on the first tile of an attention
  // window, tokens before it get score -inf (selected, never multiplied) and
  // their values are zeroed, whatever the slots hold.
  auto softmax_pv = [&](f32x4_t a, TileRegs<C::KCH>& t, bool last) __attribute__((always_inline)) {
    float s[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (lo_cols) a[r] += swap_half_row(a[r]);   // the other half of the score
      s[r] = a[r] * sscale;
    }
    if (last || (cw.j == 0 && lo_tok > 16 * cw.lo) ||
        (MQ && 16 * (cw.j + cw.lo + 1) > L - TQ)) {
      const int t0 = 16 * (cw.j + cw.lo) + 4 * lq;   // token of this lane's first score
      const int nv = L - t0;                         // its tokens r < nv are in the context
      const int nlo = lo_tok - t0;                   // and those r >= nlo in the window
      // and those r < nc are visible to the column's new token (causal)
      const int nc = MQ ? L - TQ + lane_qi + 1 - t0 : nv;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (r >= nc || r < nlo) s[r] = -INFINITY;
      u32x4_t keep;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t m = 0;
#pragma unroll
        for (int by = 0; by < 4; ++by) {
          const int e = ((4 * q + by) % (4 * C::ELEM)) / C::ELEM;   // token of byte
          m |= (e < nv && e >= nlo) ? (0xffu << (8 * by)) : 0u;
        }
        keep[q] = m;
      }
#pragma unroll
      for (int c = 0; c < C::KCH; ++c) t.v[c] &= keep;
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = max_over_lq(mx);
    const float m_new = fmaxf(m_run, mx);
    const float mb = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = exp2_fast(m_run - mb);
    m_run = m_new;
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = exp2_fast(s[r] - mb);
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) acc[nt] *= alpha;

    // The normaliser sums the probabilities as the P V product sees them
    // (rounded to bf16 or f16 for the matrix cores), so that the output's
    // weights sum to one exactly.
    if constexpr (KV == KV_BF16) {
      u32x2_t pw2;
      pw2[0] = pack_bf16x2(s[0], s[1]);
      pw2[1] = pack_bf16x2(s[2], s[3]);
      const float h0 = __uint_as_float(pw2[0] << 16), h1 = __uint_as_float(pw2[0] & 0xffff0000u);
      const float h2 = __uint_as_float(pw2[1] << 16), h3 = __uint_as_float(pw2[1] & 0xffff0000u);
      // with low parts, the two columns of a pair together carry p to 16
      // bits: the normaliser sums p itself; without, the rounded p
      const float ps = lo_cols ? (s[0] + s[1]) + (s[2] + s[3]) : (h0 + h1) + (h2 + h3);
      l_run = __builtin_fmaf(l_run, alpha, ps);
      if (lo_cols && lo_lane) {
        pw2[0] = pack_bf16x2(s[0] - h0, s[1] - h1);
        pw2[1] = pack_bf16x2(s[2] - h2, s[3] - h3);
      }
      const s16x4_t pb = __builtin_bit_cast(s16x4_t, pw2);
#pragma unroll
      for (int c = 0; c < C::KCH; ++c)
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          u32x2_t vw;
          vw[0] = t.v[c][2 * k];
          vw[1] = t.v[c][2 * k + 1];
          acc[2 * c + k] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
              __builtin_bit_cast(s16x4_t, vw), pb, acc[2 * c + k], 0, 0, 0);
        }
    } else if constexpr (KV == KV_FP8) {
      u32x2_t pw2;
      pw2[0] = pack_f16x2(s[0], s[1]);
      pw2[1] = pack_f16x2(s[2], s[3]);
      const f16x4_t ph = __builtin_bit_cast(f16x4_t, pw2);
      const float ps = ((float)ph[0] + (float)ph[1]) + ((float)ph[2] + (float)ph[3]);
      l_run = __builtin_fmaf(l_run, alpha, ps);
#pragma unroll
      for (int c = 0; c < C::KCH; ++c)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          acc[4 * c + k] = __builtin_amdgcn_mfma_f32_16x16x16f16(fp8x4_to_f16x4(t.v[c][k]), ph,
                                                                 acc[4 * c + k], 0, 0, 0);
    } else {
      l_run = __builtin_fmaf(l_run, alpha, (s[0] + s[1]) + (s[2] + s[3]));
#pragma unroll
      for (int c = 0; c < C::KCH; ++c) {
        const f32x4_t vf = __builtin_bit_cast(f32x4_t, t.v[c]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[e], s[e], acc[c], 0, 0, 0);
      }
    }
  };

  // The G output rows of sequence (b, h), normalised and cast: queued as
  // an item laid out like the rows in memory ([head][dim]), or stored now.
  auto store_out = [&](int b, int h, const f32x4_t (&o)[C::NT], float scale) __attribute__((always_inline)) {
    const int at = q_reserve(out_words);
    if (at >= 0) q_header(at, Q_OUT, out_words, b * hkv + h, 0, 0);
    if (lr >= NC) return;
    const int64_t row = (((int64_t)b * TQ + lane_qi) * out_row_stride + h * G + (lr - lane_qi * G)) * D;
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
      const int d = 16 * nt + 4 * lq;
      const int e = (at + 1) * (16 / IO_BYTES) + lr * D + d;     // io element index in sQ[wid]
      if constexpr (C::IO_BF16) {
        u32x2_t w;
        w[0] = bf16_rne(o[nt][0] * scale) | (bf16_rne(o[nt][1] * scale) << 16);
        w[1] = bf16_rne(o[nt][2] * scale) | (bf16_rne(o[nt][3] * scale) << 16);
        if (at >= 0) *reinterpret_cast<u32x2_t*>(sQw + e / 2) = w;
        else *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(p.out) + row + d) = w;
      } else {
        if (at >= 0) *reinterpret_cast<f32x4_t*>(sQw + e) = o[nt] * scale;
        else *reinterpret_cast<f32x4_t*>(static_cast<float*>(p.out) + row + d) = o[nt] * scale;
      }
    }
    if (at < 0) wait_vector_memory();
  };

  auto end_piece = [&]() __attribute__((always_inline)) {
    if constexpr (lo_cols) {   // column g + 8 holds the low-part products of column g
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[nt][r] += swap_half_row(acc[nt][r]);
    }
    const float lt = sum_over_lq(l_run);
    if (!split) {
      store_out(cw.b, cw.h, acc, lt > 0.f ? vsc / lt : 0.f);
      return;
    }
    // The wavefront's first piece is queued (more tiles follow); its last
    // piece ends its tiles and is stored now.
    const int at = slot == 0 ? q_reserve(part_words) : -1;
    if (at >= 0) {
      q_header(at, Q_PART, part_words, cw.b * hkv + cw.h, 0, 0);
      if (lr < NC) {
        f32x4_t* accq = reinterpret_cast<f32x4_t*>(&sQ[wid][at + 1]);
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) accq[(lr * D + 16 * nt + 4 * lq) / 4] = acc[nt] * vsc;
        if (lq == 0) {
          float* ml = reinterpret_cast<float*>(&sQ[wid][at + 1 + NC * D / 4]);
          ml[2 * lr] = m_run;
          ml[2 * lr + 1] = lt;
        }
      }
    } else {
      float* part = p.partials + ((int64_t)wave * 2 + slot) * PF;
      if (lr < NC) {
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt)
          *reinterpret_cast<f32x4_t*>(part + lr * D + 16 * nt + 4 * lq) = acc[nt] * vsc;
        if (lq == 0) {
          part[16 * D + 2 * lr] = m_run;
          part[16 * D + 2 * lr + 1] = lt;
        }
      }
      wait_vector_memory();
    }
    if (j0 == 0) split_seq = make_int4(cw.b, cw.h, cw.n, slot);
  };

  PKV_STAMP(3);
  // ---- main loop: consume tile i from slot i % R, refill it with tile i + R.
  // Loads are issued unconditionally (past the range they read the dummy
  // buffer) so that the wait before each tile is a fixed count of the loads
  // issued after it.
  for (int base = 0; base < T; base += R) {
    {
      const int left8 = (8 * (T - base) + T - 1) / T;    // ceil(8 * tiles left / T)
      set_priority(uniform(left8 > 4 ? 3 : left8 > 2 ? 2 : left8 > 1 ? 1 : 0));
    }
    static_for([&](auto U) __attribute__((always_inline)) {
      constexpr int u = decltype(U)::value;
      const int i = base + u;
      const bool live = i < T;
      if (live && (i == 0 || cw.j == 0)) begin_piece(i);
      const bool last = cw.j == cw.n - 1;
      if (live && last && app) patch(ring[u]);
      const f32x4_t a = scores(ring[u]);
      issue_k(ring[u]);
      softmax_pv(a, ring[u], last);
      issue_v(ring[u]);
      if (live) {
        if (i == T - 1 || last) end_piece();
        walk_next(cw, sP, sLo, B, hkv, cost);
      }
    }, std::make_integer_sequence<int, R>{});
  }

  PKV_STAMP(4);
  // ---- the queued writes, in order
  for (int off = 0; off < q_used;) {
    const u32x4_t hd = sQ[wid][off];
    const uint32_t type = (uint32_t)uniform((int)(hd[0] & 15u));
    const int words = uniform((int)(hd[0] >> 4));
    const int seq = uniform((int)hd[1]);
    const int b = seq / hkv, h = seq - b * hkv;
    const u32x4_t* pl = &sQ[wid][off + 1];
    if (type == Q_OUT) {
      // the G rows of each new token are contiguous in `out`
      const int seg = words / TQ;
      for (int qi = 0; qi < TQ; ++qi) {
        char* dst = static_cast<char*>(p.out) +
                    (((int64_t)b * TQ + qi) * out_row_stride + h * G) * D * IO_BYTES;
        for (int w = lane; w < seg; w += 64)
          *reinterpret_cast<u32x4_t*>(dst + (int64_t)w * 16) = pl[qi * seg + w];
      }
    } else if (type == Q_APPEND) {
      write_append(h, uniform((int)hd[2]), uniform((int)hd[3]), pl,
                   reinterpret_cast<const uint32_t*>(pl + C::KROWS));
    } else {                                   // partial state of the first piece (slot 0)
      float* part = p.partials + (int64_t)wave * 2 * PF;
      for (int w = lane; w < NC * D / 4; w += 64) *reinterpret_cast<u32x4_t*>(part + 4 * w) = pl[w];
      if (lane < NC) {
        const float* ml = reinterpret_cast<const float*>(pl + NC * D / 4);
        part[16 * D + 2 * lane] = ml[2 * lane];
        part[16 * D + 2 * lane + 1] = ml[2 * lane + 1];
      }
    }
    off += 1 + words;
  }

  if (bad_block | bad_len | bad_pos) {
    if (lane == 0) {
      if (bad_block) p.err[0] = 1u;
      if (bad_pos) p.err[1] = 1u;
      if (bad_len) p.err[2] = 1u;
    }
  }

  int4 split_hdr = make_int4(0, 0, 0, 0);
  if (split_seq.x >= 0) {
    const int sb = uniform(split_seq.x), sh = uniform(split_seq.y), sn = uniform(split_seq.z);
    const int64_t last = first_unit(sP, sb, sh, sn - 1, sn, cost);
    const int np = (int)(wave_of_unit(last, U, W, ww) - wave + 1);
    split_hdr = make_int4(1, sb * hkv + sh, np, uniform(split_seq.w));
  }
  if (lane == 0) p.headers[wave] = split_hdr;
#ifdef PKV_TIMELINE
  PKV_STAMP(5);
  record(stamp1, stamp2, stamp3, stamp4, stamp5, T);
#endif
}

// Merge the partial softmax states of each split sequence, found from the
// header its first wavefront left:
// out = sum_k 2^(m_k - M) acc_k / sum_k 2^(m_k - M) l_k,  M = max_k m_k.
// A piece's accumulators are G*D floats in [head][dim] order, 16-byte
// chunks of which lane l takes l + 64c.  Each lane has KC load slots per
// piece and a batch holds 32/KC pieces in flight, with the running maximum
// rescaling the sums between batches.
//
// A sequence of many pieces (a long request spread over many wavefronts)
// would take its merge wavefront one round trip per batch.  From kShareMin
// pieces on (more than one batch), the merge wavefronts of the kHelpers
// wavefronts after its first one, each of which holds only a middle piece of
// it and so has no header of its own, share the work by columns: merge
// wavefront j of the 1 + kHelpers takes the j-th quarter of the chunks of
// every piece and writes those output elements.  No two write the same
// element and none waits for another.  With a quarter of the chunks a lane
// needs nc = 2^lkp slots per piece, and its other slots hold further pieces
// (R = KC / nc per batch slot), whose partial sums are combined at the end.
template <bool IO_BF16, int D, int KC>
__global__ __launch_bounds__(kBlockThreads) void decode_merge_kernel(DecodeParams p) {
  constexpr int PF = partial_floats(D);
  constexpr int PPB = 32 / KC;                  // batch slots of pieces
  constexpr int kHelpers = 3;
  // pieces from which the merge is shared: more than one batch, and enough
  // that wavefronts 1..kHelpers after the first hold middle pieces
  constexpr int kShareMin = PPB + 1 > kHelpers + 2 ? PPB + 1 : kHelpers + 2;
  const int lane = threadIdx.x & 63;
  const int G = p.group, hkv = p.n_kv_heads, TQ = p.n_qtok;
  // With several new tokens per request, merge wavefront mw takes the G
  // columns of new token qi = mw % TQ of the sequence whose header
  // wavefront mw / TQ left, so each merges G columns as with one token.
  const int mw = uniform(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));
  const int w = TQ > 1 ? mw / TQ : mw;
  const int qi = TQ > 1 ? mw - w * TQ : 0;
  // this wavefront's header and the kHelpers before it, in one round trip
  int4 hj[kHelpers + 1];
#pragma unroll
  for (int j = 0; j <= kHelpers; ++j) hj[j] = w - j >= 0 ? p.headers[w - j] : make_int4(0, 0, 0, 0);
  int ws = -1, part = 0, nparts = 1, seq = 0, np = 0, slot0 = 0;
  if (uniform(hj[0].x)) {
    ws = w;
    seq = uniform(hj[0].y);
    np = uniform(hj[0].z);
    slot0 = uniform(hj[0].w);
    nparts = np >= kShareMin ? kHelpers + 1 : 1;
  } else {
#pragma unroll
    for (int j = 1; j <= kHelpers; ++j) {
      if (ws < 0 && uniform(hj[j].x) && uniform(hj[j].z) >= kShareMin) {
        ws = w - j;
        part = j;
        nparts = kHelpers + 1;
        seq = uniform(hj[j].y);
        np = uniform(hj[j].z);
        slot0 = uniform(hj[j].w);
      }
    }
  }
  if (ws < 0) return;
  const int b = seq / hkv, h = seq - (seq / hkv) * hkv;
  const int nchunk = G * D / 4;               // query head x D of new token qi (a multiple of 16)
  const int cbase = qi * nchunk;              // its first chunk in a piece
  // piece pc's partial state: slot slot0 of wavefront ws for pc = 0, slot 0
  // of wavefront ws + pc after it
  const float* part0 = p.partials + (int64_t)ws * 2 * PF;
  auto piece = [&](int pc) __attribute__((always_inline)) -> const float* {
    return part0 + (pc == 0 ? slot0 * PF : pc * (2 * PF));
  };
  auto write_out = [&](int c, const f32x4_t& nsum, float dsum) __attribute__((always_inline)) {
    const float inv = dsum > 0.f ? 1.0f / dsum : 0.f;
    const int hc = (4 * c) / D;
    const int d = 4 * c - hc * D;
    const int64_t row = (((int64_t)b * TQ + qi) * hkv * G + h * G + hc) * D;
    if constexpr (IO_BF16) {
      u32x2_t o;
      o[0] = bf16_rne(nsum[0] * inv) | (bf16_rne(nsum[1] * inv) << 16);
      o[1] = bf16_rne(nsum[2] * inv) | (bf16_rne(nsum[3] * inv) << 16);
      *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(p.out) + row + d) = o;
    } else {
      *reinterpret_cast<f32x4_t*>(static_cast<float*>(p.out) + row + d) = nsum * inv;
    }
  };
  float M[KC], den[KC];
  f32x4_t num[KC];
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    M[k] = -INFINITY;
    den[k] = 0.f;
    num[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  // one batch of pieces: slot (j, k) holds chunk ch[k] of piece pc0 + pstep * j + poff[k]
  auto batch = [&](int pc0, int pstep, const int (&poff)[KC], const int (&ch)[KC],
                   const int (&hd)[KC], const bool (&ok)[KC]) __attribute__((always_inline)) {
    f32x4_t a[PPB][KC];
    f32x2_t ml[PPB][KC];
#pragma unroll
    for (int j = 0; j < PPB; ++j) {
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        const float* pp = piece(min(pc0 + pstep * j + poff[k], np - 1));
        a[j][k] = ok[k] ? *reinterpret_cast<const f32x4_t*>(pp + 4 * (cbase + ch[k]))
                        : f32x4_t{0.f, 0.f, 0.f, 0.f};
        ml[j][k] = *reinterpret_cast<const f32x2_t*>(pp + 16 * D + 2 * (qi * G + hd[k]));
      }
    }
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      float mb = M[k];
#pragma unroll
      for (int j = 0; j < PPB; ++j)
        if (pc0 + pstep * j + poff[k] < np) mb = fmaxf(mb, ml[j][k][0]);
      const float base = mb == -INFINITY ? 0.f : mb;
      const float sc = exp2_fast(M[k] - base);
      den[k] *= sc;
      num[k] *= sc;
#pragma unroll
      for (int j = 0; j < PPB; ++j) {
        if (pc0 + pstep * j + poff[k] < np) {
          const float f = exp2_fast(ml[j][k][0] - base);
          den[k] = __builtin_fmaf(f, ml[j][k][1], den[k]);
          num[k] += f * a[j][k];
        }
      }
      M[k] = mb;
    }
  };
  int ch[KC], hd[KC], poff[KC];
  bool ok[KC];
  if (nparts == 1) {
    // the whole sequence here: slot (j, k) holds chunk lane + 64k of piece k0 + j
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      ch[k] = lane + 64 * k;
      ok[k] = ch[k] < nchunk;
      hd[k] = ok[k] ? (4 * ch[k]) / D : 0;
      poff[k] = 0;
    }
    for (int k0 = 0; k0 < np; k0 += PPB) batch(k0, 1, poff, ch, hd, ok);
#pragma unroll
    for (int k = 0; k < KC; ++k)
      if (ok[k]) write_out(ch[k], num[k], den[k]);
    return;
  }
  // a share of the columns: nsh chunks from c_lo, 2^lkp per lane; slot (j, k)
  // holds chunk c_lo + lane + 64 (k mod 2^lkp) of piece k0 + R j + (k >> lkp)
  const int nsh = nchunk / nparts;
  const int c_lo = part * nsh;
  int lkp = 0;
  while ((64 << lkp) < nsh) ++lkp;
  const int nc = 1 << lkp, R = KC >> lkp;
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    const int within = lane + 64 * (k & (nc - 1));
    ok[k] = within < nsh;
    ch[k] = c_lo + (ok[k] ? within : 0);
    hd[k] = (4 * ch[k]) / D;
    poff[k] = k >> lkp;
  }
  for (int k0 = 0; k0 < np; k0 += PPB * R) batch(k0, R, poff, ch, hd, ok);
  // slot k's sums cover chunk k mod nc over its own pieces: combine the
  // slots of each chunk
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    if (k >= nc || !ok[k]) continue;
    float mc = -INFINITY;
#pragma unroll
    for (int k2 = 0; k2 < KC; ++k2)
      if ((k2 & (nc - 1)) == k) mc = fmaxf(mc, M[k2]);
    const float base = mc == -INFINITY ? 0.f : mc;
    float dsum = 0.f;
    f32x4_t nsum = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k2 = 0; k2 < KC; ++k2) {
      if ((k2 & (nc - 1)) == k) {
        const float f = exp2_fast(M[k2] - base);
        dsum = __builtin_fmaf(f, den[k2], dsum);
        nsum += f * num[k2];
      }
    }
    write_out(ch[k], nsum, dsum);
  }
}

// 16-byte chunks per lane the merge needs for G*D accumulators: a power of
// two >= G*D / 256.  One merge wavefront per attention wavefront and new
// token; with several new tokens the wavefronts go one per workgroup, which
// dispatches the larger grid faster (4 new tokens, 64 requests: 13.0 -> 10.0
// us), while with one token four per workgroup is as fast or faster.
template <bool IO_BF16, int D>
hipError_t launch_merge(const DecodeParams& p, hipStream_t stream, hipEvent_t* ev) {
  const int need = (p.group * D / 4 + 63) / 64;
  const int threads = p.n_qtok > 1 ? 64 : kBlockThreads;     // n_waves is a multiple of 4
  const dim3 grid(p.n_waves / (threads / 64) * p.n_qtok), block(threads);
  hipEvent_t e0 = ev ? ev[2] : nullptr, e1 = ev ? ev[3] : nullptr;
  if (need <= 1) hipExtLaunchKernelGGL((decode_merge_kernel<IO_BF16, D, 1>), grid, block, 0, stream, e0, e1, 0, p);
  else if (need <= 2) hipExtLaunchKernelGGL((decode_merge_kernel<IO_BF16, D, 2>), grid, block, 0, stream, e0, e1, 0, p);
  else if (need <= 4) hipExtLaunchKernelGGL((decode_merge_kernel<IO_BF16, D, 4>), grid, block, 0, stream, e0, e1, 0, p);
  else hipExtLaunchKernelGGL((decode_merge_kernel<IO_BF16, D, 8>), grid, block, 0, stream, e0, e1, 0, p);
  return hipGetLastError();
}

// The append of a step with n_qtok > 1 new tokens per request: one wavefront
// per (request, new token i, KV head) writes the rotated key and the value of
// token i to slot L - n_qtok + i, with the same arithmetic as the fused
// append (RoPE at position positions[b] + i in separate fp32 multiplies and
// adds, then the cast to the cache type).  It runs before the attention
// kernel, so every new token is in the pool when the queries read it.
template <int KV, int D, int BS>
__global__ __launch_bounds__(kBlockThreads) void decode_append_kernel(DecodeParams p) {
  using C = Cfg<KV, D, BS>;
  const int lane = threadIdx.x & 63;
  const int hkv = p.n_kv_heads, TQ = p.n_qtok;
  const int64_t item = (int64_t)blockIdx.x * (kBlockThreads / 64) + (threadIdx.x >> 6);
  if (item >= (int64_t)p.batch * TQ * hkv) return;
  const int h = (int)(item % hkv);
  const int64_t bi = item / hkv;
  const int i = (int)(bi % TQ), b = (int)(bi / TQ);
  const int cap = p.max_blocks * BS;
  const int L = p.context_lens[b];
  const int pos0 = p.positions[b];
  if (L < TQ || L > cap) {
    if (lane == 0) p.err[2] = 1u;
    return;
  }
  if (pos0 < 0 || pos0 + TQ - 1 >= p.max_pos) {
    if (lane == 0) p.err[1] = 1u;
    return;
  }
  const int slot = L - TQ + i;
  const int blk = p.block_tables[(int64_t)b * p.max_blocks + slot / BS];
  if ((unsigned)blk >= (unsigned)p.num_blocks) {
    if (lane == 0) p.err[0] = 1u;
    return;
  }
  const float* crow = p.rope_cos + (int64_t)(pos0 + i) * C::HALF;
  const float* srow = p.rope_sin + (int64_t)(pos0 + i) * C::HALF;
  const int64_t nrow = (((int64_t)b * TQ + i) * hkv + h) * D;
  float inv_k = 1.0f, inv_v = 1.0f;
  if constexpr (KV == KV_FP8) {
    inv_k = p.fp8_scales[2 * hkv + h];
    inv_v = p.fp8_scales[3 * hkv + h];
  }
  const int r = slot & (BS - 1);
  const int64_t toff = (((int64_t)blk * hkv + h) * C::TPB + ((r / kTileTokens) & (C::TPB - 1))) *
                       C::TILE_BYTES;
  const int r16 = r & 15;
  char* kpool = static_cast<char*>(p.k_pool);
  char* vpool = static_cast<char*>(p.v_pool);
  if (lane < C::KROWS) {
    const int d0 = C::X * lane;
    const bool lo = d0 < C::HALF;
    const int pd0 = lo ? d0 + C::HALF : d0 - C::HALF;
    const int i0 = lo ? d0 : pd0;
    float x[C::X], xp[C::X], cs[C::X], sn[C::X];
    load_row_f32<C::IO_BF16, C::X>(p.k_new, nrow + d0, x);
    load_row_f32<C::IO_BF16, C::X>(p.k_new, nrow + pd0, xp);
    load_f32<C::X>(crow + i0, cs);
    load_f32<C::X>(srow + i0, sn);
    uint32_t enc[C::X];
#pragma unroll
    for (int e = 0; e < C::X; ++e) {
      const float a = x[e] * cs[e];
      const float bb = xp[e] * sn[e];
      enc[e] = encode_kv<KV>(lo ? a - bb : a + bb, inv_k);
    }
    u32x4_t row;
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) {
      uint32_t w = 0;
#pragma unroll
      for (int k = 0; k < 4 / C::ELEM; ++k) w |= enc[i2 * (4 / C::ELEM) + k] << (k * C::ELEM * 8);
      row[i2] = w;
    }
    __builtin_nontemporal_store(row, reinterpret_cast<u32x4_t*>(kpool + toff + (lane * 16 + r16) * 16));
  }
#pragma unroll
  for (int k = 0; k < D / 64; ++k) {
    const int d = lane + 64 * k;
    const uint32_t code = encode_kv<KV>(load_io<C::IO_BF16>(p.v_new, nrow + d), inv_v);
    store_pool<C::ELEM>(vpool + toff + v_elem_offset<KV, D, BS>(r16, d), code);
  }
}

template <int KV, int D, int BS>
hipError_t launch_typed(const DecodeParams& p, hipStream_t stream, hipEvent_t* ev) {
  // With events, the start/stop stamps are taken by the dispatch packets of
  // the kernels themselves (ev[0..1] attention, ev[2..3] merge).
  if (p.n_qtok > 1) {
    if constexpr (KV == KV_F32) {
      return hipErrorInvalidValue;             // several new tokens: bf16 and fp8 caches only
    } else {
      const int64_t items = (int64_t)p.batch * p.n_qtok * p.n_kv_heads;
      hipLaunchKernelGGL((decode_append_kernel<KV, D, BS>),
                         dim3((unsigned)((items + kBlockThreads / 64 - 1) / (kBlockThreads / 64))),
                         dim3(kBlockThreads), 0, stream, p);
      hipExtLaunchKernelGGL((decode_attn_kernel<KV, D, BS, true, false>), dim3(p.n_waves / 4),
                            dim3(kBlockThreads), 0, stream, ev ? ev[0] : nullptr,
                            ev ? ev[1] : nullptr, 0, p, p.block_tables, p.context_lens,
                            p.positions, static_cast<char*>(p.k_pool),
                            static_cast<char*>(p.v_pool));
    }
  } else if (KV == KV_BF16 && p.group <= 8) {
    hipExtLaunchKernelGGL((decode_attn_kernel<KV, D, BS, false, KV == KV_BF16>),
                          dim3(p.n_waves / 4), dim3(kBlockThreads), 0, stream,
                          ev ? ev[0] : nullptr, ev ? ev[1] : nullptr, 0, p, p.block_tables,
                          p.context_lens, p.positions, static_cast<char*>(p.k_pool),
                          static_cast<char*>(p.v_pool));
  } else {
    hipExtLaunchKernelGGL((decode_attn_kernel<KV, D, BS, false, false>), dim3(p.n_waves / 4),
                          dim3(kBlockThreads), 0, stream, ev ? ev[0] : nullptr,
                          ev ? ev[1] : nullptr, 0, p, p.block_tables, p.context_lens,
                          p.positions, static_cast<char*>(p.k_pool),
                          static_cast<char*>(p.v_pool));
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_merge<KV != KV_F32, D>(p, stream, ev);
}

template <int KV, int D, int BS>
hipError_t occupancy_typed(int* blocks) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(
      blocks, decode_attn_kernel<KV, D, BS, false, false>, kBlockThreads, 0);
}

template <int KV, int D>
hipError_t dispatch_bs(int bs, const DecodeParams* p, hipStream_t stream, hipEvent_t* ev,
                       int* blocks) {
  switch (bs) {
    case 16: return p ? launch_typed<KV, D, 16>(*p, stream, ev) : occupancy_typed<KV, D, 16>(blocks);
    case 32: return p ? launch_typed<KV, D, 32>(*p, stream, ev) : occupancy_typed<KV, D, 32>(blocks);
    case 64: return p ? launch_typed<KV, D, 64>(*p, stream, ev) : occupancy_typed<KV, D, 64>(blocks);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

template <>
hipError_t decode_dispatch<PKV_KV>(int head_dim, int block_size, const DecodeParams* p,
                                   hipStream_t stream, hipEvent_t* events, int* blocks) {
  switch (head_dim) {
    case 64: return dispatch_bs<PKV_KV, 64>(block_size, p, stream, events, blocks);
    case 128: return dispatch_bs<PKV_KV, 128>(block_size, p, stream, events, blocks);
    default: return hipErrorInvalidValue;
  }
}

template <>
int decode_ring_tiles_of<PKV_KV>(int head_dim) {
  switch (head_dim) {
    case 64: return Cfg<PKV_KV, 64, 16>::RING;
    case 128: return Cfg<PKV_KV, 128, 16>::RING;
    default: return 0;
  }
}

}  // namespace pkv
