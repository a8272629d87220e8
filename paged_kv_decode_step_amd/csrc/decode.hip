// decode.hip -- fused paged-KV decode step for gfx950 (MI355X).
//
// One kernel does the whole step for its share of the batch: RoPE of the new
// query and key, the append of the new K/V into the block pool, the gather of
// the cached K/V through the block table, and softmax(q K^T / sqrt(D)) V with
// an online softmax.  A second, small kernel merges the partial softmax
// states of sequences that were cut between wavefronts.
//
// The pages ask for: the block-table lookup done inside the attention kernel
// ("Scaling TensorRT-LLM: Kernel Fusion and Inflight Batching in Production",
// section "The Paged KV-Cache: vLLM Borrowed by TensorRT-LLM"); RoPE inside the
// attention kernel and intermediates kept on chip (same page, "What Gets
// Fused"); KV blocks read once and reused by every query head of the group
// ("TensorRT-LLM Guide: High-Throughput GPU Inference Engine", section
// "3. Custom Fused Attention Kernels: FMHA and XQA"); an E4M3 cache with
// precomputed scales (same page, "4. Native FP8 Quantization on NVIDIA Hopper
// & Blackwell"); attention and KV-cache update fused ("TensorRT-LLM" glossary,
// inferensys.com, paragraph on the KV cache).
//
// Mapping onto CDNA4.  The step streams the KV cache from HBM once per KV
// head; the arithmetic is a G x D by D x T contraction (scores) and a G x T by
// T x D one (values), G <= 16.  Both run on 16x16 MFMA tiles with the query
// group padded to 16 columns: the matrix cores have ~40x more throughput than
// the 8 TB/s stream needs even at 1/8 column use, while plain VALU FMAs would
// use most of the vector ALU at G = 8.  Each 64-lane wavefront owns a
// contiguous range of (request, KV head, token step) work (see plan.h) and
// double-buffers whole steps of K and V (16 KiB per step) in registers:
// 16-byte loads, no LDS round trip, in-order completion counters.
//
// Register layouts (lane = 16 * lq + lr, lr in [0,16), lq in [0,4)).  For a
// cache element of E bytes, X = 16 / E elements fill a 16-byte row, a step is
// 4X tokens split into NG = X/4 sub-steps of 16 tokens.
//  * Scores, sub-step g: A = K rows (16 tokens), B = rotated queries (16
//    heads, zero beyond G), result lane (lr, lq) holds S[token X*lq + 4g + r]
//    [head lr], r = 0..3.  A's row i is token X*(i/4) + 4g + i%4, so the same
//    lane later holds exactly the probabilities the value product needs.
//  * Contraction over d is order-free: lane (lr, lq) holds dims
//    [X*(lq + 4j), X*(lq + 4j) + X) of its key row for j < D/(4X), which is
//    one 16-byte row of the K layout [D/X][bs][X].
//  * Values: A = V^T (16 dims x tokens), B = P^T (tokens x 16 heads); lane
//    (lr, lq) holds tokens [X*lq, X*lq + X) of dim 16*nt + lr, one 16-byte
//    row of the V layout [D][bs]; the result accumulates O^T so lane (lr, lq)
//    holds O[head lr][dims 16*nt + 4*lq + r].
#include "kernels.h"
#include "plan.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <int KV> struct KvT;
template <> struct KvT<KV_F32>  { static constexpr int ELEM = 4, X = 4; };
template <> struct KvT<KV_BF16> { static constexpr int ELEM = 2, X = 8; };
template <> struct KvT<KV_FP8>  { static constexpr int ELEM = 1, X = 16; };

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- scalars
__device__ __forceinline__ float exp2_fast(float x) {
  return __builtin_amdgcn_exp2f(x);   // v_exp_f32; -inf -> 0
}

__device__ __forceinline__ float shfl_xor(float v, int m) {
  return __shfl_xor(v, m, 64);
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

// Two E4M3 codes spread as bytes [c1, 0, c0, 0] -> two f16 holding
// value * 2^-8, exactly (subnormals included).
__device__ __forceinline__ uint32_t fp8x2_spread_to_f16x2(uint32_t s) {
  return ((s >> 1) & 0x3f803f80u) | (s & 0x80008000u);
}

__device__ __forceinline__ void fp8x16_to_f16(u32x4_t c, f16x8_t& lo, f16x8_t& hi) {
  u32x4_t a, b;
  a[0] = fp8x2_spread_to_f16x2(__builtin_amdgcn_perm(0u, c[0], 0x010c000cu));
  a[1] = fp8x2_spread_to_f16x2(__builtin_amdgcn_perm(0u, c[0], 0x030c020cu));
  a[2] = fp8x2_spread_to_f16x2(__builtin_amdgcn_perm(0u, c[1], 0x010c000cu));
  a[3] = fp8x2_spread_to_f16x2(__builtin_amdgcn_perm(0u, c[1], 0x030c020cu));
  b[0] = fp8x2_spread_to_f16x2(__builtin_amdgcn_perm(0u, c[2], 0x010c000cu));
  b[1] = fp8x2_spread_to_f16x2(__builtin_amdgcn_perm(0u, c[2], 0x030c020cu));
  b[2] = fp8x2_spread_to_f16x2(__builtin_amdgcn_perm(0u, c[3], 0x010c000cu));
  b[3] = fp8x2_spread_to_f16x2(__builtin_amdgcn_perm(0u, c[3], 0x030c020cu));
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

// Encode one float into the cache storage type (bit pattern in the low bits).
template <int KV>
__device__ __forceinline__ uint32_t encode_kv(float y, float inv_scale) {
  if constexpr (KV == KV_F32) return __float_as_uint(y);
  else if constexpr (KV == KV_BF16) return bf16_rne(y);
  else return fp8_encode(y * inv_scale);
}

// Zero the elements with index >= nv in a 16-byte row of E-byte elements.
template <int ELEM>
__device__ __forceinline__ u32x4_t keep_first(u32x4_t row, int nv) {
  constexpr int EPD = 4 / ELEM;
  constexpr uint32_t M = ELEM == 4 ? 0xffffffffu : (ELEM == 2 ? 0xffffu : 0xffu);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t keep = 0;
#pragma unroll
    for (int k = 0; k < EPD; ++k)
      keep |= (i * EPD + k < nv) ? (M << (k * ELEM * 8)) : 0u;
    row[i] &= keep;
  }
  return row;
}

// ---------------------------------------------------------------- kernel
template <int KV, int D, int BS>
struct Cfg {
  static constexpr int ELEM = KvT<KV>::ELEM;
  static constexpr int X = KvT<KV>::X;       // elements per 16-byte row
  static constexpr int NG = X / 4;           // 16-token sub-steps per step
  static constexpr int STEP = 4 * X;         // tokens per step
  static constexpr int NJ = D / (4 * X);     // key rows per lane per sub-step
  static constexpr int NC = D / 16;          // 16-byte K (and V) rows per lane
  static constexpr int HALF = D / 2;
  static constexpr bool IO_BF16 = KV != KV_F32;
  static constexpr int LOG2BS = BS == 16 ? 4 : (BS == 32 ? 5 : 6);
  static constexpr int NB = STEP > BS ? STEP / BS : 1;   // blocks per step
  static constexpr int TW = 256;             // block-table window per wavefront
  static_assert(X <= BS, "a 16-byte row of V must stay inside one block");
};

// One step's worth of K and V in registers.
template <int NC>
struct StepBuf {
  u32x4_t k[NC];
  u32x4_t v[NC];
};

// Per-piece state.
struct PieceCtx {
  const char* kpool;
  const char* vpool;
  const int32_t* trow;    // block-table row of the request
  int* tw;                // this wavefront's block-table window in LDS
  int kvh, L, n_used;
  int blk_base;           // block index held in tw[0]
};

// Refill the LDS window with block ids [base, base + TW) of the request
// (0 past the request's last block; ids outside the pool become 0 and raise
// a flag).  Waits for its own loads: called once per piece and then only
// every TW blocks.
template <int TW>
__device__ __forceinline__ void fill_window(PieceCtx& c, const DecodeParams& p, int base,
                                            int lane) {
  c.blk_base = base;
  int v[TW / 64];
#pragma unroll
  for (int i = 0; i < TW / 64; ++i) {
    const int idx = base + i * 64 + lane;
    const int id = c.trow[idx < c.n_used ? idx : 0];
    v[i] = idx < c.n_used ? id : 0;
  }
#pragma unroll
  for (int i = 0; i < TW / 64; ++i) {
    const bool ok = (unsigned)v[i] < (unsigned)p.num_blocks;
    if (!ok) p.err[0] = 1u;
    c.tw[i * 64 + lane] = ok ? v[i] : 0;
  }
}

// K rows of step st: lane row lr is token X*(lr/4) + 4g + lr%4 of sub-step g.
// Slides the block-table window first when the step runs past it.
template <int KV, int D, int BS>
__device__ __forceinline__ void issue_k(StepBuf<Cfg<KV, D, BS>::NC>& buf, PieceCtx& c,
                                        const DecodeParams& p, int st, int lr, int lq,
                                        int lane) {
  using C = Cfg<KV, D, BS>;
  const int token0 = st * C::STEP;
  const int fb = token0 >> C::LOG2BS;
  if (fb + C::NB - c.blk_base > C::TW) fill_window<C::TW>(c, p, fb, lane);
  const int64_t hk = (int64_t)p.n_kv_heads;
#pragma unroll
  for (int g = 0; g < C::NG; ++g) {
    const int t = token0 + C::X * (lr >> 2) + 4 * g + (lr & 3);
    const int ph = c.tw[(t >> C::LOG2BS) - c.blk_base];
    const int slot = t & (BS - 1);
    const char* base = c.kpool +
        ((((int64_t)ph * hk + c.kvh) * (D / C::X) + lq) * BS + slot) * 16;
#pragma unroll
    for (int j = 0; j < C::NJ; ++j)
      buf.k[g * C::NJ + j] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(base + j * 4 * BS * 16));
  }
}

// V rows of step st: lane holds tokens [X*lq, X*lq + X) of dims 16*nt + lr.
// Uses the window as issue_k of the same step left it.
template <int KV, int D, int BS>
__device__ __forceinline__ void issue_v(StepBuf<Cfg<KV, D, BS>::NC>& buf, const PieceCtx& c,
                                        const DecodeParams& p, int st, int lr, int lq) {
  using C = Cfg<KV, D, BS>;
  const int t0 = st * C::STEP + C::X * lq;
  const int ph = c.tw[(t0 >> C::LOG2BS) - c.blk_base];
  const int slot0 = t0 & (BS - 1);
  const char* base = c.vpool +
      ((((int64_t)ph * p.n_kv_heads + c.kvh) * D + lr) * BS + slot0) * C::ELEM;
#pragma unroll
  for (int nt = 0; nt < C::NC; ++nt)
    buf.v[nt] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4_t*>(base + nt * 16 * BS * C::ELEM));
}

// Query operand of the score MFMA: the rotated query of head lr (zero if
// lr >= G) at the dims lane (lr, lq) contracts over.
template <int KV, int NJ> struct QOp;
template <int NJ> struct QOp<KV_BF16, NJ> { bf16x8_t v[NJ]; };
template <int NJ> struct QOp<KV_FP8, NJ>  { f16x8_t v[NJ][2]; };
template <int NJ> struct QOp<KV_F32, NJ>  { float v[NJ][4]; };

// X consecutive io-dtype elements starting at element `off` -> float.
template <bool IO_BF16, int X>
__device__ __forceinline__ void load_row_f32(const void* base, int64_t off, float (&out)[X]) {
  if constexpr (IO_BF16) {
    const u32x4_t* ptr = reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int i = 0; i < X / 8; ++i) {
      const u32x4_t w = ptr[i];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        out[8 * i + 2 * k] = __uint_as_float(w[k] << 16);
        out[8 * i + 2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
      }
    }
  } else {
    const f32x4_t* ptr = reinterpret_cast<const f32x4_t*>(static_cast<const float*>(base) + off);
#pragma unroll
    for (int i = 0; i < X / 4; ++i) {
      const f32x4_t w = ptr[i];
#pragma unroll
      for (int k = 0; k < 4; ++k) out[4 * i + k] = w[k];
    }
  }
}

template <int X>
__device__ __forceinline__ void load_f32(const float* ptr, float (&out)[X]) {
#pragma unroll
  for (int i = 0; i < X / 4; ++i) {
    const f32x4_t w = reinterpret_cast<const f32x4_t*>(ptr)[i];
#pragma unroll
    for (int k = 0; k < 4; ++k) out[4 * i + k] = w[k];
  }
}

// One step: scores from the K rows, then (after the caller's hook has
// reused the K registers for the next step) the online softmax and P V.
template <int KV, int D, int BS, class AfterScores>
__device__ __forceinline__ void compute_step(StepBuf<Cfg<KV, D, BS>::NC>& buf,
                                             const QOp<KV, Cfg<KV, D, BS>::NJ>& qop,
                                             f32x4_t (&acc)[Cfg<KV, D, BS>::NC], float& m_run,
                                             float& l_run, float sscale, int L, int st,
                                             bool last, int lq, AfterScores&& after_scores) {
  using C = Cfg<KV, D, BS>;
  const int token0 = st * C::STEP;

  // Scores for the NG sub-steps.
  float s[C::NG][4];
#pragma unroll
  for (int g = 0; g < C::NG; ++g) {
    f32x4_t a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) {
      const u32x4_t kr = buf.k[g * C::NJ + j];
      if constexpr (KV == KV_BF16) {
        a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kr),
                                                     qop.v[j], a4, 0, 0, 0);
      } else if constexpr (KV == KV_FP8) {
        f16x8_t lo, hi;
        fp8x16_to_f16(kr, lo, hi);
        a4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(lo, qop.v[j][0], a4, 0, 0, 0);
        a4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi, qop.v[j][1], a4, 0, 0, 0);
      } else {
        const f32x4_t kf = __builtin_bit_cast(f32x4_t, kr);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          a4 = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[e], qop.v[j][e], a4, 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) s[g][r] = a4[r] * sscale;
  }
  after_scores();

  if (last) {
    // Tokens at or past L: scores are -inf (selected, never multiplied) and
    // their values are zeroed, whatever the unused slots hold.
#pragma unroll
    for (int g = 0; g < C::NG; ++g)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (token0 + C::X * lq + 4 * g + r >= L) s[g][r] = -INFINITY;
    const int nv = L - (token0 + C::X * lq);
#pragma unroll
    for (int nt = 0; nt < C::NC; ++nt) buf.v[nt] = keep_first<C::ELEM>(buf.v[nt], nv);
  }

  // Online softmax over the step (log2 domain); the four lanes lq = 0..3 of
  // head lr share one running max.
  float mx = s[0][0];
#pragma unroll
  for (int g = 0; g < C::NG; ++g)
#pragma unroll
    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[g][r]);
  mx = fmaxf(mx, shfl_xor(mx, 16));
  mx = fmaxf(mx, shfl_xor(mx, 32));
  const float m_new = fmaxf(m_run, mx);
  const float mb = (m_new == -INFINITY) ? 0.0f : m_new;
  const float alpha = exp2_fast(m_run - mb);
  m_run = m_new;
  float ps = 0.f;
#pragma unroll
  for (int g = 0; g < C::NG; ++g)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s[g][r] = exp2_fast(s[g][r] - mb);
      ps += s[g][r];
    }
  l_run = __builtin_fmaf(l_run, alpha, ps);
#pragma unroll
  for (int nt = 0; nt < C::NC; ++nt) acc[nt] *= alpha;

  // P V.
  if constexpr (KV == KV_BF16) {
    u32x4_t pb;
    pb[0] = pack_bf16x2(s[0][0], s[0][1]);
    pb[1] = pack_bf16x2(s[0][2], s[0][3]);
    pb[2] = pack_bf16x2(s[1][0], s[1][1]);
    pb[3] = pack_bf16x2(s[1][2], s[1][3]);
    const bf16x8_t pbv = __builtin_bit_cast(bf16x8_t, pb);
#pragma unroll
    for (int nt = 0; nt < C::NC; ++nt)
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, buf.v[nt]),
                                                        pbv, acc[nt], 0, 0, 0);
  } else if constexpr (KV == KV_FP8) {
    u32x4_t p0, p1;
    p0[0] = pack_f16x2(s[0][0], s[0][1]);
    p0[1] = pack_f16x2(s[0][2], s[0][3]);
    p0[2] = pack_f16x2(s[1][0], s[1][1]);
    p0[3] = pack_f16x2(s[1][2], s[1][3]);
    p1[0] = pack_f16x2(s[2][0], s[2][1]);
    p1[1] = pack_f16x2(s[2][2], s[2][3]);
    p1[2] = pack_f16x2(s[3][0], s[3][1]);
    p1[3] = pack_f16x2(s[3][2], s[3][3]);
    const f16x8_t pa = __builtin_bit_cast(f16x8_t, p0);
    const f16x8_t pc = __builtin_bit_cast(f16x8_t, p1);
#pragma unroll
    for (int nt = 0; nt < C::NC; ++nt) {
      f16x8_t lo, hi;
      fp8x16_to_f16(buf.v[nt], lo, hi);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(lo, pa, acc[nt], 0, 0, 0);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi, pc, acc[nt], 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int nt = 0; nt < C::NC; ++nt) {
      const f32x4_t vf = __builtin_bit_cast(f32x4_t, buf.v[nt]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[e], s[0][e], acc[nt], 0, 0, 0);
    }
  }
}

// Append of the new token, done before the piece's loads are issued.  The
// rotated key (pinned fp32 arithmetic: two separate multiplies and one add or
// subtract, no contraction) and the value are cast to the cache type and
// stored into slot L-1.  Each element is written by the lane that later loads
// it in the last step's layout, so program order makes that load return it.
template <int KV, int D, int BS>
__device__ __forceinline__ void append_token(const DecodeParams& p, const PieceCtx& c, int b,
                                             int posn, int lr, int lq) {
  using C = Cfg<KV, D, BS>;
  const int L = c.L;
  const int rel = (L - 1) & (C::STEP - 1);        // position in the last step
  const int row_new = 4 * (rel / C::X) + (rel & 3);
  int phn = c.trow[(L - 1) >> C::LOG2BS];
  if ((unsigned)phn >= (unsigned)p.num_blocks) {
    p.err[0] = 1u;
    phn = 0;
  }
  const int slot_new = (L - 1) & (BS - 1);
  const int64_t hk = (int64_t)p.n_kv_heads;
  const int64_t row_off = ((int64_t)b * hk + c.kvh) * D;
  const float* crow = p.rope_cos + (int64_t)posn * C::HALF;
  const float* srow = p.rope_sin + (int64_t)posn * C::HALF;
  float inv_k = 1.0f, inv_v = 1.0f;
  if constexpr (KV == KV_FP8) {
    inv_k = p.fp8_scales[2 * p.n_kv_heads + c.kvh];
    inv_v = p.fp8_scales[3 * p.n_kv_heads + c.kvh];
  }
  char* kpool = const_cast<char*>(c.kpool);
  char* vpool = const_cast<char*>(c.vpool);
#pragma unroll
  for (int j = 0; j < C::NJ; ++j) {
    const int d0 = C::X * (lq + 4 * j);
    const bool lo = d0 < C::HALF;
    const int pd0 = lo ? d0 + C::HALF : d0 - C::HALF;
    const int i0 = lo ? d0 : pd0;
    float x[C::X], xp[C::X], cs[C::X], sn[C::X];
    load_row_f32<C::IO_BF16, C::X>(p.k_new, row_off + d0, x);
    load_row_f32<C::IO_BF16, C::X>(p.k_new, row_off + pd0, xp);
    load_f32<C::X>(crow + i0, cs);
    load_f32<C::X>(srow + i0, sn);
    uint32_t enc[C::X];
#pragma unroll
    for (int e = 0; e < C::X; ++e) {
      // lo half: y = x*C - x[i+D/2]*S ; hi half: y = x*C + x[i-D/2]*S
      const float a = x[e] * cs[e];
      const float bb = xp[e] * sn[e];
      const float y = lo ? a - bb : a + bb;
      enc[e] = encode_kv<KV>(y, inv_k);
    }
    u32x4_t row;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t w = 0;
#pragma unroll
      for (int k = 0; k < 4 / C::ELEM; ++k) w |= enc[i * (4 / C::ELEM) + k] << (k * C::ELEM * 8);
      row[i] = w;
    }
    if (lr == row_new) {
      char* dst = kpool + ((((int64_t)phn * hk + c.kvh) * (D / C::X) + lq + 4 * j) * BS +
                           slot_new) * 16;
      *reinterpret_cast<u32x4_t*>(dst) = row;
    }
  }
  uint32_t vbits[C::NC];
#pragma unroll
  for (int nt = 0; nt < C::NC; ++nt)
    vbits[nt] = encode_kv<KV>(load_io<C::IO_BF16>(p.v_new, row_off + 16 * nt + lr), inv_v);
  if (lq == rel / C::X) {
#pragma unroll
    for (int nt = 0; nt < C::NC; ++nt) {
      const int d = 16 * nt + lr;
      char* dst = vpool + ((((int64_t)phn * hk + c.kvh) * D + d) * BS + slot_new) * C::ELEM;
      if constexpr (C::ELEM == 4) *reinterpret_cast<uint32_t*>(dst) = vbits[nt];
      else if constexpr (C::ELEM == 2) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)vbits[nt];
      else *reinterpret_cast<uint8_t*>(dst) = (uint8_t)vbits[nt];
    }
  }
}

template <int KV, int D, int BS>
__device__ __forceinline__ void process_piece(const DecodeParams& p, int* tw, int b, int kvh,
                                              int ns, int st0, int st1, bool split, int slot,
                                              int64_t wave, int lane) {
  using C = Cfg<KV, D, BS>;
  const int lr = lane & 15, lq = lane >> 4;
  const int G = p.group;
  const int cap = p.max_blocks * BS;

  const int Lraw = p.context_lens[b];
  const bool len_ok = Lraw >= 1 && Lraw <= cap;
  const int L = Lraw < 0 ? 0 : (Lraw > cap ? cap : Lraw);
  int posn = p.positions[b];
  const bool pos_ok = posn >= 0 && posn < p.max_pos;
  posn = posn < 0 ? 0 : (posn >= p.max_pos ? p.max_pos - 1 : posn);
  if (st0 == 0) {
    if (!len_ok) p.err[2] = 1u;
    if (!pos_ok) p.err[1] = 1u;
  }

  PieceCtx c;
  c.kpool = static_cast<const char*>(p.k_pool);
  c.vpool = static_cast<const char*>(p.v_pool);
  c.trow = p.block_tables + (int64_t)b * p.max_blocks;
  c.tw = tw;
  c.kvh = kvh;
  c.L = L;
  c.n_used = (L + BS - 1) >> C::LOG2BS;

  // Rotated query of head lr at this lane's dims (fp32).  Heads past G load
  // head 0 of the group (a valid address) and are zeroed.
  const int hq = kvh * G + (lr < G ? lr : 0);
  const bool hvalid = lr < G;
  const int64_t qrow = ((int64_t)b * (p.n_kv_heads * G) + hq) * D;
  const float* crow = p.rope_cos + (int64_t)posn * C::HALF;
  const float* srow = p.rope_sin + (int64_t)posn * C::HALF;
  float qv[C::NJ][C::X];
#pragma unroll
  for (int j = 0; j < C::NJ; ++j) {
    const int d0 = C::X * (lq + 4 * j);
    const bool lo = d0 < C::HALF;
    const int pd0 = lo ? d0 + C::HALF : d0 - C::HALF;
    const int i0 = lo ? d0 : pd0;
    float x[C::X], xp[C::X], cs[C::X], sn[C::X];
    load_row_f32<C::IO_BF16, C::X>(p.q, qrow + d0, x);
    load_row_f32<C::IO_BF16, C::X>(p.q, qrow + pd0, xp);
    load_f32<C::X>(crow + i0, cs);
    load_f32<C::X>(srow + i0, sn);
#pragma unroll
    for (int e = 0; e < C::X; ++e) {
      const float y = lo ? (x[e] * cs[e] - xp[e] * sn[e]) : (x[e] * cs[e] + xp[e] * sn[e]);
      qv[j][e] = hvalid ? y : 0.0f;
    }
  }

  if (len_ok && st1 == ns) append_token<KV, D, BS>(p, c, b, posn, lr, lq);

  fill_window<C::TW>(c, p, (st0 * C::STEP) >> C::LOG2BS, lane);
  StepBuf<C::NC> buf;
  issue_k<KV, D, BS>(buf, c, p, st0, lr, lq, lane);
  issue_v<KV, D, BS>(buf, c, p, st0, lr, lq);

  float sscale = p.sm_scale_log2;
  QOp<KV, C::NJ> qop;
  if constexpr (KV == KV_BF16) {
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) {
      u32x4_t w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(qv[j][2 * i], qv[j][2 * i + 1]);
      qop.v[j] = __builtin_bit_cast(bf16x8_t, w);
    }
  } else if constexpr (KV == KV_FP8) {
    // Scale the query by a power of two so that it fits f16 with room to
    // spare; the factor goes back into the score scale.
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < C::NJ; ++j)
#pragma unroll
      for (int e = 0; e < C::X; ++e) amax = fmaxf(amax, fabsf(qv[j][e]));
    amax = fmaxf(amax, shfl_xor(amax, 16));
    amax = fmaxf(amax, shfl_xor(amax, 32));
    int ex = 0;
    if (amax > 0.f) {
      (void)__builtin_frexpf(amax, &ex);   // amax < 2^ex
      ex = ex > 15 ? ex - 15 : 0;
    }
    const float qs = __builtin_ldexpf(1.0f, -ex);
    sscale = p.sm_scale_log2 * p.fp8_scales[kvh] * __builtin_ldexpf(1.0f, 8 + ex);
#pragma unroll
    for (int j = 0; j < C::NJ; ++j)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        u32x4_t w;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          w[i] = pack_f16x2(qv[j][8 * hh + 2 * i] * qs, qv[j][8 * hh + 2 * i + 1] * qs);
        qop.v[j][hh] = __builtin_bit_cast(f16x8_t, w);
      }
  } else {
#pragma unroll
    for (int j = 0; j < C::NJ; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) qop.v[j][e] = qv[j][e];
  }

  f32x4_t acc[C::NC];
#pragma unroll
  for (int nt = 0; nt < C::NC; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // One buffer: the next step's K loads go out as soon as the scores are
  // done, its V loads as soon as P V is done.
  for (int st = st0; st < st1; ++st) {
    const bool more = st + 1 < st1;
    compute_step<KV, D, BS>(buf, qop, acc, m_run, l_run, sscale, L, st, st == ns - 1, lq,
                            [&] { if (more) issue_k<KV, D, BS>(buf, c, p, st + 1, lr, lq, lane); });
    if (more) issue_v<KV, D, BS>(buf, c, p, st + 1, lr, lq);
  }

  // Finish the piece: normalise and store, or leave a partial state.
  float lt = l_run + shfl_xor(l_run, 16);
  lt += shfl_xor(lt, 32);
  float vsc = 1.0f;
  if constexpr (KV == KV_FP8) vsc = 256.0f * p.fp8_scales[p.n_kv_heads + kvh];
  if (!hvalid) return;
  if (!split) {
    const float inv = lt > 0.f ? vsc / lt : 0.f;
#pragma unroll
    for (int nt = 0; nt < C::NC; ++nt) {
      const int d = 16 * nt + 4 * lq;
      if constexpr (C::IO_BF16) {
        u32x2_t w;
        w[0] = bf16_rne(acc[nt][0] * inv) | (bf16_rne(acc[nt][1] * inv) << 16);
        w[1] = bf16_rne(acc[nt][2] * inv) | (bf16_rne(acc[nt][3] * inv) << 16);
        *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(p.out) + qrow + d) = w;
      } else {
        *reinterpret_cast<f32x4_t*>(static_cast<float*>(p.out) + qrow + d) = acc[nt] * inv;
      }
    }
  } else {
    float* part = p.partials + ((size_t)(wave * 2 + slot) * kGroupMax + lr) * (D + 2);
#pragma unroll
    for (int nt = 0; nt < C::NC; ++nt)
      *reinterpret_cast<f32x4_t*>(part + 16 * nt + 4 * lq) = acc[nt] * vsc;
    if (lq == 0) {
      part[D] = m_run;
      part[D + 1] = lt;
    }
  }
}

template <int KV, int D, int BS>
__global__ __launch_bounds__(kBlockThreads) __attribute__((amdgpu_waves_per_eu(3, 3)))
void decode_attn_kernel(DecodeParams p) {
  using C = Cfg<KV, D, BS>;
  __shared__ int sP[kMaxBatch + 1];
  __shared__ int sScan[kBlockThreads];
  __shared__ int sTw[kBlockThreads / 64][C::TW];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kBlockThreads / 64) + (tid >> 6);
  const int B = p.batch, hkv = p.n_kv_heads;
  const int cap = p.max_blocks * BS;

  // Steps per request, prefix-summed into LDS (every workgroup does this).
  {
    const int per = (B + kBlockThreads - 1) / kBlockThreads;
    const int i0 = tid * per;
    int sum = 0;
    for (int i = 0; i < per; ++i) {
      const int b = i0 + i;
      if (b < B) sum += steps_of(p.context_lens[b], cap, C::STEP);
    }
    sScan[tid] = sum;
    __syncthreads();
    for (int off = 1; off < kBlockThreads; off <<= 1) {
      const int v = tid >= off ? sScan[tid - off] : 0;
      __syncthreads();
      sScan[tid] += v;
      __syncthreads();
    }
    int run = sScan[tid] - sum;
    for (int i = 0; i < per; ++i) {
      const int b = i0 + i;
      if (b < B) {
        sP[b] = run;
        run += steps_of(p.context_lens[b], cap, C::STEP);
      }
    }
    if (tid == kBlockThreads - 1) sP[B] = sScan[tid];
    __syncthreads();
  }

  const int64_t N = (int64_t)hkv * sP[B];
  const int64_t We = active_waves(N, p.n_waves, p.min_steps);
  if (wave >= We) {
    if (lane == 0) p.headers[wave] = make_int4(0, 0, 0, 0);
    return;
  }
  int* tw = sTw[tid >> 6];
  const int64_t start = wave_start(wave, N, We);
  const int64_t end = wave_start(wave + 1, N, We);
  int b = find_request(sP, B, start, hkv);
  int ns = sP[b + 1] - sP[b];
  int64_t rbase = (int64_t)hkv * sP[b];
  int h = (int)((start - rbase) / ns);
  int64_t pos = start;
  bool first = true;
  while (pos < end) {
    const int64_t seq_begin = rbase + (int64_t)h * ns;
    const int64_t seq_end = seq_begin + ns;
    const int64_t piece_end = seq_end < end ? seq_end : end;
    const bool split = seq_begin < start || seq_end > end;
    process_piece<KV, D, BS>(p, tw, b, h, ns, (int)(pos - seq_begin),
                             (int)(piece_end - seq_begin), split, first ? 0 : 1, wave, lane);
    if (first) {
      if (lane == 0) {
        int4 hdr = make_int4(0, 0, 0, 0);
        if (split && seq_end <= end) {
          const int64_t wf = wave_of_step(seq_begin, N, We);
          const int slot_f = wave_start(wf, N, We) == seq_begin ? 0 : 1;
          hdr = make_int4(HDR_TRIGGER, b * hkv + h, (int)wf,
                          slot_f | ((int)(wave - wf + 1) << 1));
        }
        p.headers[wave] = hdr;
      }
      first = false;
    }
    pos = piece_end;
    if (++h == hkv) {
      h = 0;
      if (++b < B) {
        ns = sP[b + 1] - sP[b];
        rbase = (int64_t)hkv * sP[b];
      }
    }
  }
}

// Merge the partial softmax states of each split sequence:
// out = sum_k 2^(m_k - M) acc_k / sum_k 2^(m_k - M) l_k,  M = max_k m_k.
template <bool IO_BF16, int D>
__global__ __launch_bounds__(128) void decode_merge_kernel(DecodeParams p) {
  const int4 hdr = p.headers[blockIdx.x];
  if (!(hdr.x & HDR_TRIGGER)) return;
  const int hkv = p.n_kv_heads, G = p.group;
  const int b = hdr.y / hkv, kvh = hdr.y % hkv;
  const int wf = hdr.z, slot_f = hdr.w & 1, np = hdr.w >> 1;
  for (int idx = threadIdx.x; idx < G * D; idx += 128) {
    const int hh = idx / D, d = idx % D;
    float M = -INFINITY;
    for (int k = 0; k < np; ++k) {
      const int slot = k == 0 ? slot_f : 0;
      const float* part = p.partials + ((size_t)((wf + k) * 2 + slot) * kGroupMax + hh) * (D + 2);
      M = fmaxf(M, part[D]);
    }
    const float mb = M == -INFINITY ? 0.f : M;
    float num = 0.f, den = 0.f;
    for (int k = 0; k < np; ++k) {
      const int slot = k == 0 ? slot_f : 0;
      const float* part = p.partials + ((size_t)((wf + k) * 2 + slot) * kGroupMax + hh) * (D + 2);
      const float f = exp2_fast(part[D] - mb);
      num = __builtin_fmaf(f, part[d], num);
      den = __builtin_fmaf(f, part[D + 1], den);
    }
    const float o = den > 0.f ? num / den : 0.f;
    const int64_t oi = ((int64_t)b * (hkv * G) + kvh * G + hh) * D + d;
    if constexpr (IO_BF16) static_cast<uint16_t*>(p.out)[oi] = (uint16_t)bf16_rne(o);
    else static_cast<float*>(p.out)[oi] = o;
  }
}

template <int KV, int D, int BS>
hipError_t launch_typed(const DecodeParams& p, hipStream_t stream, hipEvent_t* ev) {
  hipError_t e;
  if (ev && (e = hipEventRecord(ev[0], stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((decode_attn_kernel<KV, D, BS>), dim3(p.n_waves / 4), dim3(kBlockThreads),
                     0, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[1], stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<KV != KV_F32, D>), dim3(p.n_waves), dim3(128), 0,
                     stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[2], stream)) != hipSuccess) return e;
  return hipSuccess;
}

template <int KV, int D, int BS>
hipError_t occupancy_typed(int* blocks) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, decode_attn_kernel<KV, D, BS>,
                                                      kBlockThreads, 0);
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

hipError_t dispatch(int kv_kind, int head_dim, int bs, const DecodeParams* p, hipStream_t stream,
                    hipEvent_t* ev, int* blocks) {
  switch (kv_kind * 1000 + head_dim) {
    case KV_F32 * 1000 + 64:   return dispatch_bs<KV_F32, 64>(bs, p, stream, ev, blocks);
    case KV_F32 * 1000 + 128:  return dispatch_bs<KV_F32, 128>(bs, p, stream, ev, blocks);
    case KV_BF16 * 1000 + 64:  return dispatch_bs<KV_BF16, 64>(bs, p, stream, ev, blocks);
    case KV_BF16 * 1000 + 128: return dispatch_bs<KV_BF16, 128>(bs, p, stream, ev, blocks);
    case KV_FP8 * 1000 + 64:   return dispatch_bs<KV_FP8, 64>(bs, p, stream, ev, blocks);
    case KV_FP8 * 1000 + 128:  return dispatch_bs<KV_FP8, 128>(bs, p, stream, ev, blocks);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(int kv_kind, int head_dim, int block_size, const DecodeParams& p,
                         hipStream_t stream, hipEvent_t* events) {
  return dispatch(kv_kind, head_dim, block_size, &p, stream, events, nullptr);
}

hipError_t decode_occupancy(int kv_kind, int head_dim, int block_size, int* blocks) {
  return dispatch(kv_kind, head_dim, block_size, nullptr, nullptr, nullptr, blocks);
}

}  // namespace pkv
