/* c_abi_driver.c -- a caller of libpkv.so in plain C, with no Python in the
 * process: it builds three requests' contexts token by token through
 * decode_step (each step appends the new token and attends over the context so
 * far) and writes the last step's output rows, then the K and V pools, to the
 * file named by argv[1].  The inputs come from a 32-bit linear congruential
 * generator that test_gpu_c_abi.py replays.
 *
 * Shapes: 3 requests, 32 query heads over 8 KV heads, head_dim 128, blocks of
 * 16 tokens, bf16 cache and io; request b owns blocks 3b .. 3b + 2 and its
 * context grows to 40 tokens.  Exit status 0 on success. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pkv.h"

enum { B = 3, HKV = 8, HQ = 32, D = 128, BS = 16, MAXB = 3, STEPS = 40, NBLK = B * MAXB };

static uint32_t next(uint32_t* s) { return *s = *s * 1664525u + 1013904223u; }

/* a bf16 in [-1, 1): the top 16 bits of a float built from 24 random bits */
static uint16_t draw_bf16(uint32_t* s) {
  const float f = (float)(next(s) >> 8) * (1.0f / 8388608.0f) - 1.0f;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

#define HIP_OK(x)                                                             \
  do {                                                                        \
    if ((x) != hipSuccess) {                                                  \
      fprintf(stderr, "HIP call failed at line %d\n", __LINE__);              \
      return 2;                                                               \
    }                                                                         \
  } while (0)
#define PKV_OK_(x)                                                            \
  do {                                                                        \
    if ((x) != PKV_OK) {                                                      \
      fprintf(stderr, "line %d: %s\n", __LINE__, pkv_last_error());           \
      return 3;                                                               \
    }                                                                         \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 2) return 1;
  pkv_pool* pool = NULL;
  PKV_OK_(kv_pool_create(NBLK, BS, HKV, D, PKV_BF16, &pool));
  PKV_OK_(kv_pool_set_rope(pool, 5.0e5, STEPS));
  void *kb = NULL, *vb = NULL;
  int64_t strides[3];
  int32_t tile_bytes = 0;
  PKV_OK_(kv_pool_layout(pool, &kb, &vb, strides, &tile_bytes));
  const size_t pool_bytes = (size_t)NBLK * (size_t)strides[0];
  HIP_OK(hipMemset(kb, 0, pool_bytes));
  HIP_OK(hipMemset(vb, 0, pool_bytes));

  static uint16_t q[B * HQ * D], kn[B * HKV * D], vn[B * HKV * D], out[B * HQ * D];
  int32_t pos[B], lens[B], tables[B * MAXB];
  for (int i = 0; i < B * MAXB; ++i) tables[i] = i;
  void *dq, *dk, *dv, *dout, *dpos, *dlens, *dtab;
  HIP_OK(hipMalloc(&dq, sizeof q));
  HIP_OK(hipMalloc(&dk, sizeof kn));
  HIP_OK(hipMalloc(&dv, sizeof vn));
  HIP_OK(hipMalloc(&dout, sizeof out));
  HIP_OK(hipMalloc(&dpos, sizeof pos));
  HIP_OK(hipMalloc(&dlens, sizeof lens));
  HIP_OK(hipMalloc(&dtab, sizeof tables));
  HIP_OK(hipMemcpy(dtab, tables, sizeof tables, hipMemcpyHostToDevice));

  uint32_t seed = 20241203u;
  for (int step = 0; step < STEPS; ++step) {
    for (int i = 0; i < B * HQ * D; ++i) q[i] = draw_bf16(&seed);
    for (int i = 0; i < B * HKV * D; ++i) kn[i] = draw_bf16(&seed);
    for (int i = 0; i < B * HKV * D; ++i) vn[i] = draw_bf16(&seed);
    for (int b = 0; b < B; ++b) {
      pos[b] = step;
      lens[b] = step + 1;
    }
    HIP_OK(hipMemcpy(dq, q, sizeof q, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dk, kn, sizeof kn, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dv, vn, sizeof vn, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dpos, pos, sizeof pos, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dlens, lens, sizeof lens, hipMemcpyHostToDevice));
    PKV_OK_(decode_step(pool, dq, dk, dv, PKV_BF16, (const int32_t*)dpos, (const int32_t*)dtab,
                        MAXB, (const int32_t*)dlens, B, HQ, dout, NULL));
  }
  HIP_OK(hipDeviceSynchronize());
  uint32_t flags = 1;
  PKV_OK_(kv_pool_device_errors(pool, &flags));
  if (flags != 0) {
    fprintf(stderr, "device flags %u\n", flags);
    return 4;
  }
  HIP_OK(hipMemcpy(out, dout, sizeof out, hipMemcpyDeviceToHost));
  unsigned char* kp = (unsigned char*)malloc(pool_bytes);
  unsigned char* vp = (unsigned char*)malloc(pool_bytes);
  if (!kp || !vp) return 5;
  HIP_OK(hipMemcpy(kp, kb, pool_bytes, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(vp, vb, pool_bytes, hipMemcpyDeviceToHost));
  FILE* f = fopen(argv[1], "wb");
  if (!f) return 6;
  const int ok = fwrite(out, sizeof out, 1, f) == 1 && fwrite(kp, pool_bytes, 1, f) == 1 &&
                 fwrite(vp, pool_bytes, 1, f) == 1;
  fclose(f);
  free(kp);
  free(vp);
  hipFree(dq); hipFree(dk); hipFree(dv); hipFree(dout); hipFree(dpos); hipFree(dlens); hipFree(dtab);
  PKV_OK_(kv_pool_destroy(pool));
  printf("c abi driver: %d steps, %zu pool bytes\n", STEPS, pool_bytes);
  return ok ? 0 : 7;
}
