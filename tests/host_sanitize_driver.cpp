// host_sanitize_driver.cpp -- drives the library's host-only entry points
// (block allocator, argument checks, RoPE table, work-partition replay) over
// seeded random inputs, valid and invalid, for a build under AddressSanitizer,
// UndefinedBehaviorSanitizer and LeakSanitizer.  It checks only what needs no
// reference (statuses, conservation of blocks, every tile planned once); the
// exact results are the Python tests' business.  Exit status 0 = clean.
#include <stdint.h>

#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "pkv.h"

#define CHECK(cond)                                                       \
  do {                                                                    \
    if (!(cond)) {                                                        \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      std::exit(2);                                                       \
    }                                                                     \
  } while (0)

static void allocator_rounds(std::mt19937& rng) {
  for (int round = 0; round < 200; ++round) {
    const int64_t nb = 4 + rng() % 60;
    const int32_t bs = 1 << (rng() % 5);
    const int32_t ms = 1 + rng() % 12;
    pkv_block_alloc* a = nullptr;
    CHECK(pkv_alloc_create(nb, bs, ms, &a) == PKV_OK && a);
    std::vector<int32_t> live;
    for (int op = 0; op < 300; ++op) {
      const int kind = rng() % 6;
      if (kind == 0) {
        int32_t s = -1;
        if (pkv_seq_add(a, rng() % (3 * bs + 3), &s) == PKV_OK) live.push_back(s);
      } else if (kind == 1 && !live.empty()) {
        int32_t c = -1;
        if (pkv_seq_fork(a, live[rng() % live.size()], &c) == PKV_OK) live.push_back(c);
      } else if (kind == 2 && !live.empty()) {
        const size_t i = rng() % live.size();
        CHECK(pkv_seq_release(a, live[i]) == PKV_OK);
        live.erase(live.begin() + i);
      } else if (kind == 5) {
        // invalid ids and sizes are refused, and leave the state alone
        CHECK(pkv_seq_release(a, -1) == PKV_ERR_INVALID);
        CHECK(pkv_seq_release(a, ms + 3) == PKV_ERR_INVALID);
        int32_t s = 0;
        CHECK(pkv_seq_add(a, -5, &s) == PKV_ERR_INVALID);
      } else if (!live.empty()) {
        const int32_t batch = 1 + rng() % live.size();
        std::vector<int32_t> ids(live.begin(), live.begin() + batch);
        if (rng() % 8 == 0) ids.push_back(ids[0]);          // a repeated id
        const int32_t maxb = 1 + rng() % 10, maxc = rng() % (batch + 1);
        std::vector<int32_t> tab((size_t)ids.size() * maxb), lens(ids.size()), pos(ids.size()),
            cp(2 * (size_t)(maxc + 1));
        int32_t n = -1;
        const pkv_status st = pkv_alloc_prepare_step(a, ids.data(), (int32_t)ids.size(), maxb,
                                                     tab.data(), lens.data(), pos.data(),
                                                     cp.data(), maxc, &n);
        CHECK(st == PKV_OK || st == PKV_ERR_INVALID || st == PKV_ERR_OOM);
        if (st == PKV_OK) CHECK(n >= 0 && n <= maxc);
      }
      int64_t fb = -1;
      int32_t ls = -1;
      CHECK(pkv_alloc_stats(a, &fb, &ls) == PKV_OK);
      CHECK(fb >= 0 && fb <= nb && ls == (int32_t)live.size());
      for (int32_t s : live) {
        int32_t len = -1, nblk = -1;
        std::vector<int32_t> blocks(64);
        CHECK(pkv_seq_info(a, s, &len, &nblk, blocks.data(), 64) == PKV_OK);
        for (int32_t j = 0; j < nblk && j < 64; ++j) {
          int32_t rc = 0;
          CHECK(pkv_alloc_refcount(a, blocks[j], &rc) == PKV_OK && rc >= 1);
        }
      }
    }
    for (int32_t s : live) CHECK(pkv_seq_release(a, s) == PKV_OK);
    int64_t fb = -1;
    CHECK(pkv_alloc_stats(a, &fb, nullptr) == PKV_OK && fb == nb);
    CHECK(pkv_alloc_destroy(a) == PKV_OK);
  }
  pkv_block_alloc* a = nullptr;
  CHECK(pkv_alloc_create(0, 16, 4, &a) == PKV_ERR_INVALID);
}

static void plan_rounds(std::mt19937& rng) {
  for (int round = 0; round < 300; ++round) {
    const int32_t batch = 1 + rng() % 300, hkv = 1 + rng() % 8;
    const int32_t max_tokens = 1 + rng() % 20000;
    std::vector<int32_t> lens(batch);
    for (auto& L : lens) L = (int32_t)(rng() % (max_tokens + 3)) - 1;    // some out of range
    const int32_t n_waves = 4 * (1 + rng() % 300), min_units = 1 + rng() % 40;
    const int32_t cost = rng() % 9, window = rng() % 3 ? 0 : 1 + rng() % 3000;
    const int32_t odd = 1 + rng() % 100, rest = 1 + rng() % 100;
    const int32_t max_pieces = rng() % 4 ? 1 << 20 : rng() % 50;   // sometimes too few rows
    std::vector<int32_t> pieces(6 * (size_t)std::max(max_pieces, 1)), splits(4 * (size_t)n_waves);
    int32_t n = -1;
    const pkv_status st = pkv_plan_host(lens.data(), batch, hkv, max_tokens, n_waves,
                                        std::max(min_units, cost + 1), cost, 4 * (rng() % 64),
                                        100, rest, odd, 256, window, max_pieces, pieces.data(),
                                        &n, splits.data());
    CHECK(st == PKV_OK && n >= 1);
    if (n <= max_pieces) {
      // every planned tile belongs to exactly one piece, in order
      int64_t tiles = 0;
      for (int32_t i = 0; i < n; ++i) {
        const int32_t* r = &pieces[6 * (size_t)i];
        CHECK(r[1] >= 0 && r[1] < batch && r[2] >= 0 && r[2] < hkv && r[3] < r[4]);
        tiles += r[4] - r[3];
      }
      CHECK(tiles > 0);
    }
  }
  int32_t n = 0, lens[1] = {5}, splits[4];
  CHECK(pkv_plan_host(nullptr, 1, 1, 16, 1, 1, 0, 0, 1, 1, 100, 0, 0, 0, nullptr, &n, splits) ==
        PKV_ERR_INVALID);
  CHECK(pkv_plan_host(lens, 1, 1, 16, 1, 1, 65, 0, 1, 1, 100, 0, 0, 0, nullptr, &n, splits) ==
        PKV_ERR_INVALID);
}

static void check_rounds(std::mt19937& rng) {
  const pkv_dtype dts[] = {PKV_F32, PKV_BF16, PKV_FP8_E4M3, (pkv_dtype)7};
  for (int round = 0; round < 20000; ++round) {
    const pkv_dtype kv = dts[rng() % 4], io = dts[rng() % 4];
    const int32_t batch = (int32_t)(rng() % 5000) - 10, hkv = (int32_t)(rng() % 20) - 2;
    const int32_t hq = (int32_t)(rng() % 300) - 5, d = (rng() % 3) ? 128 : 96;
    const int32_t bs = 1 << (3 + rng() % 4), maxb = (int32_t)(rng() % 5000) - 2;
    const uintptr_t base = (rng() % 4) ? 0x10000 : 0x10004;
    const pkv_status st = pkv_check_decode_args(
        1 + rng() % 100000, bs, hkv, d, kv, io, (void*)base, (void*)(base + 0x1000),
        (void*)(base + 0x2000), (int32_t*)(base + 0x3000), (int32_t*)(base + 0x4000), maxb,
        (int32_t*)(base + 0x5000), batch, hq, (void*)(base + 0x6000));
    CHECK(st == PKV_OK || st == PKV_ERR_INVALID || st == PKV_ERR_UNSUPPORTED);
  }
  for (int d : {2, 64, 128}) {
    const int32_t maxp = 1 + rng() % 5000;
    std::vector<float> c((size_t)maxp * d / 2), s((size_t)maxp * d / 2);
    CHECK(pkv_rope_table_host(5.0e5, d, maxp, c.data(), s.data()) == PKV_OK);
    CHECK(c[0] == 1.0f && s[0] == 0.0f);
  }
  float one = 0;
  CHECK(pkv_rope_table_host(-1.0, 64, 1, &one, &one) == PKV_ERR_INVALID);
  CHECK(pkv_rope_table_host(1e4, 63, 1, &one, &one) == PKV_ERR_INVALID);
  CHECK(pkv_tile_tokens() == 16);
  CHECK(pkv_last_error() != nullptr);
}

int main() {
  std::mt19937 rng(20241203);
  allocator_rounds(rng);
  plan_rounds(rng);
  check_rounds(rng);
  std::printf("host entry points clean\n");
  return 0;
}
