// block_alloc.cpp -- host-side block allocator for the paged KV pool.
//
// The pages keep the cache in fixed-size blocks handed out on demand as
// tokens are generated, with waste bounded by the last, partly filled block
// of each request ("TensorRT-LLM Guide: High-Throughput GPU Inference
// Engine", section "2. Paged KV Cache & Memory Virtualization"); the
// scheduler updates each request's block table every iteration ("Scaling
// TensorRT-LLM: Kernel Fusion and Inflight Batching in Production", section
// "What the Scheduler Actually Does"); and blocks are reused across requests
// that share a prefix, such as a common system prompt ("Lesson 13.17
// TensorRT-LLM: NVIDIA's Optimized Inference Engine", section "The paged KV
// cache, in-flight batching and CUDA graphs").
//
// Here a sequence owns a list of block ids; a block may be held by several
// sequences (a shared prefix) and carries a reference count.  Before a step
// appends a token to a block that other sequences still hold, the appending
// sequence gets a fresh block and a copy of the shared one (copy on write),
// so no sequence ever sees another's appended token.  Free blocks sit on a
// stack: a fresh allocator hands out 0, 1, 2, ... and a freed block is the
// next one handed out.
#include <stdint.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <set>
#include <unordered_map>
#include <vector>

#include "../../include/pkv.h"

#include "host_errors.h"

namespace {

pkv_status afail(pkv_status s, const char* fmt, ...) {
  char buf[256];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  return pkv::set_error(s, buf);
}

}  // namespace

struct pkv_block_alloc {
  int64_t num_blocks = 0;
  int32_t block_size = 0;
  int32_t max_seqs = 0;
  std::vector<int32_t> free_stack;     // top = back()
  std::vector<int32_t> refcount;       // per block
  struct Seq {
    bool live = false;
    int32_t len = 0;
    std::vector<int32_t> blocks;
  };
  std::vector<Seq> seqs;
  std::set<int32_t> free_ids;          // the lowest is handed out first

  int32_t pop_block() {
    const int32_t b = free_stack.back();
    free_stack.pop_back();
    refcount[b] = 1;
    return b;
  }
  void drop_block(int32_t b) {
    if (--refcount[b] == 0) free_stack.push_back(b);
  }
  bool valid_seq(int32_t s) const {
    return s >= 0 && s < max_seqs && seqs[s].live;
  }
  int32_t blocks_for(int64_t len) const {
    return (int32_t)((len + block_size - 1) / block_size);
  }
};

extern "C" {

pkv_status pkv_alloc_create(int64_t num_blocks, int32_t block_size, int32_t max_seqs,
                            pkv_block_alloc** out) {
  if (!out) return afail(PKV_ERR_INVALID, "out is null");
  *out = nullptr;
  if (num_blocks < 1 || num_blocks > INT32_MAX)
    return afail(PKV_ERR_INVALID, "num_blocks must be in [1, 2^31)");
  if (block_size < 1) return afail(PKV_ERR_INVALID, "block_size must be >= 1");
  if (max_seqs < 1) return afail(PKV_ERR_INVALID, "max_seqs must be >= 1");
  pkv_block_alloc* a = new pkv_block_alloc;
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  a->max_seqs = max_seqs;
  a->free_stack.resize((size_t)num_blocks);
  for (int64_t i = 0; i < num_blocks; ++i) a->free_stack[(size_t)i] = (int32_t)(num_blocks - 1 - i);
  a->refcount.assign((size_t)num_blocks, 0);
  a->seqs.resize((size_t)max_seqs);
  for (int32_t i = 0; i < max_seqs; ++i) a->free_ids.insert(a->free_ids.end(), i);
  *out = a;
  return PKV_OK;
}

pkv_status pkv_alloc_destroy(pkv_block_alloc* a) {
  delete a;
  return PKV_OK;
}

pkv_status pkv_alloc_stats(const pkv_block_alloc* a, int64_t* free_blocks, int32_t* live_seqs) {
  if (!a) return afail(PKV_ERR_INVALID, "allocator is null");
  if (free_blocks) *free_blocks = (int64_t)a->free_stack.size();
  if (live_seqs) *live_seqs = a->max_seqs - (int32_t)a->free_ids.size();
  return PKV_OK;
}

pkv_status pkv_alloc_refcount(const pkv_block_alloc* a, int32_t block, int32_t* count) {
  if (!a || !count) return afail(PKV_ERR_INVALID, "null argument");
  if (block < 0 || block >= a->num_blocks) return afail(PKV_ERR_INVALID, "block %d out of range", block);
  *count = a->refcount[(size_t)block];
  return PKV_OK;
}

pkv_status pkv_seq_add(pkv_block_alloc* a, int32_t length, int32_t* seq) {
  if (!a || !seq) return afail(PKV_ERR_INVALID, "null argument");
  if (length < 0) return afail(PKV_ERR_INVALID, "length must be >= 0");
  if (a->free_ids.empty()) return afail(PKV_ERR_OOM, "all %d sequence ids in use", a->max_seqs);
  const int32_t nb = a->blocks_for(length);
  if ((size_t)nb > a->free_stack.size())
    return afail(PKV_ERR_OOM, "%d blocks needed, %zu free", nb, a->free_stack.size());
  const int32_t id = *a->free_ids.begin();
  a->free_ids.erase(a->free_ids.begin());
  pkv_block_alloc::Seq& s = a->seqs[(size_t)id];
  s.live = true;
  s.len = length;
  s.blocks.clear();
  for (int32_t j = 0; j < nb; ++j) s.blocks.push_back(a->pop_block());
  *seq = id;
  return PKV_OK;
}

pkv_status pkv_seq_fork(pkv_block_alloc* a, int32_t parent, int32_t* child) {
  if (!a || !child) return afail(PKV_ERR_INVALID, "null argument");
  if (!a->valid_seq(parent)) return afail(PKV_ERR_INVALID, "sequence %d is not live", parent);
  if (a->free_ids.empty()) return afail(PKV_ERR_OOM, "all %d sequence ids in use", a->max_seqs);
  const int32_t id = *a->free_ids.begin();
  a->free_ids.erase(a->free_ids.begin());
  pkv_block_alloc::Seq& c = a->seqs[(size_t)id];
  const pkv_block_alloc::Seq& p = a->seqs[(size_t)parent];
  c.live = true;
  c.len = p.len;
  c.blocks = p.blocks;
  for (int32_t b : c.blocks) ++a->refcount[(size_t)b];
  *child = id;
  return PKV_OK;
}

pkv_status pkv_seq_release(pkv_block_alloc* a, int32_t seq) {
  if (!a) return afail(PKV_ERR_INVALID, "allocator is null");
  if (!a->valid_seq(seq)) return afail(PKV_ERR_INVALID, "sequence %d is not live", seq);
  pkv_block_alloc::Seq& s = a->seqs[(size_t)seq];
  // the last block first, so that a released sequence's first block is the
  // next one handed out
  for (auto it = s.blocks.rbegin(); it != s.blocks.rend(); ++it) a->drop_block(*it);
  s.blocks.clear();
  s.len = 0;
  s.live = false;
  a->free_ids.insert(seq);
  return PKV_OK;
}

pkv_status pkv_seq_info(const pkv_block_alloc* a, int32_t seq, int32_t* length,
                        int32_t* n_blocks, int32_t* blocks, int32_t max_blocks) {
  if (!a) return afail(PKV_ERR_INVALID, "allocator is null");
  if (!a->valid_seq(seq)) return afail(PKV_ERR_INVALID, "sequence %d is not live", seq);
  const pkv_block_alloc::Seq& s = a->seqs[(size_t)seq];
  if (length) *length = s.len;
  if (n_blocks) *n_blocks = (int32_t)s.blocks.size();
  if (blocks)
    for (int32_t j = 0; j < std::min<int32_t>(max_blocks, (int32_t)s.blocks.size()); ++j)
      blocks[j] = s.blocks[(size_t)j];
  return PKV_OK;
}

pkv_status pkv_alloc_prepare_step(pkv_block_alloc* a, const int32_t* seq_ids, int32_t batch,
                                  int32_t max_blocks_per_seq, int32_t* block_tables,
                                  int32_t* context_lens, int32_t* positions, int32_t* copies,
                                  int32_t max_copies, int32_t* n_copies) {
  if (!a || !n_copies || (batch > 0 && (!seq_ids || !block_tables || !context_lens || !positions)))
    return afail(PKV_ERR_INVALID, "null argument");
  if (batch < 0) return afail(PKV_ERR_INVALID, "batch must be >= 0");
  if (max_blocks_per_seq < 1) return afail(PKV_ERR_INVALID, "max_blocks_per_seq must be >= 1");
  *n_copies = 0;
  // Everything is checked and counted before anything changes: a failing
  // call leaves the allocator as it was.
  std::vector<char> seen((size_t)a->max_seqs, 0);
  std::unordered_map<int32_t, int32_t> writers;   // shared block -> batch members appending to it
  int64_t fresh = 0;
  for (int32_t i = 0; i < batch; ++i) {
    const int32_t s = seq_ids[i];
    if (!a->valid_seq(s)) return afail(PKV_ERR_INVALID, "sequence %d (batch row %d) is not live", s, i);
    if (seen[(size_t)s]) return afail(PKV_ERR_INVALID, "sequence %d appears twice in the batch", s);
    seen[(size_t)s] = 1;
    const pkv_block_alloc::Seq& q = a->seqs[(size_t)s];
    const int64_t slot = q.len;                   // the new token's slot
    if (a->blocks_for(slot + 1) > max_blocks_per_seq)
      return afail(PKV_ERR_INVALID, "sequence %d grows to %lld tokens, above %d blocks", s,
                   (long long)(slot + 1), max_blocks_per_seq);
    if (slot % a->block_size == 0) {
      ++fresh;
    } else {
      const int32_t b = q.blocks[(size_t)(slot / a->block_size)];
      if (a->refcount[(size_t)b] > 1) ++writers[b];
    }
  }
  int64_t n_cow = 0;
  for (const auto& kv : writers) {
    // if every holder of the block appends in this step, the last one keeps it
    n_cow += kv.second - (a->refcount[(size_t)kv.first] == kv.second ? 1 : 0);
  }
  if (n_cow > max_copies || (n_cow > 0 && !copies))
    return afail(PKV_ERR_INVALID, "%lld block copies needed, room for %d", (long long)n_cow,
                 max_copies);
  if (fresh + n_cow > (int64_t)a->free_stack.size())
    return afail(PKV_ERR_OOM, "%lld blocks needed, %zu free", (long long)(fresh + n_cow),
                 a->free_stack.size());

  int32_t nc = 0;
  for (int32_t i = 0; i < batch; ++i) {
    pkv_block_alloc::Seq& q = a->seqs[(size_t)seq_ids[i]];
    const int64_t slot = q.len;
    if (slot % a->block_size == 0) {
      q.blocks.push_back(a->pop_block());
    } else {
      int32_t& b = q.blocks[(size_t)(slot / a->block_size)];
      if (a->refcount[(size_t)b] > 1) {
        const int32_t dst = a->pop_block();
        copies[2 * nc] = b;
        copies[2 * nc + 1] = dst;
        ++nc;
        --a->refcount[(size_t)b];
        b = dst;
      }
    }
    q.len = (int32_t)(slot + 1);
    int32_t* row = block_tables + (int64_t)i * max_blocks_per_seq;
    const int32_t nb = (int32_t)q.blocks.size();
    std::copy(q.blocks.begin(), q.blocks.end(), row);
    std::fill(row + nb, row + max_blocks_per_seq, -1);
    context_lens[i] = q.len;
    positions[i] = q.len - 1;
  }
  *n_copies = nc;
  return PKV_OK;
}

}  // extern "C"
