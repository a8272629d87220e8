// dispatch.cpp -- the launch interface of kernels.h over the three cache
// types, whose kernels live in objects of their own.
#include "kernels.h"

namespace pkv {

hipError_t launch_decode(int kv_kind, int head_dim, int block_size, const DecodeParams& p,
                         hipStream_t stream, hipEvent_t* events) {
  switch (kv_kind) {
    case KV_F32: return decode_dispatch<KV_F32>(head_dim, block_size, &p, stream, events, nullptr);
    case KV_BF16: return decode_dispatch<KV_BF16>(head_dim, block_size, &p, stream, events, nullptr);
    case KV_FP8: return decode_dispatch<KV_FP8>(head_dim, block_size, &p, stream, events, nullptr);
    default: return hipErrorInvalidValue;
  }
}

int decode_ring_tiles(int kv_kind, int head_dim) {
  switch (kv_kind) {
    case KV_F32: return decode_ring_tiles_of<KV_F32>(head_dim);
    case KV_BF16: return decode_ring_tiles_of<KV_BF16>(head_dim);
    case KV_FP8: return decode_ring_tiles_of<KV_FP8>(head_dim);
    default: return 0;
  }
}

hipError_t decode_occupancy(int kv_kind, int head_dim, int block_size, int* blocks) {
  switch (kv_kind) {
    case KV_F32: return decode_dispatch<KV_F32>(head_dim, block_size, nullptr, nullptr, nullptr, blocks);
    case KV_BF16: return decode_dispatch<KV_BF16>(head_dim, block_size, nullptr, nullptr, nullptr, blocks);
    case KV_FP8: return decode_dispatch<KV_FP8>(head_dim, block_size, nullptr, nullptr, nullptr, blocks);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
