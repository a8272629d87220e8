"""CPU fp64 oracle for the paged-KV decode step.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check of ``__graft_entry__`` and the CPU
baseline leg of ``bench.py`` may import this package.  The product path (the
HIP library and its Python binding) never imports, calls or links anything
here, and nothing here imports the product.

What it computes (plain definitions, no tiling, no split, no fusion):

1. RoPE tables in fp64 math rounded to fp32 (``rope``);
2. the append of the new token: RoPE of ``k_new`` in pinned fp32 arithmetic,
   cast to the KV storage type and written to slot ``L-1`` (``decode``);
3. a gather of each request's K/V through its block table into contiguous
   arrays, dequantised exactly to fp64;
4. RoPE of the query in fp64 and ``softmax(q K^T / sqrt(D)) V`` in fp64 per
   query head, with query head ``hq`` reading KV head ``hq // G``.

The pages never write the attention formula out; they name its parts: RoPE
applied inside the attention kernel and attention that keeps its
intermediates on chip ("Scaling TensorRT-LLM: Kernel Fusion and Inflight
Batching in Production", section "What Gets Fused"), a KV cache kept in
fixed-size blocks reached through per-request block tables (same page,
section "The Paged KV-Cache: vLLM Borrowed by TensorRT-LLM"), query heads
sharing KV heads (GQA) and an E4M3 FP8 cache ("TensorRT-LLM Guide:
High-Throughput GPU Inference Engine", sections "3. Custom Fused Attention
Kernels: FMHA and XQA" and "4. Native FP8 Quantization on NVIDIA Hopper &
Blackwell").  The readings taken where the pages are silent are listed in the
docstrings of the functions that take them.

Pins (tests marked ``not gpu``): codecs against all 256 FP8 codes and torch's
casts; the FP8 cache path against the E4M3 rounding bound of the raw values,
torch's SDPA on K/V dequantised by torch, a brute force and a hand-worked
step; RoPE against closed forms and the relative-position identity;
attention against closed forms (one token, identical keys, zero query),
linearity, block-permutation invariance, a padded static batch computed on a
separate dense path, ``scaled_dot_product_attention`` in float64 and an
mpmath brute force on tiny inputs; the dense-history steps against
``decode_step`` on paged layouts of the same histories; the allocator
against its invariants (reference counts equal the holders, blocks conserved,
an appending sequence's block exclusive) and a token-level simulation of the
pool.  No function here is "parity unpinned".
"""
from .codecs import (bf16_bits_from_f32, bf16_bits_to_f32, bf16_bits_to_f64,
                     fp8_code_value, fp8_encode, fp8_decode, FP8_MAX)
from .rope import inv_freq, rope_rows_f32, rope_f64, rope_k_f32
from .decode import (decode_step, decode_step_multi, gather_request, attention_request,
                     io_to_f64, io_to_f32, kv_to_f64, fp8_inverse_scale,
                     cast_to_kv)
from .variants import (padded_static_batch, split_merge,
                       brute_force_rotate_key, brute_force_attention)
from .block_alloc import BlockAllocator, AllocError
from .history import DenseHistories

__all__ = [
    "bf16_bits_from_f32", "bf16_bits_to_f32", "bf16_bits_to_f64",
    "fp8_code_value", "fp8_encode", "fp8_decode", "FP8_MAX",
    "inv_freq", "rope_rows_f32", "rope_f64", "rope_k_f32",
    "decode_step", "decode_step_multi", "gather_request", "attention_request", "io_to_f64",
    "io_to_f32", "kv_to_f64", "fp8_inverse_scale", "cast_to_kv",
    "padded_static_batch", "split_merge", "brute_force_rotate_key",
    "brute_force_attention", "BlockAllocator", "AllocError", "DenseHistories",
]
