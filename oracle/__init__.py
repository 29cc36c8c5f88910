"""Oracle for the int2 draft LM head. TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may import this package.
The product path (the HIP library and its Python binding) never imports, calls or links it.

Parity status: every function is pinned by the CPU tests in tests/test_oracle_pins.py against
values fixed by the page or by mathematics (closed forms, exact-grid constructions, brute force
on small inputs, invariants and byte counts the page prints).
"""
from .int2_head import (BLOCK_N, GROUP, bf16_to_f32, block_emit, check_shape, coarse_logits,
                        dequantize, exact_logits, f32_to_bf16, finalize, fp8_e4m3_decode, fp8_rows_f32,
                        group_sums, head, head4, logits_row, pack, pack4, pack_fp8, pack_half_split,
                        premultiplied_scales4, quantize4, quantize_fp8, rerank_exact_fp8, coarse_logits4,
                        dequantize4, unpack_half_split, check_shape4,
                        pack_quarter_split, premultiplied_scales, quantize, rerank_exact,
                        select_top_r, storage_bytes, unpack_quarter_split,
                        pack_contiguous4, unpack_contiguous4, pack_variant, coarse_logits_contiguous4,
                        dequantize_tile, coarse_logits_tile, select_tokens)

__all__ = ["BLOCK_N", "GROUP", "bf16_to_f32", "block_emit", "check_shape", "coarse_logits",
           "dequantize", "exact_logits", "f32_to_bf16", "finalize", "fp8_e4m3_decode", "fp8_rows_f32",
           "group_sums", "head", "head4", "logits_row", "pack", "pack4", "pack_fp8", "pack_half_split",
           "premultiplied_scales4", "quantize4", "quantize_fp8", "rerank_exact_fp8", "coarse_logits4",
           "dequantize4", "unpack_half_split", "check_shape4",
           "pack_quarter_split", "premultiplied_scales", "quantize", "rerank_exact",
           "select_top_r", "storage_bytes", "unpack_quarter_split",
           "pack_contiguous4", "unpack_contiguous4", "pack_variant", "coarse_logits_contiguous4",
           "dequantize_tile", "coarse_logits_tile", "select_tokens"]
