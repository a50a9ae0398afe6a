"""Weight-only block-32 int4/int8 matmul for MI355X (gfx950).

Public API (all computation runs in libwq.so's HIP kernels; PyTorch supplies
device memory and the current stream):

    pack(w, bits) -> (q, scales)        quantize + pack fp32 weights [N, K]
    unpack(q, K, bits) -> codes         int8 codes [N, K]
    gemv(x, q, scales, bits)            decode path, 1 <= M <= 16
    gemm(x, q, scales, bits)            prefill path (fp16 matrix cores)
    gemm_noalloc(x, q, scales, bits)    the same on the library's fixed per-device scratch
    linear(x, q, scales, bits)          dispatch by M
    embed(ids, q, scales, K, bits)      tied-embedding rows of a packed table, fp32
    Package / GroupedCall               64-byte-aligned package + one-launch decode step

The library is loaded on first use and must have been built
(``python -m weight_only_bit_block_amd.build``); there is no fallback.
"""
from .wq import (BLOCK, GEMV_MAX_M, GroupedCall, Package, WqError, embed, gemm, gemm_noalloc, gemv,
                 header_symbols, linear, load, pack, table_layout, table_plan, table_plan_gemm, unpack)

__all__ = ["BLOCK", "GEMV_MAX_M", "GroupedCall", "Package", "WqError", "embed", "gemm", "gemm_noalloc", "gemv",
           "header_symbols", "linear", "load", "pack", "table_layout", "table_plan", "table_plan_gemm", "unpack"]
