"""MI355X-native fused-dequant quantized GEMV/GEMM (Q4_K, Q5_K, Q6_K, NVFP4 W4A16, block-scaled FP8 W8A16).

The product runs in libqgemm.so (hand-written HIP for gfx950) behind the C ABI
of include/qgemm.h; this package is its ctypes binding.
"""
from ._lib import (FP8, LAYOUT_ROWS, LAYOUT_TILES, MAX_ROWS, NVFP4, Q4_K, Q5_K, Q6_K, QGError, QWeight, lib, qdequant, qgemm_prefill, qgemm_rows,
                   qgemv, qgemv_add, qgemv_fp8, qgemv_nvfp4, qgemv_pair, qgemv_pair_swiglu, qgemv_q4k, qgemv_q5k,
                   qgemv_q6k, qgemv_triple, pack_tiles, qg_stream_read, row_bytes)

__all__ = ["FP8", "LAYOUT_ROWS", "LAYOUT_TILES", "MAX_ROWS", "NVFP4", "Q4_K", "Q5_K", "Q6_K", "QGError", "QWeight", "lib", "qdequant", "qgemm_prefill",
           "qgemm_rows", "qgemv", "qgemv_add", "qgemv_fp8", "qgemv_nvfp4", "qgemv_pair", "qgemv_pair_swiglu",
           "qgemv_q4k", "qgemv_q5k", "qgemv_q6k", "qgemv_triple", "pack_tiles", "qg_stream_read", "row_bytes"]
