"""qwg: fused dequantize + GEMV over block-quantized weights (Q4_K, IQ3) for MI355X.

The compute path is the HIP library ``libqwg.so`` (C ABI in ``include/qwg.h``);
this package only marshals torch tensors into its calls. Importing the package
does not load the library; the first call does, and raises if it is missing.
"""
from ._binding import (Group, Iq3Group, Q4kChain, Iq3sGroup, Iq4xsGroup, MAX_BATCH, Q4kBatchedGroup, Q4kGroup, QWG_FMT_IQ3,
                       QWG_FMT_IQ3_S, QWG_FMT_IQ3_XXS, QWG_FMT_IQ4_XS, QWG_FMT_Q4K, QwgError,
                       dequant_iq3, dequant_iq3_xxs, dequant_iq3s, dequant_iq4xs, dequant_q4k,
                       encode_iq3, gemm_q4k, gemm_q4k_noalloc, gemm_q4k_tiled, gemv_iq3, gemv_iq3_tiled, gemv_iq3_xxs,
                       gemv_iq3s, gemv_iq3s_tiled, gemv_iq4xs, gemv_iq4xs_tiled, gemv_q4k, gemv_q4k_tiled, lib,
                       pack_iq3_tiles, pack_iq3_xxs_tiles, pack_iq3s_tiles, pack_iq4xs_tiles,
                       pack_q4k_tiles, plan_splits, row_bytes, tiled_bytes, workspace_release,
                       workspace_reserve)

__all__ = ["Group", "Iq3Group", "Q4kChain", "Iq3sGroup", "Iq4xsGroup", "MAX_BATCH", "Q4kBatchedGroup", "Q4kGroup", "QWG_FMT_IQ3",
           "QWG_FMT_IQ3_S", "QWG_FMT_IQ3_XXS", "QWG_FMT_IQ4_XS", "QWG_FMT_Q4K", "QwgError",
           "dequant_iq3", "dequant_iq3_xxs", "dequant_iq3s", "dequant_iq4xs", "dequant_q4k",
           "encode_iq3", "gemm_q4k", "gemm_q4k_noalloc", "gemm_q4k_tiled", "gemv_iq3", "gemv_iq3_tiled", "gemv_iq3_xxs",
           "gemv_iq3s", "gemv_iq3s_tiled", "gemv_iq4xs", "gemv_iq4xs_tiled", "gemv_q4k", "gemv_q4k_tiled", "lib",
           "pack_iq3_tiles", "pack_iq3_xxs_tiles", "pack_iq3s_tiles", "pack_iq4xs_tiles",
           "pack_q4k_tiles", "plan_splits", "row_bytes", "tiled_bytes", "workspace_release",
           "workspace_reserve"]
