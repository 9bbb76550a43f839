"""MSA (MiniMax Sparse Attention) decode for AMD Instinct MI355X (gfx950).

The decode path runs in hand-written HIP kernels behind the C ABI of
include/msa.h (libmsa.so); this package holds the kernels' sources (csrc/),
the build script and a thin ctypes binding with the same entry-point names.
"""
from ._lib import (MSAError, MSA_OK, MSA_ERR_INVALID_ARG, MSA_ERR_UNSUPPORTED, MSA_ERR_WORKSPACE, MSA_ERR_HIP,
                   Params, Cache, DeviceCache, load, to_device, alloc_workspace,
                   msa_workspace_size, msa_indexer_scores, msa_pool_select_blocks,
                   msa_sparse_attn_decode, msa_decode_layer, msa_decode_layer_single, msa_decode_layer_single_static, msa_kv_insert, msa_debug_dequant_nvfp4, msa_debug_layer_spin_limit, msa_debug_read_bandwidth,
                   msa_debug_layer_splits, msa_decode_layer_gave_up,
                   msa_debug_dequant_fp8, EXPORTED, NUM_STAGES, STAGE_NAMES, KV_BF16, KV_NVFP4,
                   IDX_BF16, IDX_FP8, IDX_NVFP4)

__all__ = ["MSAError", "MSA_OK", "MSA_ERR_INVALID_ARG", "MSA_ERR_UNSUPPORTED", "MSA_ERR_WORKSPACE", "MSA_ERR_HIP",
           "Params", "Cache", "DeviceCache", "load", "to_device", "alloc_workspace",
           "msa_workspace_size", "msa_indexer_scores", "msa_pool_select_blocks", "msa_sparse_attn_decode",
           "msa_decode_layer", "msa_decode_layer_single", "msa_decode_layer_single_static", "msa_kv_insert", "msa_debug_dequant_nvfp4", "msa_debug_dequant_fp8", "msa_debug_layer_spin_limit", "msa_debug_read_bandwidth", "msa_debug_layer_splits", "msa_decode_layer_gave_up", "EXPORTED",
           "NUM_STAGES", "STAGE_NAMES", "KV_BF16", "KV_NVFP4", "IDX_BF16", "IDX_FP8", "IDX_NVFP4"]
