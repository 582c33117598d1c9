"""Exact IO-aware attention (fused tiled forward, recompute backward) for AMD MI355X (gfx950).

The compute runs in the HIP library libflashattn.so (C ABI in include/flash_attn.h); this
package holds its Python binding, the in-tree build step and the seeded input recipe.
"""
from .flash_attn import (FA_DTYPE_BF16, FA_DTYPE_FP16, FA_DTYPE_FP32, FA_MASK_BLOCK, FlashAttnFunction,
                         flash_attention, flash_attn_bwd, flash_attn_bwd_delta, flash_attn_bwd_dkdv, flash_attn_bwd_dq,
                         flash_attn_bwd_masked, flash_attn_bwd_workspace_size, flash_attn_dropout_mask, flash_attn_fwd, flash_attn_fwd_kvsplit,
                         flash_attn_fwd_kvsplit_noalloc, flash_attn_fwd_kvsplit_workspace_size, flash_attn_fwd_masked, flash_attn_status_string,
                         load_library)

__all__ = ["FA_DTYPE_BF16", "FA_DTYPE_FP16", "FA_DTYPE_FP32", "FA_MASK_BLOCK", "FlashAttnFunction", "flash_attention", "flash_attn_bwd",
           "flash_attn_bwd_delta", "flash_attn_bwd_dkdv", "flash_attn_bwd_dq", "flash_attn_bwd_workspace_size",
           "flash_attn_fwd", "flash_attn_fwd_kvsplit", "flash_attn_fwd_kvsplit_noalloc", "flash_attn_fwd_kvsplit_workspace_size", "flash_attn_fwd_masked",
           "flash_attn_bwd_masked", "flash_attn_dropout_mask",
           "flash_attn_status_string", "load_library"]
