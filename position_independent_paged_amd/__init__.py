"""Position-free paged prefill attention for AMD Instinct MI355X (gfx950).

The compute path is libminipic.so (HIP C++, see include/minipic.h); this
package is its thin Python binding plus device staging helpers. The library
is loaded on the first call into it (or by ``load_library()``), which raises
ImportError if it has not been built: there is no fallback path.
"""
from ._binding import (BlockCache, MINIPIC_ERR_CACHE_FULL, MINIPIC_ERR_CONTRACT, minipic_describe_blocks,
                       minipic_slot_mapping, EXPORTS, MINIPIC_BF16, MINIPIC_BLK_GLOBAL, MINIPIC_BLK_PDEP, MINIPIC_EW_BLOCK,
                       MINIPIC_EW_CTX, MINIPIC_EW_POS, MINIPIC_EW_QCTX, MINIPIC_F32, MINIPIC_FLAG_ROTATE_Q,
                       LIB_PATH, MinipicError, load_library, minipic_batch, minipic_get_launch_info,
                       minipic_decode_attn, minipic_decode_prerotated, minipic_decode_workspace_size,
                       minipic_kernel_times, minipic_kernel_times_all, minipic_prefill_attn,
                       minipic_prefill_attn_static, MINIPIC_STATIC_WORKSPACE_BYTES, minipic_prefill_plan,
                       minipic_prefill_run, MINIPIC_EW_SPAN, MINIPIC_EW_PLAN,
                       minipic_reference_prerotated,
                       minipic_rope_table, minipic_set_kernel_timing, minipic_version, minipic_workspace_size,
                       minipic_write_kv)


__all__ = [
    "BlockCache", "MINIPIC_ERR_CACHE_FULL", "MINIPIC_ERR_CONTRACT", "minipic_describe_blocks", "minipic_slot_mapping",
    "EXPORTS", "LIB_PATH", "MinipicError", "load_library", "minipic_batch", "minipic_get_launch_info",
    "minipic_prefill_attn", "minipic_prefill_attn_static", "MINIPIC_STATIC_WORKSPACE_BYTES",
    "minipic_prefill_plan", "minipic_prefill_run", "MINIPIC_EW_SPAN", "MINIPIC_EW_PLAN",
    "minipic_reference_prerotated", "minipic_rope_table", "minipic_version",
    "minipic_set_kernel_timing", "minipic_kernel_times", "minipic_kernel_times_all", "minipic_decode_workspace_size",
    "minipic_decode_attn", "minipic_decode_prerotated",
    "minipic_workspace_size", "minipic_write_kv", "MINIPIC_BF16", "MINIPIC_F32", "MINIPIC_BLK_PDEP",
    "MINIPIC_BLK_GLOBAL", "MINIPIC_FLAG_ROTATE_Q", "MINIPIC_EW_BLOCK", "MINIPIC_EW_POS", "MINIPIC_EW_QCTX",
    "MINIPIC_EW_CTX",
]
