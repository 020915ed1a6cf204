"""Sliding Tile Attention forward for AMD MI355X (gfx950).

The compute path is libsta.so (HIP kernels + C ABI, see include/sta.h); the
functions re-exported here are its ctypes binding.
"""

from .binding import (  # noqa: F401
    STA_MAX_HEADS,
    StaError,
    last_error,
    load_library,
    sliding_tile_attention,
    sta_attention,
    sta_backward,
    sta_backward_noalloc,
    sta_forward,
    sta_forward_lse,
    sta_forward_fp8,
    sta_forward_fp8_lse,
    sta_forward_raster,
    sta_full_attention,
    sta_kv_pair_count,
    sta_kv_tiles,
    sta_q_tiles,
    sta_reorder_tiles,
    sta_restore_order,
    sta_tile_list_len,
    sta_window_recall,
    sta_window_recall_fp8,
    tile_major_rows,
)
