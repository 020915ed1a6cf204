"""CPU oracle for Sliding Tile Attention -- test infrastructure only.

Imported by the tests, the smoke check and the benchmark's CPU-baseline leg;
the library under ``sparse_attention_video_tile_amd`` never imports it.
"""
from .sta_oracle import *  # noqa: F401,F403
from .sta_backward_oracle import (  # noqa: F401
    q_tile_lists,
    sta_backward,
    sta_backward_key_rows,
    sta_backward_query_rows,
    sta_lse,
    window_recall,
)
from .sta_fp8_oracle import e4m3_decode, sta_attention_fp8, sta_attention_fp8_rows, sta_lse_fp8, window_recall_fp8  # noqa: F401
