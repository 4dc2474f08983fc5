"""AWQ search, INT4 pack and W4A16 on AMD MI355X (gfx950).

The engine is the HIP library libawq.so (C ABI in include/awq.h); this package holds its sources
(csrc/), the in-tree build (build.py) and a thin torch binding (api.py) with the same call names.
"""
from .api import (AwqConfig, ClipResult, PackResult, SearchResult, act_stats,
                  act_stats_noalloc, act_stats_workspace_bytes, clip_search, clip_search_gram,
                  clip_workspace_bytes, fold_scale, pack_int4, search_layer, search_layers, search_workspace_bytes,
                  stats_search_layer, w4a16_gemm, w4a16_gemm_ws, w4a16_gemm_workspace_bytes)
from ._lib import AwqError

__all__ = ["AwqConfig", "AwqError", "ClipResult", "PackResult", "SearchResult", "act_stats",
           "act_stats_noalloc", "act_stats_workspace_bytes", "clip_search", "clip_search_gram",
           "clip_workspace_bytes", "fold_scale", "pack_int4", "search_layer", "search_layers", "search_workspace_bytes",
           "stats_search_layer", "w4a16_gemm", "w4a16_gemm_ws", "w4a16_gemm_workspace_bytes"]
