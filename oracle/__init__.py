"""CPU oracle of the AWQ search, INT4 pack and W4A16 path (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this package;
the GPU library does not, and the two share no code.
"""
from .awq_oracle import (accuracy_report, act_stats, alpha_grid, argmin_lowest, clip_grid,
                         clip_search, code_range, dequant_scaled, error_matrix, fold_scale, gram,
                         group_errors, loss_gram, output_loss, pack_int4, pack_layer, quantize,
                         quantize_zp,
                         relative_gap, scale_table, search_layer, search_shared, unpack_int4,
                         unpack_uint4, w4a16)

__all__ = ["accuracy_report", "act_stats", "alpha_grid", "argmin_lowest", "clip_grid",
           "clip_search", "code_range", "dequant_scaled", "error_matrix", "fold_scale", "gram",
           "group_errors", "loss_gram", "output_loss", "pack_int4", "pack_layer", "quantize",
           "quantize_zp", "unpack_uint4",
           "relative_gap", "scale_table", "search_layer", "search_shared", "unpack_int4", "w4a16"]
