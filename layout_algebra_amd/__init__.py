"""Python binding of the MI355X tiled GEMM library (liblagemm.so).

Argument marshalling only: every step of the GEMM runs in the library's HIP
kernels.  PyTorch provides device memory and the current HIP stream; nothing
else.  The library is loaded on first use and a missing library is an error
(there is no fallback implementation).

Entry points carry the C ABI's names (include/la_gemm.h):
    gemm_plan, gemm_run, gemm_plan_workspace_bytes, gemm_run_split, gemm_run_split_noalloc, gemm_run_reduce, gemm_gate_up_run, gemm_gate_up_swiglu_run, gemm_plan_describe,
    la_rms_norm_run, la_attention_run, gemm_plan_lds_offset, gemm_plan_lds_stage_bytes, gemm_debug_lds_image,
    la_probe_mfma (matrix-core rate probe, a measurement aid), la_layout_eval, la_layout_eval_index, la_swizzle_apply, la_tile_plan_offset,
    la_layout_eval_str, la_layout_tile_str, la_layout_coalesce_str, la_layout_permute_str, la_layout_cosize_str,
    la_view_window_eval (the pages' "shape:stride" notation)
"""
from ._lib import (  # noqa: F401
    BF16, F16, F32, F8E4M3, F8E5M2, FLAG_GATE_UP, FLAG_B_KMAJOR, FLAG_LARGE_TILES, FLAG_A_TRANSPOSED, GemmError, Plan, EXPORTED_SYMBOLS, lib_path, load,
    gemm_plan, gemm_run, gemm_plan_workspace_bytes, gemm_run_split, gemm_run_split_noalloc, gemm_run_reduce, gemm_gate_up_run, gemm_gate_up_swiglu_run, gemm_plan_describe,
    gemm_plan_lds_offset,
    gemm_plan_lds_stage_bytes, gemm_debug_lds_image, la_layout_eval, la_layout_eval_index,
    la_swizzle_apply, la_tile_plan_offset, la_rms_norm_run, la_attention_run, la_probe_mfma,
    la_layout_eval_str, la_layout_tile_str, la_layout_coalesce_str, la_layout_permute_str, la_layout_cosize_str,
    la_view_window_eval,
)
