// Host-side GEMM planner: picks a kernel, builds and validates its layouts.
#pragma once

#include <string>

#include "../../include/la_gemm.h"
#include "kernel_table.hpp"
#include "launch.hpp"
#include "layout.hpp"

struct gemm_plan_s {
  gemm_desc d;
  gemm_desc kd;              // what the kernel runs on: d, or for one-byte inputs d with k, lda, ldb and the
                             // A / B batch strides counted in 16-bit units (byte pairs)
  int kid = 0;
  int in_kind = 0, out_kind = 0;
  int in_bytes = 2;          // bytes per A / B element (2: bf16 / f16, 4: binary32, 1: E4M3 / E5M2)
  int vec = 1;               // elements per global vector load of A and B
  int align_bytes = 2;       // required alignment of the A / B / W pointers
  int out_bytes = 4;         // bytes per C element
  int out_align_bytes = 4;   // required alignment of the C / G / U pointers
  bool gate_up = false;
  bool b_kmajor = false;     // B (and the gate/up weights) stored [N, K]
  bool a_trans = false;      // A (and X) stored [K, M]
  int tiles_m = 0, tiles_n = 0, grid = 0, group_m = 8;
  // gemm_run_split: K cut into `split` equal ranges, each range's FP32 partial product written by
  // kernel `split_kid` (the skinny kernel: one column strip per workgroup; or the 256-wide kernel:
  // one tile per workgroup; split_tiles_m x split_tiles_n of them, the ranges along the launch's y
  // dimension) into ws_bytes = split * m * n * 4 bytes of workspace, then summed in range order by
  // a second kernel that applies alpha, beta and the rounding.  split = 1: the plan has no split
  // form and gemm_run_split runs as gemm_run.
  int split = 1, split_kid = 0, split_tiles_m = 1, split_tiles_n = 0;
  int64_t ws_bytes = 0;
  int64_t stage_elems = 0, lds_bytes = 0;
  lak::KernelShape shape{};
  la::View lds_a, lds_b, lds_b2;     // operand block maps in (row, col) tile coordinates
  int64_t base_a = 0, base_b = 0, base_b2 = 0;  // element offsets of each block in a stage
  la::Layout glob_a, glob_b, glob_c;  // operands in global memory, tiled by the kernel's tile (covering extents)
  std::string copy_json, store_json;  // copy and store plans as described (coalesced per wave instruction)
  std::string json;
};

namespace plan {

// The full-tile direct-load kernels (LDS-staged 16-byte epilogue stores).
bool is_fast(int kid);

// Build a plan; on failure returns a status and sets *err.
gemm_status build(const gemm_desc& d, gemm_plan_s& p, std::string* err);

// Element offset of operand (0 = A, 1 = B / W_gate, 2 = W_up) element (row, col) in a stage.
gemm_status lds_offset(const gemm_plan_s& p, int operand, int64_t row, int64_t col, int64_t* out, std::string* err);

}  // namespace plan
