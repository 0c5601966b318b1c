// Interface between the host planner / C ABI and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lak {

// Everything one launch of a tiled kernel needs; plain values only.
struct TiledArgs {
  const uint16_t* A;     // [M, K] row-major, lda
  const uint16_t* B;     // [K, N] N contiguous, ldb (W_gate for gate/up)
  const uint16_t* B2;    // W_up for gate/up, else unused
  void* C;               // [M, N] row-major, ldc (G for gate/up)
  void* C2;              // U for gate/up
  int64_t M, N, K, lda, ldb, ldc;
  float alpha, beta;
  int tiles_m, tiles_n, group_m;
  int dbg_tm, dbg_tn;    // LDS-image debug launch: tile to stage
  uint16_t* dbg_out;     // LDS-image debug launch: destination of one stage
};

enum KernelId : int {
  KID_TILED_128 = 0,     // 128x128x64 tile, 4 waves of 64x64
  KID_COUNT
};

enum InKind : int { IN_BF16 = 0, IN_F16 = 1 };
enum OutKind : int { OUT_F32 = 0, OUT_BF16 = 1, OUT_F16 = 2 };

struct KernelShape {
  int bm, bn, bk;
  int waves_m, waves_n;
  int threads;
  int mfma_m, mfma_n, mfma_k;
  int sw_b, sw_m, sw_s;    // LDS swizzle (element offsets)
  int stages;
};

// Static description of each kernel id (host and device agree through this table).
KernelShape kernel_shape(int kid);

// LDS elements (16-bit) of one pipeline stage for a kernel id.
int64_t stage_elems(int kid, bool gate_up);

// Enqueue a GEMM (or, with lds_image, the debug stage dump) on `stream`.
hipError_t launch_tiled(int kid, int in_kind, int out_kind, int vec, bool gate_up,
                        const TiledArgs& args, int grid, hipStream_t stream, bool lds_image);

}  // namespace lak
