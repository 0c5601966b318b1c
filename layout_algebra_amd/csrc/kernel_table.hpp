// Host-side table of the GEMM kernels: tile shape, waves, MFMA block, LDS
// maps and copy style of each kernel id, which the planner validates and
// describes.  No kernel source includes this file.
#pragma once

#include "launch.hpp"

namespace lak {

struct KernelShape {
  int bm, bn, bk;          // bn is per weight matrix
  int nb;                  // weight matrices per launch (2 for gate/up)
  int waves_m, waves_n;
  int threads;
  int mfma_m, mfma_n, mfma_k;
  int sw_a[3];             // Swizzle{B,M,S} of the A block, element offsets over (bm,bk):(bk,1)
  int sw_b[3];             // Swizzle{B,M,S} of a B block
  int b_kmajor;            // 1: B block stored (bn,bk):(bk,1) (K contiguous); 0: (bk,bn):(bn,1)
  int direct;              // 1: global -> LDS direct loads (whole 1 KB per wave instruction)
  int full_tiles_only;     // 1: K % bk == 0 required (M and N may end inside a tile: clamped loads, masked stores)
  int stages;
  int b_follows_storage = 0;   // 1: the B block keeps the operand's orientation (K-contiguous with sw_b
                               //    for K-major B, N-contiguous with sw_bn otherwise)
  int sw_bn[3] = {0, 0, 0};    // Swizzle{B,M,S} of an N-contiguous B block, element offsets over (bk,bn):(bn,1)
  int a_trans = 0;             // 1: the A block stored (bk,bm):(bm,1) (M contiguous, A stored [K, M]) under sw_a
  int a_follows_storage = 0;   // 1: the kernel keeps A M-contiguous with sw_am when A is stored [K, M]
  int sw_am[3] = {0, 0, 0};    // Swizzle{B,M,S} of an M-contiguous A block, element offsets over (bk,bm):(bm,1)
  int wave_split = 0;          // 1 (gate/up): wave (wm, wn) owns a (bm/waves_m) x (nb*bn/waves_n) slice of the tile
                               //    seen as [W_gate block | W_up block], i.e. one weight per wave
  int in_bytes = 2;            // bytes per input element (2: bf16 / f16, 4: binary32)
  int k_sub = 0;               // K-contiguous blocks stored as bk / k_sub sub-blocks of k_sub values per row
                               //    ((rows, (k_sub, bk/k_sub)) : (k_sub, (1, rows*k_sub))); 0: one row of bk
};

// Static description of each kernel id; the planner validates these maps.
KernelShape kernel_shape(int kid);

// LDS elements of one pipeline stage (one A block and one B block per weight).
int64_t stage_elems(const KernelShape& s, bool gate_up);

}  // namespace lak
