// Row normalisation launch interface (see rms_norm.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace lak {

struct NormArgs {
  const void* X;     // [M, D], row stride ldx (elements)
  const void* G;     // [D], same element type as X
  void* Y;           // [M, D], row stride ldy
  int64_t M, D, ldx, ldy;
  float eps;
};

// x_kind, y_kind: OUT_F32, OUT_BF16 or OUT_F16.  vec: rows of X and Y and the
// gain start on 16 bytes and ldx, ldy are multiples of rms_norm_vec_elems(x_kind).
hipError_t launch_rms_norm(const NormArgs& a, int x_kind, int y_kind, bool vec, hipStream_t stream);
int rms_norm_vec_elems(int x_kind);

}  // namespace lak
