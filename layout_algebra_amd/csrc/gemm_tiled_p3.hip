// Instantiations of the general (tiled) kernel for 64 x 64 tiles with three K blocks in flight, and the dispatch (kernels in gemm_tiled.hpp).
#include "gemm_tiled.hpp"

namespace lak {

hipError_t launch_tiled(int kid, int in_kind, int out_kind, int vec, bool gate_up, bool b_kmajor, bool a_trans,
                        const TiledArgs& args, dim3 grid, hipStream_t stream, bool lds_image) {
  switch (kid) {
    case KID_TILED_128:
      return launch_tiled_128(in_kind, out_kind, vec, gate_up, b_kmajor, a_trans, args, grid, stream, lds_image);
    case KID_TILED_64:
      return launch_tiled_64(in_kind, out_kind, vec, gate_up, b_kmajor, a_trans, args, grid, stream, lds_image);
    case KID_TILED_64_P3:
      if (a_trans) return hipErrorInvalidValue;
      return p3_by_types(in_kind, out_kind, vec, gate_up, b_kmajor, args, grid, stream, lds_image);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lak
