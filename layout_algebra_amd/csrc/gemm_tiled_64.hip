// Instantiations of the general (tiled) kernel for 64 x 64 tiles (kernels in gemm_tiled.hpp).
#include "gemm_tiled.hpp"

namespace lak {

hipError_t launch_tiled_64(int in_kind, int out_kind, int vec, bool gate_up, bool b_kmajor, bool a_trans,
                           const TiledArgs& args, dim3 grid, hipStream_t stream, bool lds_image) {
  return by_types<64, 64, 2, 1>(in_kind, out_kind, vec, gate_up, b_kmajor, a_trans, args, grid, stream, lds_image);
}

}  // namespace lak
