// Instantiations of the general (tiled) kernel for 128 x 128 tiles (kernels in gemm_tiled.hpp).
#include "gemm_tiled.hpp"

namespace lak {

hipError_t launch_tiled_128(int in_kind, int out_kind, int vec, bool gate_up, bool b_kmajor, bool a_trans,
                            const TiledArgs& args, dim3 grid, hipStream_t stream, bool lds_image) {
  return by_types<128, 128, 2, 2>(in_kind, out_kind, vec, gate_up, b_kmajor, a_trans, args, grid, stream, lds_image);
}

}  // namespace lak
