// Instantiations of the fast kernels with 128-row tiles.
#include "gemm_fast.hpp"

namespace lak {

hipError_t launch_fast_128(int kid, int in_kind, int out_kind, const TiledArgs& args, dim3 grid, hipStream_t stream,
                           bool lds_image) {
  switch (kid) {
    case KID_FAST_128: return by_types<CfgFast128>(in_kind, out_kind, args, grid, stream, lds_image);
    case KID_FAST_128_KM: return by_types<CfgFast128KM>(in_kind, out_kind, args, grid, stream, lds_image);
    case KID_FAST_128_KM64: return by_types<CfgFast128KM64>(in_kind, out_kind, args, grid, stream, lds_image);
    case KID_FAST_128_K64: return by_types<CfgFast128K64>(in_kind, out_kind, args, grid, stream, lds_image);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lak
