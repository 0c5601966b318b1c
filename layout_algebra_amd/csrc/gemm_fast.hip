// Instantiations and dispatch of the fast (full-tile, direct-to-LDS) kernels: the 256-row plain
// configurations here, gate/up in gemm_fast_gu.hip, 128-row tiles in gemm_fast_128.hip.
#include "gemm_fast.hpp"

namespace lak {

hipError_t launch_fast(int kid, int in_kind, int out_kind, const TiledArgs& args, dim3 grid, hipStream_t stream,
                       bool lds_image) {
  switch (kid) {
    case KID_FAST_256: return by_types<CfgFast256>(in_kind, out_kind, args, grid, stream, lds_image);
    case KID_FAST_256_KM: return by_types<CfgFast256KM>(in_kind, out_kind, args, grid, stream, lds_image);
    case KID_FAST_256_AT: return by_types<CfgFast256AT>(in_kind, out_kind, args, grid, stream, lds_image);
    case KID_FAST_GU:
    case KID_FAST_GU_KM:
    case KID_FAST_GU_AT: return launch_fast_gu(kid, in_kind, out_kind, args, grid, stream, lds_image);
    case KID_FAST_128:
    case KID_FAST_128_KM:
    case KID_FAST_128_KM64:
    case KID_FAST_128_K64: return launch_fast_128(kid, in_kind, out_kind, args, grid, stream, lds_image);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lak
