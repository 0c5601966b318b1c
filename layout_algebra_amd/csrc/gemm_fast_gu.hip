// Instantiations of the fast gate/up kernels (waves split by weight).
#include "gemm_fast.hpp"

namespace lak {

hipError_t launch_fast_gu(int kid, int in_kind, int out_kind, const TiledArgs& args, dim3 grid, hipStream_t stream,
                          bool lds_image) {
  switch (kid) {
    case KID_FAST_GU: return by_types<CfgFastGU>(in_kind, out_kind, args, grid, stream, lds_image);
    case KID_FAST_GU_KM: return by_types<CfgFastGUKM>(in_kind, out_kind, args, grid, stream, lds_image);
    case KID_FAST_GU_AT: return by_types<CfgFastGUAT>(in_kind, out_kind, args, grid, stream, lds_image);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lak
