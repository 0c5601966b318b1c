// Instantiations and dispatch of the fast (full-tile, direct-to-LDS) kernels.
#include "gemm_fast.hpp"

namespace lak {
namespace {

template <class C, class TI, class TO>
hipError_t go_fast(const TiledArgs& a, dim3 grid, hipStream_t s, bool img) {
  constexpr int NT = C::WM * C::WN * 64;
  if (img) {
    hipLaunchKernelGGL((gemm_fast_lds_image<TI, TO, C>),
                       dim3(1), dim3(NT), 0, s, a);
  } else {
    const bool kt = a.K % C::BK != 0;
    if constexpr (C::NB == 1) {
      // row reductions (single-output plans only) run their own instantiation
      if (a.red != RED_NONE) {
        if (kt)
          hipLaunchKernelGGL((gemm_fast_pp_kernel<TI, TO, C, true, true>), grid, dim3(NT), 0, s, a);
        else
          hipLaunchKernelGGL((gemm_fast_pp_kernel<TI, TO, C, true, false>), grid, dim3(NT), 0, s, a);
        return hipGetLastError();
      }
    }
    if (kt)
      hipLaunchKernelGGL((gemm_fast_pp_kernel<TI, TO, C, false, true>), grid, dim3(NT), 0, s, a);
    else
      hipLaunchKernelGGL((gemm_fast_pp_kernel<TI, TO, C, false, false>), grid, dim3(NT), 0, s, a);
  }
  return hipGetLastError();
}

template <class C>
hipError_t by_types(int in_kind, int out_kind, const TiledArgs& a, dim3 grid, hipStream_t s, bool img) {
  if (in_kind == IN_BF16) {
    if (out_kind == OUT_F32) return go_fast<C, InBF16, OutF32>(a, grid, s, img);
    if (out_kind == OUT_BF16) return go_fast<C, InBF16, OutBF16>(a, grid, s, img);
    if (out_kind == OUT_F16) return go_fast<C, InBF16, OutF16>(a, grid, s, img);
  } else if (in_kind == IN_F16) {
    if (out_kind == OUT_F32) return go_fast<C, InF16, OutF32>(a, grid, s, img);
    if (out_kind == OUT_BF16) return go_fast<C, InF16, OutBF16>(a, grid, s, img);
    if (out_kind == OUT_F16) return go_fast<C, InF16, OutF16>(a, grid, s, img);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fast(int kid, int in_kind, int out_kind, const TiledArgs& args, dim3 grid, hipStream_t stream,
                       bool lds_image) {
  switch (kid) {
    case KID_FAST_256: return by_types<CfgFast256>(in_kind, out_kind, args, grid, stream, lds_image);
    case KID_FAST_GU: return by_types<CfgFastGU>(in_kind, out_kind, args, grid, stream, lds_image);
    case KID_FAST_256_KM: return by_types<CfgFast256KM>(in_kind, out_kind, args, grid, stream, lds_image);
    case KID_FAST_GU_KM: return by_types<CfgFastGUKM>(in_kind, out_kind, args, grid, stream, lds_image);
    case KID_FAST_256_AT: return by_types<CfgFast256AT>(in_kind, out_kind, args, grid, stream, lds_image);
    case KID_FAST_GU_AT: return by_types<CfgFastGUAT>(in_kind, out_kind, args, grid, stream, lds_image);
    case KID_FAST_128: return by_types<CfgFast128>(in_kind, out_kind, args, grid, stream, lds_image);
    case KID_FAST_128_KM: return by_types<CfgFast128KM>(in_kind, out_kind, args, grid, stream, lds_image);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lak
