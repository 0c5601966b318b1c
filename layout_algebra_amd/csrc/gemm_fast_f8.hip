// One-byte inputs (OCP E4M3 / E5M2) on the full-tile direct-load kernels
// (plain GEMM and gate/up).
//
// The operands are K-contiguous on both sides (A [M, K], B and the gate/up
// weights [N, K]), the storage the Tylo.jl page "TMA and Hopper WGMMA" gives
// its B operand; a row of one K block is 64 codes = 64 bytes, the 64-byte swizzle row that the same
// page's storage contract offers next to the 128-byte default (section "The
// same storage contract on both sides").  Every copy and every fragment read
// moves whole 16-byte chunks, so the kernels address a row of one-byte codes
// as 16-bit units holding byte pairs: the K-major 16-bit kernels' staging,
// swizzle (Swizzle{2,3,4} over 16-bit units = Swizzle{2,4,4} over bytes),
// ring, edge clamping and epilogue run unchanged on K/2, lda/2 and ldb/2, and
// only the products differ: one v_mfma_f32_32x32x64_f8f6f4 per 32-unit block
// (64 codes) instead of two 32x32x16 products (mma_block, mma1).
#include "gemm_fast.hpp"

namespace lak {
namespace {

template <class C, class TI, class TO>
hipError_t go_f8(const TiledArgs& a, dim3 grid, hipStream_t s, bool img) {
  constexpr int NT = C::WM * C::WN * 64;
  if (img) {
    hipLaunchKernelGGL((gemm_fast_lds_image<TI, TO, C>), dim3(1), dim3(NT), 0, s, a);
    return hipGetLastError();
  }
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
  return hipGetLastError();
}

template <class C, class TI>
hipError_t by_out(int out_kind, const TiledArgs& a, dim3 grid, hipStream_t s, bool img) {
  if (out_kind == OUT_F32) return go_f8<C, TI, OutF32>(a, grid, s, img);
  if (out_kind == OUT_BF16) return go_f8<C, TI, OutBF16>(a, grid, s, img);
  if (out_kind == OUT_F16) return go_f8<C, TI, OutF16>(a, grid, s, img);
  return hipErrorInvalidValue;
}

template <class C>
hipError_t by_formats(int in_kind, int out_kind, const TiledArgs& a, dim3 grid, hipStream_t s, bool img) {
  switch (in_kind - IN_F8) {
    case 0: return by_out<C, InF8<0, 0>>(out_kind, a, grid, s, img);
    case 1: return by_out<C, InF8<0, 1>>(out_kind, a, grid, s, img);
    case 2: return by_out<C, InF8<1, 0>>(out_kind, a, grid, s, img);
    case 3: return by_out<C, InF8<1, 1>>(out_kind, a, grid, s, img);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_fast_f8(int kid, int in_kind, int out_kind, const TiledArgs& args, dim3 grid, hipStream_t stream,
                          bool lds_image) {
  if (kid == KID_FAST_F8) return by_formats<CfgFast256KM>(in_kind, out_kind, args, grid, stream, lds_image);
  if (kid == KID_FAST_GU_F8) return by_formats<CfgFastGUKM>(in_kind, out_kind, args, grid, stream, lds_image);
  if (kid == KID_FAST_F8_128) return by_formats<CfgFast128KM>(in_kind, out_kind, args, grid, stream, lds_image);
  if (kid == KID_FAST_F8_128_K64) return by_formats<CfgFast128KM64>(in_kind, out_kind, args, grid, stream, lds_image);
  return hipErrorInvalidValue;
}

}  // namespace lak
