// Kernel table and dispatch across kernel families (host code).
#include "kernel_table.hpp"
#include "launch.hpp"

namespace lak {

template <class C>
static KernelShape fast_shape() {
  KernelShape s{C::BM, C::BN, C::BK, C::NB, C::WM, C::WN, C::WM * C::WN * 64, 32, 32, 16,
                {C::AB, C::AM, C::AS}, {C::BB, C::BMb, C::BS}, C::BKMAJOR ? 1 : 0, 1, 1, C::STAGES};
  s.a_trans = C::ATRANS ? 1 : 0;
  s.wave_split = C::WSPLIT ? 1 : 0;
  return s;
}

// The skinny kernels (M <= BM rows, one strip of BN columns per workgroup).  One-byte inputs run
// the K-major configurations on byte pairs: K blocks of 2 BK codes, the swizzle's chunk field one
// bit higher (16-byte chunks of codes), one 16x16x128 product per two 32-unit steps.
template <class C>
static KernelShape skinny_shape(bool one_byte) {
  KernelShape s{C::BM, C::BN, C::BK, 1, 1, 4, 256, 16, 16, 32, {C::AB, C::AM, C::AS}, {C::BB, C::BMb, C::BS},
                C::BKMAJOR ? 1 : 0, 1, 1, C::STAGES};
  if (one_byte) {
    s.bk = 2 * C::BK;
    s.mfma_k = 128;
    s.sw_a[1] += 1;
    s.sw_b[1] += 1;
    s.in_bytes = 1;
  }
  return s;
}

KernelShape kernel_shape(int kid) {
  switch (kid) {
    case KID_TILED_128:
      return KernelShape{128, 128, 64, 2, 2, 2, 256, 32, 32, 16, {3, 3, 4}, {3, 3, 4}, 1, 0, 0, 2, 1, {2, 5, 2},
                         0, 1, {2, 5, 2}};
    case KID_TILED_64:
    case KID_TILED_64_P3:
      return KernelShape{64, 64, 64, 2, 2, 1, 128, 32, 32, 16, {3, 3, 4}, {3, 3, 4}, 1, 0, 0, 2, 1, {1, 5, 2},
                         0, 1, {1, 5, 2}};
    case KID_FAST_256: return fast_shape<CfgFast256>();
    case KID_FAST_GU: return fast_shape<CfgFastGU>();
    case KID_FAST_256_KM: return fast_shape<CfgFast256KM>();
    case KID_FAST_GU_KM: return fast_shape<CfgFastGUKM>();
    case KID_FAST_256_AT: return fast_shape<CfgFast256AT>();
    case KID_FAST_GU_AT: return fast_shape<CfgFastGUAT>();
    case KID_FAST_128: return fast_shape<CfgFast128>();
    case KID_FAST_128_KM: return fast_shape<CfgFast128KM>();
    case KID_FAST_128_KM64: return fast_shape<CfgFast128KM64>();
    case KID_FAST_128_K64: return fast_shape<CfgFast128K64>();
    case KID_TILED_F32: {
      // K-contiguous blocks: two 64-byte rows of 16 binary32 values per row under Swizzle{2,2,4};
      // M/N-contiguous blocks: rows of 128 values under Swizzle{1,5,5}
      KernelShape s{128, 128, 32, 1, 2, 2, 256, 32, 32, 2, {2, 2, 4}, {2, 2, 4}, 1, 0, 0, 2, 1, {1, 5, 5},
                    0, 1, {1, 5, 5}};
      s.in_bytes = 4;
      s.k_sub = 16;
      return s;
    }
    case KID_FAST_F8_128_K64: {
      // KID_FAST_128_KM64 in one-byte elements: K blocks of 128 codes (128-byte rows) under
      // Swizzle{3,4,4} (the pair view's Swizzle{3,3,4} with 16-code chunks), two 32x32x64 products
      // per 32x32 block and K block
      KernelShape s = fast_shape<CfgFast128KM64>();
      s.bk = 2 * CfgFast128KM64::BK;
      s.mfma_k = 64;
      s.sw_a[0] = s.sw_b[0] = 3;
      s.sw_a[1] = s.sw_b[1] = 4;
      s.sw_a[2] = s.sw_b[2] = 4;
      s.in_bytes = 1;
      return s;
    }
    case KID_FAST_F8:
    case KID_FAST_F8_128:
    case KID_FAST_GU_F8: {
      // the K-major full-tile kernels seen in one-byte elements: a K block of 64 codes per row
      // (64-byte rows) under Swizzle{2,4,4} (16-byte chunks, rows 4 apart in bits 8-9), one
      // 32x32x64 product per block
      KernelShape s = kid == KID_FAST_F8 ? fast_shape<CfgFast256KM>()
                    : kid == KID_FAST_F8_128 ? fast_shape<CfgFast128KM>() : fast_shape<CfgFastGUKM>();
      s.bk = 2 * CfgFast256KM::BK;
      s.mfma_k = 64;
      s.sw_a[0] = s.sw_b[0] = 2;
      s.sw_a[1] = s.sw_b[1] = 4;
      s.sw_a[2] = s.sw_b[2] = 4;
      s.in_bytes = 1;
      return s;
    }
    case KID_SKINNY_16: return skinny_shape<CfgSkinny16>(false);
    case KID_SKINNY_32: return skinny_shape<CfgSkinny32>(false);
    case KID_SKINNY_64: return skinny_shape<CfgSkinny64>(false);
    case KID_SKINNY_16_KM: return skinny_shape<CfgSkinny16KM>(false);
    case KID_SKINNY_32_KM: return skinny_shape<CfgSkinny32KM>(false);
    case KID_SKINNY_64_KM: return skinny_shape<CfgSkinny64KM>(false);
    case KID_SKINNY_F8: return skinny_shape<CfgSkinny16KM>(true);
    case KID_SKINNY_F8_32: return skinny_shape<CfgSkinny32KM>(true);
    case KID_SKINNY_F8_64: return skinny_shape<CfgSkinny64KM>(true);
    case KID_SKINNY_128: return skinny_shape<CfgSkinny128>(false);
    case KID_SKINNY_128_KM: return skinny_shape<CfgSkinny128KM>(false);
    case KID_SKINNY_F8_128: return skinny_shape<CfgSkinny128KM>(true);
    default:
      return KernelShape{};
  }
}

int64_t stage_elems(const KernelShape& s, bool gate_up) {
  return int64_t(s.bm) * s.bk + int64_t(gate_up ? 2 : 1) * s.bn * s.bk;
}

hipError_t launch_kernel(int kid, int in_kind, int out_kind, int vec, bool gate_up, bool b_kmajor, bool a_trans,
                         const TiledArgs& args, dim3 grid, hipStream_t stream, bool lds_image) {
  switch (kid) {
    case KID_TILED_128:
    case KID_TILED_64:
    case KID_TILED_64_P3:
      return launch_tiled(kid, in_kind, out_kind, vec, gate_up, b_kmajor, a_trans, args, grid, stream, lds_image);
    case KID_FAST_256:
    case KID_FAST_GU:
    case KID_FAST_256_KM:
    case KID_FAST_GU_KM:
    case KID_FAST_256_AT:
    case KID_FAST_GU_AT:
    case KID_FAST_128:
    case KID_FAST_128_KM:
    case KID_FAST_128_KM64:
    case KID_FAST_128_K64: return launch_fast(kid, in_kind, out_kind, args, grid, stream, lds_image);
    case KID_SKINNY_16:
    case KID_SKINNY_32:
    case KID_SKINNY_64:
    case KID_SKINNY_16_KM:
    case KID_SKINNY_32_KM:
    case KID_SKINNY_64_KM:
    case KID_SKINNY_F8:
    case KID_SKINNY_F8_32:
    case KID_SKINNY_F8_64:
    case KID_SKINNY_128:
    case KID_SKINNY_128_KM:
    case KID_SKINNY_F8_128: return launch_skinny(kid, in_kind, out_kind, args, grid, stream, lds_image);
    case KID_TILED_F32: return launch_f32(out_kind, vec, b_kmajor, a_trans, args, grid, stream, lds_image);
    case KID_FAST_F8:
    case KID_FAST_F8_128:
    case KID_FAST_F8_128_K64:
    case KID_FAST_GU_F8: return launch_fast_f8(kid, in_kind, out_kind, args, grid, stream, lds_image);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lak
