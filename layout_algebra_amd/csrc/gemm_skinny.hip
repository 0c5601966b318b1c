// Skinny GEMM for gfx950: M <= 16 rows, the whole problem streams B once.
//
// With M = 16 every byte of B is used by 16 rows only (about 16 FLOP per byte
// of B), so the kernel is bound by HBM bandwidth, not by the matrix cores.
// Structure:
//  * one workgroup per 128-column strip of C and of B; the strip's B panel
//    (K x 128) streams through a ring of STAGES LDS buffers by direct
//    global -> LDS loads (1 KB per wave instruction, source-side swizzle as
//    in the fast kernel), keeping STAGES-1 K blocks (over 100 KB per CU) in
//    flight so HBM latency is covered;
//  * the 16 x BK slice of A rides along in the same stage (A is 256 KB in
//    total and stays in L2); rows >= M are fetched from row M-1 and their
//    results discarded;
//  * each of the 4 waves owns 32 columns: two v_mfma_f32_16x16x32 blocks per
//    32-wide K step, A fragments as 16-byte LDS reads, B fragments through
//    the transposing ds_read_b64_tr_b16 (B N-contiguous) or, for B stored
//    [N, K], as 16-byte reads of its K-contiguous rows like A's (the strip is
//    then 128 rows of B, each a 256-byte row per K block under A's swizzle);
//  * one-byte inputs (B stored [N, K]) run the K-major kernel on byte pairs:
//    two 16-byte reads of consecutive 32-unit steps form the 32-byte operands
//    of one v_mfma_f32_16x16x128_f8f6f4 (A and B place K alike);
//  * FP32 accumulators stay in registers; the epilogue applies alpha/beta
//    and writes only rows < M.
#include "kernel_common.hpp"
#include "launch.hpp"

namespace lak {
namespace {

typedef short i16x4_s __attribute__((ext_vector_type(4)));
#define SK_LDS __attribute__((address_space(3)))

template <int N>
__device__ __forceinline__ void sk_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

__device__ __forceinline__ void sk_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct load of 64 x 16 bytes into one LDS kilobyte.  NT marks the access
// non-temporal: B is read exactly once, so it should not displace A (and
// whatever else is resident) from the caches.
template <bool NT>
__device__ __forceinline__ void sk_dma16(const uint16_t* base, uint32_t voff, const SK_LDS uint16_t* dst) {
  const uint32_t lds_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst));
  if constexpr (NT) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2 nt"
        :
        : "s"(lds_addr), "v"(voff), "s"(base)
        : "memory", "m0");
  } else {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2"
        :
        : "s"(lds_addr), "v"(voff), "s"(base)
        : "memory", "m0");
  }
}

template <class TI, class TO, class C>
__global__ void __launch_bounds__(256) gemm_skinny_kernel(const TiledArgs g_in) {
  const TiledArgs g = at_batch(g_in);
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, S = C::STAGES;
  constexpr int NW = 4, FM = BM / 16;
  constexpr int A_ELEMS = BM * BK, B_ELEMS = BK * BN, STAGE = A_ELEMS + B_ELEMS;
  constexpr int A_LOADS = A_ELEMS / 512 / NW, B_LOADS = B_ELEMS / 512 / NW;
  constexpr int LPS = A_LOADS + B_LOADS;
  constexpr int TN = BN / NW, FN = TN / 16;
  static_assert(A_LOADS * 512 * NW == A_ELEMS && B_LOADS * 512 * NW == B_ELEMS, "whole KB per wave");
  static_assert((S - 2) * LPS < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) uint16_t lds_raw[S * STAGE];
  SK_LDS uint16_t* lds = (SK_LDS uint16_t*)lds_raw;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn;
  grouped_tile(xcd_contiguous(blockIdx.x, gridDim.x), 1, g.tiles_n, 1, tm, tn);
  const int64_t n0 = int64_t(tn) * BN;
  constexpr bool BKM = C::BKMAJOR;

  // per-lane source offsets (bytes, 32-bit) of the direct loads
  uint32_t sa[A_LOADS], sb[B_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) {
    const int L = swz<C::AB, C::AM, C::AS>((wave * A_LOADS + i) * 512 + lane * 8);
    const int r = min(L / BK, int(g.M) - 1);
    sa[i] = uint32_t((r * g.lda + L % BK) * 2);
  }
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) {
    const int L = swz<C::BB, C::BMb, C::BS>((wave * B_LOADS + i) * 512 + lane * 8);
    // B block in LDS: (k, n) at k * BN + n, or for B stored [N, K] at n * BK + k
    sb[i] = BKM ? uint32_t(((L / BK) * g.ldb + L % BK) * 2) : uint32_t(((L / BN) * g.ldb + L % BN) * 2);
  }
  auto issue = [&](int kb, int buf) {
    const int64_t k1 = int64_t(kb) * BK;
    const uint16_t* a_blk = g.A + k1;
    const uint16_t* b_blk = BKM ? g.B + n0 * g.ldb + k1 : g.B + k1 * g.ldb + n0;
    SK_LDS uint16_t* st = lds + buf * STAGE;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) sk_dma16<false>(a_blk, sa[i], st + (wave * A_LOADS + i) * 512);
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) sk_dma16<C::B_NT>(b_blk, sb[i], st + A_ELEMS + (wave * B_LOADS + i) * 512);
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{};
  const int ar = lane & 15, ak = (lane >> 4) * 8;          // A: row l % 16 of each 16-row block, 8 K values from 8 (l / 16)
  const int g4 = lane >> 4;
  const int bk = 8 * g4 + ((lane >> 2) & 3);              // B: K row this lane addresses
  const int bn = wave * TN + 4 * (lane & 3);               // B: first of its 4 N values

  const int nk = int(g.K / BK);
#pragma unroll
  for (int p = 0; p < S - 1; ++p)
    if (p < nk) issue(p, p);
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + S - 2 <= nk - 1) {
      sk_wait_vmcnt<(S - 2) * LPS>();
    } else {
      sk_wait_vmcnt<0>();
    }
    sk_barrier();
    if (kt + S - 1 < nk) issue(kt + S - 1, (kt + S - 1) % S);
    const SK_LDS uint16_t* st = lds + (kt % S) * STAGE;
    const SK_LDS uint16_t* bs = st + A_ELEMS;
    // one 32-wide K step: A and B fragments of lane l (8 K values from 8 (l / 16))
    auto a_frag = [&](int s, int i) {
      return *reinterpret_cast<const SK_LDS u32x4*>(st + swz<C::AB, C::AM, C::AS>((16 * i + ar) * BK + s * 32 + ak));
    };
    auto b_frag = [&](int s, int j) {
      if constexpr (BKM) {
        return *reinterpret_cast<const SK_LDS u32x4*>(
            bs + swz<C::BB, C::BMb, C::BS>((wave * TN + j * 16 + ar) * BK + s * 32 + ak));
      } else {
        const i16x4_s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (SK_LDS i16x4_s*)(bs + swz<C::BB, C::BMb, C::BS>((s * 32 + bk) * BN + bn + j * 16)));
        const i16x4_s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (SK_LDS i16x4_s*)(bs + swz<C::BB, C::BMb, C::BS>((s * 32 + bk + 4) * BN + bn + j * 16)));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        return u32x4{l2.x, l2.y, h2.x, h2.y};
      }
    };
    if constexpr (TI::f8) {
      // byte pairs: steps s and s + 1 (64 units = 128 codes) form one 16x16x128 product
#pragma unroll
      for (int s = 0; s < BK / 32; s += 2) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const u32x4 b0 = b_frag(s, j), b1 = b_frag(s + 1, j);
#pragma unroll
          for (int i = 0; i < FM; ++i) acc[i][j] = mfma_f8_16x16x128<TI>(a_frag(s, i), a_frag(s + 1, i), b0, b1, acc[i][j]);
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < BK / 32; ++s) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const u32x4 b = b_frag(s, j);
#pragma unroll
          for (int i = 0; i < FM; ++i) acc[i][j] = mfma_16x16x32<TI>(a_frag(s, i), b, acc[i][j]);
        }
      }
    }
  }

  // 16x16 result lane map: register r of lane l is row 4 (l / 16) + r, column l % 16 of its block.
  typedef typename TO::storage St;
  St* Cp = static_cast<St*>(g.C);
  const int red = g.red;
  float part[FM][4];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) part[i][r] = red_identity(red);
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int64_t col = n0 + wave * TN + j * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = 16 * i + 4 * (lane >> 4) + r;
        if (row < g.M) {
          const int64_t idx = row * g.ldc + col;
          float v = g.alpha * acc[i][j][r];
          if (g.beta != 0.0f) v += g.beta * from_out<TO>(Cp[idx]);
          Cp[idx] = to_out<TO>(v);
          if (red != RED_NONE) part[i][r] = red_combine(red, part[i][r], v);
        }
      }
  }
  if (red != RED_NONE) {
    // the 16 lanes of a row group hold its 16 columns of each j block
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = red_lanes<16>(red, part[i][r]);
        const int64_t row = 16 * i + 4 * (lane >> 4) + r;
        if ((lane & 15) == 0 && row < g.M) red_commit(red, g.R + row, p);
      }
  }
}

// Debug: K block 0 of column strip dbg_tn, staged by the kernel's own code.
template <class TI, class TO, class C>
__global__ void __launch_bounds__(256) gemm_skinny_lds_image(const TiledArgs g) {
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, NW = 4;
  constexpr int A_ELEMS = BM * BK, B_ELEMS = BK * BN, STAGE = A_ELEMS + B_ELEMS;
  constexpr int A_LOADS = A_ELEMS / 512 / NW, B_LOADS = B_ELEMS / 512 / NW;
  __shared__ __attribute__((aligned(1024))) uint16_t lds_raw[STAGE];
  SK_LDS uint16_t* lds = (SK_LDS uint16_t*)lds_raw;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t n0 = int64_t(g.dbg_tn) * BN;
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) {
    const int L = swz<C::AB, C::AM, C::AS>((wave * A_LOADS + i) * 512 + lane * 8);
    const int r = min(L / BK, int(g.M) - 1);
    sk_dma16<false>(g.A, uint32_t((r * g.lda + L % BK) * 2), lds + (wave * A_LOADS + i) * 512);
  }
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) {
    const int L = swz<C::BB, C::BMb, C::BS>((wave * B_LOADS + i) * 512 + lane * 8);
    const uint32_t off = C::BKMAJOR ? uint32_t(((L / BK) * g.ldb + L % BK) * 2) : uint32_t(((L / BN) * g.ldb + L % BN) * 2);
    sk_dma16<false>(C::BKMAJOR ? g.B + n0 * g.ldb : g.B + n0, off, lds + A_ELEMS + (wave * B_LOADS + i) * 512);
  }
  sk_wait_vmcnt<0>();
  sk_barrier();
  for (int i = tid; i < STAGE; i += 256) g.dbg_out[i] = lds[i];
}

template <class C, class TI, class TO>
hipError_t go_skinny(const TiledArgs& a, dim3 grid, hipStream_t s, bool img) {
  if (img) {
    hipLaunchKernelGGL((gemm_skinny_lds_image<TI, TO, C>), dim3(1), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((gemm_skinny_kernel<TI, TO, C>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <class C, class TI>
hipError_t by_out(int out_kind, const TiledArgs& a, dim3 grid, hipStream_t s, bool img) {
  if (out_kind == OUT_F32) return go_skinny<C, TI, OutF32>(a, grid, s, img);
  if (out_kind == OUT_BF16) return go_skinny<C, TI, OutBF16>(a, grid, s, img);
  if (out_kind == OUT_F16) return go_skinny<C, TI, OutF16>(a, grid, s, img);
  return hipErrorInvalidValue;
}

template <class C>
hipError_t by_in(int in_kind, int out_kind, const TiledArgs& a, dim3 grid, hipStream_t s, bool img) {
  if (in_kind == IN_BF16) return by_out<C, InBF16>(out_kind, a, grid, s, img);
  if (in_kind == IN_F16) return by_out<C, InF16>(out_kind, a, grid, s, img);
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

hipError_t launch_skinny(int kid, int in_kind, int out_kind, const TiledArgs& a, dim3 grid, hipStream_t s, bool img) {
  switch (kid) {
    case KID_SKINNY_16: return by_in<CfgSkinny16>(in_kind, out_kind, a, grid, s, img);
    case KID_SKINNY_32: return by_in<CfgSkinny32>(in_kind, out_kind, a, grid, s, img);
    case KID_SKINNY_64: return by_in<CfgSkinny64>(in_kind, out_kind, a, grid, s, img);
    case KID_SKINNY_16_KM: return by_in<CfgSkinny16KM>(in_kind, out_kind, a, grid, s, img);
    case KID_SKINNY_32_KM: return by_in<CfgSkinny32KM>(in_kind, out_kind, a, grid, s, img);
    case KID_SKINNY_64_KM: return by_in<CfgSkinny64KM>(in_kind, out_kind, a, grid, s, img);
    case KID_SKINNY_F8: return by_formats<CfgSkinny16KM>(in_kind, out_kind, a, grid, s, img);
    case KID_SKINNY_F8_32: return by_formats<CfgSkinny32KM>(in_kind, out_kind, a, grid, s, img);
    case KID_SKINNY_F8_64: return by_formats<CfgSkinny64KM>(in_kind, out_kind, a, grid, s, img);
    case KID_SKINNY_128: return by_in<CfgSkinny128>(in_kind, out_kind, a, grid, s, img);
    case KID_SKINNY_128_KM: return by_in<CfgSkinny128KM>(in_kind, out_kind, a, grid, s, img);
    case KID_SKINNY_F8_128: return by_formats<CfgSkinny128KM>(in_kind, out_kind, a, grid, s, img);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lak
