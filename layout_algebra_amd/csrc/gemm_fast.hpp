// Fast tiled GEMM for gfx950: full tiles only (M % BM == 0, N % BN == 0,
// K % 64 == 0, 16-byte aligned rows).
//
// Differences from the general kernel (gemm_tiled.hip):
//  * Operands go global -> LDS directly (global_load_lds_dwordx4): each wave
//    instruction moves 64 x 16 bytes into one contiguous kilobyte of LDS, lane
//    l landing at byte 16 l.  The swizzle is therefore applied on the source
//    side: the lane that fills physical LDS element P fetches the logical
//    element Sw(P) (an XOR swizzle is its own inverse and keeps 16-byte chunks
//    whole, so one lane still moves 8 contiguous elements of one row).
//  * B stays N-contiguous in LDS, exactly as it is stored in memory (rows of
//    BN elements for each k).  The MFMA needs 8 consecutive K values per lane,
//    so B fragments are read with ds_read_b64_tr_b16, which transposes 4 x 16
//    blocks of 16-bit values across each 16-lane group on the way out of LDS:
//    lanes 4e..4e+3 of the group point at row e (16 values) and lane i
//    receives element i of rows 0..3.  Two such reads give the 8 K values.
//  * A fragments are plain 16-byte LDS reads (K is contiguous in A).
//  * 256 x 256 (or 256 x 2*128 for gate/up) tiles with 8 waves: one tile per
//    CU at 4096^2, two waves per SIMD so one wave's MFMAs cover the other's
//    LDS traffic.
// The LDS maps are Swizzle{AB,AM,AS} o (BM,64):(64,1) for A and
// Swizzle{BB,BMb,BS} o (64,BN):(BN,1) for B (element offsets).
#pragma once

#include "kernel_common.hpp"
#include "launch.hpp"

namespace lak {

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define LAK_LDS __attribute__((address_space(3)))
#define LAK_GLB __attribute__((address_space(1)))

template <class TI, class TO, int BM, int BN, int NB, int WM, int WN,
          int AB, int AM, int AS, int BB, int BMb, int BS>
struct Fast {
  static constexpr int NW = WM * WN;
  static constexpr int NT = NW * 64;
  static constexpr int BK = 64;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int A_ELEMS = BM * BK;
  static constexpr int B_ELEMS = BK * BN;
  static constexpr int STAGE = A_ELEMS + NB * B_ELEMS;   // 16-bit elements
  static constexpr int A_LOADS = A_ELEMS / 512 / NW;       // 1 KB (512 elements) per wave instruction
  static constexpr int B_LOADS = B_ELEMS / 512 / NW;
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(A_LOADS * 512 * NW == A_ELEMS && B_LOADS * 512 * NW == B_ELEMS, "blocks must split into whole KB per wave");
  static_assert(AM >= 3 && BMb >= 3, "swizzles must keep 16-byte chunks whole");

  static __device__ __forceinline__ int a_off(int r, int k) { return swz<AB, AM, AS>(r * BK + k); }
  static __device__ __forceinline__ int b_off(int k, int n) { return swz<BB, BMb, BS>(k * BN + n); }

  // Per-lane source offsets (elements, relative to the tile's origin in the
  // current K block) of every direct load this lane issues.
  struct Src {
    uint32_t a[A_LOADS];
    uint32_t b[B_LOADS];
  };

  static __device__ __forceinline__ void make_src(Src& s, int wave, int lane, int64_t lda, int64_t ldb) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int P = (wave * A_LOADS + i) * 512 + lane * 8;     // physical element this lane fills
      const int L = swz<AB, AM, AS>(P);                        // logical element it must hold
      s.a[i] = uint32_t((L / BK) * lda + (L % BK));
    }
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const int P = (wave * B_LOADS + i) * 512 + lane * 8;
      const int L = swz<BB, BMb, BS>(P);
      s.b[i] = uint32_t((L / BN) * ldb + (L % BN));
    }
  }

  // Issue this wave's direct loads of one K block into `stage` (byte address space 3).
  static __device__ __forceinline__ void issue(const Src& s, LAK_LDS uint16_t* stage, const uint16_t* a_blk,
                                               const uint16_t* b_blk, const uint16_t* b2_blk, int wave) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i)
      __builtin_amdgcn_global_load_lds((const LAK_GLB void*)(a_blk + s.a[i]),
                                       (LAK_LDS void*)(stage + (wave * A_LOADS + i) * 512), 16, 0, 0);
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const uint16_t* bb = t == 0 ? b_blk : b2_blk;
#pragma unroll
      for (int i = 0; i < B_LOADS; ++i)
        __builtin_amdgcn_global_load_lds((const LAK_GLB void*)(bb + s.b[i]),
                                         (LAK_LDS void*)(stage + A_ELEMS + t * B_ELEMS + (wave * B_LOADS + i) * 512),
                                         16, 0, 0);
    }
  }

  static __device__ __forceinline__ u32x4 read_b128(const LAK_LDS uint16_t* p) {
    return *reinterpret_cast<const LAK_LDS u32x4*>(p);
  }
  static __device__ __forceinline__ u32x2 read_tr(const LAK_LDS uint16_t* p) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LAK_LDS i16x4*)(p));
    return __builtin_bit_cast(u32x2, v);
  }

  static __device__ __forceinline__ void compute(const LAK_LDS uint16_t* stage, f32x16 (&acc)[NB][FM][FN], int wm, int wn,
                                                 int lane) {
    const int ar = wm * TM + (lane & 31);
    const int ak = (lane >> 5) * 8;
    const int g = lane >> 4;
    const int bn = wn * TN + 16 * (g & 1) + 4 * (lane & 3);
    const int bk = 8 * (g >> 1) + ((lane >> 2) & 3);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      u32x4 a[FM];
      u32x4 b[NB][FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) a[i] = read_b128(stage + a_off(ar + i * 32, s * 16 + ak));
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        const LAK_LDS uint16_t* bs = stage + A_ELEMS + t * B_ELEMS;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const u32x2 lo = read_tr(bs + b_off(s * 16 + bk, bn + j * 32));
          const u32x2 hi = read_tr(bs + b_off(s * 16 + bk + 4, bn + j * 32));
          b[t][j] = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
      }
#pragma unroll
      for (int t = 0; t < NB; ++t)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[t][i][j] = mfma_32x32x16<TI>(a[i], b[t][j], acc[t][i][j]);
    }
  }
};

template <class TI, class TO, int BM, int BN, int NB, int WM, int WN, int AB, int AM, int AS, int BB, int BMb, int BS>
__global__ void __launch_bounds__(WM * WN * 64) gemm_fast_kernel(const TiledArgs g) {
  using F = Fast<TI, TO, BM, BN, NB, WM, WN, AB, AM, AS, BB, BMb, BS>;
  __shared__ __attribute__((aligned(1024))) uint16_t lds_raw[2 * F::STAGE];
  LAK_LDS uint16_t* lds = (LAK_LDS uint16_t*)lds_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WM, wn = wave / WM;
  int tm, tn;
  grouped_tile(xcd_contiguous(blockIdx.x, gridDim.x), g.tiles_m, g.tiles_n, g.group_m, tm, tn);
  const int64_t m0 = int64_t(tm) * BM, n0 = int64_t(tn) * BN;

  typename F::Src src;
  F::make_src(src, wave, lane, g.lda, g.ldb);
  const uint16_t* a_tile = g.A + m0 * g.lda;
  const uint16_t* b_tile = g.B + n0;
  const uint16_t* b2_tile = NB > 1 ? g.B2 + n0 : nullptr;

  f32x16 acc[NB][F::FM][F::FN];
#pragma unroll
  for (int t = 0; t < NB; ++t)
#pragma unroll
    for (int i = 0; i < F::FM; ++i)
#pragma unroll
      for (int j = 0; j < F::FN; ++j) acc[t][i][j] = f32x16{};

  const int nk = int(g.K / F::BK);
  F::issue(src, lds, a_tile, b_tile, b2_tile, wave);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) {
      const int64_t k1 = int64_t(kt + 1) * F::BK;
      F::issue(src, lds + ((kt + 1) & 1) * F::STAGE, a_tile + k1, b_tile + k1 * g.ldb,
               NB > 1 ? b2_tile + k1 * g.ldb : nullptr, wave);
    }
    F::compute(lds + (kt & 1) * F::STAGE, acc, wm, wn, lane);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the next stage has landed
    __syncthreads();
  }

  typedef typename TO::storage St;
  const int lc = lane & 31, lr4 = (lane >> 5) * 4;
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    St* C = static_cast<St*>(t == 0 ? g.C : g.C2);
#pragma unroll
    for (int i = 0; i < F::FM; ++i) {
#pragma unroll
      for (int j = 0; j < F::FN; ++j) {
        const int64_t col = n0 + wn * F::TN + j * 32 + lc;
        const int64_t rbase = m0 + wm * F::TM + i * 32 + lr4;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t idx = (rbase + 8 * (e >> 2) + (e & 3)) * g.ldc + col;
          float v = g.alpha * acc[t][i][j][e];
          if (NB == 1 && g.beta != 0.0f) v += g.beta * from_out<TO>(C[idx]);
          C[idx] = to_out<TO>(v);
        }
      }
    }
  }
}

// Debug: K block 0 of tile (dbg_tm, dbg_tn) staged by the kernel's own code, then copied out.
template <class TI, class TO, int BM, int BN, int NB, int WM, int WN, int AB, int AM, int AS, int BB, int BMb, int BS>
__global__ void __launch_bounds__(WM * WN * 64) gemm_fast_lds_image(const TiledArgs g) {
  using F = Fast<TI, TO, BM, BN, NB, WM, WN, AB, AM, AS, BB, BMb, BS>;
  __shared__ __attribute__((aligned(1024))) uint16_t lds_raw[F::STAGE];
  LAK_LDS uint16_t* lds = (LAK_LDS uint16_t*)lds_raw;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  typename F::Src src;
  F::make_src(src, wave, lane, g.lda, g.ldb);
  const int64_t m0 = int64_t(g.dbg_tm) * BM, n0 = int64_t(g.dbg_tn) * BN;
  F::issue(src, lds, g.A + m0 * g.lda, g.B + n0, NB > 1 ? g.B2 + n0 : nullptr, wave);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  for (int i = tid; i < F::STAGE; i += F::NT) g.dbg_out[i] = lds[i];
}

}  // namespace lak
