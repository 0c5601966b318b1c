// Fast tiled GEMM for gfx950: 16-byte aligned rows; M and N may end inside a
// tile (edge tiles load clamped source rows and columns and store only inside
// C, see Fast::a_limit and store_band), and K may end inside a K block (the
// remaining K % BK values are added after the main loop, Fast::k_tail).
//
// Differences from the general kernel (gemm_tiled.hpp):
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
//  * A fragments are plain 16-byte LDS reads (K is contiguous in A).  A stored
//    [K, M] (M contiguous) stays M-contiguous in LDS and is read with the same
//    transposing reads as B.
//  * Large tiles (256 x 256, or 256 x 2*128 for gate/up) with 8 waves: one
//    tile per CU at 4096^2, two waves per SIMD.  For gate/up the waves split
//    by weight: waves 0-3 own 64-column slices of the W_gate product, waves 4-7
//    the same slices of the W_up product (the same 128 x 64 wave tile as the
//    plain kernel, so both outputs leave in 128-byte row segments).
//  * A multi-stage LDS ring (STAGES buffers) keeps STAGES-1 K blocks in
//    flight.
//  * Ping-pong wave groups: the 8 waves form two groups of four (one wave of
//    each group per SIMD); while one group runs a K block's MFMAs the other
//    reads its fragments and issues its direct loads (gemm_fast_pp_kernel).
//  * One-byte inputs (gemm_fast_f8.hip) run the K-major configurations on
//    byte pairs seen as 16-bit units; only the products change (mma_block,
//    mma1: one 32x32x64 product per K block instead of two 32x32x16).
// The LDS maps are Swizzle{AB,AM,AS} o (BM,BK):(BK,1) for A and
// Swizzle{BB,BMb,BS} o (BK,BN):(BN,1) for B (element offsets).
#pragma once

#include "kernel_common.hpp"
#include "launch.hpp"

namespace lak {

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define LAK_LDS __attribute__((address_space(3)))
#define LAK_GLB __attribute__((address_space(1)))

template <class TI, class C>
struct Fast {
  static constexpr int BM = C::BM, BN = C::BN, NB = C::NB, WM = C::WM, WN = C::WN, BK = C::BK;
  static constexpr int STAGES = C::STAGES;
  static constexpr bool BKM = C::BKMAJOR;                 // B stored [N, K] (K contiguous) instead of [K, N]
  static constexpr bool ATR = C::ATRANS;                  // A stored [K, M] (M contiguous) instead of [M, K]
  static constexpr int NW = WM * WN;
  static constexpr int NT = NW * 64;
  // waves split by weight (gate/up): NBW weights per wave, WNW waves along N per weight
  static constexpr bool WSPLIT = C::WSPLIT;
  static constexpr int NBW = WSPLIT ? 1 : NB, WNW = WSPLIT ? WN / NB : WN;
  static_assert(!WSPLIT || (NB == 2 && WN % NB == 0), "waves split by weight need two weights");
  static constexpr int TM = BM / WM, TN = BN / WNW;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int SUB = BK / 16;                      // MFMA K sub-steps per K block
  static constexpr int A_ELEMS = BM * BK;
  static constexpr int B_ELEMS = BK * BN;
  static constexpr int STAGE = A_ELEMS + NB * B_ELEMS;     // 16-bit elements
  // LDS of the kernel (16-bit elements): the stage ring, or for waves split by weight the SwiGLU
  // exchange of the epilogue (two regions of 4 x FN x 64 x 16 floats plus a window per wave) if larger
  static constexpr int XCHG = WSPLIT ? (2 * 4 * (BN / (WN / NB) / 32) * 64 * 16 + NW * 32 * (BN / (WN / NB) + 8)) * 2 : 0;
  static constexpr int LDS_ELEMS = STAGES * STAGE > XCHG ? STAGES * STAGE : XCHG;
  static constexpr int A_LOADS = A_ELEMS / 512 / NW;       // 1 KB (512 elements) per wave instruction
  static constexpr int B_LOADS = B_ELEMS / 512 / NW;
  static constexpr int LOADS_PER_STAGE = A_LOADS + NB * B_LOADS;
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(A_LOADS * 512 * NW == A_ELEMS && B_LOADS * 512 * NW == B_ELEMS, "blocks must split into whole KB per wave");
  static_assert(C::AM >= 3 && C::BMb >= 3, "swizzles must keep 16-byte chunks whole");
  static_assert(BK % 16 == 0 && STAGES >= 2, "K block and pipeline depth");
  static_assert((STAGES - 2) * LOADS_PER_STAGE < 64, "vmcnt range");

  // A block in LDS: K-contiguous rows of BK per m, or (A stored [K, M]) M-contiguous rows of BM per k.
  static __device__ __forceinline__ int a_off(int r, int k) {
    return ATR ? swz<C::AB, C::AM, C::AS>(k * BM + r) : swz<C::AB, C::AM, C::AS>(r * BK + k);
  }
  // Global A: origin of the tile at row m0, and the element step of K block k1.
  static __device__ __forceinline__ const uint16_t* a_origin(const uint16_t* A, int64_t m0, int64_t lda) {
    return ATR ? A + m0 : A + m0 * lda;
  }
  static __device__ __forceinline__ int64_t a_step(int64_t k1, int64_t lda) { return ATR ? k1 * lda : k1; }
  // B block in LDS: N-contiguous rows of BN per k, or (K-major B) K-contiguous rows of BK per n.
  static __device__ __forceinline__ int b_off(int k, int n) {
    return BKM ? swz<C::BB, C::BMb, C::BS>(n * BK + k) : swz<C::BB, C::BMb, C::BS>(k * BN + n);
  }
  // Global B: origin of the tile at column n0, and the element step of K block k1.
  static __device__ __forceinline__ const uint16_t* b_origin(const uint16_t* B, int64_t n0, int64_t ldb) {
    return BKM ? B + n0 * ldb : B + n0;
  }
  static __device__ __forceinline__ int64_t b_step(int64_t k1, int64_t ldb) { return BKM ? k1 : k1 * ldb; }

  // Per-lane source offsets (elements, relative to the tile's origin in the
  // current K block) of every direct load this lane issues.
  struct Src {
    uint32_t a[A_LOADS];
    uint32_t b[B_LOADS];
  };

  // Source limits of a tile at (m0, n0) that may cross M or N (K is a multiple
  // of BK): the last row of A (A stored [K, M]: the last 8-element chunk along
  // M) and the last 8-element chunk of a B row (B stored [N, K]: the last row)
  // a lane may read.  Elements past the edge are loaded from the clamped
  // position instead: they only ever meet rows or columns of C that are not
  // stored (C[i, j] depends on row i of A and column j of B alone), and every
  // address stays inside the operand.
  static __device__ __forceinline__ int a_limit(int64_t M, int64_t m0) {
    const int64_t left = M - m0;                       // >= 1
    return ATR ? int(min<int64_t>(BM, (left + 7) & ~int64_t(7)) - 8) : int(min<int64_t>(BM, left) - 1);
  }
  static __device__ __forceinline__ int b_limit(int64_t N, int64_t n0) {
    const int64_t left = N - n0;                       // >= 1
    return BKM ? int(min<int64_t>(BN, left) - 1) : int(min<int64_t>(BN, (left + 7) & ~int64_t(7)) - 8);
  }

  static __device__ __forceinline__ void make_src(Src& s, int wave, int lane, int64_t lda, int64_t ldb, int a_lim,
                                                  int b_lim) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int P = (wave * A_LOADS + i) * 512 + lane * 8;     // physical element this lane fills
      const int L = swz<C::AB, C::AM, C::AS>(P);               // logical element it must hold
      s.a[i] = ATR ? uint32_t((L / BM) * lda + min(L % BM, a_lim)) : uint32_t(min(L / BK, a_lim) * lda + (L % BK));
    }
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const int P = (wave * B_LOADS + i) * 512 + lane * 8;
      const int L = swz<C::BB, C::BMb, C::BS>(P);
      s.b[i] = BKM ? uint32_t(min(L / BK, b_lim) * ldb + (L % BK)) : uint32_t((L / BN) * ldb + min(L % BN, b_lim));
    }
  }

  // One direct load: 64 lanes x 16 bytes from base + voff (bytes, per lane)
  // into the kilobyte of LDS at byte address `lds_addr` (wave-uniform, via M0).
  // Written as inline assembly so that the compiler's wait-count pass does not
  // see an LDS write it cannot disambiguate: it would otherwise stall every
  // later LDS read until all loads in flight have landed.  Completion is
  // tracked explicitly with vmcnt waits before each barrier.
  static __device__ __forceinline__ void dma16(const uint16_t* base, uint32_t voff, const LAK_LDS uint16_t* dst) {
    const uint32_t lds_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst));
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2"
        :
        : "s"(lds_addr), "v"(voff), "s"(base)
        : "memory", "m0");
  }

  // Issue this wave's direct loads of one K block into `stage`.
  static __device__ __forceinline__ void issue(const Src& s, LAK_LDS uint16_t* stage, const uint16_t* a_blk,
                                               const uint16_t* b_blk, const uint16_t* b2_blk, int wave) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) dma16(a_blk, s.a[i] * 2u, stage + (wave * A_LOADS + i) * 512);
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const uint16_t* bb = t == 0 ? b_blk : b2_blk;
#pragma unroll
      for (int i = 0; i < B_LOADS; ++i) dma16(bb, s.b[i] * 2u, stage + A_ELEMS + t * B_ELEMS + (wave * B_LOADS + i) * 512);
    }
  }

  static __device__ __forceinline__ u32x4 read_b128(const LAK_LDS uint16_t* p) {
    return *reinterpret_cast<const LAK_LDS u32x4*>(p);
  }
  static __device__ __forceinline__ u32x2 read_tr(const LAK_LDS uint16_t* p) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LAK_LDS i16x4*)(p));
    return __builtin_bit_cast(u32x2, v);
  }

  // Lane-dependent parts of the fragment addresses.
  struct Lane {
    int ar, ak, bn, bk, br, am, tw;
    __device__ __forceinline__ Lane(int wm, int wn_all, int lane) {
      tw = WSPLIT ? wn_all / WNW : 0;            // weight block this wave reads (split waves)
      const int wn = WSPLIT ? wn_all % WNW : wn_all;
      ar = wm * TM + (lane & 31);                // A: row l % 32 of each 32-row block
      ak = (lane >> 5) * 8;                      // A: K half of the 16-wide sub-step
      const int g = lane >> 4;                   // B (N-contiguous): 16-lane group
      bn = wn * TN + 16 * (g & 1) + 4 * (lane & 3);
      am = wm * TM + 16 * (g & 1) + 4 * (lane & 3);   // A (M-contiguous): as bn, along M
      bk = 8 * (g >> 1) + ((lane >> 2) & 3);
      br = wn * TN + (lane & 31);                // B (K-contiguous): column l % 32 of each 32-column block
    }
  };

  struct Frags {
    u32x4 a[FM];
    u32x4 b[NBW][FN];
  };

  static __device__ __forceinline__ void read_frags(const LAK_LDS uint16_t* stage, int s, const Lane& ln, Frags& f) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if constexpr (ATR) {
        // M-contiguous A rows: transposing reads, lane mapping as for N-contiguous B
        const u32x2 lo = read_tr(stage + a_off(ln.am + i * 32, s * 16 + ln.bk));
        const u32x2 hi = read_tr(stage + a_off(ln.am + i * 32, s * 16 + ln.bk + 4));
        f.a[i] = u32x4{lo.x, lo.y, hi.x, hi.y};
      } else {
        f.a[i] = read_b128(stage + a_off(ln.ar + i * 32, s * 16 + ln.ak));
      }
    }
#pragma unroll
    for (int t = 0; t < NBW; ++t) {
      const LAK_LDS uint16_t* bs = stage + A_ELEMS + (WSPLIT ? ln.tw : t) * B_ELEMS;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (BKM) {
          // K-contiguous B rows: one plain 16-byte read gives the lane its 8 K values
          f.b[t][j] = read_b128(bs + b_off(s * 16 + ln.ak, ln.br + j * 32));
        } else {
          const u32x2 lo = read_tr(bs + b_off(s * 16 + ln.bk, ln.bn + j * 32));
          const u32x2 hi = read_tr(bs + b_off(s * 16 + ln.bk + 4, ln.bn + j * 32));
          f.b[t][j] = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
      }
    }
  }

  // Eight K values k .. k+7 of one row of a K-contiguous operand (p points at
  // element k), zero from K on; k is a multiple of 8 and the row starts on 16
  // bytes, so a whole chunk is one 16-byte load.
  static __device__ __forceinline__ u32x4 tail_contig(const uint16_t* p, int64_t valid) {
    if (valid >= 8) return *reinterpret_cast<const u32x4*>(p);
    uint16_t e[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) e[q] = q < valid ? p[q] : uint16_t(0);
    return u32x4{e[0] | (uint32_t(e[1]) << 16), e[2] | (uint32_t(e[3]) << 16), e[4] | (uint32_t(e[5]) << 16),
                 e[6] | (uint32_t(e[7]) << 16)};
  }
  // The same along a column of an operand stored K-outer (element k + q at p[q * ld]).
  static __device__ __forceinline__ u32x4 tail_strided(const uint16_t* p, int64_t ld, int64_t valid) {
    uint16_t e[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) e[q] = q < valid ? p[q * ld] : uint16_t(0);
    return u32x4{e[0] | (uint32_t(e[1]) << 16), e[2] | (uint32_t(e[3]) << 16), e[4] | (uint32_t(e[5]) << 16),
                 e[6] | (uint32_t(e[7]) << 16)};
  }

  // K values past the last whole K block (K % BK of them), added after the main
  // loop straight from global memory into MFMA fragments: lane l of a 32-row
  // (or 32-column) block holds row (column) l % 32 and the 8 K values from
  // 8 (l / 32) on of each 16-wide step, zero from K on; rows past M and
  // columns past N read the last valid one (they reach no stored output).
  // Nothing goes through LDS, so the main loop's schedule is untouched.  Per
  // step the B fragments are loaded first, then one A fragment at a time with
  // its products, which keeps the tail within the main loop's registers.
  static __device__ __forceinline__ void k_tail(f32x16 (&acc)[NBW][FM][FN], const TiledArgs& g, int64_t m0, int64_t n0,
                                                int wm, int wn_all, int lane) {
    const int64_t k0 = (g.K / BK) * BK;
    const int tw = WSPLIT ? wn_all / WNW : 0;
    const int wn = WSPLIT ? wn_all % WNW : wn_all;
    const int l32 = lane & 31, h8 = (lane >> 5) * 8;
#pragma unroll
    for (int s = 0; s < SUB; ++s) {
      if (k0 + 16 * s >= g.K) break;                    // wave-uniform
      const int64_t kl = k0 + 16 * s + h8;              // this lane's first K value of the step
      const int64_t valid = g.K - kl;
      u32x4 fb[NBW][FN];
#pragma unroll
      for (int t = 0; t < NBW; ++t) {
        const uint16_t* B = (WSPLIT ? tw : t) == 0 ? g.B : g.B2;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int64_t n = min<int64_t>(n0 + wn * TN + j * 32 + l32, g.N - 1);
          fb[t][j] = BKM ? tail_contig(B + n * g.ldb + kl, valid) : tail_strided(B + kl * g.ldb + n, g.ldb, valid);
        }
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int64_t m = min<int64_t>(m0 + wm * TM + i * 32 + l32, g.M - 1);
        const u32x4 fa =
            ATR ? tail_strided(g.A + kl * g.lda + m, g.lda, valid) : tail_contig(g.A + m * g.lda + kl, valid);
#pragma unroll
        for (int t = 0; t < NBW; ++t)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[t][i][j] = mma1(fa, fb[t][j], acc[t][i][j]);
      }
    }
  }

  // One product of a 16-value step of 16-bit elements; for one-byte elements
  // (16-bit units holding byte pairs) the step is 32 values in the lower half
  // of a 64-deep product whose upper half is zero.
  static __device__ __forceinline__ f32x16 mma1(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (TI::f8) return mfma_f8_32x32x64<TI>(a, u32x4{}, b, u32x4{}, c);
    else return mfma_32x32x16<TI>(a, b, c);
  }

  // The products of one whole K block: SUB steps of 16 16-bit values, or for
  // one-byte elements one 64-deep product over both steps' reads.
  static __device__ __forceinline__ void mma_block(const Frags (&f)[SUB], f32x16 (&acc)[NBW][FM][FN]) {
    if constexpr (TI::f8) {
      // a 64-deep one-byte product takes the two 16-byte reads of a 32-unit step pair
      static_assert(SUB % 2 == 0, "one-byte products pair the sub-steps");
#pragma unroll
      for (int s = 0; s < SUB; s += 2)
#pragma unroll
        for (int t = 0; t < NBW; ++t)
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
              acc[t][i][j] = mfma_f8_32x32x64<TI>(f[s].a[i], f[s + 1].a[i], f[s].b[t][j], f[s + 1].b[t][j], acc[t][i][j]);
    } else {
#pragma unroll
      for (int s = 0; s < SUB; ++s) mma(f[s], acc);
    }
  }

  static __device__ __forceinline__ void mma(const Frags& f, f32x16 (&acc)[NBW][FM][FN]) {
#pragma unroll
    for (int t = 0; t < NBW; ++t)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[t][i][j] = mfma_32x32x16<TI>(f.a[i], f.b[t][j], acc[t][i][j]);
  }
};

// vmcnt(n) with the other counters left alone (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier without a memory fence (a fence would also wait for the
// direct loads still in flight).  The empty asm statements with a memory
// clobber keep the compiler from moving LDS accesses across it; LDS reads
// issued before it have been waited for by their consumers.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS reads are complete
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}


// Epilogue through LDS: each wave writes alpha * acc of one 32-row band of its
// sub-tile (32 x TN, FP32) into its own padded LDS window, reads it back as
// rows, and writes 8 consecutive outputs per lane (16 bytes for 16-bit types),
// so every row segment leaves as whole vectors instead of one element per lane
// and register.  beta * C_old is added on the way out, reading C_old with the
// same vectors (only when beta != 0).  All LDS reads of the main loop must be
// finished before the first wave writes its window.  The stores carry the
// non-temporal hint: the output is not read again by this kernel, and with one
// tile per CU the whole of it drains at the end of the launch (4096^3:
// 108.1 -> 106.7 us, gate/up 607.9 -> 592.6 us measured).
// RED: also fold the row reduction `red` of the FP32 values into R (a separate
// instantiation, so that launches without it run exactly the plain epilogue).
// Rows from M on and columns from N on are not written (C_old is not read
// there either); a row segment of 8 cut by N is written element by element.
template <class TO, class F, bool RED = false>
__device__ __forceinline__ void store_band(const f32x16 (&accb)[F::FN], void* Cv, int64_t ldc, int64_t M, int64_t N,
                                           float alpha, float beta, bool use_beta, int64_t row0, int64_t col0,
                                           LAK_LDS float* win, int lane, int red = RED_NONE, float* R = nullptr) {
  constexpr int TN = F::TN;
  constexpr int PITCH = TN + 8;                      // floats: rows r and r+4 land 32 banks apart
  typedef typename TO::storage St;
  St* C = static_cast<St*>(Cv);
  const int lc = lane & 31, lr4 = (lane >> 5) * 4;
#pragma unroll
  for (int j = 0; j < F::FN; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) win[(8 * (e >> 2) + lr4 + (e & 3)) * PITCH + j * 32 + lc] = alpha * accb[j][e];
  __builtin_amdgcn_s_waitcnt(0xC07F);                // this wave's LDS writes are done
  constexpr int CH = TN / 8;                         // 8-element chunks per row
  constexpr int ROWS_PER_PASS = 64 / CH;
#pragma unroll
  for (int q = 0; q < 32 / ROWS_PER_PASS; ++q) {
    const int r = q * ROWS_PER_PASS + lane / CH;
    const int c = (lane % CH) * 8;
    const LAK_LDS float* src = win + r * PITCH + c;
    const f32x4 lo = *reinterpret_cast<const LAK_LDS f32x4*>(src);
    const f32x4 hi = *reinterpret_cast<const LAK_LDS f32x4*>(src + 4);
    float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    const int64_t row = row0 + r;
    const int64_t nleft = N - (col0 + c);              // valid columns from this chunk on
    if (row >= M || nleft <= 0) continue;
    St* dst = C + row * ldc + col0 + c;
    const bool whole = nleft >= 8;
    if (use_beta) {
      if (whole) {
        if constexpr (sizeof(St) == 4) {
          const f32x4 o0 = *reinterpret_cast<const f32x4*>(dst);
          const f32x4 o1 = *reinterpret_cast<const f32x4*>(dst + 4);
          const float o[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] += beta * o[e];
        } else {
          const u32x4 ow = *reinterpret_cast<const u32x4*>(dst);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] += beta * from_out<TO>(static_cast<St>((ow[e >> 1] >> (16 * (e & 1))) & 0xffffu));
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e < nleft) v[e] += beta * from_out<TO>(dst[e]);
      }
    }
    if constexpr (RED) {
      // row reduction: the lane's valid values, then the CH lanes sharing row r (a lane whose
      // chunk lies past N has left the loop; the reduction runs over the lanes still active)
      float p = v[0];
#pragma unroll
      for (int e = 1; e < 8; ++e)
        if (e < nleft) p = red_combine(red, p, v[e]);
      if (whole && N - col0 >= F::TN && M - row0 >= 32) {
        p = red_lanes<CH>(red, p);
        if (lane % CH == 0) red_commit(red, R + row, p);
      } else {
        red_commit(red, R + row, p);
      }
    }
    if (whole) {
      if constexpr (sizeof(St) == 4) {
        __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(dst));
        __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, reinterpret_cast<f32x4*>(dst + 4));
      } else {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = uint32_t(to_out<TO>(v[2 * e])) | (uint32_t(to_out<TO>(v[2 * e + 1])) << 16);
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(dst));
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e < nleft) dst[e] = to_out<TO>(v[e]);
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);                // reads done before the next band overwrites the window
}

template <class TO, class F, bool RED = false>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[F::FM][F::FN], void* Cv, int64_t ldc, int64_t M, int64_t N,
                                           float alpha, float beta, bool use_beta, int64_t row0, int64_t col0,
                                           LAK_LDS float* win, int lane, int red = RED_NONE, float* R = nullptr) {
#pragma unroll
  for (int i = 0; i < F::FM; ++i)
    store_band<TO, F, RED>(acc[i], Cv, ldc, M, N, alpha, beta, use_beta, row0 + i * 32, col0, win, lane, red, R);
}

// SwiGLU epilogue of waves split by weight (see epilogue): wave of weight TW (0: W_gate, 1: W_up)
// gives bands GIVE and takes its partner's half of bands OWN, through regions rg[TW] (written)
// and rg[1 - TW] (read), each of 4 waves x FN blocks x 4 quads x 64 lanes of f32x4.
template <class TO, class F, int TW>
__device__ __forceinline__ void swiglu_exchange(f32x16 (&acc)[F::NBW][F::FM][F::FN], const TiledArgs& g, LAK_LDS f32x4* rg,
                                                int64_t row0, int64_t col0, LAK_LDS float* xwin, int slot, int lane) {
  constexpr int REG = 4 * F::FN * 4 * 64;
  LAK_LDS f32x4* give = rg + TW * REG;
  const LAK_LDS f32x4* take = rg + (1 - TW) * REG;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    // the W_gate wave gives band it and evaluates band it + 2; the W_up wave the other way round
    const int give_band = TW == 0 ? it : it + 2, own_band = TW == 0 ? it + 2 : it;
#pragma unroll
    for (int j = 0; j < F::FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x16& a = acc[0][give_band][j];
        give[((slot * F::FN + j) * 4 + q) * 64 + lane] = f32x4{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
      }
    block_barrier();                                 // both halves of the exchange are in LDS
    f32x16 h[F::FN];
#pragma unroll
    for (int j = 0; j < F::FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 o = take[((slot * F::FN + j) * 4 + q) * 64 + lane];
        const f32x16& m = acc[0][own_band][j];
        const float ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)   // gate first: the wave's own value for TW == 0, the partner's otherwise
          h[j][4 * q + e] = TW == 0 ? swiglu(m[4 * q + e], ov[e]) : swiglu(ov[e], m[4 * q + e]);
      }
    store_band<TO, F>(h, g.C, g.ldc, g.M, g.N, 1.0f, 0.0f, false, row0 + own_band * 32, col0, xwin, lane);
    block_barrier();                                 // every wave has read its half before the next band is given
  }
}

template <class TO, class F, bool RED = false>
__device__ __forceinline__ void epilogue(f32x16 (&acc)[F::NBW][F::FM][F::FN], const TiledArgs& g, int64_t m0, int64_t n0,
                                         int wm, int wn, int wave, int lane, LAK_LDS uint16_t* lds) {
  constexpr int NB = F::NB;
  static_assert(F::NW * 32 * (F::TN + 8) * 4 <= F::STAGES * F::STAGE * 2, "epilogue windows must fit in the stage buffers");
  LAK_LDS float* win = reinterpret_cast<LAK_LDS float*>(lds) + wave * 32 * (F::TN + 8);
  const int64_t row0 = m0 + wm * F::TM;
  if constexpr (F::WSPLIT) {
    // waves split by weight: wave (wm, wn) holds the W_gate (wn < WNW) or W_up product of
    // columns (wn mod WNW) * TN .. + TN of the tile
    const int tw = wn / F::WNW;
    const int64_t col0 = n0 + (wn % F::WNW) * F::TN;
    if (g.act == 0) {
      store_tile<TO, F>(acc[0], tw == 0 ? g.C : g.C2, g.ldc, g.M, g.N, 1.0f, 0.0f, false, row0, col0, win, lane);
      return;
    }
    // SwiGLU: silu(g) * u needs the W_gate and W_up accumulators of an element together, and they
    // sit in the paired waves w and w + 4 (same wm, same column slice).  Each pair splits the
    // work: for bands 0 and 1 (32 rows each) the W_gate wave hands its FP32 values to the W_up
    // wave, for bands 2 and 3 the other way round, through two LDS regions in the lanes' own
    // register order; each wave evaluates its bands in FP32 and stores H through its window
    // (after the regions).  All waves pass the same four barriers.
    static_assert(F::NW == 8 && F::WNW * F::WM == 4 && F::FM == 4, "four waves per weight, four bands");
    constexpr int REG = 4 * F::FN * 4 * 64;          // f32x4 per region: 4 waves x FN blocks x 4 quads x 64 lanes
    static_assert((2 * REG * 4 + F::NW * 32 * (F::TN + 8)) * 4 <= F::LDS_ELEMS * 2, "SwiGLU exchange must fit in LDS");
    LAK_LDS float* xwin = reinterpret_cast<LAK_LDS float*>(lds) + 2 * REG * 4 + wave * 32 * (F::TN + 8);
    // one instantiation per weight, so every band index below is a compile-time constant (a
    // runtime index into the accumulator array would move it to scratch memory)
    if (tw == 0) {
      swiglu_exchange<TO, F, 0>(acc, g, reinterpret_cast<LAK_LDS f32x4*>(lds), row0, col0, xwin, wave & 3, lane);
    } else {
      swiglu_exchange<TO, F, 1>(acc, g, reinterpret_cast<LAK_LDS f32x4*>(lds), row0, col0, xwin, wave & 3, lane);
    }
    return;
  } else {
    const int64_t col0 = n0 + wn * F::TN;
    if constexpr (NB == 2) {
      if (g.act == 1) {
        // fused activation: the gate and up accumulators of one element sit in the same lane
#pragma unroll
        for (int i = 0; i < F::FM; ++i)
#pragma unroll
          for (int j = 0; j < F::FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[0][i][j][e] = swiglu(acc[0][i][j][e], acc[1][i][j][e]);
        store_tile<TO, F>(acc[0], g.C, g.ldc, g.M, g.N, 1.0f, 0.0f, false, row0, col0, win, lane);
        return;
      }
    }
#pragma unroll
    for (int t = 0; t < NB; ++t)
      store_tile<TO, F, RED && NB == 1>(acc[t], t == 0 ? g.C : g.C2, g.ldc, g.M, g.N, g.alpha, g.beta, NB == 1 && g.beta != 0.0f,
                                        row0, col0, win, lane, g.red, g.R);
  }
}

// Ping-pong schedule.  The 8 waves form two groups of 4 (one wave of each
// group per SIMD).  Each K block is handled in two phases per group:
//   M: read all fragments of the block from LDS into registers and issue this
//      wave's share of the global->LDS loads of a later block;
//   C: run the block's MFMAs back to back.
// Group 1 runs one phase behind group 0, so on every SIMD one wave feeds the
// matrix core while the other moves data.  Every phase starts with a
// workgroup barrier (s_barrier without a memory fence, so direct loads stay in
// flight); group 1 adds one barrier at the start, group 0 one at the end.
// Phase t = 2j is group 0's M(j): before its barrier every wave has waited
// for its own loads of block j.  M(kt) refills the buffer of block kt-1, which
// both groups finished reading before the barrier that opened it.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <class F>
__device__ __forceinline__ void wait_block(int kt, int nk) {
  // loads issued after block kt: blocks kt+1 .. min(kt+STAGES-2, nk-1)
  if (kt + F::STAGES - 2 <= nk - 1) {
    wait_vmcnt<(F::STAGES - 2) * F::LOADS_PER_STAGE>();
  } else {
    wait_vmcnt<0>();
  }
}

// KT: K ends inside a K block (K % BK != 0), so the kernel adds the last values
// after the main loop; a separate instantiation because the tail's registers
// would otherwise push the whole-block kernels into spills.
template <class TI, class TO, class C, bool RED = false, bool KT = false>
__global__ void __launch_bounds__(C::WM * C::WN * 64) gemm_fast_pp_kernel(const TiledArgs g_in) {
  const TiledArgs g = at_batch(g_in);
  using F = Fast<TI, C>;
  constexpr int NB = C::NB;
  static_assert(C::WM * C::WN == 8, "ping-pong needs two groups of four waves");
  __shared__ __attribute__((aligned(1024))) uint16_t lds_raw[F::LDS_ELEMS];
  LAK_LDS uint16_t* lds = (LAK_LDS uint16_t*)lds_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;
  const int wm = wave % C::WM, wn = wave / C::WM;
  int tm, tn;
  grouped_tile(xcd_contiguous(blockIdx.x, gridDim.x), g.tiles_m, g.tiles_n, g.group_m, tm, tn);
  const int64_t m0 = int64_t(tm) * C::BM, n0 = int64_t(tn) * C::BN;

  typename F::Src src;
  F::make_src(src, wave, lane, g.lda, g.ldb, F::a_limit(g.M, m0), F::b_limit(g.N, n0));
  const typename F::Lane ln(wm, wn, lane);
  const uint16_t* a_tile = F::a_origin(g.A, m0, g.lda);
  const uint16_t* b_tile = F::b_origin(g.B, n0, g.ldb);
  const uint16_t* b2_tile = NB > 1 ? F::b_origin(g.B2, n0, g.ldb) : nullptr;

  f32x16 acc[F::NBW][F::FM][F::FN];
#pragma unroll
  for (int t = 0; t < F::NBW; ++t)
#pragma unroll
    for (int i = 0; i < F::FM; ++i)
#pragma unroll
      for (int j = 0; j < F::FN; ++j) acc[t][i][j] = f32x16{};

  const int nk = int(g.K / F::BK);
#pragma unroll
  for (int p = 0; p < F::STAGES - 1; ++p) {
    if (p < nk) {
      const int64_t k1 = int64_t(p) * F::BK;
      F::issue(src, lds + p * F::STAGE, a_tile + F::a_step(k1, g.lda), b_tile + F::b_step(k1, g.ldb),
               NB > 1 ? b2_tile + F::b_step(k1, g.ldb) : nullptr, wave);
    }
  }
  if (group == 1) {
    wait_block<F>(0, nk);
    phase_barrier();                       // t = 0: group 1 idles while group 0 reads block 0
  }
  typename F::Frags f[F::SUB];
  for (int kt = 0; kt < nk; ++kt) {
    if (group == 0) wait_block<F>(kt, nk);
    phase_barrier();                       // M(kt)
#pragma unroll
    for (int s = 0; s < F::SUB; ++s) F::read_frags(lds + (kt % F::STAGES) * F::STAGE, s, ln, f[s]);
    const int kn = kt + F::STAGES - 1;
    if (kn < nk) {
      const int64_t k1 = int64_t(kn) * F::BK;
      F::issue(src, lds + (kn % F::STAGES) * F::STAGE, a_tile + F::a_step(k1, g.lda), b_tile + F::b_step(k1, g.ldb),
               NB > 1 ? b2_tile + F::b_step(k1, g.ldb) : nullptr, wave);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0): fragments in registers
    if (group == 1) {
      if (kt + 1 < nk) wait_block<F>(kt + 1, nk);
    }
    phase_barrier();                       // C(kt)
    F::mma_block(f, acc);
  }
  if (group == 0) phase_barrier();         // t = 2 nk: group 0 idles while group 1 finishes
  if constexpr (KT) F::k_tail(acc, g, m0, n0, wm, wn, lane);

  // After the last phase barrier every M phase (all LDS reads) is complete,
  // so the waves may reuse the stage buffers as epilogue windows.
  epilogue<TO, F, RED>(acc, g, m0, n0, wm, wn, wave, lane, lds);
}

// Debug: K block 0 of tile (dbg_tm, dbg_tn) staged by the kernel's own code, then copied out.
template <class TI, class TO, class C>
__global__ void __launch_bounds__(C::WM * C::WN * 64) gemm_fast_lds_image(const TiledArgs g) {
  using F = Fast<TI, C>;
  __shared__ __attribute__((aligned(1024))) uint16_t lds_raw[F::STAGE];
  LAK_LDS uint16_t* lds = (LAK_LDS uint16_t*)lds_raw;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t m0 = int64_t(g.dbg_tm) * C::BM, n0 = int64_t(g.dbg_tn) * C::BN;
  typename F::Src src;
  F::make_src(src, wave, lane, g.lda, g.ldb, F::a_limit(g.M, m0), F::b_limit(g.N, n0));
  F::issue(src, lds, F::a_origin(g.A, m0, g.lda), F::b_origin(g.B, n0, g.ldb),
           C::NB > 1 ? F::b_origin(g.B2, n0, g.ldb) : nullptr, wave);
  wait_vmcnt<0>();
  block_barrier();
  for (int i = tid; i < F::STAGE; i += F::NT) g.dbg_out[i] = lds[i];
}

// ------------------------------------------------------------------ launch
// Launch of one configuration for every input / output type (instantiated by gemm_fast.hip,
// gemm_fast_gu.hip and gemm_fast_128.hip, one translation unit per group of configurations).
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

hipError_t launch_fast_gu(int kid, int in_kind, int out_kind, const TiledArgs& args, dim3 grid, hipStream_t stream,
                          bool lds_image);
hipError_t launch_fast_128(int kid, int in_kind, int out_kind, const TiledArgs& args, dim3 grid, hipStream_t stream,
                           bool lds_image);

}  // namespace lak
