// GEMM with binary32 inputs for gfx950: C = alpha * A * B + beta * C, A and B
// binary32, products and sums on the matrix cores in FP32
// (v_mfma_f32_32x32x2_f32).
//
// Structure (per workgroup, one 128 x 128 output tile, 4 waves of 64 x 64):
//   * K is walked in blocks of 32.  Each thread stages 4-element (16-byte)
//     chunks global -> registers -> LDS: one 16-byte load when rows start on
//     16 bytes and no chunk is cut by an edge (V == 4), else four 4-byte
//     loads (V == 1).  Every element outside the matrix is loaded from a
//     zero word instead (the zero-filled edge semantics of the Tylo.jl page
//     "TMA and Hopper WGMMA", section "Copy and completion"); only addresses
//     are selected, so no load waits under a branch.
//   * In LDS an operand stored K-contiguous (A [M, K], B [N, K]) is kept
//     K-contiguous as two sub-blocks of 16 values: one 64-byte row per M row
//     (N column), the 64-byte binary32 plan of the Tylo.jl page "TMA and
//     Hopper WGMMA" (section "The same storage contract on both sides": inner
//     extent 16 four-byte elements, outer extent 128 rows), under
//     Swizzle{2,2,4}: element (r, k) of sub-block h sits at
//     2048 h + 16 r + (k XOR 4 ((r >> 2) mod 4)).  The page's map for these
//     rows is Swizzle{2,2,3}, made for 32 banks: on gfx950's 64 banks a
//     16-byte read of 16 consecutive rows under it touches only 8 distinct
//     16-byte slots (only row bits 0-2 enter the slot), a 2-way conflict;
//     taking the XOR from row bits 2-3 spreads the 16 rows over all 64 banks.
//     An operand stored along M or N (A [K, M], B [K, N]) is kept that way, one
//     row of 128 values per k, under Swizzle{1,5,5}: element (k, c) at
//     128 k + (c XOR 32 ((k >> 3) mod 2)), so that the two K rows one
//     fragment read touches (k and k + 8) fall into different halves of the
//     banks.
//   * The K values of one 16-value sub-block are split between the two
//     32-lane halves of a wave: MFMA j (0..7) multiplies, in lanes 32 g ..
//     32 g + 31, the K value 8 g + j.  A dot product does not depend on the
//     order of its terms, and A and B use the same split, so each lane of a
//     K-contiguous operand reads its 8 values as two 16-byte LDS reads; an
//     M/N-contiguous operand is read one 4-byte value per lane and MFMA.
//   * Two LDS stages of 32 KiB: while the MFMAs consume stage s, the next
//     block is written from registers to stage s^1 and the one after it is
//     loaded; one workgroup barrier per block, placed between the two
//     sub-blocks' MFMAs so that every fragment read is issued a sub-block
//     ahead of its use (the two synchronisations of the Tylo.jl page
//     "Layouts, storage and ownership", section "Plans describe work, callers
//     establish readiness").  Two workgroups share a CU.
//   * Each wave owns 2 x 2 blocks of 32 x 32 FP32 accumulators for the whole K
//     loop (Phobos "Tiles and shared memory", section "Tiles in registers").
//   * Epilogue: alpha * acc + beta * C_old in FP32 (C_old read only when
//     beta != 0), rounded to nearest even for 16-bit outputs, written only
//     inside [0,M) x [0,N), with the optional row reduction.
#include "kernel_common.hpp"
#include "launch.hpp"

namespace lak {

// Sixteen zero bytes in device memory: staging loads of elements outside the
// matrix read from here.
__device__ __attribute__((aligned(16))) float kZeroWords[4];

template <class TO, int V, bool AT, bool BKM>
struct TiledF32 {
  static constexpr int BM = 128, BN = 128, BK = 32, KS = 16;    // KS: values per 64-byte row
  static constexpr int WM = 2, WN = 2, NT = WM * WN * 64;
  static constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  static constexpr int A_ELEMS = BM * BK, B_ELEMS = BN * BK, STAGE = A_ELEMS + B_ELEMS;
  static constexpr int CH = BM * BK / 4 / NT;     // 4-element chunks per thread and operand (both 128 x 32)
  static_assert(BM == BN && CH * NT * 4 == BM * BK, "both blocks split evenly over the threads");
  static_assert(V == 4 || V == 1, "staging width");

  // LDS word offset of (r, k) in a K-contiguous block: two 64-byte-row sub-blocks.
  static __device__ __forceinline__ int off_k(int r, int k) { return swz<2, 2, 4>((k >> 4) * (BM * KS) + r * KS + (k & 15)); }
  // LDS word offset of (k, c) in an M/N-contiguous block: rows of 128 values.
  static __device__ __forceinline__ int off_c(int k, int c) { return swz<1, 5, 5>(k * BM + c); }

  // Chunk `slot` of a thread as (row, column) of the operand block as it sits in
  // memory: rows of 32 K values (K-contiguous) or of 128 M/N values.
  // K-contiguous: one wave instruction covers 8 rows x 32 values; each
  // 16-lane group stages 4 rows x 4 chunks of one sub-block (256 bytes, all 64
  // banks), the two groups of a 4-row band the two halves of those rows.
  static __device__ __forceinline__ void chunk_k(int idx, int& r, int& k) {
    const int l = idx & 63, q = l >> 4, w = l & 15;
    r = (idx >> 6) * 8 + (q >> 1) * 4 + (w >> 2);
    k = (q & 1) * KS + (w & 3) * 4;
  }
  // M/N-contiguous: one wave instruction covers 2 rows of 128 values.
  static __device__ __forceinline__ void chunk_c(int idx, int& k, int& c) {
    k = idx >> 5;
    c = (idx & 31) * 4;
  }

  struct Regs {
    f32x4 a[CH], b[CH];
  };
  // LDS read instructions for one sub-block's fragments: 2 per 32-row block of a
  // K-contiguous operand, 8 per block of an M/N-contiguous one.
  static constexpr int READS = (AT ? 8 : 2) * FM + (BKM ? 2 : 8) * FN;

  // Four consecutive elements of a row starting at p, of which the first
  // `nvalid` (0..4) lie inside the matrix.
  static __device__ __forceinline__ f32x4 load4(const float* p, int nvalid) {
    if constexpr (V == 4) {
      return *reinterpret_cast<const f32x4*>(nvalid > 0 ? p : kZeroWords);
    } else {
      f32x4 v;
      v.x = *(nvalid > 0 ? p : kZeroWords);
      v.y = *(nvalid > 1 ? p + 1 : kZeroWords);
      v.z = *(nvalid > 2 ? p + 2 : kZeroWords);
      v.w = *(nvalid > 3 ? p + 3 : kZeroWords);
      return v;
    }
  }

  // Stage operand block (rows0 .. +R, K block k0) of a matrix with `rows`
  // rows: K-contiguous when kc, else along its rows (k0 then indexes rows).
  static __device__ __forceinline__ int nvalid(int64_t left) { return int(max<int64_t>(0, min<int64_t>(4, left))); }

  static __device__ __forceinline__ void load(Regs& r, const TiledArgs& g, int m0, int n0, int64_t k0, int tid) {
    const float* A = reinterpret_cast<const float*>(g.A);
    const float* B = reinterpret_cast<const float*>(g.B);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int idx = tid + NT * j;
      if constexpr (AT) {
        int k, c;
        chunk_c(idx, k, c);
        const int64_t gk = k0 + k, gm = m0 + c;
        r.a[j] = load4(A + gk * g.lda + gm, gk < g.K ? nvalid(g.M - gm) : 0);
      } else {
        int rr, k;
        chunk_k(idx, rr, k);
        const int64_t gm = m0 + rr, gk = k0 + k;
        r.a[j] = load4(A + gm * g.lda + gk, gm < g.M ? nvalid(g.K - gk) : 0);
      }
      if constexpr (BKM) {
        int rr, k;
        chunk_k(idx, rr, k);
        const int64_t gn = n0 + rr, gk = k0 + k;
        r.b[j] = load4(B + gn * g.ldb + gk, gn < g.N ? nvalid(g.K - gk) : 0);
      } else {
        int k, c;
        chunk_c(idx, k, c);
        const int64_t gk = k0 + k, gn = n0 + c;
        r.b[j] = load4(B + gk * g.ldb + gn, gk < g.K ? nvalid(g.N - gn) : 0);
      }
    }
  }

  static __device__ __forceinline__ void store(const Regs& r, float* stage, int tid) {
    float* sb = stage + A_ELEMS;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int idx = tid + NT * j;
      int p, q;
      if constexpr (AT) {
        chunk_c(idx, p, q);
        *reinterpret_cast<f32x4*>(stage + off_c(p, q)) = r.a[j];
      } else {
        chunk_k(idx, p, q);
        *reinterpret_cast<f32x4*>(stage + off_k(p, q)) = r.a[j];
      }
      if constexpr (BKM) {
        chunk_k(idx, p, q);
        *reinterpret_cast<f32x4*>(sb + off_k(p, q)) = r.b[j];
      } else {
        chunk_c(idx, p, q);
        *reinterpret_cast<f32x4*>(sb + off_c(p, q)) = r.b[j];
      }
    }
  }

  // The 8 K values of sub-block h this lane multiplies (8 g .. 8 g + 7) for
  // row / column `rc` of an operand block.
  template <bool KC>
  static __device__ __forceinline__ void frag(const float* blk, int rc, int h, int g8, float (&v)[8]) {
    if constexpr (KC) {
      const f32x4 lo = *reinterpret_cast<const f32x4*>(blk + off_k(rc, h * KS + g8));
      const f32x4 hi = *reinterpret_cast<const f32x4*>(blk + off_k(rc, h * KS + g8 + 4));
      v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
      v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = blk[off_c(h * KS + g8 + j, rc)];
    }
  }

  // Fragments of one 16-value sub-block: this lane's 8 K values of its rows of A and columns of B.
  struct Frags {
    float a[FM][8], b[FN][8];
  };

  static __device__ __forceinline__ void read_frags(const float* stage, int h, Frags& f, int wm, int wn, int lane) {
    const int l32 = lane & 31, g8 = (lane >> 5) * 8;
#pragma unroll
    for (int i = 0; i < FM; ++i) frag<!AT>(stage, wm * TM + i * 32 + l32, h, g8, f.a[i]);
#pragma unroll
    for (int j = 0; j < FN; ++j) frag<BKM>(stage + A_ELEMS, wn * TN + j * 32 + l32, h, g8, f.b[j]);
  }

  static __device__ __forceinline__ void mma(const Frags& f, f32x16 (&acc)[FM][FN]) {
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[i][s], f.b[j][s], acc[i][j], 0, 0, 0);
  }
};

// Workgroup barrier without a memory fence (global loads stay in flight).
__device__ __forceinline__ void f32_stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <class TO, int V, bool AT, bool BKM>
__global__ void __launch_bounds__(256, 2) gemm_f32_kernel(const TiledArgs g_in) {
  const TiledArgs g = at_batch<4>(g_in);
  using T = TiledF32<TO, V, AT, BKM>;
  __shared__ __attribute__((aligned(1024))) float lds[2 * T::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave % T::WM, wn = wave / T::WM;
  int tm, tn;
  grouped_tile(xcd_contiguous(blockIdx.x, gridDim.x), g.tiles_m, g.tiles_n, g.group_m, tm, tn);
  const int m0 = tm * T::BM, n0 = tn * T::BN;

  f32x16 acc[T::FM][T::FN];
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j) acc[i][j] = f32x16{};

  // Software pipeline over K blocks (stage s = kt & 1), with the fragments of
  // the first sub-block of block kt already in registers (f0):
  //   read the second sub-block's fragments (f1) while the first sub-block's
  //   MFMAs run; write block kt+1 (loaded one step earlier) to stage s^1;
  //   barrier; start loading block kt+2 and read the first sub-block of stage
  //   s^1 into f0 while the second sub-block's MFMAs run.
  // The barrier sits between the two halves of the MFMA stream, and the reads
  // of both stages are issued a sub-block (32 MFMAs) before they are used, so
  // no LDS read latency is exposed.  The barrier orders every wave's reads of stage s
  // before the next iteration's writes into it, and the writes of stage s^1
  // before its reads.  Global loads have two sub-blocks to arrive.  Loads and
  // LDS writes also run past the last block (every element then reads as zero
  // and the stage written is never multiplied), so neither sits under a branch.
  // With 4-byte staging (V == 1: four loads and addresses per chunk) the two
  // fragment sets do not fit the 256 registers of two waves per SIMD; that
  // path reads each sub-block's fragments just before its MFMAs instead.
  const int nk = int((g.K + T::BK - 1) / T::BK);
  typename T::Regs r;
  typename T::Frags f0, f1;
  T::load(r, g, m0, n0, 0, tid);
  T::store(r, lds, tid);
  f32_stage_barrier();
  if constexpr (V == 4) {
    T::load(r, g, m0, n0, T::BK, tid);
    T::read_frags(lds, 0, f0, wm, wn, lane);
    // Instruction order inside each half (sched_group_barrier): the fragment
    // reads two per MFMA from the first MFMA on, then in the first half the
    // LDS writes one per MFMA, in the second half the global loads one per
    // MFMA; measured 5 % faster than the compiler's own order, which sinks
    // reads and loads towards their first use.
    constexpr int NR = T::READS / 2, NW = 2 * T::CH, NMMA = 8 * T::FM * T::FN;
    static_assert(NR + NW <= NMMA, "one MFMA per group");
    for (int kt = 0; kt < nk; ++kt) {
      const float* cur = lds + (kt & 1) * T::STAGE;
      float* nxt = lds + ((kt + 1) & 1) * T::STAGE;
      T::read_frags(cur, 1, f1, wm, wn, lane);
      T::mma(f0, acc);
      T::store(r, nxt, tid);
#pragma unroll
      for (int q = 0; q < NR; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // LDS reads
      }
#pragma unroll
      for (int q = 0; q < NW; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // LDS writes
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NMMA - NR - NW, 0);
      f32_stage_barrier();
      T::load(r, g, m0, n0, int64_t(kt + 2) * T::BK, tid);
      T::read_frags(nxt, 0, f0, wm, wn, lane);
      T::mma(f1, acc);
#pragma unroll
      for (int q = 0; q < NR; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
#pragma unroll
      for (int q = 0; q < NW; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // global loads
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NMMA - NR - NW, 0);
    }
  } else {
    for (int kt = 0; kt < nk; ++kt) {
      const float* cur = lds + (kt & 1) * T::STAGE;
      T::load(r, g, m0, n0, int64_t(kt + 1) * T::BK, tid);
      T::read_frags(cur, 0, f0, wm, wn, lane);
      T::mma(f0, acc);
      T::read_frags(cur, 1, f1, wm, wn, lane);
      T::mma(f1, acc);
      T::store(r, lds + ((kt + 1) & 1) * T::STAGE, tid);
      f32_stage_barrier();
    }
  }
  epilogue_mfma32<TO, T::FM, T::FN>(g, acc, m0 + wm * T::TM, n0 + wn * T::TN, lane, g.red);
}

// Debug: stage K block 0 of tile (dbg_tm, dbg_tn) with the kernel's own
// staging code and copy the LDS stage out verbatim (32-bit words).
template <class TO, int V, bool AT, bool BKM>
__global__ void __launch_bounds__(256) gemm_f32_lds_image(const TiledArgs g) {
  using T = TiledF32<TO, V, AT, BKM>;
  __shared__ __attribute__((aligned(1024))) float lds[T::STAGE];
  const int tid = threadIdx.x;
  typename T::Regs r;
  T::load(r, g, g.dbg_tm * T::BM, g.dbg_tn * T::BN, 0, tid);
  T::store(r, lds, tid);
  __syncthreads();
  uint32_t* out = reinterpret_cast<uint32_t*>(g.dbg_out);
  for (int i = tid; i < T::STAGE; i += T::NT) out[i] = __builtin_bit_cast(uint32_t, lds[i]);
}

namespace {

template <class TO, int V, bool AT, bool BKM>
hipError_t go_f32(const TiledArgs& a, dim3 grid, hipStream_t s, bool img) {
  if (img) {
    hipLaunchKernelGGL((gemm_f32_lds_image<TO, V, AT, BKM>), dim3(1), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((gemm_f32_kernel<TO, V, AT, BKM>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <class TO, int V>
hipError_t f32_by_order(bool km, bool at, const TiledArgs& a, dim3 grid, hipStream_t s, bool img) {
  if (at) return km ? go_f32<TO, V, true, true>(a, grid, s, img) : go_f32<TO, V, true, false>(a, grid, s, img);
  return km ? go_f32<TO, V, false, true>(a, grid, s, img) : go_f32<TO, V, false, false>(a, grid, s, img);
}

template <class TO>
hipError_t f32_by_vec(int vec, bool km, bool at, const TiledArgs& a, dim3 grid, hipStream_t s, bool img) {
  if (vec == 4) return f32_by_order<TO, 4>(km, at, a, grid, s, img);
  if (vec == 1) return f32_by_order<TO, 1>(km, at, a, grid, s, img);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_f32(int out_kind, int vec, bool b_kmajor, bool a_trans, const TiledArgs& args, dim3 grid,
                      hipStream_t stream, bool lds_image) {
  if (out_kind == OUT_F32) return f32_by_vec<OutF32>(vec, b_kmajor, a_trans, args, grid, stream, lds_image);
  if (out_kind == OUT_BF16) return f32_by_vec<OutBF16>(vec, b_kmajor, a_trans, args, grid, stream, lds_image);
  if (out_kind == OUT_F16) return f32_by_vec<OutF16>(vec, b_kmajor, a_trans, args, grid, stream, lds_image);
  return hipErrorInvalidValue;
}

}  // namespace lak
