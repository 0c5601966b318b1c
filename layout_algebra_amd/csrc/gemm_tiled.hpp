// Tiled GEMM kernels for gfx950: C = alpha * A * B + beta * C.
//
// Structure (per workgroup, one BM x BN output tile):
//   * K is walked in blocks of 64.  A block of A (BM x 64) and of B (64 x BN)
//     is staged cooperatively by every thread, global -> registers -> LDS,
//     in 8-element chunks, one 16-byte load each (aligned when rows start on
//     16 bytes and no chunk is cut by an edge; else at 2-byte alignment, a
//     chunk cut by an edge loading the 8 elements that end at its last valid
//     one and shifting them into place on their way to LDS), or 2-byte loads
//     for rows of at most 8 elements; a zero stands for every element
//     outside [0,M) x [0,K) or [0,K) x [0,N) (the
//     zero-filled edge semantics of the Tylo.jl page "TMA and Hopper WGMMA",
//     section "Copy and completion").
//   * In LDS both operands are stored K-contiguous, one 128-byte row of 64
//     16-bit values per M row (A) or N column (B), under Swizzle{3,3,4}:
//     element (r, k) sits at 64 r + (k XOR 8 ((r >> 1) mod 8)).  The 128-byte
//     row map of the Tylo.jl page "TMA and Hopper WGMMA" (section "The same
//     storage contract on both sides") is Swizzle{3,3,3}, made for 32 banks;
//     gfx950's LDS has 64, so rows r and r+8 of that map share banks and a
//     16-byte fragment read of 16 rows is 2-way conflicted.  Taking the XOR
//     from one row bit higher spreads those 16 rows over all 64 banks.  This
//     holds A, and B stored K-contiguous ([N, K]).  B stored N-contiguous
//     ([K, N]) stays N-contiguous in LDS, one row of BN values per k, under
//     Swizzle{1,5,2} (BN = 64) or Swizzle{2,5,2} (BN = 128), and its fragments
//     are read with ds_read_b64_tr_b16, which transposes 4 x 16 blocks of
//     16-bit values across each 16-lane group (lanes 4e..4e+3 address row e;
//     lane i receives element i of rows 0..3): staging writes whole 16-byte
//     row chunks and both the writes and the transposing reads are free of
//     bank conflicts.  A stored [K, M] (M contiguous) is kept M-contiguous the
//     same way, one row of BM values per k under the same swizzle, staged in
//     8-element chunks along M and read with the same transposing reads.
//   * Two LDS stages: while the MFMAs consume stage s the next block is
//     loaded into registers and written to stage s^1; one workgroup barrier
//     per block keeps every wave's reads of a stage ahead of its refill
//     (the two synchronisations the Tylo.jl page "Layouts, storage and
//     ownership" requires in section "Plans describe work, callers establish
//     readiness").
//   * Each wave owns a (BM/WM) x (BN/WN) sub-tile as a grid of
//     v_mfma_f32_32x32x16 blocks whose FP32 accumulators stay in registers
//     for the whole K loop (Phobos "Tiles and shared memory", section "Tiles in
//     registers"); A and B fragments are reused across that grid.
//   * Epilogue: alpha * acc + beta * C_old in FP32 (C_old read only when
//     beta != 0), rounded to nearest even for 16-bit outputs, written only
//     inside [0,M) x [0,N).
// The kernels' instantiations are spread over gemm_tiled_{64,128,p3}.hip (one
// translation unit per tile configuration, compiled in parallel).
#pragma once

#include <type_traits>

#include "kernel_common.hpp"
#include "launch.hpp"

namespace lak {

typedef short i16x4_t __attribute__((ext_vector_type(4)));
#define TILED_LDS __attribute__((address_space(3)))

// Sixteen zero bytes in device memory: staging loads of elements outside the
// matrix read from here, so the loaded registers need no masking afterwards.
static __device__ __attribute__((aligned(16))) uint16_t kZeroChunk[8];

// Eight 16-bit elements of one staging load, packed in pairs.
struct Chunk8 { u32x4 w; };   // one aligned 16-byte load
struct Chunk2 { u32x4 w; };   // one 16-byte load at 2-byte alignment (a cut chunk: shifted window)
struct Chunk1 { u32x4 w; };   // eight 2-byte loads

template <class TI, class TO, int BM, int BN, int WM, int WN, int V, bool GU, bool BKM, bool AT = false>
struct Tiled {
  static constexpr int NT = WM * WN * 64;
  static constexpr int BK = 64;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int NB = GU ? 2 : 1;
  static constexpr int A_ELEMS = BM * BK;
  static constexpr int B_ELEMS = BN * BK;
  static constexpr int STAGE = A_ELEMS + NB * B_ELEMS;
  static constexpr int A_CHUNKS = BM * BK / 8 / NT;
  static constexpr int BN8 = BN / 8;
  static constexpr int B_CHUNKS = BN * BK / 8 / NT;         // 8-element B chunks per thread (along K or N)
  static constexpr int BSW = BN == 64 ? 1 : 2;              // N-contiguous B block: Swizzle{BSW,5,2}
  static constexpr int BM8 = BM / 8;
  static constexpr int ASW = BM == 64 ? 1 : 2;              // M-contiguous A block: Swizzle{ASW,5,2}
  static_assert(!AT || (!BKM && V != 1), "A stored [K, M] pairs with B stored [K, N] and 16-byte staging");
  static_assert(!AT || NT % BM8 == 0, "a thread's A chunks share their index along M");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(A_CHUNKS * NT * 8 == BM * BK, "A block must split evenly over threads");
  static_assert(B_CHUNKS * NT * 8 == BN * BK, "B block must split evenly over threads");
  static_assert(BN == 64 || BN == 128, "N-contiguous B swizzle is chosen for 64- and 128-wide blocks");
  static_assert(V == 8 || V == 2 || V == 1, "staging width");
  typedef typename std::conditional<V == 8, Chunk8, typename std::conditional<V == 2, Chunk2, Chunk1>::type>::type Chunk;

  // LDS element offset of (row, k) inside one operand block.
  static __device__ __forceinline__ int lds_off(int row, int k) { return swz<3, 3, 4>(row * BK + k); }
  // LDS element offset of (k, n) inside an N-contiguous B block.
  static __device__ __forceinline__ int b_off_n(int k, int n) { return swz<BSW, 5, 2>(k * BN + n); }
  // LDS element offset of (k, m) inside an M-contiguous A block.
  static __device__ __forceinline__ int a_off_m(int k, int m) { return swz<ASW, 5, 2>(k * BM + m); }

  // Staging registers of one K block.
  struct Regs {
    Chunk a[A_CHUNKS];
    Chunk b[NB][B_CHUNKS];
  };

  // Chunks of one block cut by an edge (V == 2), the same for every row of the
  // block: the chunk index along K of A (and of K-major B) in the last K block,
  // and the column chunk of N-contiguous B in the tile holding N's edge (-1:
  // none), with the places each is shifted down on its way to LDS.  A thread's
  // chunks all share one such index (tid mod 8 along K, tid mod BN/8 along N),
  // so a thread shifts either all of an operand's chunks or none.
  struct Cut {
    int a_ch, a_sh, b_nc, b_sh;
  };
  static_assert(NT % BN8 == 0 && NT % 8 == 0, "a thread's chunks share their index along K and N");

  // Element q of the result is element q + sh of w (0 past the end), sh in 1..7.
  static __device__ __forceinline__ u32x4 shift_down(u32x4 w, int sh) {
    const uint32_t v[4] = {w.x, w.y, w.z, w.w};
    const int d = sh >> 1;
    uint32_t o[5];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t v1 = i + 1 < 4 ? v[i + 1] : 0u, v2 = i + 2 < 4 ? v[i + 2] : 0u, v3 = i + 3 < 4 ? v[i + 3] : 0u;
      o[i] = d == 0 ? v[i] : d == 1 ? v1 : d == 2 ? v2 : v3;
    }
    o[4] = 0u;
    if (sh & 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = (o[i] >> 16) | (o[i + 1] << 16);
    }
    return u32x4{o[0], o[1], o[2], o[3]};
  }

  static __device__ __forceinline__ u32x4 pack8(const uint16_t* e) {
    u32x4 w;
    w.x = e[0] | (uint32_t(e[1]) << 16);
    w.y = e[2] | (uint32_t(e[3]) << 16);
    w.z = e[4] | (uint32_t(e[5]) << 16);
    w.w = e[6] | (uint32_t(e[7]) << 16);
    return w;
  }

  // Eight consecutive elements starting at p, of which the first `nvalid` (0..8)
  // lie inside the matrix; the others read as 0.
  // V == 8 (rows on 16 bytes, no chunk cut by an edge, so nvalid is 0 or 8):
  // one 16-byte load whose aligned bytes all lie inside the matrix, or of the
  // zero chunk.
  // V == 2 (any 2-byte alignment, rows of more than 8 elements): one 16-byte
  // load at 2-byte alignment (gfx9 devices run with unaligned global access
  // enabled; the compiler emits a single global_load_dwordx4): the chunk
  // itself when whole, the zero chunk when empty, and for a chunk cut by an
  // edge the 8 elements that end at its last valid one, which lie in the same
  // row and are shifted down into place on their way to LDS (see Cut).
  // In both, only the address is selected and the data is left untouched
  // until it is written to LDS, so no wait follows the load: a load under a
  // divergent branch, or a select on its result, makes the compiler wait for
  // it at once, and with it for every load issued before.
  // V == 1 (rows of at most 8 elements): eight 2-byte loads at immediate
  // offsets from one address for a whole chunk; a chunk cut by an edge loads
  // its valid elements one by one.  (For longer rows this measured slower
  // than V == 2: the per-chunk branch costs more than the loads.)
  static __device__ __forceinline__ void load8(Chunk8& c, const uint16_t* p, int nvalid) {
    c.w = *reinterpret_cast<const u32x4*>(nvalid > 0 ? p : kZeroChunk);
  }
  static __device__ __forceinline__ void load8(Chunk2& c, const uint16_t* p, int nvalid) {
    const int k = nvalid > 0 && nvalid < 8 ? 8 - nvalid : 0;
    __builtin_memcpy(&c.w, nvalid > 0 ? p - k : kZeroChunk, 16);
  }
  static __device__ __forceinline__ void load8(Chunk1& c, const uint16_t* p, int nvalid) {
    uint16_t e[8];
    if (nvalid >= 8) {
#pragma unroll
      for (int q = 0; q < 8; ++q) e[q] = p[q];
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) e[q] = q < nvalid ? p[q] : uint16_t(0);
    }
    c.w = pack8(e);
  }

  static __device__ __forceinline__ void load(Regs& r, const TiledArgs& g, int m0, int n0, int64_t k0, int tid) {
#pragma unroll
    for (int j = 0; j < A_CHUNKS; ++j) {
      const int idx = tid + NT * j;
      if constexpr (AT) {
        // A stored [K, M]: rows k of M values, 8-element chunks along M
        const int kr = idx / BM8, mc = idx % BM8;
        const int64_t gk = k0 + kr;
        const int64_t gm = m0 + mc * 8;
        const int nvalid = gk < g.K ? int(max<int64_t>(0, min<int64_t>(8, g.M - gm))) : 0;
        load8(r.a[j], g.A + gk * g.lda + gm, nvalid);
      } else {
        const int row = idx >> 3, ch = idx & 7;
        const int64_t gm = m0 + row;
        const int64_t gk = k0 + ch * 8;
        const int nvalid = gm < g.M ? int(max<int64_t>(0, min<int64_t>(8, g.K - gk))) : 0;
        load8(r.a[j], g.A + gm * g.lda + gk, nvalid);
      }
    }
#pragma unroll
    for (int s = 0; s < NB; ++s) {
      const uint16_t* B = s == 0 ? g.B : g.B2;
      if constexpr (BKM) {
        // B stored [N, K]: rows n of K values, staged exactly like A
#pragma unroll
        for (int j = 0; j < B_CHUNKS; ++j) {
          const int idx = tid + NT * j;
          const int row = idx >> 3, ch = idx & 7;
          const int64_t gn = n0 + row;
          const int64_t gk = k0 + ch * 8;
          const int nvalid = gn < g.N ? int(max<int64_t>(0, min<int64_t>(8, g.K - gk))) : 0;
          load8(r.b[s][j], B + gn * g.ldb + gk, nvalid);
        }
        continue;
      }
      // B stored [K, N]: rows k of N values, 8-element chunks along N
#pragma unroll
      for (int j = 0; j < B_CHUNKS; ++j) {
        const int idx = tid + NT * j;
        const int kr = idx / BN8, nc = idx % BN8;
        const int64_t gk = k0 + kr;
        const int64_t gn = n0 + nc * 8;
        const int nvalid = gk < g.K ? int(max<int64_t>(0, min<int64_t>(8, g.N - gn))) : 0;
        load8(r.b[s][j], B + gk * g.ldb + gn, nvalid);
      }
    }
  }

  // Write the staged block to LDS; `cut` (uniform, V == 2 only): its chunks cut by an edge.
  static __device__ __forceinline__ void store(const Regs& r, uint16_t* stage, int tid, const Cut& cut) {
    u32x4 a[A_CHUNKS], b[NB][B_CHUNKS];
#pragma unroll
    for (int j = 0; j < A_CHUNKS; ++j) a[j] = r.a[j].w;
#pragma unroll
    for (int s = 0; s < NB; ++s)
#pragma unroll
      for (int j = 0; j < B_CHUNKS; ++j) b[s][j] = r.b[s][j].w;
    if constexpr (V == 2) {
      // one branch per operand; the data has arrived by now
      if ((AT ? tid % BM8 : tid & 7) == cut.a_ch) {
#pragma unroll
        for (int j = 0; j < A_CHUNKS; ++j) a[j] = shift_down(a[j], cut.a_sh);
      }
      const bool cut_b = BKM ? (tid & 7) == cut.a_ch : (tid % BN8) == cut.b_nc;
      if (cut_b) {
        const int sh = BKM ? cut.a_sh : cut.b_sh;
#pragma unroll
        for (int s = 0; s < NB; ++s)
#pragma unroll
          for (int j = 0; j < B_CHUNKS; ++j) b[s][j] = shift_down(b[s][j], sh);
      }
    }
#pragma unroll
    for (int j = 0; j < A_CHUNKS; ++j) {
      const int idx = tid + NT * j;
      if constexpr (AT) {
        *reinterpret_cast<u32x4*>(stage + a_off_m(idx / BM8, (idx % BM8) * 8)) = a[j];
      } else {
        *reinterpret_cast<u32x4*>(stage + lds_off(idx >> 3, (idx & 7) * 8)) = a[j];
      }
    }
#pragma unroll
    for (int s = 0; s < NB; ++s) {
      uint16_t* dst = stage + A_ELEMS + s * B_ELEMS;
#pragma unroll
      for (int j = 0; j < B_CHUNKS; ++j) {
        const int idx = tid + NT * j;
        if constexpr (BKM) {
          *reinterpret_cast<u32x4*>(dst + lds_off(idx >> 3, (idx & 7) * 8)) = b[s][j];
        } else {
          *reinterpret_cast<u32x4*>(dst + b_off_n(idx / BN8, (idx % BN8) * 8)) = b[s][j];
        }
      }
    }
  }

  // Four consecutive N values of one K row of an N-contiguous B block, transposed across the
  // 16-lane group (see the file header).
  static __device__ __forceinline__ u32x2 read_tr(const uint16_t* p) {
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TILED_LDS i16x4_t*)(p));
    return __builtin_bit_cast(u32x2, v);
  }

  static __device__ __forceinline__ void compute(const uint16_t* stage, f32x16 (&acc)[NB][FM][FN], int wm, int wn, int lane) {
    const int lr = lane & 31, lk = (lane >> 5) * 8;
    // N-contiguous B: lane l of 16-lane group g addresses row 8 (g / 2) + (l / 4) % 4 (+ 4 for the
    // second read) at column 16 (g % 2) + 4 (l % 4) of each 32-column block, and receives the 8 K
    // values of column l % 32 that the MFMA's B operand expects of lane l.
    const int g4 = lane >> 4;
    const int bn = wn * TN + 16 * (g4 & 1) + 4 * (lane & 3);
    const int bk = 8 * (g4 >> 1) + ((lane >> 2) & 3);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      u32x4 a[FM], b[NB][FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if constexpr (AT) {
          // M-contiguous A: transposing reads, lane mapping as for N-contiguous B along M
          const int am = wm * TM + 16 * (g4 & 1) + 4 * (lane & 3) + i * 32;
          const u32x2 lo = read_tr(stage + a_off_m(s * 16 + bk, am));
          const u32x2 hi = read_tr(stage + a_off_m(s * 16 + bk + 4, am));
          a[i] = u32x4{lo.x, lo.y, hi.x, hi.y};
        } else {
          a[i] = *reinterpret_cast<const u32x4*>(stage + lds_off(wm * TM + i * 32 + lr, s * 16 + lk));
        }
      }
#pragma unroll
      for (int t = 0; t < NB; ++t)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          if constexpr (BKM) {
            b[t][j] = *reinterpret_cast<const u32x4*>(stage + A_ELEMS + t * B_ELEMS + lds_off(wn * TN + j * 32 + lr, s * 16 + lk));
          } else {
            const uint16_t* bs = stage + A_ELEMS + t * B_ELEMS;
            const u32x2 lo = read_tr(bs + b_off_n(s * 16 + bk, bn + j * 32));
            const u32x2 hi = read_tr(bs + b_off_n(s * 16 + bk + 4, bn + j * 32));
            b[t][j] = u32x4{lo.x, lo.y, hi.x, hi.y};
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

// Workgroup barrier without a memory fence: this wave's LDS accesses are
// complete (lgkmcnt(0)) but its global loads may stay in flight.  The empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <class TI, class TO, int BM, int BN, int WM, int WN, int V, bool GU, bool BKM, bool P3, bool AT = false>
__global__ void __launch_bounds__(WM * WN * 64) gemm_tiled_kernel(const TiledArgs g_in) {
  const TiledArgs g = at_batch(g_in);
  using T = Tiled<TI, TO, BM, BN, WM, WN, V, GU, BKM, AT>;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * T::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  int tm, tn;
  grouped_tile(xcd_contiguous(blockIdx.x, gridDim.x), g.tiles_m, g.tiles_n, g.group_m, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  f32x16 acc[T::NB][T::FM][T::FN];
#pragma unroll
  for (int t = 0; t < T::NB; ++t)
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j) acc[t][i][j] = f32x16{};

  // 64 x 64 tiles of a plain GEMM with 16-byte loads keep two register sets:
  // block kt+2 is loaded while block kt is multiplied and block kt+1 (loaded
  // one step earlier) is written to LDS, so every block has two steps to
  // arrive.  Everything else keeps one set: block kt+1 is loaded while block
  // kt is multiplied.  (Two sets would spill for gate/up and halve the
  // workgroups per CU for 128 x 128 tiles, which measured slower on full
  // grids; with 2-byte loads two blocks are more loads than a wave can keep
  // counted in flight, 63.)  Loads and LDS writes happen on every step, also
  // past the last block, where every element reads as zero and the stage
  // written is never read again, so that neither sits under a branch and the
  // compiler can count exactly which loads are still in flight.  The barriers
  // carry no memory fence: a fence would also wait for the prefetch.
  const int nk = int((g.K + T::BK - 1) / T::BK);
  // chunks cut by an edge (V == 2): along K in the last block when K is not a multiple of 8,
  // along N in every block of the tile that holds N's edge when N is not (N-contiguous B), and
  // for A stored [K, M] along M in every block of the tile that holds M's edge (A's K runs
  // along its rows there, so it has no K cut)
  const int64_t n_left = g.N - n0, m_left = g.M - m0;
  const bool n_cut = !BKM && n_left < BN && (n_left & 7) != 0;
  const bool m_cut = AT && m_left < BM && (m_left & 7) != 0;
  auto cut = [&](int blk) {
    typename T::Cut c{-1, 0, -1, 0};
    const int64_t k_left = g.K - int64_t(blk) * T::BK;
    if (!AT && blk < nk && k_left < T::BK && (k_left & 7) != 0) {
      c.a_ch = int(k_left >> 3);
      c.a_sh = 8 - int(k_left & 7);
    }
    if (blk < nk && m_cut) {
      c.a_ch = int(m_left >> 3);
      c.a_sh = 8 - int(m_left & 7);
    }
    if (blk < nk && n_cut) {
      c.b_nc = int(n_left >> 3);
      c.b_sh = 8 - int(n_left & 7);
    }
    return c;
  };
  if constexpr (V != 1 && BM == 64 && !GU && P3) {
    // three register sets: blocks kt+1 and kt+2 in flight while block kt is
    // multiplied (240 registers, one wave per SIMD: the planner takes this
    // only for grids of one to two workgroups per CU, where it measured
    // 6-9 % faster; larger grids lose the second workgroup per SIMD)
    typename T::Regs r0, r1, r2;
    T::load(r0, g, m0, n0, 0, tid);
    T::load(r1, g, m0, n0, T::BK, tid);
    T::load(r2, g, m0, n0, 2 * T::BK, tid);
    T::store(r0, lds, tid, cut(0));
    stage_barrier();
    for (int kt = 0; kt < nk; kt += 3) {
      // block kt in stage kt % 2, blocks kt+1 and kt+2 in flight in r1 and r2
      uint16_t* s0 = lds + (kt & 1) * T::STAGE;
      uint16_t* s1 = lds + ((kt + 1) & 1) * T::STAGE;
      T::load(r0, g, m0, n0, int64_t(kt + 3) * T::BK, tid);
      T::compute(s0, acc, wm, wn, lane);
      T::store(r1, s1, tid, cut(kt + 1));
      stage_barrier();
      if (kt + 1 >= nk) break;
      T::load(r1, g, m0, n0, int64_t(kt + 4) * T::BK, tid);
      T::compute(s1, acc, wm, wn, lane);
      T::store(r2, s0, tid, cut(kt + 2));
      stage_barrier();
      if (kt + 2 >= nk) break;
      T::load(r2, g, m0, n0, int64_t(kt + 5) * T::BK, tid);
      T::compute(s0, acc, wm, wn, lane);
      T::store(r0, s1, tid, cut(kt + 3));
      stage_barrier();
    }
  } else if constexpr (V != 1 && BM == 64 && !GU) {
    typename T::Regs r0, r1;
    T::load(r0, g, m0, n0, 0, tid);
    T::load(r1, g, m0, n0, T::BK, tid);
    T::store(r0, lds, tid, cut(0));
    stage_barrier();
    for (int kt = 0; kt < nk; kt += 2) {
      // block kt in stage 0, block kt+1 in flight in r1
      T::load(r0, g, m0, n0, int64_t(kt + 2) * T::BK, tid);
      T::compute(lds, acc, wm, wn, lane);
      T::store(r1, lds + T::STAGE, tid, cut(kt + 1));
      stage_barrier();
      if (kt + 1 >= nk) break;
      // block kt+1 in stage 1, block kt+2 in flight in r0
      T::load(r1, g, m0, n0, int64_t(kt + 3) * T::BK, tid);
      T::compute(lds + T::STAGE, acc, wm, wn, lane);
      T::store(r0, lds, tid, cut(kt + 2));
      stage_barrier();
    }
  } else {
    typename T::Regs r;
    T::load(r, g, m0, n0, 0, tid);
    T::store(r, lds, tid, cut(0));
    stage_barrier();
    for (int kt = 0; kt < nk; ++kt) {
      T::load(r, g, m0, n0, int64_t(kt + 1) * T::BK, tid);
      T::compute(lds + (kt & 1) * T::STAGE, acc, wm, wn, lane);
      T::store(r, lds + ((kt + 1) & 1) * T::STAGE, tid, cut(kt + 1));
      stage_barrier();
    }
  }

  // Epilogue straight from the accumulator lane map (epilogue_mfma32 for a
  // plain GEMM; gate/up writes G and U, or silu(G) * U, with no row reduction).
  if constexpr (GU) {
    typedef typename TO::storage St;
    const int lc = lane & 31, lr4 = (lane >> 5) * 4;
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
#pragma unroll
      for (int j = 0; j < T::FN; ++j) {
        const int64_t col = n0 + wn * T::TN + j * 32 + lc;
        const int64_t rbase = m0 + wm * T::TM + i * 32 + lr4;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t row = rbase + 8 * (e >> 2) + (e & 3);
          if (col >= g.N || row >= g.M) continue;
          const int64_t idx = row * g.ldc + col;
          if (g.act == 1) {
            static_cast<St*>(g.C)[idx] = to_out<TO>(swiglu(acc[0][i][j][e], acc[1][i][j][e]));
          } else {
            static_cast<St*>(g.C)[idx] = to_out<TO>(acc[0][i][j][e]);
            static_cast<St*>(g.C2)[idx] = to_out<TO>(acc[1][i][j][e]);
          }
        }
      }
    }
  } else {
    epilogue_mfma32<TO, T::FM, T::FN>(g, acc[0], m0 + wm * T::TM, n0 + wn * T::TN, lane, g.red);
  }
}

// Debug: stage K block 0 of tile (dbg_tm, dbg_tn) with the kernel's own
// staging code and copy the LDS stage out verbatim.
template <class TI, class TO, int BM, int BN, int WM, int WN, int V, bool GU, bool BKM, bool AT = false>
__global__ void __launch_bounds__(WM * WN * 64) gemm_tiled_lds_image(const TiledArgs g) {
  using T = Tiled<TI, TO, BM, BN, WM, WN, V, GU, BKM, AT>;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[T::STAGE];
  const int tid = threadIdx.x;
  typename T::Regs r;
  T::load(r, g, g.dbg_tm * BM, g.dbg_tn * BN, 0, tid);
  T::store(r, lds, tid, [&] {
    typename T::Cut c{-1, 0, -1, 0};
    const int64_t k_left = g.K, n_left = g.N - int64_t(g.dbg_tn) * BN, m_left = g.M - int64_t(g.dbg_tm) * BM;
    if (!AT && k_left < T::BK && (k_left & 7) != 0) { c.a_ch = int(k_left >> 3); c.a_sh = 8 - int(k_left & 7); }
    if (AT && m_left < BM && (m_left & 7) != 0) { c.a_ch = int(m_left >> 3); c.a_sh = 8 - int(m_left & 7); }
    if (!BKM && n_left < BN && (n_left & 7) != 0) { c.b_nc = int(n_left >> 3); c.b_sh = 8 - int(n_left & 7); }
    return c;
  }());
  __syncthreads();
  for (int i = tid; i < T::STAGE; i += T::NT) g.dbg_out[i] = lds[i];
}

// ------------------------------------------------------------------ dispatch
// The general kernel's tile configurations, each in its own translation unit (launch_tiled, in
// gemm_tiled_p3.hip, picks one by kernel id).
hipError_t launch_tiled_128(int in_kind, int out_kind, int vec, bool gate_up, bool b_kmajor, bool a_trans,
                            const TiledArgs& args, dim3 grid, hipStream_t stream, bool lds_image);
hipError_t launch_tiled_64(int in_kind, int out_kind, int vec, bool gate_up, bool b_kmajor, bool a_trans,
                           const TiledArgs& args, dim3 grid, hipStream_t stream, bool lds_image);

namespace {

template <class TI, class TO, int BM, int BN, int WM, int WN, int V, bool GU, bool BKM, bool P3 = false, bool AT = false>
hipError_t go(const TiledArgs& a, dim3 grid, hipStream_t s, bool img) {
  if (img) {
    hipLaunchKernelGGL((gemm_tiled_lds_image<TI, TO, BM, BN, WM, WN, V, GU, BKM, AT>), dim3(1), dim3(WM * WN * 64), 0, s, a);
  } else {
    hipLaunchKernelGGL((gemm_tiled_kernel<TI, TO, BM, BN, WM, WN, V, GU, BKM, P3, AT>), grid, dim3(WM * WN * 64), 0, s, a);
  }
  return hipGetLastError();
}

template <class TI, class TO, int BM, int BN, int WM, int WN, int V>
hipError_t by_gu_km(bool gu, bool km, bool at, const TiledArgs& a, dim3 grid, hipStream_t s, bool img) {
  if (at) {
    // A stored [K, M]: B stored [K, N], 16-byte staging (the planner rejects the rest)
    if constexpr (V != 1) {
      if (km) return hipErrorInvalidValue;
      return gu ? go<TI, TO, BM, BN, WM, WN, V, true, false, false, true>(a, grid, s, img)
                : go<TI, TO, BM, BN, WM, WN, V, false, false, false, true>(a, grid, s, img);
    }
    return hipErrorInvalidValue;
  }
  if (gu) return km ? go<TI, TO, BM, BN, WM, WN, V, true, true>(a, grid, s, img) : go<TI, TO, BM, BN, WM, WN, V, true, false>(a, grid, s, img);
  return km ? go<TI, TO, BM, BN, WM, WN, V, false, true>(a, grid, s, img) : go<TI, TO, BM, BN, WM, WN, V, false, false>(a, grid, s, img);
}

template <class TI, class TO, int BM, int BN, int WM, int WN>
hipError_t by_vec_gu(int vec, bool gu, bool km, bool at, const TiledArgs& a, dim3 grid, hipStream_t s, bool img) {
  if (vec == 8) return by_gu_km<TI, TO, BM, BN, WM, WN, 8>(gu, km, at, a, grid, s, img);
  if (vec == 2) return by_gu_km<TI, TO, BM, BN, WM, WN, 2>(gu, km, at, a, grid, s, img);
  if (vec == 1) return by_gu_km<TI, TO, BM, BN, WM, WN, 1>(gu, km, at, a, grid, s, img);
  return hipErrorInvalidValue;
}

template <int BM, int BN, int WM, int WN>
hipError_t by_types(int in_kind, int out_kind, int vec, bool gu, bool km, bool at, const TiledArgs& a, dim3 grid,
                    hipStream_t s, bool img) {
  if (in_kind == IN_BF16) {
    if (out_kind == OUT_F32) return by_vec_gu<InBF16, OutF32, BM, BN, WM, WN>(vec, gu, km, at, a, grid, s, img);
    if (out_kind == OUT_BF16) return by_vec_gu<InBF16, OutBF16, BM, BN, WM, WN>(vec, gu, km, at, a, grid, s, img);
    if (out_kind == OUT_F16) return by_vec_gu<InBF16, OutF16, BM, BN, WM, WN>(vec, gu, km, at, a, grid, s, img);
  } else if (in_kind == IN_F16) {
    if (out_kind == OUT_F32) return by_vec_gu<InF16, OutF32, BM, BN, WM, WN>(vec, gu, km, at, a, grid, s, img);
    if (out_kind == OUT_BF16) return by_vec_gu<InF16, OutBF16, BM, BN, WM, WN>(vec, gu, km, at, a, grid, s, img);
    if (out_kind == OUT_F16) return by_vec_gu<InF16, OutF16, BM, BN, WM, WN>(vec, gu, km, at, a, grid, s, img);
  }
  return hipErrorInvalidValue;
}

// 64 x 64 tiles with three K blocks in flight: plain GEMMs with 16-byte loads only.
template <class TI, class TO>
hipError_t p3_by_vec(int vec, bool gu, bool km, const TiledArgs& a, dim3 grid, hipStream_t s, bool img) {
  if (gu) return hipErrorInvalidValue;
  if (vec == 8)
    return km ? go<TI, TO, 64, 64, 2, 1, 8, false, true, true>(a, grid, s, img)
              : go<TI, TO, 64, 64, 2, 1, 8, false, false, true>(a, grid, s, img);
  if (vec == 2)
    return km ? go<TI, TO, 64, 64, 2, 1, 2, false, true, true>(a, grid, s, img)
              : go<TI, TO, 64, 64, 2, 1, 2, false, false, true>(a, grid, s, img);
  return hipErrorInvalidValue;
}

inline hipError_t p3_by_types(int in_kind, int out_kind, int vec, bool gu, bool km, const TiledArgs& a, dim3 grid,
                              hipStream_t s, bool img) {
  if (in_kind == IN_BF16) {
    if (out_kind == OUT_F32) return p3_by_vec<InBF16, OutF32>(vec, gu, km, a, grid, s, img);
    if (out_kind == OUT_BF16) return p3_by_vec<InBF16, OutBF16>(vec, gu, km, a, grid, s, img);
    if (out_kind == OUT_F16) return p3_by_vec<InBF16, OutF16>(vec, gu, km, a, grid, s, img);
  } else if (in_kind == IN_F16) {
    if (out_kind == OUT_F32) return p3_by_vec<InF16, OutF32>(vec, gu, km, a, grid, s, img);
    if (out_kind == OUT_BF16) return p3_by_vec<InF16, OutBF16>(vec, gu, km, a, grid, s, img);
    if (out_kind == OUT_F16) return p3_by_vec<InF16, OutF16>(vec, gu, km, a, grid, s, img);
  }
  return hipErrorInvalidValue;
}

}  // namespace

}  // namespace lak
