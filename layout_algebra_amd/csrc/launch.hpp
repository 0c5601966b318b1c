// Interface between the host planner / C ABI and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lak {

// Row-reduction operations of the GEMM epilogue.
enum : int { RED_NONE = 0, RED_SUM = 1, RED_MAX = 2, RED_MIN = 3 };

// Everything one launch needs; plain values only.
struct TiledArgs {
  const uint16_t* A;     // [M, K] row-major, lda (binary32 inputs: the same address, read as 32-bit words)
  const uint16_t* B;     // [K, N] N contiguous, ldb (W_gate for gate/up)
  const uint16_t* B2;    // W_up for gate/up, else unused
  void* C;               // [M, N] row-major, ldc (G for gate/up)
  void* C2;              // U for gate/up
  int64_t M, N, K, lda, ldb, ldc;
  float alpha, beta;
  int act;               // gate/up only: 0 = write G and U, 1 = write silu(G) * U to C
  int red;               // row reduction of the FP32 outputs into R: RED_NONE, RED_SUM, RED_MAX, RED_MIN
  float* R;              // [M] per matrix (batch entry z at R + z * M), prefilled with the identity of `red`
  int64_t sa, sb, sc;    // batched launches: element strides between consecutive A, B (and B2), C (and C2)
  int out_bytes;         // bytes per C element (for the C batch stride)
  int tiles_m, tiles_n, group_m;
  int dbg_tm, dbg_tn;    // LDS-image debug launch: tile to stage
  uint16_t* dbg_out;     // LDS-image debug launch: destination of one stage
};

// The matrices of batch entry blockIdx.y (grid dimension y = batch count);
// IB: bytes per input element (the A / B pointers count 16-bit units).
template <int IB = 2>
__device__ __forceinline__ TiledArgs at_batch(const TiledArgs& g) {
  static_assert(IB == 2 || IB == 4, "16- or 32-bit input elements");
  TiledArgs r = g;
  const int64_t z = blockIdx.y;
  r.A = g.A + z * g.sa * (IB / 2);
  r.B = g.B + z * g.sb * (IB / 2);
  r.B2 = g.B2 ? g.B2 + z * g.sb * (IB / 2) : nullptr;
  r.C = g.C ? static_cast<void*>(static_cast<char*>(g.C) + z * g.sc * g.out_bytes) : nullptr;
  r.C2 = g.C2 ? static_cast<void*>(static_cast<char*>(g.C2) + z * g.sc * g.out_bytes) : nullptr;
  r.R = g.R ? g.R + z * g.M : nullptr;
  return r;
}

enum KernelId : int {
  KID_TILED_128 = 0,     // any shape: 128x128x64, 4 waves of 64x64, register-staged, B transposed while staging
  KID_FAST_256 = 1,      // full tiles: 256x256x32, 8 waves of 128x64, direct-to-LDS, transposing B reads
  KID_FAST_GU = 2,       // full tiles, gate/up: 256 x (128 + 128) x 32, 8 waves of 128 x (32 + 32)
  KID_SKINNY_16 = 3,     // M <= 16: 16 x 128 column strips over all of K, 4 waves of 16 x 32, HBM-bound
  KID_FAST_256_KM = 4,   // KID_FAST_256 for B stored [N, K] (K contiguous)
  KID_FAST_GU_KM = 5,    // KID_FAST_GU for weights stored [N, K]
  KID_TILED_64 = 6,      // any shape, small grids: 64x64x64, 2 waves of 32x64, as KID_TILED_128 otherwise
  KID_TILED_64_P3 = 7,   // KID_TILED_64 with three K blocks in flight (plain GEMM, 16-byte loads)
  KID_FAST_256_AT = 8,   // KID_FAST_256 for A stored [K, M] (M contiguous)
  KID_FAST_GU_AT = 9,    // KID_FAST_GU for X stored [K, M]
  KID_TILED_F32 = 10,    // binary32 A and B, any shape: 128x128x32, 4 waves of 64x64, v_mfma_f32_32x32x2_f32
  KID_FAST_F8 = 11,      // one-byte A [M, K] and B [N, K]: KID_FAST_256_KM on byte pairs, 256x256x64, v_mfma_f32_32x32x64_f8f6f4
  KID_FAST_GU_F8 = 12,   // one-byte gate/up, weights [N, K]: KID_FAST_GU_KM on byte pairs
  KID_SKINNY_16_KM = 13, // KID_SKINNY_16 for B stored [N, K]: B strips of 128 K-contiguous rows
  KID_SKINNY_F8 = 14,    // one-byte M <= 16, B [N, K]: KID_SKINNY_16_KM on byte pairs, v_mfma_f32_16x16x128_f8f6f4
  KID_SKINNY_32 = 15,    // KID_SKINNY_16 with 32 rows of A (M <= 32)
  KID_SKINNY_64 = 16,    // ... 64 rows (M <= 64)
  KID_SKINNY_32_KM = 17, // KID_SKINNY_16_KM with 32 rows of A
  KID_SKINNY_64_KM = 18, // ... 64 rows
  KID_SKINNY_F8_32 = 19, // KID_SKINNY_32_KM on byte pairs
  KID_SKINNY_F8_64 = 20, // KID_SKINNY_64_KM on byte pairs
  KID_SKINNY_128 = 21,   // KID_SKINNY_16 with 128 rows of A (M <= 128)
  KID_SKINNY_128_KM = 22,// KID_SKINNY_16_KM with 128 rows of A
  KID_SKINNY_F8_128 = 23,// KID_SKINNY_128_KM on byte pairs
  KID_FAST_128 = 24,     // KID_FAST_256 with 128-row tiles: 8 waves of 64 x 64
  KID_FAST_128_KM = 25,  // KID_FAST_128 for B stored [N, K]
  KID_FAST_F8_128 = 26,  // KID_FAST_128_KM on byte pairs (one-byte inputs)
  KID_FAST_128_KM64 = 27,  // KID_FAST_128_KM with K blocks of 64 (128-byte row segments of A and B)
  KID_FAST_128_K64 = 28,   // KID_FAST_128 with K blocks of 64 (128-byte row segments of A)
  KID_FAST_F8_128_K64 = 29,  // KID_FAST_128_KM64 on byte pairs (K blocks of 128 codes)
  KID_COUNT
};

// One-byte inputs: IN_F8 + 2 * (A is E5M2) + (B is E5M2).
enum InKind : int { IN_BF16 = 0, IN_F16 = 1, IN_F32 = 2, IN_F8 = 3 };
enum OutKind : int { OUT_F32 = 0, OUT_BF16 = 1, OUT_F16 = 2 };

// Compile-time parameters of the fast kernels (one source of truth for the
// template instantiations and the planner's table).
// Swizzles were chosen with the LDS bank-conflict counter: gfx950 serves LDS
// reads from 64 four-byte banks (256 bytes per cycle), so a 16-byte read of
// 16 lanes must touch 16 distinct 16-byte slots of a 256-byte window.
struct CfgFast256 {
  static constexpr int BM = 256, BN = 256, NB = 1, WM = 2, WN = 4, BK = 32, STAGES = 4;
  static constexpr bool BKMAJOR = false, ATRANS = false, WSPLIT = false;
  static constexpr int AB = 2, AM = 3, AS = 4;   // A: Swizzle{2,3,4} over 64-byte rows
  static constexpr int BB = 2, BMb = 5, BS = 3;  // B: Swizzle{2,5,3} over 512-byte rows
};
// Gate/up: waves split by weight (WSPLIT): waves 0-3 (wn 0, 1) hold 128 x 64 slices of the
// W_gate product, waves 4-7 (wn 2, 3) the same slices of the W_up product.
struct CfgFastGU {
  static constexpr int BM = 256, BN = 128, NB = 2, WM = 2, WN = 4, BK = 32, STAGES = 4;
  static constexpr bool BKMAJOR = false, ATRANS = false, WSPLIT = true;
  static constexpr int AB = 2, AM = 3, AS = 4;   // A: Swizzle{2,3,4} over 64-byte rows
  static constexpr int BB = 2, BMb = 5, BS = 2;  // B: Swizzle{2,5,2} over 256-byte rows
};
// K-major B ([N, K], the storage of the Tylo.jl Hopper page): B blocks are K-contiguous rows
// like A blocks, read with plain 16-byte LDS reads, under the same swizzle as A.
struct CfgFast256KM : CfgFast256 {
  static constexpr bool BKMAJOR = true;
  static constexpr int BB = 2, BMb = 3, BS = 4;
};
// 128 x 256 tiles (twice the tiles of the 256-wide kernel for mid-size M): 8 waves (2 x 4) of 64 x 64,
// the same K blocks, swizzles and ping-pong; 4 stages of 24 KiB.
struct CfgFast128 : CfgFast256 {
  static constexpr int BM = 128;
};
struct CfgFast128KM : CfgFast256KM {
  static constexpr int BM = 128;
};
// The same tiles with K blocks of 64 (16-bit inputs, K a multiple of 64): 3 stages of 48 KiB, A (and
// K-major B) rows of 128 bytes under Swizzle{3,3,4}.  Measured against K blocks of 32 on one box
// (bf16 -> bf16, us, B [N, K] / [K, N]): 1024 x 4096 x 14336 168.6 -> 150.2 / 174.1 -> 155.4;
// 256 x 28672 x 8192 179.0 -> 153.3 / 162.4 -> 147.0; 384 x 11008 x 4096 58.0 -> 52.1 / 58.6 -> 53.7;
// 1024 x 4096 x 2048 29.8 -> 29.6 / 32.1 -> 30.6.
struct CfgFast128K64 : CfgFast128 {
  static constexpr int BK = 64, STAGES = 3;
  static constexpr int AB = 3, AM = 3, AS = 4;   // A: 128-byte rows; B keeps its 512-byte rows
};
struct CfgFast128KM64 : CfgFast128KM {
  static constexpr int BK = 64, STAGES = 3;
  static constexpr int AB = 3, AM = 3, AS = 4;   // 128-byte rows
  static constexpr int BB = 3, BMb = 3, BS = 4;
};
struct CfgFastGUKM : CfgFastGU {
  static constexpr bool BKMAJOR = true;
  static constexpr int BB = 2, BMb = 3, BS = 4;
};

// A stored [K, M] (M contiguous): the A block keeps the storage's orientation in
// LDS, rows of BM values per k, under the swizzle of the N-contiguous 256-wide B
// block (Swizzle{2,5,3} over 512-byte rows), and is read with transposing reads.
struct CfgFast256AT : CfgFast256 {
  static constexpr bool ATRANS = true;
  static constexpr int AB = 2, AM = 5, AS = 3;
};
struct CfgFastGUAT : CfgFastGU {
  static constexpr bool ATRANS = true;
  static constexpr int AB = 2, AM = 5, AS = 3;
};

struct CfgSkinny16 {
  static constexpr int BM = 16, BN = 128, BK = 128, STAGES = 4;
  static constexpr bool B_NT = true;             // non-temporal B loads: +10% HBM throughput (measured)
  static constexpr bool BKMAJOR = false;
  static constexpr int AB = 4, AM = 3, AS = 4;   // A: Swizzle{4,3,4} over 256-byte rows (16 rows -> 16 slots)
  static constexpr int BB = 3, BMb = 4, BS = 3;  // B: Swizzle{3,4,3} over 256-byte rows
};
// B stored [N, K]: strips of 64 B rows, each a K-contiguous 512-byte row per K block of 256,
// read like A's (plain 16-byte reads of 16 consecutive rows) under the same swizzle; two stages
// (80 KB) so that two workgroups share a CU.  Measured on 16 x 28672 x 8192 bf16 (one box): 128
// rows x 256-byte rows x 4 stages 83.4 us, 128 x 512 B x 2 stages 74.4, 64 x 512 B x 4 stages
// 73.4, x 3 stages 73.0, x 2 stages 71.0 (6.6 TB/s), 64 x 1 KB x 2 stages 77.9, 64 x 256 B x
// 4 stages 77.3: longer runs of each row per visit and more workgroups in flight both count.
struct CfgSkinny16KM : CfgSkinny16 {
  static constexpr int BN = 64, BK = 256, STAGES = 2;
  static constexpr bool BKMAJOR = true;
  static constexpr int AB = 4, AM = 3, AS = 5;   // 512-byte rows: 16 rows -> 16 slots
  static constexpr int BB = 4, BMb = 3, BS = 5;
};
// 32 and 64 rows of A (M <= 32, M <= 64: batches of a few dozen rows), each wave holding two or
// four 16-row blocks per 16 columns.  Measured on M x 28672 x 8192 bf16 against the general kernel
// these shapes took before (one box): M = 32 B [K, N] 78.7 us (3 stages; 4 stages 79.1) against
// 105.9, B [N, K] 78.5 us (64-row strips, K blocks of 128, 3 stages, 72 KB) against 104.4 (512-byte
// rows, 2 stages: 83.9); M = 64 B [K, N] 85.9 against 116.6, B [N, K] 91.3 (K blocks of 128, 2
// stages, 64 KB; 256-deep blocks 94.0, 128-row strips 93.5) against 106.4.
struct CfgSkinny32 : CfgSkinny16 {
  static constexpr int BM = 32, STAGES = 3;      // 120 KB
};
struct CfgSkinny64 : CfgSkinny16 {
  static constexpr int BM = 64, STAGES = 3;      // 144 KB
};
struct CfgSkinny32KM : CfgSkinny16KM {
  static constexpr int BM = 32, BK = 128, STAGES = 3;   // 72 KB: two workgroups per CU
  static constexpr int AS = 4, BS = 4;           // 256-byte rows
};
struct CfgSkinny64KM : CfgSkinny16KM {
  static constexpr int BM = 64, BK = 128, STAGES = 2;   // 64 KB: two workgroups per CU
  static constexpr int AS = 4, BS = 4;
};
// 128 rows of A: 128-column strips, K blocks of 64 (128-byte rows: Swizzle{3,3,4}, rows 2k and
// 2k+1 share a 256-byte window), 4 stages (128 KB).  Measured on 128 x 28672 x 8192 bf16 (one box):
// B [K, N] 97.9 us (3 stages 102.0; K blocks of 128, 2 stages 109.0) against 188.4 on the general
// kernel; B [N, K] 104.8 us (3 stages 106.4; 64-column strips with K blocks of 128, 3 stages 129.9)
// against 148.8.
struct CfgSkinny128 : CfgSkinny16 {
  static constexpr int BM = 128, BK = 64, STAGES = 4;
  static constexpr int AB = 3, AM = 3, AS = 4;
};
struct CfgSkinny128KM : CfgSkinny16KM {
  static constexpr int BM = 128, BN = 128, BK = 64, STAGES = 4;
  static constexpr int AB = 3, AM = 3, AS = 4;
  static constexpr int BB = 3, BMb = 3, BS = 4;
};

// Fill R[0, n) with the identity of `red` (0, -inf or +inf) on `stream`: a
// kernel, not a memset, so that HIP graphs may capture it.
hipError_t launch_reduce_init(float* R, int64_t n, int red, hipStream_t stream);

// C = alpha * sum over z < S of P[z * M * N ...] + beta * C (P: S FP32 slices of M x N, row stride N;
// N a multiple of 4, P 16-byte aligned; S one of 1, 2, 4, 8, 16), rounded to C's type.
hipError_t launch_split_sum(const float* P, int S, int64_t M, int64_t N, void* C, int64_t ldc, int out_kind,
                            float alpha, float beta, hipStream_t stream);

// Bytes of the per-GPU workspace array behind gemm_run_split_noalloc: the largest split form the
// planner makes (at most 256 workgroups of at most 128 x 256 FP32 values each) with room to spare.
constexpr int64_t kSplitScratchBytes = int64_t(64) << 20;

// Device address of the current device's workspace array (looked up once per device).
hipError_t split_scratch(void** out);

// Matrix-core rate probe (measurement aid): `workgroups` x 4 waves, each
// issuing mfma_per_wave (a multiple of 16) MFMAs on fragments from `ops`.
hipError_t launch_mfma_probe(const void* ops, int64_t n_frags, float* sink, int64_t workgroups, int64_t mfma_per_wave,
                             int in_kind, hipStream_t stream);

// Enqueue a GEMM (or, with lds_image, the debug stage dump) on `stream`.
hipError_t launch_kernel(int kid, int in_kind, int out_kind, int vec, bool gate_up, bool b_kmajor, bool a_trans,
                         const TiledArgs& args, dim3 grid, hipStream_t stream, bool lds_image);

// Per-family launchers.
hipError_t launch_tiled(int kid, int in_kind, int out_kind, int vec, bool gate_up, bool b_kmajor, bool a_trans,
                        const TiledArgs& args, dim3 grid, hipStream_t stream, bool lds_image);
hipError_t launch_fast(int kid, int in_kind, int out_kind, const TiledArgs& args, dim3 grid,
                       hipStream_t stream, bool lds_image);
hipError_t launch_skinny(int kid, int in_kind, int out_kind, const TiledArgs& args, dim3 grid, hipStream_t stream,
                         bool lds_image);
hipError_t launch_fast_f8(int kid, int in_kind, int out_kind, const TiledArgs& args, dim3 grid, hipStream_t stream,
                          bool lds_image);
hipError_t launch_f32(int out_kind, int vec, bool b_kmajor, bool a_trans, const TiledArgs& args, dim3 grid,
                      hipStream_t stream, bool lds_image);

}  // namespace lak
