// Device-side building blocks shared by the gfx950 GEMM kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace lak {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Input element tags: 16-bit patterns in memory ...
struct InBF16 { static constexpr bool f8 = false; };
struct InF16 { static constexpr bool f8 = false; };
// ... or one-byte codes, A and B each in the OCP 8-bit format FA / FB
// (0: E4M3, 1: E5M2, the matrix core's format selectors for A and B).
template <int FA, int FB>
struct InF8 {
  static constexpr bool f8 = true;
  static constexpr int fmt_a = FA, fmt_b = FB;
};

// Output element tags.
struct OutF32 { typedef float storage; };
struct OutBF16 { typedef uint16_t storage; };
struct OutF16 { typedef uint16_t storage; };

// v_mfma_f32_32x32x16_{bf16,f16}: 32x32 FP32 block += (32x16) x (16x32).
// Operand lane map: lane l holds row (A) / column (B) l % 32 and eight
// consecutive K values starting at 8 * (l / 32).  Result lane map: register r
// of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l % 32.
template <class TI>
__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c);
template <>
__device__ __forceinline__ f32x16 mfma_32x32x16<InBF16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma_32x32x16<InF16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// v_mfma_f32_32x32x64_f8f6f4 on 8-bit A and B: 32x32 FP32 block += (32x64) x
// (64x32).  Lane l holds row (A) / column (B) l % 32 and 32 K values, the
// result lane map is that of the 32x32x16 products.  A and B place K the same
// way (byte q of lane l of A meets byte q of lane l's half of B), so any
// assignment of K values to (lane half, byte) that both operands share gives
// the product; callers concatenate two 16-byte K-contiguous reads.  Scale
// operands 0 select the unscaled form of the instruction (no block scaling).
template <class TI>
__device__ __forceinline__ f32x16 mfma_f8_32x32x64(u32x4 a_lo, u32x4 a_hi, u32x4 b_lo, u32x4 b_hi, f32x16 c) {
  const i32x8 a{int(a_lo.x), int(a_lo.y), int(a_lo.z), int(a_lo.w), int(a_hi.x), int(a_hi.y), int(a_hi.z), int(a_hi.w)};
  const i32x8 b{int(b_lo.x), int(b_lo.y), int(b_lo.z), int(b_lo.w), int(b_hi.x), int(b_hi.y), int(b_hi.z), int(b_hi.w)};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, TI::fmt_a, TI::fmt_b, 0, 0, 0, 0);
}

// v_mfma_f32_16x16x128_f8f6f4 on 8-bit A and B: 16x16 FP32 block += (16x128) x
// (128x16).  Lane l holds row (A) / column (B) l % 16 and 32 K values; A and B
// place K the same way (byte q of lane l of A meets byte q of lane l's group of
// B), the result lane map is that of the 16x16x32 products.  Scale operands 0
// select the unscaled form.
template <class TI>
__device__ __forceinline__ f32x4 mfma_f8_16x16x128(u32x4 a_lo, u32x4 a_hi, u32x4 b_lo, u32x4 b_hi, f32x4 c) {
  const i32x8 a{int(a_lo.x), int(a_lo.y), int(a_lo.z), int(a_lo.w), int(a_hi.x), int(a_hi.y), int(a_hi.z), int(a_hi.w)};
  const i32x8 b{int(b_lo.x), int(b_lo.y), int(b_lo.z), int(b_lo.w), int(b_hi.x), int(b_hi.y), int(b_hi.z), int(b_hi.w)};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, TI::fmt_a, TI::fmt_b, 0, 0, 0, 0);
}

// v_mfma_f32_16x16x32_{bf16,f16}: lane l holds row/column l % 16 and eight
// consecutive K values starting at 8 * (l / 16); result register r of lane l
// is row 4*(l/16) + r, column l % 16.
template <class TI>
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c);
template <>
__device__ __forceinline__ f32x4 mfma_16x16x32<InBF16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma_16x16x32<InF16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Round-to-nearest-even conversions of the FP32 result (the language's own
// float -> __bf16 / _Float16 conversions, which gfx950 implements in hardware).
template <class TO>
__device__ __forceinline__ typename TO::storage to_out(float v);
template <>
__device__ __forceinline__ float to_out<OutF32>(float v) { return v; }
template <>
__device__ __forceinline__ uint16_t to_out<OutBF16>(float v) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v)); }
template <>
__device__ __forceinline__ uint16_t to_out<OutF16>(float v) { return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v)); }

template <class TO>
__device__ __forceinline__ float from_out(typename TO::storage v);
template <>
__device__ __forceinline__ float from_out<OutF32>(float v) { return v; }
template <>
__device__ __forceinline__ float from_out<OutBF16>(uint16_t v) { return static_cast<float>(__builtin_bit_cast(__bf16, v)); }
template <>
__device__ __forceinline__ float from_out<OutF16>(uint16_t v) { return static_cast<float>(__builtin_bit_cast(_Float16, v)); }

// Row reductions of the FP32 outputs (sum, maximum, minimum along a row);
// the operation codes RED_* live in launch.hpp.

__device__ __forceinline__ float red_identity(int op) {
  return op == RED_SUM ? 0.0f : op == RED_MAX ? -__builtin_inff() : __builtin_inff();
}
__device__ __forceinline__ float red_combine(int op, float a, float b) {
  return op == RED_SUM ? a + b : op == RED_MAX ? fmaxf(a, b) : fminf(a, b);
}
// Combine v over aligned groups of W consecutive lanes (W a power of two <= 64);
// every lane of a group ends with the group's value.
template <int W>
__device__ __forceinline__ float red_lanes(int op, float v) {
#pragma unroll
  for (int m = W / 2; m >= 1; m >>= 1) v = red_combine(op, v, __shfl_xor(v, m, 64));
  return v;
}
// Fold one partial into the row's result in global memory.
__device__ __forceinline__ void red_commit(int op, float* p, float v) {
  if (op == RED_SUM) {
    atomicAdd(p, v);
  } else if (op == RED_MAX) {
    atomicMax(p, v);
  } else {
    atomicMin(p, v);
  }
}

// Epilogue of one wave's FM x FN grid of 32 x 32 accumulator blocks, straight
// from the accumulator lane map (register e of lane l: row 8*(e/4) + 4*(l/32) +
// e%4, column l % 32 of its block): C = alpha * acc + beta * C_old in FP32
// (C_old read only when beta != 0), written only inside [0,M) x [0,N), and,
// when red != RED_NONE, every row's partial folded into R.  r0 / c0: the
// wave's first row and column in C.  The 16 old values of a block are all
// requested before the first is used, from clamped addresses (element 0 for
// positions outside C), so their latencies overlap; only the stores are
// predicated.
template <class TO, int FM, int FN>
__device__ __forceinline__ void epilogue_mfma32(const TiledArgs& g, const f32x16 (&acc)[FM][FN], int64_t r0, int64_t c0,
                                                int lane, int red) {
  typedef typename TO::storage St;
  const int lc = lane & 31, lr4 = (lane >> 5) * 4;
  // row reduction: per-lane partials of the 16 rows of each 32-row block
  // (columns j*32 + lc of the wave's sub-tile), then across the 32 lanes of each half
  float part[FM][16];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) part[i][e] = red_identity(red);
  St* C = static_cast<St*>(g.C);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t col = c0 + j * 32 + lc;
      const int64_t rbase = r0 + i * 32 + lr4;
      int64_t idx[16];
      bool ok[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = rbase + 8 * (e >> 2) + (e & 3);
        ok[e] = col < g.N && row < g.M;
        idx[e] = row * g.ldc + col;
      }
      float v[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] = g.alpha * acc[i][j][e];
      if (g.beta != 0.0f) {
        St old[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) old[e] = C[ok[e] ? idx[e] : 0];
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] += g.beta * from_out<TO>(old[e]);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if (ok[e]) C[idx[e]] = to_out<TO>(v[e]);
        if (red != RED_NONE && ok[e]) part[i][e] = red_combine(red, part[i][e], v[e]);
      }
    }
  }
  if (red != RED_NONE) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = red_lanes<32>(red, part[i][e]);
        const int64_t row = r0 + i * 32 + lr4 + 8 * (e >> 2) + (e & 3);
        if (lc == 0 && row < g.M) red_commit(red, g.R + row, p);
      }
  }
}

// SwiGLU combination of one gate and one up accumulator, in FP32:
// silu(g) * u with silu(g) = g / (1 + e^-g).
__device__ __forceinline__ float swiglu(float gate, float up) { return gate / (1.0f + expf(-gate)) * up; }

// Swizzle{B,M,S} on element offsets: XOR bits [M+S, M+S+B) into [M, M+B).
template <int B, int M, int S>
__device__ __forceinline__ constexpr int swz(int off) {
  return off ^ ((off >> S) & (((1 << B) - 1) << M));
}

// Workgroups are handed to the 8 XCDs round-robin (workgroup b runs on XCD
// b % 8).  Renumber so that each XCD receives one contiguous range of tile
// ids, keeping neighbouring tiles -- which share A rows and B columns -- in the
// same L2.  Ids past the last multiple of 8 keep their own number.
__device__ __forceinline__ int xcd_contiguous(int b, int nb) {
  const int full = nb & ~7;
  if (b >= full) return b;
  const int per = full >> 3;
  return (b & 7) * per + (b >> 3);
}

// Grouped ordering: walk `group` tile-rows together, column by column, so
// that consecutive ids reuse the same A panels and nearby B panels.
__device__ __forceinline__ void grouped_tile(int id, int tiles_m, int tiles_n, int group, int& tm, int& tn) {
  const int per_group = group * tiles_n;
  const int g = id / per_group;
  const int first = g * group;
  const int rows = min(group, tiles_m - first);
  const int in = id - g * per_group;
  tm = first + in % rows;
  tn = in / rows;
}

}  // namespace lak
