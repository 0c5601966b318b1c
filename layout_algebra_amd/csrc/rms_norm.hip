// Row normalisation for gfx950: Y[i, :] = X[i, :] * inv[i] * G with
// inv[i] = 1 / sqrt(sum_j X[i, j]^2 / D + eps), the kernel of the Phobos page
// "Tiles and shared memory" (section "A complete kernel": a row sum of squares,
// the inverse root of its mean plus eps, the row scaled by it and by the gain).
//
// The pages' kernel gives each workgroup 8 rows held in a shared tile and lets
// the compiler place a barrier before the row sum.  Here the work is HBM-bound
// (one read and one write per element), so the MI355X mapping is one wave per
// row with no LDS at all: each lane holds its slice of the row in registers,
// the sum of squares is reduced across the 64 lanes with cross-lane swaps, and
// the same registers produce the outputs.  Every lane ends the butterfly with
// the same sum (each step adds the same two values in both partners).
//  * Rows of up to NCH chunks (a chunk is 64 lanes x VEC elements) stay in
//    registers, ROWS rows per wave at a time so several loads are in flight;
//    longer rows are read twice (sum of squares, then outputs), the second
//    read mostly from L2.
//  * VEC = 16 bytes of X per lane (4 f32 or 8 16-bit values) when rows start
//    on 16 bytes, else 1; the last partial chunk of a row is element-wise.
//  * Arithmetic in FP32: squares summed with fused multiply-adds per lane,
//    then across lanes; ss / D, + eps, sqrt and 1 / r each correctly rounded;
//    y = (x * inv) * g, rounded once to Y's type (nearest even).
//  * X is loaded and Y stored non-temporally (each is touched once): measured
//    5.37 -> 5.70 TB/s for f32 rows of 256 and 4.08 -> 5.90 TB/s for bf16
//    rows of 4096, above a device-to-device copy of the same bytes (5.1-5.3).
//    Keeping the gain as FP32 in LDS instead of registers measured no better.
//  * The grid is capped at 8 workgroups of 4 waves per CU; waves stride over
//    the rows, keeping the gain vector in registers.
#include "norm.hpp"
#include "kernel_common.hpp"

namespace lak {
namespace {

template <class S, int N>
struct alignas(N * sizeof(S) >= 16 ? 16 : N * sizeof(S)) Pack {
  S v[N];
};

// Options of the register-path kernel.
enum : int { OPT_NT = 1,      // non-temporal X loads and Y stores (streamed once)
             OPT_G_LDS = 2 };  // gain converted to FP32 once per workgroup and kept in LDS

template <class TX, int VEC, bool NT = false>
__device__ __forceinline__ void load_chunk(const typename TX::storage* row, int64_t col, int64_t D,
                                           Pack<typename TX::storage, VEC>& out) {
  typedef typename TX::storage S;
  if (col + VEC <= D) {
    if constexpr (NT && sizeof(Pack<S, VEC>) == 16) {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + col));
      out = __builtin_bit_cast(Pack<S, VEC>, v);
    } else {
      out = *reinterpret_cast<const Pack<S, VEC>*>(row + col);
    }
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e) out.v[e] = col + e < D ? row[col + e] : S(0);
  }
}

template <class TY, int VEC, bool NT = false>
__device__ __forceinline__ void store_chunk(typename TY::storage* row, int64_t col, int64_t D,
                                            const Pack<typename TY::storage, VEC>& v) {
  typedef typename TY::storage S;
  constexpr int BYTES = int(sizeof(Pack<S, VEC>));
  if (col + VEC <= D) {
    if constexpr (NT && BYTES % 16 == 0) {
      u32x4* dst = reinterpret_cast<u32x4*>(row + col);
      const u32x4* src = reinterpret_cast<const u32x4*>(&v);
#pragma unroll
      for (int i = 0; i < BYTES / 16; ++i) __builtin_nontemporal_store(src[i], dst + i);
    } else if constexpr (NT && BYTES == 8) {
      __builtin_nontemporal_store(__builtin_bit_cast(u32x2, v), reinterpret_cast<u32x2*>(row + col));
    } else {
      *reinterpret_cast<Pack<S, VEC>*>(row + col) = v;
    }
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e)
      if (col + e < D) row[col + e] = v.v[e];
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ float inv_rms(float ss, float d, float eps) { return 1.0f / sqrtf(ss / d + eps); }

// Rows of at most NCH chunks, held in registers; ROWS rows per wave at a time.
template <class TX, class TY, int VEC, int NCH, int ROWS, int OPT>
__global__ void __launch_bounds__(256) rms_norm_reg_kernel(const NormArgs a) {
  typedef typename TX::storage SX;
  typedef typename TY::storage SY;
  constexpr int CW = 64 * VEC;
  constexpr bool NT = (OPT & OPT_NT) != 0;
  constexpr bool GL = (OPT & OPT_G_LDS) != 0;
  constexpr int GL_ELEMS = GL ? NCH * CW : 1;
  __shared__ __attribute__((aligned(16))) float g_lds[GL_ELEMS];
  const int lane = threadIdx.x & 63;
  const int64_t wave = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t nwaves = int64_t(gridDim.x) * 4;
  const int64_t D = a.D;
  const float df = float(D);
  const SX* X = static_cast<const SX*>(a.X);
  const SX* G = static_cast<const SX*>(a.G);
  SY* Y = static_cast<SY*>(a.Y);

  Pack<SX, VEC> g[GL ? 1 : NCH];
  if constexpr (GL) {
    for (int64_t j = threadIdx.x; j < GL_ELEMS; j += 256) g_lds[j] = j < D ? from_out<TX>(G[j]) : 0.0f;
    __syncthreads();
  } else {
#pragma unroll
    for (int c = 0; c < NCH; ++c) load_chunk<TX, VEC>(G, int64_t(c) * CW + lane * VEC, D, g[c]);
  }

  for (int64_t r0 = wave * ROWS; r0 < a.M; r0 += nwaves * ROWS) {
    Pack<SX, VEC> x[ROWS][NCH];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const int64_t row = r0 + r < a.M ? r0 + r : a.M - 1;   // a short last group repeats a valid row
#pragma unroll
      for (int c = 0; c < NCH; ++c) load_chunk<TX, VEC, NT>(X + row * a.ldx, int64_t(c) * CW + lane * VEC, D, x[r][c]);
    }
    float inv[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      float ss = 0.0f;
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float v = from_out<TX>(x[r][c].v[e]);
          ss = __builtin_fmaf(v, v, ss);
        }
      inv[r] = inv_rms(wave_sum(ss), df, a.eps);
    }
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      if (r0 + r >= a.M) break;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        Pack<SY, VEC> y;
        float gv[VEC];
        if constexpr (GL) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) gv[e] = g_lds[c * CW + lane * VEC + e];
        } else {
#pragma unroll
          for (int e = 0; e < VEC; ++e) gv[e] = from_out<TX>(g[c].v[e]);
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) y.v[e] = to_out<TY>(from_out<TX>(x[r][c].v[e]) * inv[r] * gv[e]);
        store_chunk<TY, VEC, NT>(Y + (r0 + r) * a.ldy, int64_t(c) * CW + lane * VEC, D, y);
      }
    }
  }
}

// Long rows: the sum of squares in one pass over the row, the outputs in a
// second (8 chunks of loads in flight per step).
template <class TX, class TY, int VEC>
__global__ void __launch_bounds__(256) rms_norm_stream_kernel(const NormArgs a) {
  typedef typename TX::storage SX;
  typedef typename TY::storage SY;
  constexpr int CW = 64 * VEC, STEP = 8;
  const int lane = threadIdx.x & 63;
  const int64_t wave = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t nwaves = int64_t(gridDim.x) * 4;
  const int64_t D = a.D;
  const float df = float(D);
  const SX* G = static_cast<const SX*>(a.G);

  for (int64_t row = wave; row < a.M; row += nwaves) {
    const SX* xr = static_cast<const SX*>(a.X) + row * a.ldx;
    SY* yr = static_cast<SY*>(a.Y) + row * a.ldy;
    float ss = 0.0f;
    for (int64_t c0 = 0; c0 < D; c0 += int64_t(STEP) * CW) {
      Pack<SX, VEC> x[STEP];
#pragma unroll
      for (int c = 0; c < STEP; ++c) load_chunk<TX, VEC>(xr, c0 + int64_t(c) * CW + lane * VEC, D, x[c]);
#pragma unroll
      for (int c = 0; c < STEP; ++c)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float v = from_out<TX>(x[c].v[e]);
          ss = __builtin_fmaf(v, v, ss);
        }
    }
    const float inv = inv_rms(wave_sum(ss), df, a.eps);
    for (int64_t c0 = 0; c0 < D; c0 += int64_t(STEP) * CW) {
      Pack<SX, VEC> x[STEP], g[STEP];
#pragma unroll
      for (int c = 0; c < STEP; ++c) {
        load_chunk<TX, VEC, true>(xr, c0 + int64_t(c) * CW + lane * VEC, D, x[c]);   // last use of X
        load_chunk<TX, VEC>(G, c0 + int64_t(c) * CW + lane * VEC, D, g[c]);
      }
#pragma unroll
      for (int c = 0; c < STEP; ++c) {
        Pack<SY, VEC> y;
#pragma unroll
        for (int e = 0; e < VEC; ++e) y.v[e] = to_out<TY>(from_out<TX>(x[c].v[e]) * inv * from_out<TX>(g[c].v[e]));
        store_chunk<TY, VEC, true>(yr, c0 + int64_t(c) * CW + lane * VEC, D, y);
      }
    }
  }
}

constexpr int kMaxBlocks = 256 * 8;
constexpr int kNormOpt = OPT_NT;

template <class K>
hipError_t go(K kernel, const NormArgs& a, int64_t waves_needed, hipStream_t s) {
  int64_t blocks = (waves_needed + 3) / 4;
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <class TX, class TY, int VEC, int OPT = kNormOpt>
hipError_t by_len(const NormArgs& a, hipStream_t s) {
  const int64_t nch = (a.D + 64 * VEC - 1) / (64 * VEC);
  if (nch <= 1) return go(rms_norm_reg_kernel<TX, TY, VEC, 1, 4, OPT>, a, (a.M + 3) / 4, s);
  if (nch <= 2) return go(rms_norm_reg_kernel<TX, TY, VEC, 2, 2, OPT>, a, (a.M + 1) / 2, s);
  if (nch <= 4) return go(rms_norm_reg_kernel<TX, TY, VEC, 4, 1, OPT>, a, a.M, s);
  if (nch <= 8) return go(rms_norm_reg_kernel<TX, TY, VEC, 8, 1, OPT>, a, a.M, s);
  return go(rms_norm_stream_kernel<TX, TY, VEC>, a, a.M, s);
}

template <class TX, class TY>
hipError_t by_vec(const NormArgs& a, bool vec, hipStream_t s) {
  constexpr int V = 16 / int(sizeof(typename TX::storage));
  return vec ? by_len<TX, TY, V>(a, s) : by_len<TX, TY, 1>(a, s);
}

template <class TX>
hipError_t by_out(const NormArgs& a, int y_kind, bool vec, hipStream_t s) {
  switch (y_kind) {
    case OUT_F32: return by_vec<TX, OutF32>(a, vec, s);
    case OUT_BF16: return by_vec<TX, OutBF16>(a, vec, s);
    case OUT_F16: return by_vec<TX, OutF16>(a, vec, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_rms_norm(const NormArgs& a, int x_kind, int y_kind, bool vec, hipStream_t s) {
  switch (x_kind) {
    case OUT_F32: return by_out<OutF32>(a, y_kind, vec, s);
    case OUT_BF16: return by_out<OutBF16>(a, y_kind, vec, s);
    case OUT_F16: return by_out<OutF16>(a, y_kind, vec, s);
    default: return hipErrorInvalidValue;
  }
}

int rms_norm_vec_elems(int x_kind) { return x_kind == OUT_F32 ? 4 : 8; }

}  // namespace lak
