// Matrix-core rate probe: a measurement aid beside the GEMM, not part of it.
//
// Every lane loads eight 16-byte operand fragments (four A-side, four B-side)
// from a caller buffer and then issues v_mfma_f32_32x32x16 (bf16 / f16),
// v_mfma_f32_32x32x2_f32 (binary32, the first word of each fragment) or
// v_mfma_f32_32x32x64_f8f6f4 on E4M3 codes (two fragments per 32-byte operand)
// in sixteen independent accumulator chains, with no memory traffic in between.  Timed
// against the same number of MFMAs per SIMD as a GEMM launch, it gives the
// rate the matrix cores sustain on those operand values at whatever clock the
// chip settles to under that load (the power drawn by the multipliers depends
// on the operand bits).  One workgroup of four waves per CU: one wave per SIMD.
#include "kernel_common.hpp"
#include "launch.hpp"

namespace lak {
namespace {

template <class TI>
__global__ void __launch_bounds__(256) mfma_probe_kernel(const u32x4* __restrict__ ops, int64_t n_frags,
                                                          float* __restrict__ sink, int64_t iters) {
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  u32x4 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = ops[(t * 8 + i) % n_frags];
    b[i] = ops[(t * 8 + 4 + i) % n_frags];
  }
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_32x32x16<TI>(a[i], b[j], acc[i][j]);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[i][j][e];
  sink[t] = s;
}

// Binary32: v_mfma_f32_32x32x2_f32 in sixteen chains, one 4-byte operand per
// lane and side (the first word of each fragment).
__global__ void __launch_bounds__(256) mfma_probe_f32_kernel(const u32x4* __restrict__ ops, int64_t n_frags,
                                                              float* __restrict__ sink, int64_t iters) {
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  float a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = __builtin_bit_cast(float, ops[(t * 8 + i) % n_frags].x);
    b[i] = __builtin_bit_cast(float, ops[(t * 8 + 4 + i) % n_frags].x);
  }
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[i][j][e];
  sink[t] = s;
}

// One-byte E4M3 codes: v_mfma_f32_32x32x64_f8f6f4 in sixteen chains; operand
// i of each side is fragments i and (i + 1) % 4 of that side, concatenated.
__global__ void __launch_bounds__(256) mfma_probe_f8_kernel(const u32x4* __restrict__ ops, int64_t n_frags,
                                                             float* __restrict__ sink, int64_t iters) {
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  u32x4 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = ops[(t * 8 + i) % n_frags];
    b[i] = ops[(t * 8 + 4 + i) % n_frags];
  }
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = mfma_f8_32x32x64<InF8<0, 0>>(a[i], a[(i + 1) % 4], b[j], b[(j + 1) % 4], acc[i][j]);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[i][j][e];
  sink[t] = s;
}

}  // namespace

hipError_t launch_mfma_probe(const void* ops, int64_t n_frags, float* sink, int64_t workgroups, int64_t mfma_per_wave,
                             int in_kind, hipStream_t stream) {
  const u32x4* p = static_cast<const u32x4*>(ops);
  const int64_t iters = mfma_per_wave / 16;
  if (in_kind == IN_BF16) {
    hipLaunchKernelGGL(mfma_probe_kernel<InBF16>, dim3(unsigned(workgroups)), dim3(256), 0, stream, p, n_frags, sink, iters);
  } else if (in_kind == IN_F32) {
    hipLaunchKernelGGL(mfma_probe_f32_kernel, dim3(unsigned(workgroups)), dim3(256), 0, stream, p, n_frags, sink, iters);
  } else if (in_kind == IN_F8) {
    hipLaunchKernelGGL(mfma_probe_f8_kernel, dim3(unsigned(workgroups)), dim3(256), 0, stream, p, n_frags, sink, iters);
  } else {
    hipLaunchKernelGGL(mfma_probe_kernel<InF16>, dim3(unsigned(workgroups)), dim3(256), 0, stream, p, n_frags, sink, iters);
  }
  return hipGetLastError();
}

}  // namespace lak
