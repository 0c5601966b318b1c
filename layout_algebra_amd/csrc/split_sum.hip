// Second pass of a GEMM whose K sum was cut into S ranges (gemm_run_split):
//   C = alpha * (P[0] + P[1] + ... + P[S-1]) + beta * C
// P holds the S FP32 partial products of the same m x n output, each over one
// contiguous range of K, as S slices of m * n values (row stride n).  The sum
// is the GEMM's own reduction over k regrouped by range (the accumulation
// order is the only difference to a single pass).  Each thread takes four
// consecutive columns of one row: S 16-byte reads summed in range order (the
// result does not depend on scheduling), then alpha, beta and the rounding of
// the GEMM epilogue.
#include "kernel_common.hpp"
#include "launch.hpp"

namespace lak {
namespace {

template <class TO>
__global__ void __launch_bounds__(256) split_sum_kernel(const float* __restrict__ P, int S, int64_t M, int64_t N,
                                                        void* C, int64_t ldc, float alpha, float beta) {
  const int64_t nq = N >> 2;
  const int64_t q = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (q >= M * nq) return;
  const int64_t row = q / nq, col = (q - row * nq) * 4;
  const int64_t slice = M * N;
  const float* p = P + row * N + col;
  f32x4 s = *reinterpret_cast<const f32x4*>(p);
  for (int z = 1; z < S; ++z) s += *reinterpret_cast<const f32x4*>(p + z * slice);
  typedef typename TO::storage St;
  St* c = static_cast<St*>(C) + row * ldc + col;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float v = alpha * s[e];
    if (beta != 0.0f) v += beta * from_out<TO>(c[e]);
    c[e] = to_out<TO>(v);
  }
}

}  // namespace

hipError_t launch_split_sum(const float* P, int S, int64_t M, int64_t N, void* C, int64_t ldc, int out_kind,
                            float alpha, float beta, hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (S < 1 || N % 4 || ldc < N) return hipErrorInvalidValue;
  const int64_t blocks = (M * (N / 4) + 255) / 256;
  if (blocks > int64_t(INT32_MAX)) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks));
  switch (out_kind) {
    case OUT_F32: hipLaunchKernelGGL(split_sum_kernel<OutF32>, grid, dim3(256), 0, stream, P, S, M, N, C, ldc, alpha, beta); break;
    case OUT_BF16: hipLaunchKernelGGL(split_sum_kernel<OutBF16>, grid, dim3(256), 0, stream, P, S, M, N, C, ldc, alpha, beta); break;
    case OUT_F16: hipLaunchKernelGGL(split_sum_kernel<OutF16>, grid, dim3(256), 0, stream, P, S, M, N, C, ldc, alpha, beta); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lak
