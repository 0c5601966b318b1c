// Second pass of a GEMM whose K sum was cut into S ranges (gemm_run_split):
//   C = alpha * (P[0] + P[1] + ... + P[S-1]) + beta * C
// P holds the S FP32 partial products of the same m x n output, each over one
// contiguous range of K, as S slices of m * n values (row stride n).  The sum
// is the GEMM's own reduction over k regrouped by range (the accumulation
// order is the only difference to a single pass).  Each thread takes four
// consecutive columns of one row: its S 16-byte reads are all issued before the
// first is used (S is a template parameter: one memory latency per thread, not
// S of them), summed in range order (the result does not depend on
// scheduling), then alpha, beta and the rounding of the GEMM epilogue.
#include <mutex>

#include "kernel_common.hpp"
#include "launch.hpp"

namespace lak {
namespace {

// Workspace of gemm_run_split_noalloc: one array per GPU, held by the loaded code object until the
// process ends.  Host code never passes the array's name to a kernel (on the host it names a
// stand-in, not the device memory): split_scratch() looks up each device's address once.
static __device__ __align__(256) unsigned char scratch[kSplitScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

template <class TO, int S>
__global__ void __launch_bounds__(256) split_sum_kernel(const float* __restrict__ P, int64_t M, int64_t N, void* C,
                                                        int64_t ldc, float alpha, float beta) {
  const int64_t nq = N >> 2;
  const int64_t q = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (q >= M * nq) return;
  const int64_t row = q / nq, col = (q - row * nq) * 4;
  const int64_t slice = M * N;
  const float* p = P + row * N + col;
  f32x4 v[S];
#pragma unroll
  for (int z = 0; z < S; ++z) v[z] = *reinterpret_cast<const f32x4*>(p + z * slice);
  f32x4 s = v[0];
#pragma unroll
  for (int z = 1; z < S; ++z) s += v[z];
  typedef typename TO::storage St;
  St* c = static_cast<St*>(C) + row * ldc + col;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float x = alpha * s[e];
    if (beta != 0.0f) x += beta * from_out<TO>(c[e]);
    c[e] = to_out<TO>(x);
  }
}

template <class TO>
hipError_t go_sum(const float* P, int S, int64_t M, int64_t N, void* C, int64_t ldc, float alpha, float beta, dim3 grid,
                  hipStream_t stream) {
  switch (S) {
    case 1: hipLaunchKernelGGL((split_sum_kernel<TO, 1>), grid, dim3(256), 0, stream, P, M, N, C, ldc, alpha, beta); break;
    case 2: hipLaunchKernelGGL((split_sum_kernel<TO, 2>), grid, dim3(256), 0, stream, P, M, N, C, ldc, alpha, beta); break;
    case 4: hipLaunchKernelGGL((split_sum_kernel<TO, 4>), grid, dim3(256), 0, stream, P, M, N, C, ldc, alpha, beta); break;
    case 8: hipLaunchKernelGGL((split_sum_kernel<TO, 8>), grid, dim3(256), 0, stream, P, M, N, C, ldc, alpha, beta); break;
    case 16: hipLaunchKernelGGL((split_sum_kernel<TO, 16>), grid, dim3(256), 0, stream, P, M, N, C, ldc, alpha, beta); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t split_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_split_sum(const float* P, int S, int64_t M, int64_t N, void* C, int64_t ldc, int out_kind,
                            float alpha, float beta, hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (S < 1 || N % 4 || ldc < N) return hipErrorInvalidValue;
  const int64_t blocks = (M * (N / 4) + 255) / 256;
  if (blocks > int64_t(INT32_MAX)) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks));
  switch (out_kind) {
    case OUT_F32: return go_sum<OutF32>(P, S, M, N, C, ldc, alpha, beta, grid, stream);
    case OUT_BF16: return go_sum<OutBF16>(P, S, M, N, C, ldc, alpha, beta, grid, stream);
    case OUT_F16: return go_sum<OutF16>(P, S, M, N, C, ldc, alpha, beta, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lak
