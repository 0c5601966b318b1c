// Prefill of the row-reduction result: R[i] = identity of the operation (0 for
// a sum, -inf for a maximum, +inf for a minimum), so that the GEMM epilogues
// can fold their partial results into R with atomics in any order.  A plain
// fill kernel rather than a memset keeps the whole run capturable in a HIP graph.
#include "kernel_common.hpp"
#include "launch.hpp"

namespace lak {

__global__ void __launch_bounds__(256) reduce_init_kernel(float* R, int64_t n, int red) {
  const float v = red_identity(red);
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) R[i] = v;
}

hipError_t launch_reduce_init(float* R, int64_t n, int red, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(reduce_init_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, R, n, red);
  return hipGetLastError();
}

}  // namespace lak
