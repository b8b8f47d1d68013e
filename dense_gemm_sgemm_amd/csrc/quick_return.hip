// The quick-return kernels: C = beta * C for an fp32 call with K == 0 or
// alpha == 0 (C = 0 when beta == 0, C is then not read), and C = 0 for an
// fp16 call with K == 0.  An empty sum is zero; the BLAS convention makes
// beta == 0 overwrite C whatever it holds.
#include "internal.h"

namespace mi355gemm {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------- fp32 -------
// C = beta * C (C = 0 when beta == 0): the K == 0 / alpha == 0 result.
__global__ __launch_bounds__(kThreads) void sgemm_scale_kernel(F32Args p) {
  const int64_t total = (int64_t)p.M * p.N;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * kThreads) {
    const int64_t m = e / p.N, n = e % p.N;
    float* c = p.C + m * p.ldc + n;
    *c = (p.beta != 0.f) ? p.beta * *c : 0.f;
  }
}

// ---------------------------------------------------------------- fp16 -------
__global__ __launch_bounds__(kThreads) void hgemm_zero_kernel(Args16 p) {
  const int64_t total = (int64_t)p.M * p.N;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * kThreads) {
    const int64_t m = e / p.N, n = e % p.N;
    p.C[m * p.ldc + n] = (half_t)0.f;
  }
}

unsigned fill_blocks(int M, int N) {
  const int64_t want = ((int64_t)M * N + kThreads - 1) / kThreads;
  return (unsigned)(want < 4096 ? want : 4096);
}

}  // namespace

hipError_t launch_f32_scale(const F32Args& a, hipStream_t stream) {
  F32Args p = a;
  void* args[] = {&p};
  return hipLaunchKernel((const void*)sgemm_scale_kernel, dim3(fill_blocks(a.M, a.N)),
                         dim3(kThreads), args, 0, stream);
}

hipError_t launch_f16_zero(const Args16& a, hipStream_t stream) {
  Args16 p = a;
  void* args[] = {&p};
  return hipLaunchKernel((const void*)hgemm_zero_kernel, dim3(fill_blocks(a.M, a.N)),
                         dim3(kThreads), args, 0, stream);
}

}  // namespace mi355gemm
