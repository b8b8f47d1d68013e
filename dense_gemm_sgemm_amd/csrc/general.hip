// General kernels: correct for every shape, leading dimension and alignment.
//
// These are the LDS-tiled kernels of page 1 ("第 6 章 Shared Memory & Tile",
// sections 6.2 and 6.3.1: a block owns an output tile, stages K-slabs of A and
// B in shared memory and each thread accumulates a small register tile) with
// every global load predicated (zero-filled outside the matrix) and every
// store masked -- the boundary rule of exercise 7 in section 6.9.  They back
// the fast MFMA kernels wherever a shape or an alignment does not fit those,
// and they implement the K == 0 / alpha == 0 quick returns.
#include "internal.h"

namespace mi355gemm {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;        // output tile is kTile x kTile, 4 x 4 per thread

// ---------------------------------------------------------------- fp32 -------
constexpr int kF32Bk = 16;

__global__ __launch_bounds__(kThreads) void sgemm_general_kernel(F32Args p, int64_t tile_base) {
  // A is staged k-major so that the inner loop reads rows of both tiles.
  __shared__ float As[kF32Bk][kTile + 4];
  __shared__ float Bs[kF32Bk][kTile + 4];
  const int tid = threadIdx.x;
  const int tx = tid % 16, ty = tid / 16;
  const int64_t tile = tile_base + blockIdx.x, tiles_n = (p.N + kTile - 1) / kTile;
  const int m0 = (int)(tile / tiles_n) * kTile, n0 = (int)(tile % tiles_n) * kTile;

  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

  for (int k0 = 0; k0 < p.K; k0 += kF32Bk) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + ty + 16 * r, k = k0 + tx;
      As[tx][ty + 16 * r] = (m < p.M && k < p.K) ? p.A[(int64_t)m * p.lda + k] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kr = tid / 64 + 4 * r, n = n0 + tid % 64, k = k0 + kr;
      Bs[kr][tid % 64] = (k < p.K && n < p.N) ? p.B[(int64_t)k * p.ldb + n] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kF32Bk; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty + 16 * i;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx + 16 * j;
      if (n >= p.N) continue;
      float* c = p.C + (int64_t)m * p.ldc + n;
      float v = p.alpha * acc[i][j];
      if (p.beta != 0.f) v = fmaf(p.beta, *c, v);
      *c = v;
    }
  }
}

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
__global__ __launch_bounds__(kThreads) void hgemm_zero_kernel(F16Args p) {
  const int64_t total = (int64_t)p.M * p.N;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * kThreads) {
    const int64_t m = e / p.N, n = e % p.N;
    p.C[m * p.ldc + n] = (half_t)0.f;
  }
}

int64_t tile_count(int M, int N) {
  return (int64_t)((M + kTile - 1) / kTile) * ((N + kTile - 1) / kTile);
}

unsigned fill_blocks(int M, int N) {
  const int64_t want = ((int64_t)M * N + kThreads - 1) / kThreads;
  return (unsigned)(want < 4096 ? want : 4096);
}

}  // namespace

hipError_t launch_f32_general(const F32Args& a, hipStream_t stream) {
  return launch_tiles((const void*)sgemm_general_kernel, a, tile_count(a.M, a.N), kThreads, 0,
                      stream);
}

hipError_t launch_f32_scale(const F32Args& a, hipStream_t stream) {
  F32Args p = a;
  void* args[] = {&p};
  return hipLaunchKernel((const void*)sgemm_scale_kernel, dim3(fill_blocks(a.M, a.N)),
                         dim3(kThreads), args, 0, stream);
}

hipError_t launch_f16_zero(const F16Args& a, hipStream_t stream) {
  F16Args p = a;
  void* args[] = {&p};
  return hipLaunchKernel((const void*)hgemm_zero_kernel, dim3(fill_blocks(a.M, a.N)),
                         dim3(kThreads), args, 0, stream);
}

}  // namespace mi355gemm
