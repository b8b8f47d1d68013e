// Transposition of a matrix of 16-bit words into a K-contiguous copy, the
// step that lets the A * B^T kernels serve the other operand layouts.  Page
// "从零开始的 AI Infra: 算子基础与GPU架构" (section "19. 去掉转置") changes a
// layout once so that neighbouring threads read neighbouring elements; here
// the copy goes the other way, into the layout the matrix-core kernels read.
//
// dst[c * ldd + r] = src[r * lds + c] for r < rows, c < cols, in 64 x 64 tiles
// through LDS: each thread reads 16 bytes of a source row (8 consecutive
// columns) and writes 16 bytes of a destination row (8 consecutive source
// rows), so both sides of HBM see whole 128-byte row segments.  Elements
// outside the matrix are neither read nor written.
#include "internal.h"

namespace mi355gemm {
namespace {

constexpr int kT = 64;
constexpr int kThreads = 256;
constexpr int kPad = 2;   // LDS row = 66 words: 8 consecutive rows of one column fall in 2-way banks

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

struct TransposeArgs {
  const half_t* src;
  half_t* dst;
  int64_t lds, ldd;
  int rows, cols;
};

__global__ __launch_bounds__(kThreads) void transpose16_kernel(TransposeArgs p, int64_t tile_base) {
  __shared__ half_t tile[kT][kT + kPad];
  const int t = threadIdx.x;
  const int tiles_c = (p.cols + kT - 1) / kT;
  const int64_t idx = tile_base + blockIdx.x;
  const int r0 = (int)(idx / tiles_c) * kT, c0 = (int)(idx % tiles_c) * kT;

  // Source rows r0 + t / 8 + 32 i, columns c0 + 8 (t % 8) .. + 7.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = t / 8 + 32 * i, c = 8 * (t % 8);
    h8 v = {};
    if (r0 + r < p.rows && c0 + c < p.cols) {
      const half_t* s = p.src + (int64_t)(r0 + r) * p.lds + c0 + c;
      if (c0 + c + 8 <= p.cols) {
        __builtin_memcpy(&v, s, 16);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (c0 + c + e < p.cols) v[e] = s[e];
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[r][c + e] = v[e];
  }
  __syncthreads();

  // Destination rows c0 + t / 8 + 32 i (source columns), 8 source rows from
  // r0 + 8 (t % 8).
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = t / 8 + 32 * i, r = 8 * (t % 8);
    if (c0 + c >= p.cols || r0 + r >= p.rows) continue;
    h8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tile[r + e][c];
    half_t* d = p.dst + (int64_t)(c0 + c) * p.ldd + r0 + r;
    if (r0 + r + 8 <= p.rows) {
      __builtin_memcpy(d, &v, 16);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (r0 + r + e < p.rows) d[e] = v[e];
    }
  }
}

}  // namespace

hipError_t launch_transpose16(const half_t* src, int64_t lds, int rows, int cols, half_t* dst,
                              int64_t ldd, hipStream_t stream) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  const TransposeArgs p{src, dst, lds, ldd, rows, cols};
  const int64_t tiles = (int64_t)((rows + kT - 1) / kT) * ((cols + kT - 1) / kT);
  return launch_tiles((const void*)transpose16_kernel, p, tiles, kThreads, 0, stream);
}

}  // namespace mi355gemm
