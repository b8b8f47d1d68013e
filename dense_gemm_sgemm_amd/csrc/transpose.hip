// Transposition of a matrix of 16-bit words into a K-contiguous copy, the
// step that lets the A * B^T kernels serve the other operand layouts.  Page
// "从零开始的 AI Infra: 算子基础与GPU架构" (section "19. 去掉转置") changes a
// layout once so that neighbouring threads read neighbouring elements; here
// the copy goes the other way, into the layout the matrix-core kernels read.
//
// dst[c * ldd + r] = src[r * lds + c] for r < rows, c < cols, one 64 x 64 tile
// per wave and no LDS: lane (i, j) = (l / 8, l % 8) loads the 8 x 8 block at
// source rows 8 i .. 8 i + 7 and columns 8 j .. 8 j + 7 of its tile as eight
// 16-byte row pieces, transposes it in registers, and stores it as eight
// 16-byte pieces of destination rows 8 j .. 8 j + 7.  Every load and store
// instruction of a wave covers 8 rows x 128 contiguous bytes.  The
// destination may be padded: every element of its rows_p x cols_p extent
// (source orientation) is written, zero outside the source matrix, which is
// never read outside.

#include "internal.h"

namespace mi355gemm {
namespace {

constexpr int kT = 64;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;   // transpose tiles per workgroup

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct TransposeArgs {
  const half_t* src;
  half_t* dst;
  int64_t lds, ldd;
  int rows, cols;       // the source matrix
  int rows_p, cols_p;   // the extent written (>= rows, cols)
};

// Two copies in one launch (transpositions or padding copies): blocks below
// split_block copy `first`, the others `second`.
struct PadPair {
  TransposeArgs first, second;
  int64_t split_block;
};

// One lane's 8 x 8 block: source rows r0 .. r0 + 7, columns c0 .. c0 + 7.
// INSIDE: the wave's whole tile lies inside the source matrix (hence inside
// the written extent) and takes whole 16-byte pieces; edge tiles check every
// row and element.
template <bool INSIDE>
__device__ __forceinline__ void transpose_block(const TransposeArgs& p, int r0, int c0) {
  // x[e] word q: source row r0 + e, columns c0 + 2q (low half) and c0 + 2q + 1.
  u32x4 x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const half_t* s = p.src + (int64_t)(r0 + e) * p.lds + c0;
    h8 v = {};
    if (INSIDE) {
      __builtin_memcpy(&v, s, 16);
    } else if (r0 + e < p.rows) {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (c0 + k < p.cols) v[k] = s[k];
    }
    x[e] = __builtin_bit_cast(u32x4, v);
  }
  // Destination row c0 + k holds source column c0 + k: word q of it pairs
  // rows r0 + 2q (low half) and r0 + 2q + 1.
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int sh = 16 * (k & 1);
    u32x4 w;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = ((x[2 * q][k >> 1] >> sh) & 0xFFFFu) | (((x[2 * q + 1][k >> 1] >> sh) & 0xFFFFu) << 16);
    half_t* d = p.dst + (int64_t)(c0 + k) * p.ldd + r0;
    if (INSIDE) {
      __builtin_memcpy(d, &w, 16);
    } else if (c0 + k < p.cols_p) {
      const h8 v = __builtin_bit_cast(h8, w);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (r0 + e < p.rows_p) d[e] = v[e];
    }
  }
}

int64_t transpose_blocks(int rows_p, int cols_p) {
  const int64_t tiles = (int64_t)((rows_p + kT - 1) / kT) * ((cols_p + kT - 1) / kT);
  return (tiles + kWaves - 1) / kWaves;
}

__global__ __launch_bounds__(kThreads) void transpose16_kernel(PadPair pair, int64_t block_base) {
  int64_t block = block_base + blockIdx.x;
  const bool first = block < pair.split_block;
  const TransposeArgs& p = first ? pair.first : pair.second;
  if (!first) block -= pair.split_block;
  const int lane = threadIdx.x & 63;
  const int tiles_c = (p.cols_p + kT - 1) / kT;
  const int64_t tiles = (int64_t)((p.rows_p + kT - 1) / kT) * tiles_c;
  const int64_t idx = block * kWaves + (threadIdx.x >> 6);
  if (idx >= tiles) return;
  const int tr = (int)(idx / tiles_c) * kT, tc = (int)(idx % tiles_c) * kT;
  const int r0 = tr + 8 * (lane >> 3), c0 = tc + 8 * (lane & 7);
  if (tr + kT <= p.rows && tc + kT <= p.cols)
    transpose_block<true>(p, r0, c0);
  else
    transpose_block<false>(p, r0, c0);
}

}  // namespace

hipError_t launch_transpose16(const PadCopy& first, const PadCopy* second, hipStream_t stream) {
  auto args = [](const PadCopy& c) {
    return TransposeArgs{c.src, c.dst, c.lds, c.ldd, c.rows, c.cols,
                         c.rows_p > c.rows ? c.rows_p : c.rows, c.cols_p > c.cols ? c.cols_p : c.cols};
  };
  PadPair p;
  p.first = args(first);
  p.split_block = transpose_blocks(p.first.rows_p, p.first.cols_p);
  int64_t blocks = p.split_block;
  if (second) {
    p.second = args(*second);
    blocks += transpose_blocks(p.second.rows_p, p.second.cols_p);
  } else {
    p.second = p.first;
  }
  if (blocks <= 0) return hipSuccess;
  return launch_tiles((const void*)transpose16_kernel, p, blocks, kThreads, 0, stream);
}

}  // namespace mi355gemm
