// 16-bit (fp16 or bf16) C = A * B^T for every shape, leading dimension and
// alignment, on the matrix cores.
//
// The boundary rule is the one of page 1 ("第 6 章 Shared Memory & Tile",
// exercise 7 of section 6.9): loads outside the matrix read zero, stores
// outside it are dropped.  Its motivating case on the NT page ("从零开始的 AI
// Infra: 算子基础与GPU架构", sections 19 and 29) is a shape that is not a
// multiple of any tile; here also K may be odd, so that rows start at any
// 2-byte address.
//
//  * a workgroup of 4 waves (2 x 2) owns a 128 x 128 tile of C, each wave
//    64 x 64 built from 16 x 16 blocks of v_mfma_f32_16x16x32_f16; two
//    workgroups share a CU;
//  * K is walked in slabs of 64.  Each thread fetches 4 chunks of 8 halves of
//    A and 4 of B per slab into registers -- one 16-byte load per chunk that
//    lies inside its row, element loads for the chunk that straddles K, zero
//    for chunks outside the matrix -- and writes them to LDS one slab ahead
//    of the MFMAs (two LDS stages, one barrier per slab).  The 16-byte global
//    accesses carry only the alignment of the data (2 bytes for an odd K);
//    the target runs with unaligned access enabled, which the compiler itself
//    relies on for such loads;
//  * LDS rows are 128 bytes, chunk c of row r at position c ^ ((r >> 1) & 7),
//    the layout of the full-tile kernel, so the MFMA operand reads (lane l:
//    row l % 16, chunk 4 s + l / 16) are free of bank conflicts;
//  * the epilogue rounds to half, stages 16 rows at a time per wave through
//    LDS and writes row segments of 8 halves: whole segments with one store,
//    the segment that straddles N element by element, nothing past M or N;
//  * the EPI instance applies the fused write-back act(acc + bias) +
//    residual in fp32 before the rounding, reading bias and residual element
//    by element inside the matrix.
#include "hgemm_tile.hpp"

namespace mi355gemm {
namespace hedge {

using hgemm::f4;
using hgemm::h4;
using hgemm::h8;
using hgemm::map_tile;

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int WM = 64, WN = 64, kBlocks = 4;              // 4 x 4 blocks per wave
constexpr int kRow = 2 * BK;                              // bytes per LDS slab row
constexpr int kStage = (BM + BN) * kRow;                  // 32 KiB
constexpr int kChunksPerThread = BM * (BK / 8) / kThreads;   // 4 per operand
constexpr int kOutRowBytes = 2 * WN;                      // staging row: 64 halves
constexpr int GM = 8;

// One chunk of 8 halves of row `row` starting at column k: zero outside the
// matrix, element loads where the chunk crosses K.
__device__ __forceinline__ h8 load_chunk(const half_t* base, int64_t ld, int rows, int K, int row,
                                         int k) {
  h8 v = {};
  if (row < rows && k < K) {
    const half_t* src = base + (int64_t)row * ld + k;
    if (k + 8 <= K) {
      __builtin_memcpy(&v, src, 16);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (k + e < K) v[e] = src[e];
    }
  }
  return v;
}

// MODE 0 writes C = half(acc), MODE 1 the fused write-back, MODE 2 the fp32
// partial product of one split-K range (workgroup b: range b / tiles, tile
// b % tiles) to the tile-padded workspace.
template <int MODE, int FMT>
__global__ __launch_bounds__(kThreads, 2) void hgemm_nt_edge_kernel(Args16 p, int64_t tile_base) {
  constexpr bool EPI = MODE == 1;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * kStage];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = (wave >> 1) * WM, wn = (wave & 1) * WN;
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  int64_t item = tile_base + blockIdx.x;
  int split = 0;
  if constexpr (MODE == 2) {
    const int64_t tiles = (int64_t)tiles_m * tiles_n;
    split = (int)(item / tiles);
    item -= split * tiles;
  }
  int tm, tn;
  map_tile<GM>(item, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // Chunk assignment: thread t fetches rows (t >> 3) + 32 i, chunk t & 7.
  const int crow = tid >> 3, cchunk = tid & 7;
  h8 ra[kChunksPerThread], rb[kChunksPerThread];
  auto fetch = [&](int t) __attribute__((always_inline)) {
    const int k = t * BK + 8 * cchunk;
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
      ra[i] = load_chunk(p.A, p.lda, p.M, p.K, m0 + crow + 32 * i, k);
      rb[i] = load_chunk(p.B, p.ldb, p.N, p.K, n0 + crow + 32 * i, k);
    }
  };
  auto stash = [&](int stage) __attribute__((always_inline)) {
    unsigned char* st = lds + stage * kStage;
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
      const int r = crow + 32 * i;
      const int pos = 16 * (cchunk ^ ((r >> 1) & 7));
      *(h8*)(st + r * kRow + pos) = ra[i];
      *(h8*)(st + (BM + r) * kRow + pos) = rb[i];
    }
  };

  const int r = lane & 15, g = lane >> 4;
  const int fr = (r >> 1) & 7;
  f4 acc[kBlocks][kBlocks];
#pragma unroll
  for (int i = 0; i < kBlocks; ++i)
#pragma unroll
    for (int j = 0; j < kBlocks; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int stage) __attribute__((always_inline)) {
    const unsigned char* st = lds + stage * kStage;
#pragma unroll
    for (int s = 0; s < BK / 32; ++s) {
      const int pos = 16 * ((4 * s + g) ^ fr);
      h8 fa[kBlocks], fb[kBlocks];
#pragma unroll
      for (int i = 0; i < kBlocks; ++i) fa[i] = *(const h8*)(st + (wm + 16 * i + r) * kRow + pos);
#pragma unroll
      for (int j = 0; j < kBlocks; ++j)
        fb[j] = *(const h8*)(st + (BM + wn + 16 * j + r) * kRow + pos);
#pragma unroll
      for (int i = 0; i < kBlocks; ++i)
#pragma unroll
        for (int j = 0; j < kBlocks; ++j)
          acc[i][j] = hgemm::mfma16<FMT>(fb[j], fa[i], acc[i][j]);
    }
  };

  // Slabs t0 .. t1 - 1: all of K, or this workgroup's split-K range.
  int t0 = 0, t1 = (p.K + BK - 1) / BK;
  if constexpr (MODE == 2) {
    t0 = split * p.sk.per;
    t1 = t0 + p.sk.per < t1 ? t0 + p.sk.per : t1;
  }
  fetch(t0);
  stash(0);
  __syncthreads();
  for (int t = t0; t < t1; ++t) {
    if (t + 1 < t1) fetch(t + 1);
    compute((t - t0) & 1);
    if (t + 1 < t1) stash((t + 1 - t0) & 1);
    __syncthreads();
  }

  if constexpr (MODE == 2) {
    // acc[i][j][v] is row m0 + wm + 16 i + r, column n0 + wn + 16 j + 4 g + v:
    // one 16-byte store per block into the padded workspace, no bounds.
    float* ws = p.sk.ws + split * p.sk.split_stride;
#pragma unroll
    for (int i = 0; i < kBlocks; ++i)
#pragma unroll
      for (int j = 0; j < kBlocks; ++j)
        *(f4*)(ws + (int64_t)(m0 + wm + 16 * i + r) * p.sk.ld + n0 + wn + 16 * j + 4 * g) =
            acc[i][j];
    return;
  }

  // Epilogue: acc[i][j][v] is C[m0 + wm + 16 i + r][n0 + wn + 16 j + 4 g + v].
  // Row block i at a time: quads are rounded and written (8 bytes per lane)
  // to this wave's 16-row staging area, chunk c of staging row R at slot
  // c ^ (R & 7); then each lane writes 8 consecutive halves of one row.
  unsigned char* out = lds + wave * (16 * kOutRowBytes);
  const int orow = lane >> 3, ochunk = lane & 7;
#pragma unroll
  for (int i = 0; i < kBlocks; ++i) {
#pragma unroll
    for (int j = 0; j < kBlocks; ++j) {
      h4 o;
      if constexpr (EPI) {
        // fused write-back, element by element inside the matrix
        const int m = m0 + wm + 16 * i + r, n = n0 + wn + 16 * j + 4 * g;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const bool in = m < p.M && n + v < p.N;
          float x = acc[i][j][v];
          if (p.bias && in) x += word_to_f32<FMT>(p.bias[n + v]);
          x = epi_act(x, p.act);
          if (p.res && in) x += word_to_f32<FMT>(p.res[(int64_t)m * p.ldr + n + v]);
          o[v] = f32_to_word<FMT>(x);
        }
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) o[v] = f32_to_word<FMT>(acc[i][j][v]);
      }
      const int c = 2 * j + (g >> 1);
      *(h4*)(out + r * kOutRowBytes + 16 * (c ^ (r & 7)) + 8 * (g & 1)) = o;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int R = 8 * q + orow;
      const h8 v = *(const h8*)(out + R * kOutRowBytes + 16 * (ochunk ^ (R & 7)));
      const int m = m0 + wm + 16 * i + R, n = n0 + wn + 8 * ochunk;
      if (m < p.M && n < p.N) {
        half_t* dst = p.C + (int64_t)m * p.ldc + n;
        if (n + 8 <= p.N) {
          __builtin_memcpy(dst, &v, 16);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (n + e < p.N) dst[e] = v[e];
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
}

}  // namespace hedge

namespace {
const void* edge_kernel(int mode, int fmt) {
  using hedge::hgemm_nt_edge_kernel;
  if (fmt == kFmtBF16)
    return mode == 0 ? (const void*)hgemm_nt_edge_kernel<0, kFmtBF16>
         : mode == 1 ? (const void*)hgemm_nt_edge_kernel<1, kFmtBF16>
                     : (const void*)hgemm_nt_edge_kernel<2, kFmtBF16>;
  return mode == 0 ? (const void*)hgemm_nt_edge_kernel<0, kFmtF16>
       : mode == 1 ? (const void*)hgemm_nt_edge_kernel<1, kFmtF16>
                   : (const void*)hgemm_nt_edge_kernel<2, kFmtF16>;
}
}  // namespace

hipError_t launch_f16_edge(const Args16& a, bool epi, hipStream_t stream) {
  const int64_t tiles = (int64_t)((a.M + hedge::BM - 1) / hedge::BM) *
                        ((a.N + hedge::BN - 1) / hedge::BN);
  return launch_tiles(edge_kernel(epi ? 1 : 0, a.fmt), a, tiles, hedge::kThreads, 0, stream);
}

hipError_t launch_f16_partials(const Args16& a, hipStream_t stream) {
  const int64_t tiles = (int64_t)((a.M + hedge::BM - 1) / hedge::BM) *
                        ((a.N + hedge::BN - 1) / hedge::BN);
  return launch_tiles(edge_kernel(2, a.fmt), a, tiles * a.sk.splits, hedge::kThreads, 0, stream);
}

}  // namespace mi355gemm
