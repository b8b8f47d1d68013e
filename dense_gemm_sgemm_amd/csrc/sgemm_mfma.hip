// fp32 SGEMM on the CDNA4 matrix cores: C = alpha * A * B + beta * C.
//
// Structure (prior art: the 2-D register-tiled, multi-stage SGEMM of the page
// "异步拷贝与 Hopper/Blackwell 新特性", section "cp.async 与多级流水"; the
// per-thread 8x8 FMA tile of that kernel becomes a per-wave tile of
// v_mfma_f32_16x16x4_f32 products here):
//
//  * a 256-thread workgroup (4 waves, 2 x 2) owns a BM x BN tile of C
//    (128 x 128, or 64 x 64 when the larger tiles would leave CUs idle);
//  * K is walked in slabs of 16 (32 for the 64 x 64 full tiles when K allows);
//    each slab of A (BM x BK) and B (BK x BN) is
//    fetched with 16-byte loads into registers one slab ahead and written to
//    the other half of a double-buffered LDS ring, so one barrier per slab
//    separates writers from readers;
//  * a wave's tile is blocks of 16 x 16; per 16 k of a slab each block takes
//    4 MFMAs (K = 4 each).  Lane l = 16 g + r feeds the MFMA row/column r
//    and, in MFMA step s of part q, the slab column k = 16 q + 4 g + s: the
//    same bijection for both operands, so the four steps sum all 16 k of the
//    part.  With that mapping a lane's four A values are one 16-byte LDS read;
//  * epilogue: alpha * acc (+ beta * C when beta != 0, C is not read
//    otherwise) straight from the accumulators (lane l, register v holds row
//    4 g + v, column r of a block).
//
// Two variants of every tile size: the full-tile kernel (M % BM == N % BN ==
// K % 16 == 0, 16-byte aligned rows and leading dimensions that are
// multiples of 4) loads and stores unchecked; the edge
// kernel serves every other shape, leading dimension and alignment with the
// boundary rule of page 1 ("第 6 章 Shared Memory & Tile", exercise 7 of
// section 6.9): loads outside the matrix read zero, stores outside it are
// dropped.  Its 16-byte loads of rows that are only 4-byte aligned rely on
// the target's unaligned-access mode (the compiler emits the same loads for
// such data itself); chunks that cross K or N are read element by element.
#include "internal.h"
#include "hgemm_tile.hpp"

namespace mi355gemm {
namespace {

constexpr int BK = 16;   // K granularity of the full-tile kernel
constexpr int kThreads = 256;

typedef float f4 __attribute__((ext_vector_type(4)));

// One LDS stage of a BKT-deep slab.  A rows are BKT + 4 floats apart for
// BKT = 16 (measured fastest there) and BKT + 8 for BKT = 32 (bank-conflict
// free 16-byte fragment reads); B rows BN + 4 floats apart: 4 rows apart = 16
// banks apart.
template <int BM, int BN, int BKT>
struct Stage {
  static constexpr int kAStride = BKT == 16 ? BKT + 4 : BKT + 8;
  static constexpr int kBStride = BN + 4;
  float a[BM * kAStride];
  float b[BKT * kBStride];
};

// Four consecutive floats of row `row`, columns col .. col + 3, of a matrix
// with `rows` rows and `cols` columns: zero outside, element loads where the
// chunk crosses the last column.
__device__ __forceinline__ f4 load4(const float* base, int64_t ld, int rows, int cols, int row,
                                    int col) {
  f4 v = {0.f, 0.f, 0.f, 0.f};
  if (row < rows && col < cols) {
    const float* src = base + (int64_t)row * ld + col;
    if (col + 4 <= cols) {
      __builtin_memcpy(&v, src, 16);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (col + e < cols) v[e] = src[e];
    }
  }
  return v;
}

// SPLIT instances write the fp32 partial product of one split-K range
// (workgroup b: range b / tiles, tile b % tiles) to the tile-padded
// workspace instead of C.
template <int BM, int BN, bool EDGE, bool SPLIT = false, int BKT = 16>
__global__ __launch_bounds__(kThreads, 2) void sgemm_mfma_kernel(F32Args p, int64_t tile_base) {
  constexpr int BK = BKT;   // slab depth of this instance
  typedef Stage<BM, BN, BKT> S;
  constexpr int WM = BM / 2, WN = BN / 2;              // wave tile
  constexpr int IB = WM / 16, JB = WN / 16;            // blocks per wave
  constexpr int kA = BM * BK / 4 / kThreads;           // A chunks per thread per slab
  constexpr int kB = BK * BN / 4 / kThreads;           // B chunks per thread per slab
  constexpr int kBRowChunks = BN / 4;
  __shared__ __attribute__((aligned(16))) S st[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int wm = (wave >> 1) * WM, wn = (wave & 1) * WN;

  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  int64_t item = tile_base + blockIdx.x;
  int split = 0;
  if constexpr (SPLIT) {
    const int64_t tiles = (int64_t)tiles_m * tiles_n;
    split = (int)(item / tiles);
    item -= split * tiles;
  }
  int tm, tn;
  hgemm::map_tile<8>(item, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // Global -> register assignment.
  // A slab BM x BK: chunk e -> row e / (BK / 4), column 4 (e % (BK / 4)).
  // B slab 16 x BN: chunk e -> row e / (BN / 4), column 4 (e % (BN / 4)).
  int arow[kA], acol[kA], brow[kB], bcol[kB], lA[kA], lB[kB];
#pragma unroll
  for (int i = 0; i < kA; ++i) {
    const int e = tid + kThreads * i;
    arow[i] = e / (BK / 4);
    acol[i] = (e % (BK / 4)) * 4;
    lA[i] = arow[i] * S::kAStride + acol[i];
  }
#pragma unroll
  for (int i = 0; i < kB; ++i) {
    const int e = tid + kThreads * i;
    brow[i] = e / kBRowChunks;
    bcol[i] = (e % kBRowChunks) * 4;
    lB[i] = brow[i] * S::kBStride + bcol[i];
  }

  f4 ra[kA], rb[kB];
  auto fetch = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kA; ++i) {
      if (EDGE) ra[i] = load4(p.A, p.lda, p.M, p.K, m0 + arow[i], k0 + acol[i]);
      else ra[i] = *(const f4*)(p.A + (int64_t)(m0 + arow[i]) * p.lda + k0 + acol[i]);
    }
#pragma unroll
    for (int i = 0; i < kB; ++i) {
      if (EDGE) rb[i] = load4(p.B, p.ldb, p.K, p.N, k0 + brow[i], n0 + bcol[i]);
      else rb[i] = *(const f4*)(p.B + (int64_t)(k0 + brow[i]) * p.ldb + n0 + bcol[i]);
    }
  };
  auto stash = [&](S& s) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kA; ++i) *(f4*)&s.a[lA[i]] = ra[i];
#pragma unroll
    for (int i = 0; i < kB; ++i) *(f4*)&s.b[lB[i]] = rb[i];
  };

  f4 acc[IB][JB];
#pragma unroll
  for (int i = 0; i < IB; ++i)
#pragma unroll
    for (int j = 0; j < JB; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  // Slabs t0 .. t1 - 1: all of K, or this workgroup's split-K range.
  int t0 = 0, t1 = (p.K + BK - 1) / BK;
  if constexpr (SPLIT) {
    t0 = split * p.sk.per;
    t1 = t0 + p.sk.per < t1 ? t0 + p.sk.per : t1;
  }
  fetch(t0 * BK);
  stash(st[0]);
  __syncthreads();

  for (int t = t0; t < t1; ++t) {
    const S& cur = st[(t - t0) & 1];
    if (t + 1 < t1) fetch((t + 1) * BK);

    // 16-deep sub-slabs q of the slab, k = 16 q + 4 g + s.
#pragma unroll
    for (int q = 0; q < BK / 16; ++q) {
      f4 av[IB];
#pragma unroll
      for (int i = 0; i < IB; ++i)
        av[i] = *(const f4*)&cur.a[(wm + 16 * i + r) * S::kAStride + 16 * q + 4 * g];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float bv[JB];
#pragma unroll
        for (int j = 0; j < JB; ++j) bv[j] = cur.b[(16 * q + 4 * g + s) * S::kBStride + wn + 16 * j + r];
#pragma unroll
        for (int i = 0; i < IB; ++i)
#pragma unroll
          for (int j = 0; j < JB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i][s], bv[j], acc[i][j], 0, 0, 0);
      }
    }

    if (t + 1 < t1) stash(st[(t + 1 - t0) & 1]);
    __syncthreads();
  }

  if constexpr (SPLIT) {
    float* ws = p.sk.ws + split * p.sk.split_stride;
#pragma unroll
    for (int i = 0; i < IB; ++i)
#pragma unroll
      for (int j = 0; j < JB; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          ws[(int64_t)(m0 + wm + 16 * i + 4 * g + v) * p.sk.ld + n0 + wn + 16 * j + r] =
              acc[i][j][v];
    return;
  }

  const float alpha = p.alpha, beta = p.beta;
#pragma unroll
  for (int i = 0; i < IB; ++i)
#pragma unroll
    for (int j = 0; j < JB; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + wm + 16 * i + 4 * g + v, n = n0 + wn + 16 * j + r;
        if (EDGE && (m >= p.M || n >= p.N)) continue;
        float* c = p.C + (int64_t)m * p.ldc + n;
        float out = alpha * acc[i][j][v];
        if (beta != 0.f) out = fmaf(beta, *c, out);
        *c = out;
      }
}

// Tile size for an M x N product: 128 x 128 while that gives every CU work,
// 64 x 64 below.
bool small_tiles(int M, int N, int cus) {
  const int64_t tiles128 = (int64_t)((M + 127) / 128) * ((N + 127) / 128);
  return tiles128 < cus;
}

template <int BM, int BN, bool EDGE, int BKT = 16>
hipError_t launch_tiled(const F32Args& a, hipStream_t stream) {
  const int64_t tiles = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  return launch_tiles((const void*)sgemm_mfma_kernel<BM, BN, EDGE, false, BKT>, a, tiles, kThreads,
                      0, stream);
}

}  // namespace

bool f32_mfma_fits(int M, int N, int K, const void* A, int64_t lda, const void* B, int64_t ldb,
                   const void* C, int64_t ldc) {
  return M % 64 == 0 && N % 64 == 0 && K % BK == 0 && aligned16(A) && aligned16(B) &&
         aligned16(C) && lda % 4 == 0 && ldb % 4 == 0 && ldc % 4 == 0;
}

hipError_t launch_f32_mfma(const F32Args& a, int cus, hipStream_t stream) {
  if (!small_tiles(a.M, a.N, cus) && a.M % 128 == 0 && a.N % 128 == 0)
    return launch_tiled<128, 128, false>(a, stream);
  // The small tiles run one workgroup per CU; 32-deep slabs halve their
  // barriers (1024^3: 28 us against 30 us).
  if (a.K % 32 == 0) return launch_tiled<64, 64, false, 32>(a, stream);
  return launch_tiled<64, 64, false>(a, stream);
}

hipError_t launch_f32_edge(const F32Args& a, int cus, hipStream_t stream) {
  if (small_tiles(a.M, a.N, cus)) return launch_tiled<64, 64, true>(a, stream);
  return launch_tiled<128, 128, true>(a, stream);
}

// Split-K partial products over 128 x 128 tiles: the full-tile kernel where
// the shape and alignment allow it, the edge kernel otherwise.
hipError_t launch_f32_partials(const F32Args& a, hipStream_t stream) {
  const int64_t tiles = (int64_t)((a.M + 127) / 128) * ((a.N + 127) / 128);
  const bool full = a.M % 128 == 0 && a.N % 128 == 0 &&
                    f32_mfma_fits(a.M, a.N, a.K, a.A, a.lda, a.B, a.ldb, a.C, a.ldc);
  const void* k = full ? (const void*)sgemm_mfma_kernel<128, 128, false, true>
                       : (const void*)sgemm_mfma_kernel<128, 128, true, true>;
  return launch_tiles(k, a, tiles * a.sk.splits, kThreads, 0, stream);
}

}  // namespace mi355gemm
