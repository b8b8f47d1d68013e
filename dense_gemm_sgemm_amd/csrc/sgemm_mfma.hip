// fp32 SGEMM on the CDNA4 matrix cores: C = alpha * A * B + beta * C.
//
// Structure (prior art: the 2-D register-tiled, multi-stage SGEMM of the page
// "异步拷贝与 Hopper/Blackwell 新特性", section "cp.async 与多级流水"; the
// per-thread 8x8 FMA tile of that kernel becomes a per-wave 64x64 tile of
// v_mfma_f32_16x16x4_f32 products here):
//
//  * a 256-thread workgroup (4 waves, 2 x 2) owns a 128 x 128 tile of C;
//  * K is walked in slabs of 16; each slab of A (128 x 16) and B (16 x 128) is
//    fetched with 128-bit coalesced loads into registers one slab ahead and
//    written to the other half of a double-buffered LDS ring, so one barrier
//    per slab separates writers from readers;
//  * a wave's 64 x 64 tile is 4 x 4 blocks of 16 x 16; per slab each block
//    takes 4 MFMAs (K = 4 each).  Lane l = 16 g + r feeds the MFMA row/column
//    r and, in MFMA step s, the slab column k = 4 g + s: the same bijection for
//    both operands, so the four steps sum all 16 k of the slab.  With that
//    mapping a lane's four A values are one 16-byte LDS read;
//  * epilogue: alpha * acc (+ beta * C when beta != 0) straight from the
//    accumulators (lane l, register v holds row 4 g + v, column r of a block).
//
// Host-checked preconditions (f32_mfma_fits): M % 128 == N % 128 == K % 16 ==
// 0, 16-byte aligned A, B, C and leading dimensions that are multiples of 4.
#include "internal.h"

namespace mi355gemm {
namespace {

constexpr int BM = 128, BN = 128, BK = 16;
constexpr int kThreads = 256;
constexpr int WM = 64, WN = 64;          // wave tile
constexpr int kAStride = BK + 4;         // floats per A row in LDS
constexpr int kBStride = BN + 4;         // floats per B row in LDS: 4 rows apart = 16 banks apart

typedef float f4 __attribute__((ext_vector_type(4)));

struct Stage {
  float a[BM * kAStride];
  float b[BK * kBStride];
};

__global__ __launch_bounds__(kThreads, 2) void sgemm_mfma_kernel(F32Args p, int64_t tile_base) {
  __shared__ __attribute__((aligned(16))) Stage st[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int wm = (wave >> 1) * WM, wn = (wave & 1) * WN;

  const int64_t tile = tile_base + blockIdx.x;
  const int tiles_n = p.N / BN;
  const int m0 = (int)(tile / tiles_n) * BM, n0 = (int)(tile % tiles_n) * BN;

  // Global -> register assignment: two float4 of A and two of B per thread.
  // A slab 128 x 16: chunk e -> row e / 4, column 4 (e % 4).
  // B slab 16 x 128: chunk e -> row e / 32, column 4 (e % 32).
  const float* gA[2];
  const float* gB[2];
  int lA[2], lB[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = tid + kThreads * i;
    const int ar = e >> 2, ac = (e & 3) * 4;
    gA[i] = p.A + (int64_t)(m0 + ar) * p.lda + ac;
    lA[i] = ar * kAStride + ac;
    const int br = e >> 5, bc = (e & 31) * 4;
    gB[i] = p.B + (int64_t)br * p.ldb + n0 + bc;
    lB[i] = br * kBStride + bc;
  }
  const int64_t bstep = (int64_t)BK * p.ldb;

  f4 ra[2], rb[2];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      ra[i] = *(const f4*)(gA[i] + k0);
      rb[i] = *(const f4*)(gB[i] + (int64_t)(k0 / BK) * bstep);
    }
  };
  auto stash = [&](Stage& s) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      *(f4*)&s.a[lA[i]] = ra[i];
      *(f4*)&s.b[lB[i]] = rb[i];
    }
  };

  f4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  const int nk = p.K / BK;
  fetch(0);
  stash(st[0]);
  __syncthreads();

  for (int t = 0; t < nk; ++t) {
    const Stage& cur = st[t & 1];
    if (t + 1 < nk) fetch((t + 1) * BK);

    f4 av[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) av[i] = *(const f4*)&cur.a[(wm + 16 * i + r) * kAStride + 4 * g];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float bv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = cur.b[(4 * g + s) * kBStride + wn + 16 * j + r];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i][s], bv[j], acc[i][j], 0, 0, 0);
    }

    if (t + 1 < nk) stash(st[(t + 1) & 1]);
    __syncthreads();
  }

  const float alpha = p.alpha, beta = p.beta;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float* c = p.C + (int64_t)(m0 + wm + 16 * i + 4 * g + v) * p.ldc + n0 + wn + 16 * j + r;
        float out = alpha * acc[i][j][v];
        if (beta != 0.f) out = fmaf(beta, *c, out);
        *c = out;
      }
}

}  // namespace

bool f32_mfma_fits(int M, int N, int K, const void* A, int64_t lda, const void* B, int64_t ldb,
                   const void* C, int64_t ldc) {
  return M % BM == 0 && N % BN == 0 && K % BK == 0 && aligned16(A) && aligned16(B) &&
         aligned16(C) && lda % 4 == 0 && ldb % 4 == 0 && ldc % 4 == 0;
}

hipError_t launch_f32_mfma(const F32Args& a, hipStream_t stream) {
  const int64_t tiles = (int64_t)(a.M / BM) * (a.N / BN);
  return launch_tiles((const void*)sgemm_mfma_kernel, a, tiles, kThreads, 0, stream);
}

}  // namespace mi355gemm
