// fp16 C = A * B^T (A[M][K], B[N][K] row-major) on the CDNA4 matrix cores,
// fp32 accumulation, fp16 output rounded to nearest even.
//
// Prior art: the step-by-step A800 kernel of the page "从零开始的 AI Infra:
// 算子基础与GPU架构" -- shared-memory tiles (section 3), tensor-core fragments
// (section 7), 16-byte loads (sections 8-9), a multi-stage buffer ring
// (sections 10-12), B consumed in its stored [n][k] layout (section 19) and a
// XOR-swizzled, padding-free shared layout (section 21).  Re-done for gfx950:
//
//  * a 512-thread workgroup (8 waves, 2 along M x 4 along N) owns a 256 x 256
//    tile of C; each wave owns 128 x 64 = 8 x 4 blocks of 16 x 16;
//  * K is walked in slabs of 64.  A slab of A and of B (256 rows x 128 bytes
//    each) is fetched with 128-bit coalesced loads (8 lanes per row) into
//    registers one slab ahead, then written to the other half of a double
//    buffered LDS ring (2 x 64 KiB): one barrier per slab;
//  * LDS rows are 128 bytes = 8 chunks of 16 bytes, no padding.  Chunk c of
//    row r is stored at chunk c ^ f(r), f(r) = (r mod 8) xor (bit 3 of r):
//    the 16 rows that one ds_read_b128 of an MFMA operand touches then cover
//    every bank group once, both for 32 and for 64 four-byte banks;
//  * the tile product is v_mfma_f32_16x16x32_f16.  Both operands are K-major
//    16 x 32 fragments, one 16-byte LDS read per lane: lane l = 16 g + r
//    supplies row r and k = 8 g .. 8 g + 7 of the 32 -- the same k bijection
//    for both operands, so each MFMA sums all 32;
//  * B is passed as the MFMA's first operand, so a lane's four accumulator
//    registers hold four consecutive columns n of one row m: the epilogue
//    rounds them to half and stores 8 bytes per lane.
//
// Host-checked preconditions (f16_mfma_fits): M % 256 == N % 256 == K % 64 ==
// 0, 16-byte aligned A, B, C and leading dimensions that are multiples of 8.
#include "internal.h"

namespace mi355gemm {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kThreads = 512;
constexpr int WM = 128, WN = 64;          // wave tile
constexpr int kChunks = BK / 8;           // 16-byte chunks per LDS row
constexpr int kLoads = BM * kChunks / kThreads;  // 16-byte loads per thread per operand

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

struct Stage {
  h8 a[BM * kChunks];
  h8 b[BN * kChunks];
};

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__global__ __launch_bounds__(kThreads) void hgemm_nt_mfma_kernel(F16Args p, int64_t tile_base) {
  __shared__ Stage st[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int wm = (wave >> 2) * WM, wn = (wave & 3) * WN;

  const int64_t tile = tile_base + blockIdx.x;
  const int tiles_n = p.N / BN;
  const int m0 = (int)(tile / tiles_n) * BM, n0 = (int)(tile % tiles_n) * BN;

  // Global -> register -> LDS assignment: chunk e = tid + 512 i of a slab is
  // row e / 8, chunk e % 8.
  const h8* gA[kLoads];
  const h8* gB[kLoads];
  int lds[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int e = tid + kThreads * i;
    const int row = e >> 3, c = e & 7;
    gA[i] = (const h8*)(p.A + (int64_t)(m0 + row) * p.lda + 8 * c);
    gB[i] = (const h8*)(p.B + (int64_t)(n0 + row) * p.ldb + 8 * c);
    lds[i] = row * kChunks + (c ^ swz(row));
  }

  h8 ra[kLoads], rb[kLoads];
  auto fetch = [&](int k0) {
    const int kc = k0 / 8;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      ra[i] = gA[i][kc];
      rb[i] = gB[i][kc];
    }
  };
  auto stash = [&](Stage& s) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      s.a[lds[i]] = ra[i];
      s.b[lds[i]] = rb[i];
    }
  };

  // Operand read offsets: row (wm | wn) + 16 * block + r, chunk (4 kk + g) ^ f(r).
  const int fr = swz(r);
  const int a_base = (wm + r) * kChunks, b_base = (wn + r) * kChunks;
  const int pc0 = (0 + g) ^ fr, pc1 = (4 + g) ^ fr;

  f4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  const int nk = p.K / BK;
  fetch(0);
  stash(st[0]);
  __syncthreads();

  for (int t = 0; t < nk; ++t) {
    const Stage& cur = st[t & 1];
    if (t + 1 < nk) fetch((t + 1) * BK);

#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int pc = kk ? pc1 : pc0;
      h8 av[8], bv[4];
#pragma unroll
      for (int i = 0; i < 8; ++i) av[i] = cur.a[a_base + 16 * kChunks * i + pc];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = cur.b[b_base + 16 * kChunks * j + pc];
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bv[j], av[i], acc[i][j], 0, 0, 0);
    }

    if (t + 1 < nk) stash(st[(t + 1) & 1]);
    __syncthreads();
  }

  // acc[i][j][v] = C[m0 + wm + 16 i + r][n0 + wn + 16 j + 4 g + v].
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    half_t* crow = p.C + (int64_t)(m0 + wm + 16 * i + r) * p.ldc + n0 + wn + 4 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h4 o;
#pragma unroll
      for (int v = 0; v < 4; ++v) o[v] = (half_t)acc[i][j][v];
      *(h4*)(crow + 16 * j) = o;
    }
  }
}

}  // namespace

bool f16_mfma_fits(int M, int N, int K, const void* A, int64_t lda, const void* B, int64_t ldb,
                   const void* C, int64_t ldc) {
  return M % BM == 0 && N % BN == 0 && K % BK == 0 && aligned16(A) && aligned16(B) &&
         aligned16(C) && lda % 8 == 0 && ldb % 8 == 0 && ldc % 8 == 0;
}

hipError_t launch_f16_mfma(const F16Args& a, hipStream_t stream) {
  const int64_t tiles = (int64_t)(a.M / BM) * (a.N / BN);
  return launch_tiles((const void*)hgemm_nt_mfma_kernel, a, tiles, kThreads, 0, stream);
}

}  // namespace mi355gemm
