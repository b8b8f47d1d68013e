// 16-bit (fp16 or bf16) C = A * B^T for products with few output tiles: at
// most as many 64 x 64 tiles as CUs, where the full-tile kernels (128 x 128
// and larger) would leave most CUs idle, and the plain call has no memory for
// split-K partial sums.  Measured against the full tiles: 512 x 1024 x 8192
// 33.5 against 73.1 us, 1024^2 x 2048 15.3 against 23.1 us, 128^2 x 16384 31
// against 159 us.
//
// The split of K happens inside a workgroup instead (the idea of page 1, "第
// 6 章 Shared Memory & Tile", section 6.5.6, split-K, with the partial sums
// in LDS): one 256-thread workgroup per BT x BT tile of C (BT = 32, or 16
// while 32 x 32 tiles would leave CUs idle), four or sixteen times the
// workgroups of 64 x 64 tiles.
//
//  * K is walked in chunks of up to 256 (K a multiple of 128): every thread
//    loads its 16-byte pieces of the chunk's A and B rows into registers, the
//    next chunk's loads are issued before the current chunk's products, and
//    the chunk goes to LDS with rows padded by 16 bytes (row r at r * 528
//    bytes: the 16 rows a fragment read touches fall on 16 distinct groups of
//    four banks);
//  * wave w computes the whole tile over its quarter of every chunk (64 or
//    32 K values: one or two k-steps of v_mfma_f32_16x16x32_f16 per block);
//    lane l supplies row l % 16 and k = 8 (l / 16) .. + 7 of a step for both
//    operands (the full-tile kernels' k bijection);
//  * at the end the four partial tiles go to LDS and each thread adds its
//    outputs' four partials in the fixed order 0..3 (deterministic), rounds
//    once to the storage format and stores them.
//
// Preconditions (checked by the host): M, N multiples of 32, at most as many
// 64 x 64 tiles as CUs, K a multiple of 128, A, B and C 16-byte aligned with leading dimensions that are
// multiples of 8, no fused write-back.
#include "hgemm_tile.hpp"

namespace mi355gemm {
namespace hsmall {

using hgemm::f4;
using hgemm::h4;
using hgemm::h8;

constexpr int KC = 256;           // K per chunk
constexpr int kThreads = 256;
constexpr int kPitch = KC + 8;    // halves per LDS row

template <int BT, int FMT>
__global__ __launch_bounds__(kThreads, 1) void hgemm_small_kernel(Args16 p, int64_t tile_base) {
  constexpr int IB = BT / 16;                         // blocks per dimension
  constexpr int kRowChunks = KC / 8;                  // 16-byte pieces per chunk row
  constexpr int kLoads = BT * kRowChunks / kThreads;  // pieces per thread per operand
  constexpr int kRowStep = kThreads / kRowChunks;     // rows between a thread's pieces
  constexpr int kPartPitch = BT + 4;                  // floats per partial-tile row
  constexpr int kPart = BT * kPartPitch;              // floats per partial tile
  static_assert(kLoads >= 1 && BT % kRowStep == 0, "chunk pieces");
  static_assert(4 * kPart * 4 <= 2 * BT * kPitch * 2, "partial tiles fit over the chunk");
  __shared__ __attribute__((aligned(16))) half_t lds[2 * BT * kPitch];
  half_t* sa = lds;
  half_t* sb = lds + BT * kPitch;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  int tm, tn;
  hgemm::map_tile<8>(tile_base + blockIdx.x, p.M / BT, p.N / BT, tm, tn);
  const int m0 = tm * BT, n0 = tn * BT;

  // Piece u of this thread: row (tid / kRowChunks) + kRowStep u of the tile,
  // K values 8 (tid % kRowChunks) .. + 7 of the chunk.
  const int prow = tid / kRowChunks, pcol = 8 * (tid % kRowChunks);
  const half_t* a_src = p.A + (int64_t)(m0 + prow) * p.lda + pcol;
  const half_t* b_src = p.B + (int64_t)(n0 + prow) * p.ldb + pcol;
  h8 ra[kLoads], rb[kLoads];
  auto load_chunk = [&](int k0, int kc) __attribute__((always_inline)) {
    if (pcol < kc) {
#pragma unroll
      for (int u = 0; u < kLoads; ++u) {
        ra[u] = *(const h8*)(a_src + (int64_t)(kRowStep * u) * p.lda + k0);
        rb[u] = *(const h8*)(b_src + (int64_t)(kRowStep * u) * p.ldb + k0);
      }
    }
  };
  auto store_chunk = [&](int kc) __attribute__((always_inline)) {
    if (pcol < kc) {
#pragma unroll
      for (int u = 0; u < kLoads; ++u) {
        *(h8*)(sa + (prow + kRowStep * u) * kPitch + pcol) = ra[u];
        *(h8*)(sb + (prow + kRowStep * u) * kPitch + pcol) = rb[u];
      }
    }
  };

  f4 acc[IB][IB];
#pragma unroll
  for (int i = 0; i < IB; ++i)
#pragma unroll
    for (int j = 0; j < IB; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  int kc = p.K < KC ? p.K : KC;
  load_chunk(0, kc);
  for (int k0 = 0; k0 < p.K; k0 += KC) {
    store_chunk(kc);
    __builtin_amdgcn_s_waitcnt(hgemm::kWaitLgkm0);
    asm volatile("s_barrier" ::: "memory");
    const int next = k0 + KC;
    const int kc_next = p.K - next < KC ? p.K - next : KC;
    if (next < p.K) load_chunk(next, kc_next);
    // this wave's quarter of the chunk, in k-steps of 32
    const int kq = kc / 4;
    for (int s = 0; s < kq / 32; ++s) {
      const int kk = w * kq + 32 * s + 8 * g;
      h8 fa[IB], fb[IB];
#pragma unroll
      for (int i = 0; i < IB; ++i) fa[i] = *(const h8*)(sa + (16 * i + r) * kPitch + kk);
#pragma unroll
      for (int j = 0; j < IB; ++j) fb[j] = *(const h8*)(sb + (16 * j + r) * kPitch + kk);
#pragma unroll
      for (int i = 0; i < IB; ++i)
#pragma unroll
        for (int j = 0; j < IB; ++j) acc[i][j] = hgemm::mfma16<FMT>(fb[j], fa[i], acc[i][j]);
    }
    __builtin_amdgcn_s_waitcnt(hgemm::kWaitLgkm0);
    asm volatile("s_barrier" ::: "memory");   // the chunk's LDS is free again
    kc = kc_next;
  }

  // acc[i][j][v] is this wave's part of C[m0 + 16 i + r][n0 + 16 j + 4 g + v]:
  // the four partial tiles go to LDS (over the chunk), then each thread adds
  // the four partials of its outputs in wave order, rounds once and stores.
  float* part = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int i = 0; i < IB; ++i)
#pragma unroll
    for (int j = 0; j < IB; ++j)
      *(f4*)(part + w * kPart + (16 * i + r) * kPartPitch + 16 * j + 4 * g) = acc[i][j];
  __builtin_amdgcn_s_waitcnt(hgemm::kWaitLgkm0);
  asm volatile("s_barrier" ::: "memory");
  constexpr int kOut = BT * BT / kThreads;   // outputs per thread: 4 (BT = 32) or 1
  const int o = tid * kOut, row = o / BT, col = o % BT;
  float sum[kOut];
#pragma unroll
  for (int e = 0; e < kOut; ++e) sum[e] = part[row * kPartPitch + col + e];
#pragma unroll
  for (int v = 1; v < 4; ++v)
#pragma unroll
    for (int e = 0; e < kOut; ++e) sum[e] += part[v * kPart + row * kPartPitch + col + e];
  half_t* c = p.C + (int64_t)(m0 + row) * p.ldc + n0 + col;
  if constexpr (kOut == 4) {
    h4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = f32_to_word<FMT>(sum[e]);
    *(h4*)c = out;
  } else {
    *c = f32_to_word<FMT>(sum[0]);
  }
}

}  // namespace hsmall

bool f16_small_fits(int M, int N, int K, const void* A, int64_t lda, const void* B, int64_t ldb,
                    const void* C, int64_t ldc, int cus) {
  const int64_t tiles64 = (int64_t)((M + 63) / 64) * ((N + 63) / 64);
  return M % 32 == 0 && N % 32 == 0 && K % 128 == 0 && K > 0 && tiles64 <= cus &&
         aligned16(A) && aligned16(B) && aligned16(C) && lda % 8 == 0 && ldb % 8 == 0 &&
         ldc % 8 == 0;
}

hipError_t launch_f16_small(const Args16& a, int cus, hipStream_t stream) {
  const int64_t tiles32 = (int64_t)(a.M / 32) * (a.N / 32);
  if (tiles32 < cus) {
    const void* k = a.fmt == kFmtBF16 ? (const void*)hsmall::hgemm_small_kernel<16, kFmtBF16>
                                      : (const void*)hsmall::hgemm_small_kernel<16, kFmtF16>;
    return launch_tiles(k, a, 4 * tiles32, hsmall::kThreads, 0, stream);
  }
  const void* k = a.fmt == kFmtBF16 ? (const void*)hsmall::hgemm_small_kernel<32, kFmtBF16>
                                    : (const void*)hsmall::hgemm_small_kernel<32, kFmtF16>;
  return launch_tiles(k, a, tiles32, hsmall::kThreads, 0, stream);
}

}  // namespace mi355gemm
