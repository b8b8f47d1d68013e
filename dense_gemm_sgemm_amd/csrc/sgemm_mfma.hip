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
// Large products whose K is a multiple of 64 take the streaming kernel
// further down instead (direct-to-LDS copies by dedicated copying waves).
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

#include <utility>

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

// ---------------------------------------------------------------------------
// The streaming kernel for large fp32 products (M, N multiples of 128 with
// at least as many 128 x 128 tiles as CUs, K a multiple of 64; or, RAG, any
// M, N >= 128 and K a multiple of 4): one persistent 512-thread workgroup per
// CU walks its 128 x 128 tiles as one stream of 64-deep K slabs.
//
//  * waves 0-3 (one per SIMD) compute: each owns 64 x 64 of the tile, 16
//    blocks of v_mfma_f32_16x16x4_f32 with 16 accumulators in rotation;
//  * waves 4-7 only copy -- the producer / consumer split of the page "第 6 章
//    Shared Memory & Tile" (section 6.10.1), with the workgroup barrier in
//    place of mbarriers: every slab of A (128 x 64) and B (64 x 128) goes
//    global -> LDS with global_load_lds_dwordx4 into a two-stage ring
//    (2 x 64 KiB), one barrier per slab.  A copying wave shares its SIMD with
//    a computing wave, so its copies carry no vector address arithmetic: the
//    source is a wave-uniform base in scalar registers plus a lane offset
//    computed once (a vector add per copy waits behind the other wave's
//    matrix instructions and stalls the stream);
//  * LDS layouts: A row a (64 floats, 16 chunks of 16 bytes) holds logical
//    chunk c at position c ^ (a & 15); B row k (128 floats, 32 chunks) holds
//    logical chunk c at position c ^ (4 ((k >> 2) & 3)).  One copy fills 4 A
//    rows or 2 B rows (1 KiB, lane i writing position i); the permutation is
//    realised by the global addresses the lanes load;
//  * operands: per 16-deep part q of a slab, lane l = 16 g + r reads A row
//    r of block i at k = 16 q + 4 g .. + 3 (one 16-byte read) and B column r
//    of block j at k = 16 q + 4 g + s, s = 0..3 (four 4-byte reads); MFMA
//    step s takes element s of both -- the k bijection of the register-staged
//    kernel above, so both kernels sum in the same order and agree bit for
//    bit.  Both reads are free of bank conflicts with these layouts;
//  * B is the MFMA's first operand, so a lane's accumulator quad holds four
//    consecutive columns of one row of C: one 16-byte store per block;
//  * the barrier of slab t sits after 240 of its 256 MFMAs: before it every
//    computing wave has read all of slab t and the copying waves have landed
//    slab t + 1; after it they copy slab t + 2 into slab t's stage while the
//    computing waves read the first fragments of slab t + 1;
//  * RAG (the boundary rule of page 1, "第 6 章 Shared Memory & Tile",
//    exercise 7 of section 6.9: arbitrary M, N, K): the last tile row and
//    column are shifted back to end at M and N, so every row a copy reads
//    exists, and store only the rows and columns no earlier tile owns; the
//    last slab of a K that is not a multiple of 64 copies its chunks and rows
//    past K from the last ones inside (in bounds), and the copying wave that
//    wrote them zeroes them in LDS before the barrier that publishes the slab
//    (whole 16-byte chunks, since K is a multiple of 4).
namespace stream {
constexpr int BM = 128, BN = 128, BKS = 64;
constexpr int kStageA = BM * BKS * 4, kStageB = BKS * BN * 4;   // bytes
constexpr int kStage = kStageA + kStageB;
constexpr int kThreads = 512;          // 4 computing + 4 copying waves
constexpr int kCopiers = 4;
constexpr int kCopies = 64 / kCopiers;   // copy instructions per copying wave per slab

typedef __attribute__((address_space(3))) void lds_void_t;

using hgemm::static_for;   // compile-time loop indices (hgemm_tile.hpp)

// A wave-uniform pointer, held in scalar registers.
__device__ __forceinline__ const char* uniform_ptr(const char* q) {
  const uint64_t v = (uint64_t)q;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(((uint64_t)hi << 32) | lo);
}

// One direct-to-LDS copy: lane i loads 16 bytes from sbase + voff and they
// land at dst + 16 i.  Written out so that the scalar-base form is the one
// issued.  M0 (the LDS destination, read when the copy issues) is set here
// one wait state ahead of the copy, as the hardware requires, and restored
// after it, since the compiler reserves M0 and does not track a change made
// inside an asm statement.  Completion is the caller's explicit vmcnt wait.
__device__ __forceinline__ void copy16(const char* sbase, uint32_t voff, lds_void_t* dst) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(m0v)
      : "memory");
}

constexpr int kWaitVmLgkm0 = 0x0070;   // s_waitcnt vmcnt(0) lgkmcnt(0)
constexpr int kWaitLgkm0 = 0xC07F;     // s_waitcnt lgkmcnt(0)

template <bool RAG>
__global__ __launch_bounds__(kThreads, 2) void sgemm_stream_kernel(F32Args p, int64_t tiles) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * kStage];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tiles_m = RAG ? (p.M + BM - 1) / BM : p.M / BM;
  const int tiles_n = RAG ? (p.N + BN - 1) / BN : p.N / BN;
  const int64_t stride = gridDim.x;
  const int ntiles = (int)((tiles - blockIdx.x + stride - 1) / stride);
  const int nk = RAG ? (p.K + BKS - 1) / BKS : p.K / BKS;
  const int kv = p.K - (nk - 1) * BKS;   // K values in the last slab (RAG: 4 .. 64)
  const int total = ntiles * nk;         // slabs of this workgroup's stream
  // Tile jt of this workgroup: origin (m0, n0) of the rows and columns it
  // computes, and (mlo, nlo), the first it stores (RAG: the last tile row
  // and column start at M - 128 and N - 128 and leave the rows and columns
  // of the tile before them to it).
  auto origin = [&](int jt, int& m0, int& n0, int& mlo, int& nlo) __attribute__((always_inline)) {
    int tm, tn;
    hgemm::map_tile<8>(blockIdx.x + (int64_t)jt * stride, tiles_m, tiles_n, tm, tn);
    mlo = tm * BM;
    nlo = tn * BN;
    m0 = RAG && mlo > p.M - BM ? p.M - BM : mlo;
    n0 = RAG && nlo > p.N - BN ? p.N - BN : nlo;
  };
  // Slab it of the stream reaches past K.
  auto tail_slab = [&](int it) __attribute__((always_inline)) {
    return RAG && kv < BKS && it % nk == nk - 1;
  };

  if (wave >= 4) {
    // Copying wave cw issues A copies c = cw + 4 i (rows 4 c .. 4 c + 3; lane
    // l writes row 4 c + l / 16 at position l % 16, so it loads logical chunk
    // (l % 16) ^ ((4 c + l / 16) & 15), where c & 3 = cw) and B copies
    // c = cw + 4 i (rows 2 c, 2 c + 1; lane l writes row 2 c + l / 32 at
    // position l % 32, logical chunk (l % 32) ^ (4 ((c >> 1) & 3)), where
    // (c >> 1) & 3 = ((cw >> 1) + 2 i) & 3).
    const int cw = wave - 4;
    const uint32_t la = (uint32_t)((lane >> 4) * p.lda * 4);
    const uint32_t lb = (uint32_t)((lane >> 5) * p.ldb * 4);
    const uint32_t offA = la + 16 * ((lane & 15) ^ ((4 * cw + (lane >> 4)) & 15));
    const uint32_t offB0 = lb + 16 * ((lane & 31) ^ (4 * ((cw >> 1) & 3)));
    const uint32_t offB1 = lb + 16 * ((lane & 31) ^ (4 * (((cw >> 1) + 2) & 3)));
    // RAG: this lane's A chunk (the same logical chunk in every A copy of the
    // wave) lies past K in the last slab when 4 lc >= kv; it then loads the
    // slab's last chunk inside K instead.
    const int lcA = (lane & 15) ^ ((4 * cw + (lane >> 4)) & 15);
    const bool a_past = 4 * lcA >= kv;
    const uint32_t offA_tail = a_past ? la + 16 * (kv / 4 - 1) : offA;
    auto copy_slab = [&](int it) __attribute__((always_inline)) {
      int m0, n0, mlo, nlo;
      origin(it / nk, m0, n0, mlo, nlo);
      const int t = it % nk;
      const bool tail = tail_slab(it);
      const char* a = (const char*)(p.A + (int64_t)m0 * p.lda + t * BKS);
      const char* b = (const char*)(p.B + (int64_t)(t * BKS) * p.ldb + n0);
      unsigned char* st = lds + (it & 1) * kStage;
      const uint32_t oa = tail ? offA_tail : offA;
#pragma unroll
      for (int i = 0; i < kCopies / 2; ++i) {
        const int c = cw + kCopiers * i;
        copy16(uniform_ptr(a + (int64_t)c * 16 * p.lda), oa, (lds_void_t*)(st + c * 1024));
      }
#pragma unroll
      for (int i = 0; i < kCopies / 2; ++i) {
        const int c = cw + kCopiers * i;
        // B rows 2 c, 2 c + 1 of the slab (in the last slab, rows kv - 2 and
        // kv - 1 stand in for rows past K)
        const int row = tail && 2 * c + 1 >= kv ? kv - 2 : 2 * c;
        copy16(uniform_ptr(b + (int64_t)row * 4 * p.ldb), (i & 1) ? offB1 : offB0,
               (lds_void_t*)(st + kStageA + c * 1024));
      }
    };
    // RAG: after the last slab has landed, this wave's chunks and rows past K
    // become zeros (each lane rewrites the 16 bytes its own copies wrote).
    auto zero_tail = [&](int it) __attribute__((always_inline)) {
      unsigned char* st = lds + (it & 1) * kStage;
#pragma unroll
      for (int i = 0; i < kCopies / 2; ++i) {
        const int c = cw + kCopiers * i;
        if (a_past) *(f4*)(st + c * 1024 + 16 * lane) = f4{0.f, 0.f, 0.f, 0.f};
        if (2 * c + (lane >> 5) >= kv)
          *(f4*)(st + kStageA + c * 1024 + 16 * lane) = f4{0.f, 0.f, 0.f, 0.f};
      }
    };
    // Slab 0 before the opening barrier; then, after the barrier of slab
    // t - 1 (the opening one for t = 0), slab t + 1 into the stage slab t - 1
    // used, landed before the barrier of slab t.
    copy_slab(0);
    __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0);
    if constexpr (RAG) {
      if (tail_slab(0)) zero_tail(0);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    }
    asm volatile("s_barrier" ::: "memory");
    for (int it = 0; it < total; ++it) {
      if (it + 1 < total) copy_slab(it + 1);
      __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0);
      if constexpr (RAG) {
        if (it + 1 < total && tail_slab(it + 1)) zero_tail(it + 1);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      }
      asm volatile("s_barrier" ::: "memory");
    }
    return;
  }

  const int g = lane >> 4, r = lane & 15;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  f4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};
  // Two register sets of one 16-deep part: A blocks (16 bytes each) and the
  // B values (s, j).
  f4 av[2][4];
  float bv[2][4][4];
  // Read q of part `part` (q < 4: A block q; else B value ((q - 4) / 4, (q - 4) % 4)).
  auto read_one = [&](const unsigned char* st, int set, int part, int q) __attribute__((always_inline)) {
    if (q < 4) {
      const int row = wm + 16 * q + r;   // row & 15 == r
      av[set][q] = *(const f4*)(st + row * 256 + (((4 * part + g) ^ r) * 16));
    } else {
      const int s = (q - 4) >> 2, j = (q - 4) & 3;
      const int k = 16 * part + 4 * g + s;   // (k >> 2) & 3 == g
      const int chunk = ((wn + 16 * j) >> 2) + (r >> 2);
      bv[set][s][j] = *(const float*)(st + kStageA + k * 512 + (4 * (chunk ^ (4 * g)) + (r & 3)) * 4);
    }
  };

  asm volatile("s_barrier" ::: "memory");   // slab 0 has landed
#pragma unroll
  for (int q = 0; q < 20; ++q) read_one(lds, 0, 0, q);

  // One slab in issue order: MFMA m of 256 is part m / 64, step s, block
  // (i, j); the reads of part q + 1 go out during part q (one per three
  // MFMAs), the barrier before MFMA 240, the next slab's first part after it.
  auto slab = [&](int gs) __attribute__((always_inline)) {
    const unsigned char* cur = lds + (gs & 1) * kStage;
    const unsigned char* nxt = lds + ((gs + 1) & 1) * kStage;
    __builtin_amdgcn_sched_barrier(0);
    static_for<256>([&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      constexpr int part = m / 64, s = (m % 64) / 16, i = (m % 16) / 4, j = m % 4;
      if constexpr (m == 240) {
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      }
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(bv[part & 1][s][j], av[part & 1][i][s],
                                                       acc[i][j], 0, 0, 0);
      if constexpr (part < 3 && (m % 64) % 3 == 0 && (m % 64) / 3 < 20)
        read_one(cur, (part + 1) & 1, part + 1, (m % 64) / 3);
      if constexpr (m >= 240) {
        read_one(nxt, 0, 0, m - 240);
        if constexpr (m - 240 < 4) read_one(nxt, 0, 0, 16 + (m - 240));
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // acc[i][j][v] is C[m0 + wm + 16 i + r][n0 + wn + 16 j + 4 g + v].
  const float alpha = p.alpha, beta = p.beta;
  int gs = 0;
  for (int jt = 0; jt < ntiles; ++jt) {
    int m0, n0, mlo, nlo;
    origin(jt, m0, n0, mlo, nlo);
    for (int t = 0; t < nk; ++t, ++gs) slab(gs);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = m0 + wm + 16 * i + r, n = n0 + wn + 16 * j + 4 * g;
        float* c = p.C + (int64_t)m * p.ldc + n;
        const f4 out0 = alpha * acc[i][j];
        if (!RAG || (m >= mlo && n >= nlo)) {
          f4 out = out0;
          if (beta != 0.f) {
            const f4 old = *(const f4*)c;
#pragma unroll
            for (int v = 0; v < 4; ++v) out[v] = fmaf(beta, old[v], out[v]);
          }
          *(f4*)c = out;
        } else if (m >= mlo && n + 4 > nlo) {
          // a quad that straddles the first column this tile owns
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            if (n + v < nlo) continue;
            float o = out0[v];
            if (beta != 0.f) o = fmaf(beta, c[v], o);
            c[v] = o;
          }
        }
        acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};
      }
  }
}
}  // namespace stream

// The streaming kernel for the products the 128 x 128 kernel does not take
// (M, N multiples of 64 with fewer 128 x 128 tiles than CUs, or not multiples
// of 128; K a multiple of 64): 64 x 64 tiles, so that mid-size products give
// every CU work, with the structure of the kernel above -- one
// persistent 512-thread workgroup per CU, 4 computing and 4 copying waves,
// direct-to-LDS copies of 64-deep slabs in the scalar-base form.  A 64 x 64
// tile split four ways would leave each wave 4 accumulators, too few to cover
// the matrix instruction's latency; instead each computing wave w owns the
// whole tile (16 accumulators) for the 16-deep part w of every slab, and at
// the end of the tile the four partial tiles are added in LDS in the fixed
// order w = 0, 1, 2, 3.
//
//  * LDS: three slab stages (A 64 x 64 and B 64 x 64, 32 KiB each stage),
//    then 4 x 16 KiB of partial tiles.  A row a holds logical chunk c at
//    c ^ (a & 15), B row k at c ^ (4 ((k >> 2) & 3)), partial-tile row a at
//    c ^ (a & 15): every read and write of them is free of bank conflicts;
//  * barrier B_t opens slab t: slab t + 1 has landed, and every computing
//    wave has read slab t (its fragments went to registers during slab
//    t - 1), so the copying waves refill slab t's stage with slab t + 3;
//  * during slab t a computing wave runs its 64 MFMAs on slab t and reads
//    its part of slab t + 1;
//  * after a tile's last slab each computing wave stores its partial tile,
//    all eight waves meet (the copying waves count the slabs of each tile),
//    and computing wave w adds the four partials of rows 16 w .. 16 w + 15
//    and writes them to C, 16 bytes per lane.
namespace stream64 {
constexpr int BT = 64, BKS = 64;
constexpr int kStage = 2 * BT * BKS * 4;    // A and B of one slab: 32 KiB
constexpr int kStages = 3;
constexpr int kPartial = BT * BT * 4;       // one wave's partial tile: 16 KiB
constexpr int kLds = kStages * kStage + 4 * kPartial;
constexpr int kThreads = 512;
constexpr int kCopies = 8;                  // per copying wave per slab: 4 of A, 4 of B
static_assert(kLds <= 160 * 1024, "LDS");
static_assert(kCopies < 16, "a vmcnt immediate below 16");

__global__ __launch_bounds__(kThreads, 2) void sgemm_stream64_kernel(F32Args p, int64_t tiles) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kLds];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tiles_m = p.M / BT, tiles_n = p.N / BT;
  const int64_t stride = gridDim.x;
  const int ntiles = (int)((tiles - blockIdx.x + stride - 1) / stride);
  const int nk = p.K / BKS;
  const int total = ntiles * nk;
  auto origin = [&](int jt, int& m0, int& n0) __attribute__((always_inline)) {
    int tm, tn;
    hgemm::map_tile<8>(blockIdx.x + (int64_t)jt * stride, tiles_m, tiles_n, tm, tn);
    m0 = tm * BT;
    n0 = tn * BT;
  };
  unsigned char* partials = lds + kStages * kStage;

  if (wave >= 4) {
    // Copy c (0..15) of A fills rows 4 c .. 4 c + 3 and copy c of B rows
    // 4 c .. 4 c + 3 (rows of 256 bytes; lane l writes row 4 c + l / 16 at
    // position l % 16).  Copying wave cw issues c = cw + 4 i, so c & 3 = cw
    // and one lane offset serves all its copies of each operand.
    const int cw = wave - 4;
    const int row = lane >> 4, pos = lane & 15;
    const uint32_t offA = (uint32_t)(row * p.lda * 4) + 16 * (pos ^ ((4 * cw + row) & 15));
    const uint32_t offB = (uint32_t)(row * p.ldb * 4) + 16 * (pos ^ (4 * (cw & 3)));
    auto copy_slab = [&](int it) __attribute__((always_inline)) {
      int m0, n0;
      origin(it / nk, m0, n0);
      const int t = it % nk;
      const char* a = (const char*)(p.A + (int64_t)m0 * p.lda + t * BKS);
      const char* b = (const char*)(p.B + (int64_t)(t * BKS) * p.ldb + n0);
      unsigned char* st = lds + (it % kStages) * kStage;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = cw + 4 * i;
        stream::copy16(stream::uniform_ptr(a + (int64_t)c * 16 * p.lda), offA,
                       (stream::lds_void_t*)(st + c * 1024));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = cw + 4 * i;
        stream::copy16(stream::uniform_ptr(b + (int64_t)c * 16 * p.ldb), offB,
                       (stream::lds_void_t*)(st + BT * BKS * 4 + c * 1024));
      }
    };
    // Slabs 0 and 1 before the opening barrier, slab 2 after it; after B_t
    // slab t + 3.  Before B_t slab t + 1 must have landed: all copies but
    // the latest slab's (slab t + 2, if it exists) are complete.
    copy_slab(0);
    if (total > 1) copy_slab(1);
    __builtin_amdgcn_s_waitcnt(stream::kWaitVmLgkm0);
    asm volatile("s_barrier" ::: "memory");
    if (total > 2) copy_slab(2);
    for (int it = 0; it < total; ++it) {
      if (it + 2 < total) {
        // vmcnt(kCopies) lgkmcnt(0): slab it + 2's copies may stay in flight
        __builtin_amdgcn_s_waitcnt(0x0070 | kCopies);
      } else {
        __builtin_amdgcn_s_waitcnt(stream::kWaitVmLgkm0);
      }
      asm volatile("s_barrier" ::: "memory");   // B_it
      if (it + 3 < total) copy_slab(it + 3);
      if (it % nk == nk - 1) asm volatile("s_barrier" ::: "memory");   // the tile's reduction
    }
    __builtin_amdgcn_s_waitcnt(stream::kWaitVmLgkm0);
    return;
  }

  const int g = lane >> 4, r = lane & 15;
  const int w = wave;   // this wave's 16-deep part of every slab
  f4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};
  f4 av[2][4];          // set 0: the current slab, set 1: the next
  float bv[2][4][4];
  // Read q of this wave's part of a slab: q < 4 A block q (row 16 q + r,
  // k = 16 w + 4 g .. + 3), else B value (s, j) = ((q - 4) / 4, (q - 4) % 4)
  // (row k = 16 w + 4 g + s, column 16 j + r).
  auto read_one = [&](const unsigned char* st, int set, int q) __attribute__((always_inline)) {
    if (q < 4) {
      const int row = 16 * q + r;
      av[set][q] = *(const f4*)(st + row * 256 + (((4 * w + g) ^ r) * 16));
    } else {
      const int s = (q - 4) >> 2, j = (q - 4) & 3;
      const int k = 16 * w + 4 * g + s;   // (k >> 2) & 3 == g
      const int chunk = 4 * j + (r >> 2);
      bv[set][s][j] = *(const float*)(st + BT * BKS * 4 + k * 256 + (4 * (chunk ^ (4 * g)) + (r & 3)) * 4);
    }
  };

  asm volatile("s_barrier" ::: "memory");   // slabs 0 and 1 have landed
#pragma unroll
  for (int q = 0; q < 20; ++q) read_one(lds, 0, q);

  const float alpha = p.alpha, beta = p.beta;
  int gs = 0;
  for (int jt = 0; jt < ntiles; ++jt) {
    int m0, n0;
    origin(jt, m0, n0);
    for (int t = 0; t < nk; ++t, ++gs) {
      __builtin_amdgcn_s_waitcnt(stream::kWaitLgkm0);
      asm volatile("s_barrier" ::: "memory");   // B_gs
      const unsigned char* nxt = lds + ((gs + 1) % kStages) * kStage;
      __builtin_amdgcn_sched_barrier(0);
      hgemm::static_for<64>([&](auto mc) __attribute__((always_inline)) {
        constexpr int m = decltype(mc)::value;
        constexpr int s = m / 16, i = (m % 16) / 4, j = m % 4;
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(bv[0][s][j], av[0][i][s], acc[i][j], 0, 0, 0);
        if constexpr (m % 3 == 0 && m / 3 < 20) read_one(nxt, 1, m / 3);
        __builtin_amdgcn_sched_barrier(0);
      });
      // the next slab's fragments become the current set (register moves:
      // a set index that changes from slab to slab would need indexed
      // register access)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[0][i] = av[1][i];
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[0][i][j] = bv[1][i][j];
      }
    }
    // acc[i][j][v] is this wave's part of C[m0 + 16 i + r][n0 + 16 j + 4 g + v].
    unsigned char* mine = partials + w * kPartial;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        *(f4*)(mine + (16 * i + r) * 256 + (((4 * j + g) ^ r) * 16)) = acc[i][j];
        acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};
      }
    __builtin_amdgcn_s_waitcnt(stream::kWaitLgkm0);
    asm volatile("s_barrier" ::: "memory");   // the tile's reduction
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = 16 * w + 4 * u + g, chunk = r;
      const int off = row * 256 + ((chunk ^ (row & 15)) * 16);
      f4 sum = *(const f4*)(partials + off);
#pragma unroll
      for (int v = 1; v < 4; ++v) sum += *(const f4*)(partials + v * kPartial + off);
      const int m = m0 + row, n = n0 + 4 * chunk;
      float* c = p.C + (int64_t)m * p.ldc + n;
      {
        f4 out = alpha * sum;
        if (beta != 0.f) {
          const f4 old = *(const f4*)c;
#pragma unroll
          for (int e = 0; e < 4; ++e) out[e] = fmaf(beta, old[e], out[e]);
        }
        *(f4*)c = out;
      }
    }
  }
}
}  // namespace stream64

// Products too small to give every CU a 64 x 64 tile (256^3: 16 tiles).  One
// 256-thread workgroup per BT x BT tile of C (BT = 32, or 16 when even 32 x 32
// tiles leave CUs idle), four or sixteen times as many workgroups as 64 x 64
// tiles; each of its four waves computes the whole tile over its own quarter
// of every K chunk, so the tile's K is walked four ways at once (the per-wave
// split of the pages' split-K, section 6.5.6 of page 1, inside one
// workgroup), and the four partial tiles are added through LDS in the fixed
// order 0, 1, 2, 3 (results repeat bitwise).
//
//  * K is taken in chunks of up to 256 (a multiple of 64): every thread loads
//    BT / 4 chunks of 4 floats of A (rows of the tile) and BT / 4 of B (K
//    rows) with 16-byte loads, all issued before the first is written to LDS,
//    and the next chunk's loads are issued before the current chunk's
//    products;
//  * LDS rows are padded by 4 floats: A [BT][260] (a lane's four k of one row
//    are one conflict-free 16-byte read), B [256][BT + 4] (the four K rows of
//    a lane group land 16 banks apart);
//  * wave w takes k = w * kc / 4 .. (w + 1) * kc / 4 of a chunk of kc,
//    (BT / 16)^2 blocks of v_mfma_f32_16x16x4_f32 with the MFMA step bijection
//    of the register-staged kernel (step s of 16-k part q: lane group g takes
//    k = 16 q + 4 g + s for both operands), B as the first operand so that a
//    lane's accumulator quad holds four consecutive columns of one row;
//  * the write-back is the other kernels' alpha * sum (+ beta * C, C read
//    only when beta != 0), one 16-byte store per output quad.
namespace smallk {
constexpr int KC = 256;
constexpr int kThreads = 256;

template <int BT>
__global__ __launch_bounds__(kThreads, 1) void sgemm_small_kernel(F32Args p, int64_t tile_base) {
  constexpr int IB = BT / 16;                         // blocks per wave per dimension
  constexpr int kAPitch = KC + 4, kBPitch = BT + 4;   // floats
  constexpr int kLoads = BT * KC / 4 / kThreads;      // 16-byte chunks per thread per operand
  constexpr int kBRowChunks = BT / 4;                 // chunks per K row of B
  constexpr int kBRowStep = kThreads / kBRowChunks;   // K rows between a thread's B chunks
  __shared__ __attribute__((aligned(16))) float sa[BT * kAPitch];
  __shared__ __attribute__((aligned(16))) float sb[KC * kBPitch];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int tiles_m = p.M / BT, tiles_n = p.N / BT;
  int tm, tn;
  hgemm::map_tile<8>(tile_base + blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BT, n0 = tn * BT;

  // Chunk u of this thread: A row (tid / 64) + 4 u, k 4 (tid % 64) .. + 3;
  // B K row tid / kBRowChunks + kBRowStep u, columns 4 (tid % kBRowChunks) .. + 3.
  const int brow = tid / kBRowChunks, bcol = 4 * (tid % kBRowChunks);
  const float* a_src = p.A + (int64_t)(m0 + (tid >> 6)) * p.lda + 4 * (tid & 63);
  const float* b_src = p.B + (int64_t)brow * p.ldb + n0 + bcol;
  f4 ra[kLoads], rb[kLoads];
  auto load_chunk = [&](int k0, int kc) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      // A: rows 4 u + tid / 64 hold k 4 (tid % 64) .. + 3 of the chunk, which
      // exist while 4 (tid % 64) < kc; B: K row brow + kBRowStep u < kc
      if (4 * (tid & 63) < kc) ra[u] = *(const f4*)(a_src + (int64_t)(4 * u) * p.lda + k0);
      if (brow + kBRowStep * u < kc)
        rb[u] = *(const f4*)(b_src + (int64_t)(k0 + kBRowStep * u) * p.ldb);
    }
  };
  auto store_chunk = [&](int kc) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      if (4 * (tid & 63) < kc)
        *(f4*)(sa + ((tid >> 6) + 4 * u) * kAPitch + 4 * (tid & 63)) = ra[u];
      if (brow + kBRowStep * u < kc)
        *(f4*)(sb + (brow + kBRowStep * u) * kBPitch + bcol) = rb[u];
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
    __builtin_amdgcn_s_waitcnt(stream::kWaitLgkm0);
    asm volatile("s_barrier" ::: "memory");
    const int next = k0 + KC;
    const int kc_next = p.K - next < KC ? p.K - next : KC;
    if (next < p.K) load_chunk(next, kc_next);
    // this wave's quarter of the chunk: 16-k parts q
    const int parts = kc / 64;
    const int kw = w * (kc / 4);
    for (int q = 0; q < parts; ++q) {
      const int kk = kw + 16 * q + 4 * g;
      f4 av[IB];
#pragma unroll
      for (int i = 0; i < IB; ++i) av[i] = *(const f4*)(sa + (16 * i + r) * kAPitch + kk);
      f4 bv[IB];
#pragma unroll
      for (int j = 0; j < IB; ++j)
#pragma unroll
        for (int s = 0; s < 4; ++s) bv[j][s] = sb[(kk + s) * kBPitch + 16 * j + r];
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < IB; ++i)
#pragma unroll
          for (int j = 0; j < IB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(bv[j][s], av[i][s], acc[i][j], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(stream::kWaitLgkm0);
    asm volatile("s_barrier" ::: "memory");   // the chunk's LDS is free again
    kc = kc_next;
  }

  // acc[i][j][v] is this wave's part of C[m0 + 16 i + r][n0 + 16 j + 4 g + v]:
  // the four partial tiles go to LDS (over A's rows), then each output quad
  // (row t / (BT / 4), columns 4 (t % (BT / 4)) .. + 3 for thread t) adds the
  // four partials in wave order.
  constexpr int kPart = BT * kBPitch;   // floats per partial tile
  static_assert(4 * kPart <= BT * kAPitch, "partials fit over A");
#pragma unroll
  for (int i = 0; i < IB; ++i)
#pragma unroll
    for (int j = 0; j < IB; ++j)
      *(f4*)(sa + w * kPart + (16 * i + r) * kBPitch + 16 * j + 4 * g) = acc[i][j];
  __builtin_amdgcn_s_waitcnt(stream::kWaitLgkm0);
  asm volatile("s_barrier" ::: "memory");
  constexpr int kQuads = BT * BT / 4;
  if (kQuads >= kThreads || tid < kQuads) {
    const int row = tid / (BT / 4), col = 4 * (tid % (BT / 4));
    f4 sum = *(const f4*)(sa + row * kBPitch + col);
#pragma unroll
    for (int v = 1; v < 4; ++v) sum += *(const f4*)(sa + v * kPart + row * kBPitch + col);
    float* c = p.C + (int64_t)(m0 + row) * p.ldc + n0 + col;
    const float alpha = p.alpha, beta = p.beta;
    f4 out = alpha * sum;
    if (beta != 0.f) {
      const f4 old = *(const f4*)c;
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = fmaf(beta, old[e], out[e]);
    }
    *(f4*)c = out;
  }
  static_assert(BT * BT / 4 <= kThreads, "one output quad per thread at most");
}
}  // namespace smallk

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

// The streaming kernels over a.M x a.N (multiples of 64; a.K of 64): 128 x 128
// tiles where there are at least as many as CUs, 64 x 64 otherwise.  One
// persistent workgroup per CU.
hipError_t launch_stream(const F32Args& a, int cus, hipStream_t stream) {
  const bool big = !small_tiles(a.M, a.N, cus) && a.M % 128 == 0 && a.N % 128 == 0;
  const int bt = big ? stream::BM : stream64::BT;
  const int64_t tiles = (int64_t)(a.M / bt) * (a.N / bt);
  const int64_t grid = tiles < cus ? tiles : cus;
  F32Args p = a;
  int64_t t = tiles;
  void* args[] = {&p, &t};
  const void* kernel = big ? (const void*)stream::sgemm_stream_kernel<false>
                           : (const void*)stream64::sgemm_stream64_kernel;
  static_assert(stream::kThreads == stream64::kThreads, "one block size");
  return hipLaunchKernel(kernel, dim3((unsigned)grid), dim3(stream::kThreads), args, 0, stream);
}

}  // namespace

bool f32_mfma_fits(int M, int N, int K, const void* A, int64_t lda, const void* B, int64_t ldb,
                   const void* C, int64_t ldc) {
  return M % 64 == 0 && N % 64 == 0 && K % BK == 0 && aligned16(A) && aligned16(B) &&
         aligned16(C) && lda % 4 == 0 && ldb % 4 == 0 && ldc % 4 == 0;
}

// The streaming kernels' lane offsets (3 rows into A or B, in bytes) must fit
// in 32 bits.
constexpr int64_t kStreamMaxLd = int64_t(1) << 28;

bool f32_stream_fits(int M, int N, int K, const void* A, int64_t lda, const void* B, int64_t ldb,
                     const void* C, int64_t ldc) {
  return f32_mfma_fits(M, N, K, A, lda, B, ldb, C, ldc) && K % 64 == 0 && lda < kStreamMaxLd &&
         ldb < kStreamMaxLd;
}

// The small-tile kernel: whole tiles, K a multiple of 64, and at most half
// as many 64 x 64 tiles as CUs (it then runs at least twice as many
// workgroups as the 64 x 64 kernels would, on every CU); 16 x 16 tiles when
// even 32 x 32 tiles would leave CUs idle.  Long K included: 512 x 512 x 16384
// in 144 us against 272 us on the 64 x 64 streaming tiles (256 x 256 x 16384:
// 66 against 271 us; even at K = 4096).  Between a quarter and half as many
// 64 x 64 tiles as CUs, against the 64 x 64 streaming tiles (same box):
// 512 x 1024 x 2048 30.2 against 38.4 us, 640^2 x 4096 54.7 against 71.0 us,
// 512 x 1024 x 8192 104.4 against 137.5 us, 768 x 512 x 1024 16.3 against
// 21.4 us; with as many tiles as CUs the streaming tiles stay ahead (1024^3:
// 22.9 against 31.2 us).
static bool f32_small32_fits(int M, int N, int K, const void* A, int64_t lda, const void* B,
                             int64_t ldb, const void* C, int64_t ldc, int cus) {
  const int64_t tiles64 = (int64_t)((M + 63) / 64) * ((N + 63) / 64);
  return M % 32 == 0 && N % 32 == 0 && K % 64 == 0 && 2 * tiles64 <= cus &&
         aligned16(A) && aligned16(B) && aligned16(C) && lda % 4 == 0 && ldb % 4 == 0 &&
         ldc % 4 == 0;
}

hipError_t launch_f32_mfma(const F32Args& a, int cus, hipStream_t stream) {
  if (f32_small32_fits(a.M, a.N, a.K, a.A, a.lda, a.B, a.ldb, a.C, a.ldc, cus)) {
    const int64_t tiles32 = (int64_t)(a.M / 32) * (a.N / 32);
    if (tiles32 < cus)
      return launch_tiles((const void*)smallk::sgemm_small_kernel<16>, a, 4 * tiles32,
                          smallk::kThreads, 0, stream);
    return launch_tiles((const void*)smallk::sgemm_small_kernel<32>, a, tiles32,
                        smallk::kThreads, 0, stream);
  }
  if (f32_stream_fits(a.M, a.N, a.K, a.A, a.lda, a.B, a.ldb, a.C, a.ldc))
    return launch_stream(a, cus, stream);
  if (!small_tiles(a.M, a.N, cus) && a.M % 128 == 0 && a.N % 128 == 0)
    return launch_tiled<128, 128, false>(a, stream);
  // The small tiles run one workgroup per CU; 32-deep slabs halve their
  // barriers (1024^3: 28 us against 30 us).
  if (a.K % 32 == 0) return launch_tiled<64, 64, false, 32>(a, stream);
  return launch_tiled<64, 64, false>(a, stream);
}

// The streaming kernel's ragged form (RAG): M, N at least 128 with at least
// as many 128 x 128 tiles as CUs, K a multiple of 4, the fast path's
// alignment.
bool f32_stream_ragged_fits(int M, int N, int K, const void* A, int64_t lda, const void* B,
                            int64_t ldb, const void* C, int64_t ldc, int cus) {
  return M >= 128 && N >= 128 && K >= 4 && K % 4 == 0 && !small_tiles(M, N, cus) &&
         aligned16(A) && aligned16(B) && aligned16(C) && lda % 4 == 0 && ldb % 4 == 0 &&
         ldc % 4 == 0 && lda < kStreamMaxLd && ldb < kStreamMaxLd;
}

hipError_t launch_f32_edge(const F32Args& a, int cus, hipStream_t stream) {
  if (f32_stream_ragged_fits(a.M, a.N, a.K, a.A, a.lda, a.B, a.ldb, a.C, a.ldc, cus)) {
    const int64_t tiles = (int64_t)((a.M + stream::BM - 1) / stream::BM) *
                          ((a.N + stream::BN - 1) / stream::BN);
    const int64_t grid = tiles < cus ? tiles : cus;
    F32Args p = a;
    int64_t t = tiles;
    void* args[] = {&p, &t};
    return hipLaunchKernel((const void*)stream::sgemm_stream_kernel<true>, dim3((unsigned)grid),
                           dim3(stream::kThreads), args, 0, stream);
  }
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
