// Tile kernel template for fp16 C = A * B^T (A[M][K], B[N][K] row-major) on
// the CDNA4 matrix cores, fp32 accumulation, fp16 output (nearest even).
//
// Prior art: the step-by-step A800 kernel of the page "从零开始的 AI Infra:
// 算子基础与GPU架构" -- shared-memory tiles (section 3), tensor-core fragments
// (section 7), 16-byte loads (sections 8-9), an asynchronous copy ring
// (sections 9-12), output staging through shared memory (section 13), B
// consumed in its stored [n][k] layout (section 19) and a XOR-swizzled,
// padding-free shared layout (section 21).  Re-done for gfx950:
//
//  * a workgroup of WAVES_M x WAVES_N waves owns a BM x BN tile of C; each
//    wave owns (BM / WAVES_M) x (BN / WAVES_N), built from 16 x 16 blocks of
//    v_mfma_f32_16x16x32_f16;
//  * K is walked in slabs of BK = 64.  Slabs of A and B go global -> LDS with
//    global_load_lds_dwordx4 (the loaded 16 bytes land in LDS without passing
//    through registers) into a two-stage ring, software-pipelined with two
//    register sets of MFMA operands (see the main loop): one wait and one
//    barrier per slab, placed between the slab's two k-steps;
//  * LDS holds each slab row (BK halves = 128 bytes) as 8 chunks of 16 bytes
//    with chunk c of row r at position c ^ ((r >> 1) & 7).  One copy
//    instruction fills 1 KiB = 8 rows, lane i writing position i; the
//    permutation is realised by the global address each lane loads;
//  * with 64 four-byte banks, a ds_read_b128 serves 16 lanes per cycle in the
//    groups {0-3, 12-15, 20-23, 24-27}, {4-7, 8-11, 16-19, 28-31} (and the
//    same + 32).  The MFMA operand read (lane l: row l % 16, chunk
//    4 s + l / 16) then touches 16 distinct bank quads per group;
//  * both operands are K-major fragments read with one 16-byte LDS load per
//    lane: lane l supplies row l % 16 and k = 8 (l / 16) .. + 7 of the 32 --
//    the same k bijection for A and B, so each MFMA sums its whole K;
//  * B is the MFMA's first operand, so a lane's accumulator quad holds four
//    consecutive columns of one row.  The epilogue rounds them to half,
//    writes them to a per-wave LDS staging area (8 bytes per lane, chunk
//    c of staging row r at slot c ^ (r & 15): conflict-free both ways) and
//    stores whole row segments of the wave tile to C, 16 bytes per lane;
//  * tiles are handed out in an order that keeps each XCD's L2 warm (see
//    map_tile).
//
// Preconditions (checked by the host): M % BM == N % BN == K % BK == 0,
// 16-byte aligned A, B, C, leading dimensions that are multiples of 8.
#pragma once

#include <type_traits>

#include "internal.h"

namespace mi355gemm {
namespace hgemm {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

// Tile order.  The dispatcher deals consecutive workgroups round-robin to the
// 8 XCDs (each with its own L2).  Workgroup b is remapped so that each XCD
// gets a contiguous range of the linear tile order, and that order walks GM
// tile-rows at a time, column-major inside each group: the tiles an XCD runs
// concurrently then share a few A row-panels and B column-panels.  A pure
// permutation of [0, tiles), so correctness never depends on the dispatcher.
template <int GM>
__device__ __forceinline__ void map_tile(int64_t b, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int64_t T = (int64_t)tiles_m * tiles_n;
  const int64_t x = b % 8, j = b / 8, q = T / 8, rem = T % 8;
  const int64_t L = x * q + (x < rem ? x : rem) + j;
  const int64_t per_group = (int64_t)GM * tiles_n;
  const int64_t g = L / per_group, w = L % per_group;
  const int64_t left = tiles_m - g * GM;
  const int rows = (int)(left < GM ? left : GM);
  tm = (int)(g * GM + w % rows);
  tn = (int)(w / rows);
}

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N>
struct Config {
  static constexpr int kWaves = WAVES_M * WAVES_N;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int kChunks = BK / 8;                    // 16-byte chunks per slab row
  static constexpr int kRowsPerCopy = 64 / kChunks;         // rows one copy instruction fills
  static constexpr int kCopiesA = BM / kRowsPerCopy;        // copy instructions per slab of A
  static constexpr int kCopiesB = BN / kRowsPerCopy;
  static constexpr int kPerWaveA = (kCopiesA + kWaves - 1) / kWaves;
  static constexpr int kPerWaveB = (kCopiesB + kWaves - 1) / kWaves;
  static constexpr int kBlocksM = WM / 16, kBlocksN = WN / 16;
  static constexpr int kSteps = BK / 32;                    // MFMA k-steps per slab
  static constexpr int kStageBytes = (BM + BN) * BK * 2;
  static constexpr int kOutRowBytes = 256;                  // staging row: 16 slots of 16 bytes
  static constexpr int kStageBytesOut = kWaves * WM * kOutRowBytes;
  static constexpr int kLdsBytes =
      2 * kStageBytes > kStageBytesOut ? 2 * kStageBytes : kStageBytesOut;
  static_assert(BK == 64, "the slab swizzle and the two-step pipeline assume 128-byte rows");
  static_assert(WN % 16 == 0 && WN * 2 <= kOutRowBytes, "wave tile columns");
  static_assert(WM % 16 == 0 && BM % kRowsPerCopy == 0 && BN % kRowsPerCopy == 0, "tile rows");
  static_assert(kLdsBytes <= 160 * 1024, "LDS");
};

__device__ __forceinline__ int slab_swz(int row) { return (row >> 1) & 7; }

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8; a field at its maximum does not wait).
constexpr int kWaitVmLgkm0 = 0x0070;   // vmcnt(0) lgkmcnt(0)
constexpr int kWaitLgkm0 = 0xC07F;     // lgkmcnt(0)

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int GM>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void hgemm_nt_kernel(F16Args p,
                                                                       int64_t tile_base) {
  typedef Config<BM, BN, BK, WAVES_M, WAVES_N> C;
  constexpr int kChunks = C::kChunks;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[C::kLdsBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int wm = (wave / WAVES_N) * C::WM, wn = (wave % WAVES_N) * C::WN;
  int tm, tn;
  map_tile<GM>(tile_base + blockIdx.x, p.M / BM, p.N / BN, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // Copy assignment: copy instruction c of a slab fills rows [8 c, 8 c + 8);
  // wave w issues copies w, w + kWaves, ...  Lane l writes row 8 c + l / 8 at
  // position l % 8, so it loads logical chunk (l % 8) ^ swz(row).
  const half_t* srcA[C::kPerWaveA];
  const half_t* srcB[C::kPerWaveB];
  int dstA[C::kPerWaveA], dstB[C::kPerWaveB];   // byte offset of the copy's first row
#pragma unroll
  for (int i = 0; i < C::kPerWaveA; ++i) {
    const int cp = i * C::kWaves + wave;
    const int row0 = (cp < C::kCopiesA ? cp : 0) * C::kRowsPerCopy;
    const int row = row0 + lane / kChunks, c = (lane % kChunks) ^ slab_swz(row);
    srcA[i] = p.A + (int64_t)(m0 + row) * p.lda + 8 * c;
    dstA[i] = row0 * BK * 2;
  }
#pragma unroll
  for (int i = 0; i < C::kPerWaveB; ++i) {
    const int cp = i * C::kWaves + wave;
    const int row0 = (cp < C::kCopiesB ? cp : 0) * C::kRowsPerCopy;
    const int row = row0 + lane / kChunks, c = (lane % kChunks) ^ slab_swz(row);
    srcB[i] = p.B + (int64_t)(n0 + row) * p.ldb + 8 * c;
    dstB[i] = BM * BK * 2 + row0 * BK * 2;
  }
  auto copy_slab = [&](int stage, int k0) {
    unsigned char* base = lds + stage * C::kStageBytes;
#pragma unroll
    for (int i = 0; i < C::kPerWaveA; ++i)
      if (C::kCopiesA % C::kWaves == 0 || i * C::kWaves + wave < C::kCopiesA)
        __builtin_amdgcn_global_load_lds((gbl_void_t*)(srcA[i] + k0),
                                         (lds_void_t*)(base + dstA[i]), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < C::kPerWaveB; ++i)
      if (C::kCopiesB % C::kWaves == 0 || i * C::kWaves + wave < C::kCopiesB)
        __builtin_amdgcn_global_load_lds((gbl_void_t*)(srcB[i] + k0),
                                         (lds_void_t*)(base + dstB[i]), 16, 0, 0);
  };
  // All of this wave's copies have landed in LDS, and all of its LDS reads
  // have returned; then every wave of the workgroup meets.  The waits use the
  // builtin (which the compiler's own wait insertion understands); the
  // barrier is an asm statement with a memory clobber so that no memory
  // access is moved across it.
  auto wait_and_sync = [&]() {
    __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0);
    asm volatile("s_barrier" ::: "memory");
  };

  // Operand reads: row (wm | wn) + 16 block + l % 16, chunk (4 s + l / 16) ^ swz.
  const int r = lane & 15, g = lane >> 4;
  const int fr = slab_swz(r);
  const int a_off = (wm + r) * kChunks, b_off = (BM + wn + r) * kChunks;   // in 16-byte units

  f4 acc[C::kBlocksM][C::kBlocksN];
#pragma unroll
  for (int i = 0; i < C::kBlocksM; ++i)
#pragma unroll
    for (int j = 0; j < C::kBlocksN; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  // Two register sets of operand fragments: set s holds k-step s of a slab.
  h8 fa[2][C::kBlocksM], fb[2][C::kBlocksN];
  auto load_frags = [&](int set, int stage, int s) {
    const h8* st = (const h8*)(lds + stage * C::kStageBytes);
    const int pc = (4 * s + g) ^ fr;
#pragma unroll
    for (int i = 0; i < C::kBlocksM; ++i) fa[set][i] = st[a_off + 16 * kChunks * i + pc];
#pragma unroll
    for (int j = 0; j < C::kBlocksN; ++j) fb[set][j] = st[b_off + 16 * kChunks * j + pc];
  };
  auto mfma_step = [&](int set) {
#pragma unroll
    for (int i = 0; i < C::kBlocksM; ++i)
#pragma unroll
      for (int j = 0; j < C::kBlocksN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fb[set][j], fa[set][i], acc[i][j], 0, 0, 0);
  };

  // Software pipeline over k-steps (two per slab).  The one barrier per slab
  // sits between the slab's two steps: before it, every wave has landed its
  // copy of slab t + 1 and has finished reading slab t (its step-1
  // fragments are in registers); after it, slab t's stage is refilled with
  // slab t + 2 and slab t + 1's first fragments are loaded while slab t's
  // second step runs.  Every fragment load overlaps the previous step's MFMAs
  // and every copy has one slab of MFMAs to land.
  //
  // Within each half the copies and LDS reads are interleaved one by one with
  // the MFMAs (sched_group_barrier), so that the two waves sharing a SIMD's
  // matrix pipe -- which the barrier keeps in the same phase -- never both
  // stop issuing MFMAs to issue memory instructions.  sched_barrier(0) fences
  // keep the phases apart.
  constexpr int kMfma = C::kBlocksM * C::kBlocksN;
  constexpr int kReads = C::kBlocksM + C::kBlocksN;
  constexpr int kCopies = C::kPerWaveA + C::kPerWaveB;
  static_assert(kReads + kCopies <= kMfma, "interleave pattern");
  auto slab = [&](int t, auto copy, auto next) {
    // First half: step 0 of slab t, with the loads of step 1.
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    load_frags(1, t & 1, 1);
    mfma_step(0);
#pragma unroll
    for (int q = 0; q < kReads; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kMfma - kReads, 0);
    __builtin_amdgcn_sched_barrier(0);
    wait_and_sync();
    __builtin_amdgcn_sched_barrier(0);
    // Second half: step 1 of slab t, with the copy of slab t + 2 and the
    // loads of slab t + 1's step 0.
    if constexpr (decltype(copy)::value) copy_slab(t & 1, (t + 2) * BK);
    if constexpr (decltype(next)::value) load_frags(0, (t + 1) & 1, 0);
    mfma_step(1);
    constexpr int kR = decltype(next)::value ? kReads : 0;
    constexpr int kV = decltype(copy)::value ? kCopies : 0;
#pragma unroll
    for (int q = 0; q < (kR > kV ? kR : kV); ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (q < kV) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // one copy
      if (q < kR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kMfma - (kR > kV ? kR : kV), 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  typedef std::integral_constant<bool, true> yes;
  typedef std::integral_constant<bool, false> no;

  const int nk = p.K / BK;
  copy_slab(0, 0);
  wait_and_sync();
  if (nk > 1) copy_slab(1, BK);
  load_frags(0, 0, 0);
  for (int t = 0; t + 2 < nk; ++t) slab(t, yes(), yes());
  if (nk >= 2) slab(nk - 2, no(), yes());
  slab(nk - 1, no(), no());

  // Epilogue.  acc[i][j][v] = C[m0 + wm + 16 i + r][n0 + wn + 16 j + 4 g + v].
  // Staging row R (= 16 i + r) of this wave: 16 slots of 16 bytes, chunk c
  // (8 columns) stored in slot c ^ (R & 15).
  unsigned char* stage_out = lds + wave * (C::WM * C::kOutRowBytes);
#pragma unroll
  for (int i = 0; i < C::kBlocksM; ++i) {
    const int R = 16 * i + r;
#pragma unroll
    for (int j = 0; j < C::kBlocksN; ++j) {
      h4 o;
#pragma unroll
      for (int v = 0; v < 4; ++v) o[v] = (half_t)acc[i][j][v];
      const int c = 2 * j + (g >> 1);
      *(h4*)(stage_out + R * C::kOutRowBytes + 16 * (c ^ (R & 15)) + 8 * (g & 1)) = o;
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  // Lanes 16 q' .. 16 q' + 15 store staging row R, 16 bytes each, for the WN / 8
  // chunks the row holds.
  const int cc = lane & 15;
#pragma unroll
  for (int q = 0; q < C::WM / 4; ++q) {
    const int R = 4 * q + (lane >> 4);
    const h8 v = *(const h8*)(stage_out + R * C::kOutRowBytes + 16 * (cc ^ (R & 15)));
    if (C::WN == 128 || cc < C::WN / 8)
      *(h8*)(p.C + (int64_t)(m0 + wm + R) * p.ldc + n0 + wn + 8 * cc) = v;
  }
}

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int GM>
hipError_t launch(const F16Args& a, hipStream_t stream) {
  typedef Config<BM, BN, BK, WAVES_M, WAVES_N> C;
  const int64_t tiles = (int64_t)(a.M / BM) * (a.N / BN);
  return launch_tiles((const void*)hgemm_nt_kernel<BM, BN, BK, WAVES_M, WAVES_N, GM>, a, tiles,
                      C::kThreads, 0, stream);
}

template <int BM, int BN, int BK>
bool fits(int M, int N, int K, const void* A, int64_t lda, const void* B, int64_t ldb,
          const void* Cp, int64_t ldc) {
  return M % BM == 0 && N % BN == 0 && K % BK == 0 && aligned16(A) && aligned16(B) &&
         aligned16(Cp) && lda % 8 == 0 && ldb % 8 == 0 && ldc % 8 == 0;
}

}  // namespace hgemm
}  // namespace mi355gemm
