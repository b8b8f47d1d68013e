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
//    map_tile);
//  * the EPI instances fuse the write-back of page 1 ("第 6 章 Shared Memory
//    & Tile", section 6.5.4) into the rounding step: each accumulator quad
//    gets its columns' bias, the activation and its residual quad in fp32
//    before it is rounded to half.
//
// Preconditions (checked by the host): M % BM == N % BN == K % BK == 0,
// 16-byte aligned A, B, C, leading dimensions that are multiples of 8.
//
// RAG instances take any M >= BM, N >= BN and K > BK with K % 8 == 0, A and
// B rows at 16-byte addresses and C at any 2-byte address (the boundary rule
// of page 1, "第 6 章 Shared Memory & Tile", exercise 7 of section 6.9): the
// last tile row and column are shifted back to end at M and N -- every row a
// copy reads exists -- and store only the rows and columns no earlier tile
// owns; the last slab of K copies its chunks past K from the last chunk
// inside, and the copying wave that wrote them zeroes them in LDS after its
// wait and before the barrier that publishes the slab.
#pragma once

#include <type_traits>
#include <utility>

#include "internal.h"

namespace mi355gemm {
namespace hgemm {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));

// One 16 x 16 x 32 matrix-core product of 16-bit operands in format FMT,
// accumulated in fp32.  Operands travel as 8 16-bit words.
template <int FMT>
__device__ __forceinline__ f4 mfma16(h8 a, h8 b, f4 c) {
  if constexpr (FMT == kFmtF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, a),
                                                   __builtin_bit_cast(b8, b), c, 0, 0, 0);
  }
}
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

// One direct-to-LDS copy written out as an asm statement: lane i loads 16
// bytes from sbase + voff (sbase wave-uniform) and they land at dst + 16 i.
// The compiler sees no LDS write in it, so it adds none of its own waits for
// it; the kernels that use it (those with transposing LDS reads, which the
// compiler would otherwise make wait for every copy in flight) complete it
// with their explicit vmcnt wait before the barrier that publishes a slab.
// M0 (the LDS destination, read when the copy issues) is set one wait state
// ahead and restored after, since the compiler reserves M0 and does not track
// a change made inside an asm statement.
__device__ __forceinline__ void copy16_asm(const char* sbase, uint32_t voff, lds_void_t* dst) {
  // (readfirstlane returns a signed int: each half goes through uint32_t so
  // that the low half is zero-extended, not sign-extended, into the address)
  const uint64_t v = (uint64_t)sbase;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  const uint64_t base = ((uint64_t)hi << 32) | lo;
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(base), "s"(m0v)
      : "memory");
}

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

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int COPY_SEL = 0>
struct Config {
  static constexpr int kWaves = WAVES_M * WAVES_N;
  // Waves that issue the slab copies: all of them (COPY_SEL 0), or half of
  // them -- waves 0 .. kWaves/2 - 1 (COPY_SEL 1) or the even waves (COPY_SEL 2).
  static constexpr int kCopyWaves = COPY_SEL == 0 ? kWaves : kWaves / 2;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int kChunks = BK / 8;                    // 16-byte chunks per slab row
  static constexpr int kRowsPerCopy = 64 / kChunks;         // rows one copy instruction fills
  static constexpr int kCopiesA = BM / kRowsPerCopy;        // copy instructions per slab of A
  static constexpr int kCopiesB = BN / kRowsPerCopy;
  static constexpr int kPerWaveA = (kCopiesA + kCopyWaves - 1) / kCopyWaves;
  static constexpr int kPerWaveB = (kCopiesB + kCopyWaves - 1) / kCopyWaves;
  static constexpr int kBlocksM = WM / 16, kBlocksN = WN / 16;
  static constexpr int kSteps = BK / 32;                    // MFMA k-steps per slab
  static constexpr int kStageBytes = (BM + BN) * BK * 2;
  static constexpr int kOutRowBytes = 256;                  // staging row: 16 slots of 16 bytes
  static_assert(BK == 64, "the slab swizzle and the two-step pipeline assume 128-byte rows");
  static_assert(WN % 16 == 0 && WN * 2 <= kOutRowBytes, "wave tile columns");
  static_assert(WM % 16 == 0 && BM % kRowsPerCopy == 0 && BN % kRowsPerCopy == 0, "tile rows");
};

__device__ __forceinline__ int slab_swz(int row) { return (row >> 1) & 7; }

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8; a field at its maximum does not wait).
constexpr int kWaitVmLgkm0 = 0x0070;   // vmcnt(0) lgkmcnt(0)
constexpr int kWaitLgkm0 = 0xC07F;     // lgkmcnt(0)

// Kernel arguments: the product, and the tiles this launch covers.  The
// launch has `grid` workgroups; workgroup b handles tiles b, b + grid, ...
// (< tiles), one after another, as one continuous stream of K slabs.
struct TileArgs {
  Args16 p;
  int64_t tiles;
};

// Waves of the kernel that share each SIMD: 8-wave workgroups put two on
// each; 4-wave 128 x 128 tiles run two workgroups per CU (the launcher's
// slot count), so their register budget must leave room for the second.
constexpr int waves_per_simd(int bm, int bn, int waves) {
  return waves == 8 ? 2 : (bm * bn <= 128 * 128 ? 2 : 1);
}

// f(std::integral_constant<int, 0>()), ..., f(std::integral_constant<int, N - 1>()):
// a loop whose index is a compile-time constant in the body.
template <typename F, int... Q>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Q...>) {
  (f(std::integral_constant<int, Q>()), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>());
}

// SPLIT instances walk (tile, K range) work items -- item i is range
// i / tiles of tile i % tiles, p.sk.per slabs from slab (i / tiles) * per --
// and store each item's fp32 partial tile to the split-K workspace instead of
// writing C.
//
// LAY 1 instances read B stored [K][N] (C = A * B), LAY 2 instances A
// stored [K][M] (C = A^T * B^T) and LAY 3 instances both (C = A^T * B) in
// place: the page's kernel consumes the operand in the layout it is stored in
// rather than transposing it first ("从零开始的 AI Infra: 算子基础与GPU架构",
// section 19).  Such an operand's slab is kept in LDS as 64 k-rows of 512
// bytes (32 chunks of 16 bytes: the tile's 256, 224 or 192 values, then
// unused positions; 256 bytes for a 128-value tile side), chunk c of k-row k
// at position c ^ tsw(k) with
// tsw(k) = 2 (k & 3) | 8 (((k >> 3) ^ (k >> 4)) & 1), and its fragments are
// read with gfx950's transposing LDS read (ds_read_b64_tr_b16): in each
// group of 16 lanes, lane 4 a + b receives element b of the 8-byte reads of
// lanes a, a + 4, a + 8 and a + 12.  Lane l (group g = l / 16, i = l % 16)
// reads k-row 32 s + 8 g + 4 h + i / 4 at values x0 + 4 (i % 4) .. + 3 for
// h = 0, 1, and so holds k = 32 s + 8 g .. + 7 of value x0 + i: the same k
// bijection as the K-contiguous operand's fragments.  Among any two of the
// four lane groups the sixteen rows' chunk pairs fall on distinct bank quads.
// The copies of these instances are issued from copy16_asm (the compiler
// would otherwise wait for every copy in flight before each transposing
// read).  Preconditions as above, with the K-major operands' rows at 16-byte
// addresses: whole tiles with K % 64 == 0, or RAG, whose last slab is copied
// from K - 64 when K % 64 != 0 (K > 64; K % 8 == 0 if an operand is
// K-contiguous) and has its repeated positions zeroed.
template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int GM, int COPY_SEL, int OPT, bool EPI,
          int FMT, bool SPLIT = false, bool RAG = false, int LAY = 0>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, waves_per_simd(BM, BN, WAVES_M * WAVES_N))
void hgemm_nt_kernel(TileArgs ta) {
  static_assert(!(RAG && SPLIT), "ragged tiles store C");
  typedef Config<BM, BN, BK, WAVES_M, WAVES_N, COPY_SEL> C;
  constexpr bool kAT = LAY == 2 || LAY == 3, kBT = LAY == 1 || LAY == 3;   // stored K-major
  static_assert(LAY == 0 || (!SPLIT && C::kCopyWaves == 4),
                "K-major operands: four copying waves, no split-K");
  static_assert((!kBT || (BN <= 256 && BN % 32 == 0)) && (!kAT || (BM <= 256 && BM % 32 == 0)),
                "K-major slab rows of at most 256 values");
  // A stage: A's area, then B's.  A K-major operand takes 64 k-rows of kTP
  // bytes -- 256 for 128 values, else 512 (up to 256 values, padded) -- and
  // one copy instruction fills 1024 / kTP of them.
  constexpr int kTPA = BM <= 128 ? 256 : 512, kTPB = BN <= 128 ? 256 : 512;
  constexpr int kAreaA = kAT ? BK * kTPA : BM * BK * 2;
  constexpr int kAreaB = kBT ? BK * kTPB : BN * BK * 2;
  constexpr int kStage = kAreaA + kAreaB;
  static_assert(kBT || kAreaA == BM * BK * 2, "K-contiguous B fragments are read past A's area");
  constexpr int kCopiesA = kAT ? BK * kTPA / 1024 : C::kCopiesA;
  constexpr int kCopiesB = kBT ? BK * kTPB / 1024 : C::kCopiesB;
  constexpr int kPerWaveA = (kCopiesA + C::kCopyWaves - 1) / C::kCopyWaves;
  constexpr int kPerWaveB = (kCopiesB + C::kCopyWaves - 1) / C::kCopyWaves;
  constexpr int kChunks = C::kChunks;
  const Args16& p = ta.p;
  // Two slab stages, then the epilogue staging area (16 rows of 256 bytes per
  // wave, see below).
  constexpr int kOutRows = 16;
  constexpr int kOutBytes = C::kWaves * kOutRows * C::kOutRowBytes;
  constexpr int kLds = 2 * kStage + kOutBytes;
  static_assert(kLds <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kLds];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int wm = (wave / WAVES_N) * C::WM, wn = (wave % WAVES_N) * C::WN;
  const int tiles_m = RAG ? (p.M + BM - 1) / BM : p.M / BM;
  const int tiles_n = RAG ? (p.N + BN - 1) / BN : p.N / BN;
  // K values in the last slab of a tile (RAG: 8 .. 64)
  const int kv = RAG ? p.K - ((p.K + BK - 1) / BK - 1) * BK : BK;
  const int64_t stride = gridDim.x;
  const int ntiles = (int)((ta.tiles - blockIdx.x + stride - 1) / stride);
  // Work item j of this workgroup: tile origin (m0, n0), first K slab kb and
  // split-K range sp (both 0 without SPLIT).
  // (m0, n0): the rows and columns the tile computes; (mlo, nlo): the first
  // it stores (RAG: the last tile row and column start at M - BM, N - BN).
  auto tile_origin = [&](int j, int& m0, int& n0, int& kb, int& sp, int& mlo, int& nlo)
                         __attribute__((always_inline)) {
    int64_t item = blockIdx.x + j * stride;
    sp = 0;
    if constexpr (SPLIT) {
      const int64_t tiles = (int64_t)tiles_m * tiles_n;
      sp = (int)(item / tiles);
      item -= sp * tiles;
    }
    kb = sp * (SPLIT ? p.sk.per : 0);
    int tm, tn;
    map_tile<GM>(item, tiles_m, tiles_n, tm, tn);
    mlo = tm * BM;
    nlo = tn * BN;
    m0 = RAG && mlo > p.M - BM ? p.M - BM : mlo;
    n0 = RAG && nlo > p.N - BN ? p.N - BN : nlo;
  };

  // Copy assignment: copy instruction c of a slab fills rows [8 c, 8 c + 8);
  // copying wave cw issues copies cw, cw + kCopyWaves, ...  Lane l writes row
  // 8 c + l / 8 at position l % 8, so it loads logical chunk
  // (l % 8) ^ swz(row), swz(row) = ((8 c + l / 8) >> 1) & 7
  // = (4 (c & 1) + l / 16) & 7.  A wave's copies all have c & 1 == cw & 1
  // (kCopyWaves is even), so one 32-bit offset per lane serves every copy;
  // the row base of a copy is wave-uniform.
  static_assert(C::kCopyWaves % 2 == 0 && C::kRowsPerCopy == 8, "copy addressing");
  const int cw = COPY_SEL == 0 ? wave
               : COPY_SEL == 1 ? (wave < C::kCopyWaves ? wave : -1)
                               : ((wave & 1) == 0 ? wave / 2 : -1);
  const bool copier = cw >= 0;
  const int cwp = copier ? cw : 0;
  const int lane_row = lane / kChunks;
  const int lane_chunk = (lane % kChunks) ^ ((4 * (cwp & 1) + (lane >> 4)) & 7);
  const uint32_t offA = (uint32_t)(lane_row * p.lda + 8 * lane_chunk) * 2;   // bytes
  const uint32_t offB = (uint32_t)(lane_row * p.ldb + 8 * lane_chunk) * 2;
  // RAG, the last slab of K: a lane whose chunk lies past K loads the last
  // chunk inside K instead (zeroed once it has landed).
  const bool chunk_past = RAG && 8 * lane_chunk >= kv;
  const int tail_chunk = chunk_past ? kv / 8 - 1 : lane_chunk;
  const uint32_t offA_tail = (uint32_t)(lane_row * p.lda + 8 * tail_chunk) * 2;
  const uint32_t offB_tail = (uint32_t)(lane_row * p.ldb + 8 * tail_chunk) * 2;
  const int64_t copy_strideA = (int64_t)C::kCopyWaves * C::kRowsPerCopy * p.lda * 2;
  const int64_t copy_strideB = (int64_t)C::kCopyWaves * C::kRowsPerCopy * p.ldb * 2;
  const int64_t firstA = (int64_t)cwp * C::kRowsPerCopy * p.lda * 2;
  const int64_t firstB = (int64_t)cwp * C::kRowsPerCopy * p.ldb * 2;
  // A K-major operand (LAY) with R = 1024 / kTP k-rows per copy: copy c
  // fills k-rows R c .. R c + R - 1, lane l writing k-row R c + l / (kTP / 16)
  // at position l % (kTP / 16), so it loads logical chunk
  // (l % (kTP / 16)) ^ tsw(k-row) -- the row's last chunk where that lies
  // past the tile's values (its position is never read).  Copy i of wave cw
  // is c = 4 i + cw.  R = 2: k-row 8 i + 2 cw + l / 32, k & 3 = 2 (cw & 1) +
  // l / 32 and ((k >> 3) ^ (k >> 4)) & 1 = (i ^ (i >> 1)) & 1.  R = 4: k-row
  // 16 i + 4 cw + l / 16, k & 3 = l / 16 and ((k >> 3) ^ (k >> 4)) & 1 =
  // ((cw >> 1) ^ i) & 1.  Two lane offsets per operand serve every copy.
  auto t_off = [&](int64_t ld, int width, int pitch, int hi) __attribute__((always_inline)) {
    const int cpr = pitch / 16;
    const int tlo = pitch == 512 ? 2 * (2 * (cwp & 1) + (lane >> 5)) : 2 * (lane >> 4);
    int lc = (lane % cpr) ^ (tlo | hi);
    if (lc >= width / 8) lc = width / 8 - 1;
    return (uint32_t)((lane / cpr) * ld * 2 + 16 * lc);
  };
  // whether copy i of this wave takes the offset with bit 3 set
  auto t_hi = [&](int pitch, int i) __attribute__((always_inline)) {
    return pitch == 512 ? ((i ^ (i >> 1)) & 1) != 0 : (((cwp >> 1) ^ i) & 1) != 0;
  };
  const uint32_t offTA0 = t_off(p.lda, BM, kTPA, 0), offTA1 = t_off(p.lda, BM, kTPA, 8);
  const uint32_t offTB0 = t_off(p.ldb, BN, kTPB, 0), offTB1 = t_off(p.ldb, BN, kTPB, 8);
  const int64_t firstTA = (int64_t)(1024 / kTPA) * cwp * p.lda * 2;
  const int64_t firstTB = (int64_t)(1024 / kTPB) * cwp * p.ldb * 2;
  const int64_t copy_strideTA = (int64_t)4 * (1024 / kTPA) * p.lda * 2;
  const int64_t copy_strideTB = (int64_t)4 * (1024 / kTPB) * p.ldb * 2;

  // This wave's copies of one K slab: the sources of its A and B rows and
  // the slab's LDS stage, then copy instruction c (A copies first) one at a
  // time, so that the main loop can place each one between two MFMAs.
  struct CopyBase {
    const char* a;
    const char* b;
    unsigned char* l;
    uint32_t oa, ob;   // this lane's offsets (RAG: the clamped ones in a tile's last slab)
  };
  // LAY with a K tail (RAG): the last slab is copied from K - 64 .. K - 1,
  // every row and chunk inside the matrix; its first 64 - kv positions repeat
  // the slab before and are zeroed in LDS (wait_zero_sync), so they add 0 x 0.
  auto slab_base = [&](int stage, int m0, int n0, int t, bool tail) __attribute__((always_inline)) {
    CopyBase cb;
    cb.l = lds + stage * kStage;
    const int64_t k0 = LAY != 0 && RAG && tail ? (int64_t)p.K - BK : (int64_t)t * BK;
    cb.a = kAT ? (const char*)(p.A + k0 * p.lda + m0) + firstTA
               : (const char*)(p.A + (int64_t)m0 * p.lda) + firstA + 2 * k0;
    cb.b = kBT ? (const char*)(p.B + k0 * p.ldb + n0) + firstTB
               : (const char*)(p.B + (int64_t)n0 * p.ldb) + firstB + 2 * k0;
    cb.oa = LAY == 0 && RAG && tail ? offA_tail : offA;
    cb.ob = LAY == 0 && RAG && tail ? offB_tail : offB;
    return cb;
  };
  // One copy (LAY: through the asm statement above, so that the compiler
  // adds no waits before the transposing reads).
  auto issue = [&](const char* base, uint32_t off, unsigned char* dst) __attribute__((always_inline)) {
    if constexpr (LAY != 0)
      copy16_asm(base, off, (lds_void_t*)dst);
    else
      __builtin_amdgcn_global_load_lds((gbl_void_t*)(base + off), (lds_void_t*)dst, 16, 0, 0);
  };
  auto copy_one = [&](const CopyBase& cb, int c) __attribute__((always_inline)) {
    if (c < kPerWaveA) {
      if (kCopiesA % C::kCopyWaves == 0 || c * C::kCopyWaves + cw < kCopiesA) {
        if constexpr (kAT)
          issue(cb.a + c * copy_strideTA, t_hi(kTPA, c) ? offTA1 : offTA0,
                cb.l + (c * C::kCopyWaves + cw) * 1024);
        else
          issue(cb.a + c * copy_strideA, cb.oa, cb.l + (c * C::kCopyWaves + cw) * 1024);
      }
    } else {
      const int i = c - kPerWaveA;
      if (kCopiesB % C::kCopyWaves == 0 || i * C::kCopyWaves + cw < kCopiesB) {
        if constexpr (kBT)
          issue(cb.b + i * copy_strideTB, t_hi(kTPB, i) ? offTB1 : offTB0,
                cb.l + kAreaA + (i * C::kCopyWaves + cw) * 1024);
        else
          issue(cb.b + i * copy_strideB, cb.ob,
                cb.l + kAreaA + (i * C::kCopyWaves + cw) * 1024);
      }
    }
  };
  // All of this wave's copies have landed in LDS, and all of its LDS reads
  // have returned; then every wave of the workgroup meets.  The waits use the
  // builtin (which the compiler's own wait insertion understands); the
  // barrier is an asm statement with a memory clobber so that no memory
  // access is moved across it.
  auto wait_and_sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0);
    asm volatile("s_barrier" ::: "memory");
  };
  // RAG: the same, and before the barrier this wave zeroes its chunks past K
  // of the slab in `stage` when that slab is the last of its tile.
  // LAY: this wave zeroes what its copies put in the first 64 - kv
  // positions of that slab (copied from K - 64, above): K-major k-rows below
  // 64 - kv, and K-contiguous chunks whose first k is below it.
  auto wait_zero_sync = [&](bool zero, int stage) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0);
    if constexpr (LAY != 0) {
      if (zero && copier) {
        const int ks = BK - kv;
        unsigned char* l = lds + stage * kStage;
        // the k-row a K-major copy c of this lane wrote (R = 1024 / pitch rows per copy)
        auto trow = [&](int pitch, int c) __attribute__((always_inline)) {
          return (1024 / pitch) * (c * C::kCopyWaves + cw) + lane / (pitch / 16);
        };
#pragma unroll
        for (int c = 0; c < kPerWaveA; ++c)
          if ((kCopiesA % C::kCopyWaves == 0 || c * C::kCopyWaves + cw < kCopiesA) &&
              (kAT ? trow(kTPA, c) < ks : 8 * lane_chunk < ks))
            *(h8*)(l + (c * C::kCopyWaves + cw) * 1024 + 16 * lane) = h8{};
#pragma unroll
        for (int i = 0; i < kPerWaveB; ++i)
          if ((kCopiesB % C::kCopyWaves == 0 || i * C::kCopyWaves + cw < kCopiesB) &&
              (kBT ? trow(kTPB, i) < ks : 8 * lane_chunk < ks))
            *(h8*)(l + kAreaA + (i * C::kCopyWaves + cw) * 1024 + 16 * lane) = h8{};
      }
    } else if (zero && copier && chunk_past) {
      unsigned char* l = lds + stage * kStage;
#pragma unroll
      for (int c = 0; c < kPerWaveA; ++c)
        if (kCopiesA % C::kCopyWaves == 0 || c * C::kCopyWaves + cw < kCopiesA)
          *(h8*)(l + (c * C::kCopyWaves + cw) * 1024 + 16 * lane) = h8{};
#pragma unroll
      for (int i = 0; i < kPerWaveB; ++i)
        if (kCopiesB % C::kCopyWaves == 0 || i * C::kCopyWaves + cw < kCopiesB)
          *(h8*)(l + kAreaA + (i * C::kCopyWaves + cw) * 1024 + 16 * lane) = h8{};
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    asm volatile("s_barrier" ::: "memory");
  };

  // Operand reads: row (wm | wn) + 16 block + l % 16, chunk (4 s + l / 16) ^ swz.
  const int r = lane & 15, g = lane >> 4;
  const int fr = slab_swz(r);
  const int a_off = (wm + r) * kChunks, b_off = (BM + wn + r) * kChunks;   // in 16-byte units

  // K-major operand fragments (LAY): per-lane byte offsets of block x's
  // first transposing read within the operand's stage area (block x covers
  // values x0 = w0 + 16 x .. + 15 of the wave's w0 = wm for A, wn for B).
  uint32_t toffA[kAT ? C::kBlocksM : 1], toffB[kBT ? C::kBlocksN : 1];
  {
    const int ti = lane & 15;
    const int tsw = (2 * (ti >> 2)) | (8 * ((g ^ (g >> 1)) & 1));
    auto fill = [&](uint32_t* toff, int nblocks, int w0, int pitch) __attribute__((always_inline)) {
#pragma unroll
      for (int x = 0; x < nblocks; ++x)
        toff[x] = (uint32_t)((8 * g + (ti >> 2)) * pitch +
                             16 * (((w0 >> 3) + 2 * x + ((ti & 3) >> 1)) ^ tsw) + 8 * (ti & 1));
    };
    if constexpr (kAT) fill(toffA, C::kBlocksM, wm, kTPA);
    if constexpr (kBT) fill(toffB, C::kBlocksN, wn, kTPB);
  }
  // Block x of k-step s from the operand area `area` (A's or B's part of a
  // stage, offsets toff, k-rows of `pitch` bytes): two transposing reads,
  // k-rows 4 apart.
  auto tread = [&](const unsigned char* area, const uint32_t* toff, int x, int s, int pitch)
                   __attribute__((always_inline)) {
    typedef short s4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s4 lds_s4;
    typedef __attribute__((address_space(3))) const unsigned char lds_u8;
    lds_u8* base = (lds_u8*)area + toff[x] + s * 32 * pitch;
    const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)base);
    const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(base + 4 * pitch));
    return __builtin_bit_cast(h8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f4 acc[C::kBlocksM][C::kBlocksN];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::kBlocksM; ++i)
#pragma unroll
      for (int j = 0; j < C::kBlocksN; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};
  };

  // Two register sets of operand fragments: set s holds k-step s of a slab.
  // OPT bit 1: one set of B fragments (fb[0]), for tiles whose accumulators
  // and two full sets would not fit the 256 registers of a wave.
  constexpr bool kOneB = (OPT & 2) != 0;
  h8 fa[2][C::kBlocksM], fb[kOneB ? 1 : 2][C::kBlocksN];
  auto load_frags = [&](int set, int stage, int s) __attribute__((always_inline)) {
    const h8* st = (const h8*)(lds + stage * kStage);
    const unsigned char* sa = lds + stage * kStage;
    const int pc = (4 * s + g) ^ fr;
#pragma unroll
    for (int i = 0; i < C::kBlocksM; ++i) {
      if constexpr (kAT) fa[set][i] = tread(sa, toffA, i, s, kTPA);
      else fa[set][i] = st[a_off + 16 * kChunks * i + pc];
    }
#pragma unroll
    for (int j = 0; j < C::kBlocksN; ++j) {
      if constexpr (kBT) fb[kOneB ? 0 : set][j] = tread(sa + kAreaA, toffB, j, s, kTPB);
      else fb[kOneB ? 0 : set][j] = st[b_off + 16 * kChunks * j + pc];
    }
  };
  auto mfma_step = [&](int set) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::kBlocksM; ++i)
#pragma unroll
      for (int j = 0; j < C::kBlocksN; ++j)
        acc[i][j] = mfma16<FMT>(fb[set][j], fa[set][i], acc[i][j]);
  };
  // Fragment q of a k-step (the A blocks, then the B blocks), and MFMA q of a
  // k-step (row block q / kBlocksN, column block q % kBlocksN).
  auto read_one = [&](int set, int stage, int step, int q) __attribute__((always_inline)) {
    const h8* st = (const h8*)(lds + stage * kStage);
    const unsigned char* sa = lds + stage * kStage;
    const int pc = (4 * step + g) ^ fr;
    if (q < C::kBlocksM) {
      if constexpr (kAT) fa[set][q] = tread(sa, toffA, q, step, kTPA);
      else fa[set][q] = st[a_off + 16 * kChunks * q + pc];
    } else {
      if constexpr (kBT)
        fb[set][q - C::kBlocksM] = tread(sa + kAreaA, toffB, q - C::kBlocksM, step, kTPB);
      else fb[set][q - C::kBlocksM] = st[b_off + 16 * kChunks * (q - C::kBlocksM) + pc];
    }
  };
  auto mfma_one = [&](int set, int q) __attribute__((always_inline)) {
    const int i = q / C::kBlocksN, j = q % C::kBlocksN;
    acc[i][j] = mfma16<FMT>(fb[set][j], fa[set][i], acc[i][j]);
  };

  // Epilogue of the tile with origin (m0, n0): acc[i][j][v] is
  // C[m0 + wm + 16 i + r][n0 + wn + 16 j + 4 g + v].  Row block i at a time,
  // the quads are rounded to half and written (8 bytes per lane) to this
  // wave's 16-row staging area, chunk c (8 columns) of staging row R in slot
  // c ^ R (conflict-free for the writes and for the row reads), then whole
  // row segments are stored to C with 16 bytes per lane.
  //
  // The EPI instances first load the bias and residual quads of the whole
  // wave tile (an absent operand reads as zeros), so that one memory latency
  // covers them all, then compute act(acc + bias) + residual in fp32, the
  // activation chosen once per quad.  The accumulator is never -0 (its sum
  // starts at +0), so adding a zero for an absent operand changes nothing.
  unsigned char* stage_out = lds + 2 * kStage + wave * (kOutRows * C::kOutRowBytes);
  auto epilogue = [&](int m0, int n0, int mlo, int nlo) __attribute__((always_inline)) {
    (void)mlo;
    (void)nlo;
    const int cc = lane & 15;
    h4 bq[C::kBlocksN], rq[C::kBlocksM][C::kBlocksN];
    if constexpr (EPI) {
#pragma unroll
      for (int j = 0; j < C::kBlocksN; ++j) {
        const int n = n0 + wn + 16 * j + 4 * g;
        bq[j] = h4{};
        if (p.bias) bq[j] = *(const h4*)(p.bias + n);
      }
#pragma unroll
      for (int i = 0; i < C::kBlocksM; ++i) {
        const int64_t m = m0 + wm + 16 * i + r;
#pragma unroll
        for (int j = 0; j < C::kBlocksN; ++j) {
          const int n = n0 + wn + 16 * j + 4 * g;
          rq[i][j] = h4{};
          if (p.res) rq[i][j] = *(const h4*)(p.res + m * p.ldr + n);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < C::kBlocksM; ++i) {
#pragma unroll
      for (int j = 0; j < C::kBlocksN; ++j) {
        h4 o;
        if constexpr (EPI) {
          f4 x = acc[i][j];
#pragma unroll
          for (int v = 0; v < 4; ++v) x[v] += word_to_f32<FMT>(bq[j][v]);
          if (p.act == GEMM_ACT_SILU) {
#pragma unroll
            for (int v = 0; v < 4; ++v) x[v] = epi_silu(x[v]);
          } else if (p.act == GEMM_ACT_RELU) {
#pragma unroll
            for (int v = 0; v < 4; ++v) x[v] = epi_relu(x[v]);
          }
#pragma unroll
          for (int v = 0; v < 4; ++v) o[v] = f32_to_word<FMT>(x[v] + word_to_f32<FMT>(rq[i][j][v]));
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v) o[v] = f32_to_word<FMT>(acc[i][j][v]);
        }
        const int c = 2 * j + (g >> 1);
        *(h4*)(stage_out + r * C::kOutRowBytes + 16 * (c ^ r) + 8 * (g & 1)) = o;
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int q = 0; q < kOutRows / 4; ++q) {
        const int R = 4 * q + (lane >> 4);
        const h8 v = *(const h8*)(stage_out + R * C::kOutRowBytes + 16 * (cc ^ R));
        if constexpr (RAG) {
          // only rows and columns no earlier tile owns; C at any 2-byte address
          const int m = m0 + wm + 16 * i + R, n = n0 + wn + 8 * cc;
          if ((C::WN == 128 || cc < C::WN / 8) && m >= mlo && n + 8 > nlo) {
            half_t* dst = p.C + (int64_t)m * p.ldc + n;
            if (n >= nlo) {
              __builtin_memcpy(dst, &v, 16);
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (n + e >= nlo) dst[e] = v[e];
            }
          }
        } else if (C::WN == 128 || cc < C::WN / 8) {
          h8* dst = (h8*)(p.C + (int64_t)(m0 + wm + 16 * i + R) * p.ldc + n0 + wn + 8 * cc);
          if (OPT & 1) {
            __builtin_nontemporal_store(v, dst);   // OPT bit 0: streaming stores of C
          } else {
            *dst = v;
          }
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  };

  // Split-K partial tile: acc[i][j] is row m0 + wm + 16 i + r, columns
  // n0 + wn + 16 j + 4 g .. + 3; one 16-byte store per block into the
  // workspace (padded to whole tiles, no bounds).
  auto epilogue_partial = [&](int m0, int n0, int sp) __attribute__((always_inline)) {
    float* ws = p.sk.ws + sp * p.sk.split_stride;
#pragma unroll
    for (int i = 0; i < C::kBlocksM; ++i)
#pragma unroll
      for (int j = 0; j < C::kBlocksN; ++j)
        *(f4*)(ws + (int64_t)(m0 + wm + 16 * i + r) * p.sk.ld + n0 + wn + 16 * j + 4 * g) =
            acc[i][j];
  };

  // Software pipeline over the workgroup's slab stream (ntiles x nk slabs,
  // two k-steps each).  The one barrier per slab sits between the slab's two
  // steps: before it, every wave has landed its copy of the next slab and has
  // finished reading this one (its step-1 fragments are in registers); after
  // it, this slab's stage is refilled with the slab after next (which may
  // belong to the next tile) and the next slab's first fragments are loaded
  // while this slab's second step runs.  Every fragment load overlaps the
  // previous step's MFMAs and every copy has one slab of MFMAs to land; the
  // next tile's first two slabs land while this tile finishes and stores.
  //
  // The first half interleaves its LDS reads one by one with the MFMAs
  // (sched_group_barrier).  The second half is written out in issue order --
  // MFMA q, then copy q and read q while there are any -- with
  // sched_barrier(0) fences after each group: left to itself the scheduler
  // bunches the copies (each one holds the copying wave at issue until the
  // CU's copy path takes it) and the LDS reads, both of which stall the
  // wave's MFMAs.  Copies go first, since each one has to land before the
  // next barrier.
  constexpr int kMfma = C::kBlocksM * C::kBlocksN;
  constexpr int kReads = C::kBlocksM + C::kBlocksN;
  // LDS read instructions per k-step (a K-major block takes two)
  constexpr int kReadInstr = kReads + (kAT ? C::kBlocksM : 0) + (kBT ? C::kBlocksN : 0);
  constexpr int kCopies = kPerWaveA + kPerWaveB;
  static_assert(kReadInstr <= kMfma && kCopies <= kMfma, "interleave pattern");
  const int nk = SPLIT ? p.sk.per : RAG ? (p.K + BK - 1) / BK : p.K / BK;   // slabs per work item
  // The copy target runs two slabs ahead of the compute: slab tc of the tile
  // `ahead` tiles after the current one (origins o[0..2] are refreshed once
  // per tile, outside the MFMA loop).  Past the end of the stream it stays on
  // the last slab of the last tile.
  int tc = 0, ahead = 0, cur = 0;
  int om[3], on[3], ok[3], os[3];
  int mlo0 = 0, nlo0 = 0;   // the current tile's first stored row and column
  auto refresh_origins = [&](int j) __attribute__((always_inline)) {
    cur = j;
#pragma unroll
    for (int d = 0; d < 3; ++d) {
      int mlo, nlo;
      tile_origin(j + d < ntiles ? j + d : ntiles - 1, om[d], on[d], ok[d], os[d], mlo, nlo);
      if (d == 0) {
        mlo0 = mlo;
        nlo0 = nlo;
      }
    }
  };
  refresh_origins(0);
  auto advance_copy = [&]() __attribute__((always_inline)) {
    if (++tc == nk) {
      tc = 0;
      ++ahead;
    }
  };
  // The copy target's sources and LDS stage.
  auto next_base = [&](int stage) __attribute__((always_inline)) {
    const bool past = cur + ahead >= ntiles;
    const int d = ahead < 2 ? ahead : 2;
    const int m0 = d == 0 ? om[0] : d == 1 ? om[1] : om[2];
    const int n0 = d == 0 ? on[0] : d == 1 ? on[1] : on[2];
    const int kb = d == 0 ? ok[0] : d == 1 ? ok[1] : ok[2];
    const int t = past ? nk - 1 : tc;
    return slab_base(stage, m0, n0, kb + t, RAG && kv < BK && t == nk - 1);
  };
  auto copy_next = [&](int stage) __attribute__((always_inline)) {
    const CopyBase cb = next_base(stage);
#pragma unroll
    for (int c = 0; c < kCopies; ++c) copy_one(cb, c);
  };
  // zero_next (RAG): the next slab is the last of its tile and reaches past K.
  auto slab = [&](int gs, auto next, auto is_copier, bool zero_next) __attribute__((always_inline)) {
    auto sync = [&]() __attribute__((always_inline)) {
      if constexpr (RAG) wait_zero_sync(zero_next, (gs + 1) & 1);
      else wait_and_sync();
    };
    constexpr bool kCp = decltype(is_copier)::value;
    constexpr bool kNext = decltype(next)::value;
    CopyBase cb{};
    if constexpr (kCp) cb = next_base(gs & 1);
    if constexpr (kOneB) {
      // One set of B fragments: each k-step runs its MFMAs column block by
      // column block, and B fragment j is reloaded (for the next step) right
      // after its column's last MFMA.  The barrier comes after the first
      // column of step 1, once every read of this slab's stage has been
      // issued and one column of MFMAs covers the last read's latency; reads
      // of the next slab's stage follow it.
      constexpr int MB = C::kBlocksM, NB = C::kBlocksN;
      constexpr int kB = kMfma + MB;
      static_assert(kB + kCopies <= 2 * kMfma, "copies after the barrier");
      const h8* cur_st = (const h8*)(lds + (gs & 1) * kStage);
      const h8* nxt_st = (const h8*)(lds + ((gs + 1) & 1) * kStage);
      const unsigned char* cur_sa = lds + (gs & 1) * kStage;
      const unsigned char* nxt_sa = lds + ((gs + 1) & 1) * kStage;
      const int pc1 = (4 + g) ^ fr, pc0 = g ^ fr;
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_sched_barrier(0);
      static_for<2 * kMfma>([&](auto qc) __attribute__((always_inline)) {
        constexpr int q = decltype(qc)::value;
        if constexpr (q == kB) {
          sync();
          __builtin_amdgcn_sched_barrier(0);
        }
        constexpr int step = q / kMfma, qq = q % kMfma, j = qq / MB, i = qq % MB;
        acc[i][j] = mfma16<FMT>(fb[0][j], fa[step][i], acc[i][j]);
        if constexpr (step == 0) {
          // step 1 of this slab: A fragment qq, B fragment j after its last use
          if constexpr (qq < MB) {
            if constexpr (kAT) fa[1][qq] = tread(cur_sa, toffA, qq, 1, kTPA);
            else fa[1][qq] = cur_st[a_off + 16 * kChunks * qq + pc1];
          }
          if constexpr (i == MB - 1) {
            if constexpr (kBT) fb[0][j] = tread(cur_sa + kAreaA, toffB, j, 1, kTPB);
            else fb[0][j] = cur_st[b_off + 16 * kChunks * j + pc1];
          }
        }
        if constexpr (kNext) {
          // step 0 of the next slab, after the barrier
          static_for<MB>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i2 = decltype(ic)::value;
            if constexpr (q == (kB > kMfma + i2 ? kB : kMfma + i2)) {
              if constexpr (kAT) fa[0][i2] = tread(nxt_sa, toffA, i2, 0, kTPA);
              else fa[0][i2] = nxt_st[a_off + 16 * kChunks * i2 + pc0];
            }
          });
          static_for<NB>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j2 = decltype(jc)::value;
            constexpr int last = kMfma + MB * j2 + MB - 1;
            if constexpr (q == (kB > last ? kB : last)) {
              if constexpr (kBT) fb[0][j2] = tread(nxt_sa + kAreaA, toffB, j2, 0, kTPB);
              else fb[0][j2] = nxt_st[b_off + 16 * kChunks * j2 + pc0];
            }
          });
        }
        if constexpr (kCp) {
          if constexpr (q >= kB && q - kB < kCopies) copy_one(cb, q - kB);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      advance_copy();
      return;
    }
    // First half: step 0 of slab gs, with the loads of step 1.
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    load_frags(1, gs & 1, 1);
    mfma_step(0);
#pragma unroll
    for (int q = 0; q < kReadInstr; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kMfma - kReadInstr, 0);
    __builtin_amdgcn_sched_barrier(0);
    sync();
    __builtin_amdgcn_sched_barrier(0);
    // Second half: step 1 of slab gs, with the copy of slab gs + 2 and the
    // loads of slab gs + 1's step 0.
    const int rstage = (gs + 1) & 1;
#pragma unroll
    for (int q = 0; q < kMfma; ++q) {
      mfma_one(1, q);
      if constexpr (kCp) {
        if (q < kCopies) copy_one(cb, q);
      }
      if constexpr (kNext) {
        if (q < kReads) read_one(0, rstage, 0, q);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    advance_copy();
  };
  typedef std::integral_constant<bool, true> yes;
  typedef std::integral_constant<bool, false> no;

  // Prologue: slab 0 (tile 0), then slab 1 in flight.
  if (copier) copy_next(0);
  advance_copy();
  wait_and_sync();
  if (copier) copy_next(1);
  advance_copy();
  // (ahead, tc) now names slab 2 of the stream.
  load_frags(0, 0, 0);
  zero_acc();

  // The stream: one loop over the tiles, and inside it the slab loop once
  // for waves that issue copies and once for waves that do not (a
  // wave-uniform branch keeps each body straight-line; both execute the same
  // sequence of barriers) -- the epilogue's code exists once.  A tile's last
  // slab loads no fragments: the next tile's first ones are loaded after the
  // epilogue, which keeps the epilogue's registers free.  Past the end of the
  // stream the copies repeat the last slab into a stage nothing reads any
  // more (harmless; drained before the kernel ends), so every slab has the
  // same shape.
  const bool copies = C::kCopyWaves == C::kWaves || copier;
  int gs = 0;
  for (int j = 0; j < ntiles; ++j) {
    const int m0 = om[0], n0 = on[0], sp = os[0];
    // RAG: slab nk - 1 reaches past K when kv < BK; it is the next slab of
    // slab nk - 2 (nk >= 2: K > BK).  The next tile's first slab never is.
    const int zt = RAG && kv < BK ? nk - 2 : -1;
    if (copies) {
      for (int t = 0; t + 1 < nk; ++t, ++gs) slab(gs, yes(), yes(), t == zt);
      slab(gs, no(), yes(), false);
    } else {
      for (int t = 0; t + 1 < nk; ++t, ++gs) slab(gs, yes(), no(), t == zt);
      slab(gs, no(), no(), false);
    }
    ++gs;
    if constexpr (SPLIT) {
      epilogue_partial(m0, n0, sp);
    } else {
      (void)sp;
      epilogue(m0, n0, mlo0, nlo0);
    }
    zero_acc();
    --ahead;
    refresh_origins(j + 1);
    load_frags(0, gs & 1, 0);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0);   // drain the copies past the end of the stream
}

// PERSISTENT: at most `slots` workgroups (as many as the GPU runs at once),
// each walking its tiles; otherwise one workgroup per tile.
template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int GM, int COPY_SEL, int OPT = 0,
          bool PERSISTENT = true, bool EPI = false, int FMT = kFmtF16, bool SPLIT = false,
          bool RAG = false, int LAY = 0>
hipError_t launch(const Args16& a, int slots, hipStream_t stream) {
  typedef Config<BM, BN, BK, WAVES_M, WAVES_N, COPY_SEL> C;
  const int64_t tiles = RAG ? (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN)
                            : (int64_t)(a.M / BM) * (a.N / BN) * (SPLIT ? a.sk.splits : 1);
  const int64_t max_grid = int64_t(1) << 20;
  int64_t grid = PERSISTENT ? (tiles < slots ? tiles : slots) : (tiles < max_grid ? tiles : max_grid);
  if (grid < 1) grid = 1;
  TileArgs ta{a, tiles};
  void* args[] = {&ta};
  return hipLaunchKernel(
      (const void*)
          hgemm_nt_kernel<BM, BN, BK, WAVES_M, WAVES_N, GM, COPY_SEL, OPT, EPI, FMT, SPLIT, RAG,
                          LAY>,
      dim3((unsigned)grid), dim3(C::kThreads), args, 0, stream);
}

// Leading dimensions must also keep a lane's 32-bit copy offset (up to 8 rows
// into a copy) in range: ld < 2^28 elements.
template <int BM, int BN, int BK>
bool fits(int M, int N, int K, const void* A, int64_t lda, const void* B, int64_t ldb,
          const void* Cp, int64_t ldc) {
  constexpr int64_t kMaxLd = int64_t(1) << 28;
  return M % BM == 0 && N % BN == 0 && K % BK == 0 && aligned16(A) && aligned16(B) &&
         aligned16(Cp) && lda % 8 == 0 && ldb % 8 == 0 && ldc % 8 == 0 && lda < kMaxLd &&
         ldb < kMaxLd;
}

// The fused write-back reads bias and residual 4 halves (8 bytes) at a time
// at column offsets that are multiples of 4.
inline bool epi_fits(const void* bias, const void* res, int64_t ldr) {
  const uintptr_t b = reinterpret_cast<uintptr_t>(bias), q = reinterpret_cast<uintptr_t>(res);
  return (b & 7u) == 0 && (q & 7u) == 0 && (res == nullptr || ldr % 4 == 0);
}

}  // namespace hgemm
}  // namespace mi355gemm
