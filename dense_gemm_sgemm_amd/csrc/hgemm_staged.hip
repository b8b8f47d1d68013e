// 16-bit (fp16 or bf16) C = A * B^T for large products of any shape,
// leading dimension and 2-byte alignment, with no operand copy and no
// workspace.
//
// The boundary rule is the one of page 1 ("第 6 章 Shared Memory & Tile",
// exercise 7 of section 6.9: arbitrary M, N, K; section 6.5.8: the load
// unit fills out-of-range elements with zeros); the NT page ("从零开始的 AI
// Infra: 算子基础与GPU架构", sections 19 and 29) motivates it with a shape
// that is not a multiple of any tile.  Its tile structure follows that page's
// large per-warp tiles (sections 17-18) and multi-stage pipeline (sections
// 10-12), re-done for gfx950:
//
//  * one workgroup of 4 waves per CU, one wave per SIMD, owns a 256 x BN tile
//    of C (BN = 256 or 224); each wave owns 128 x BN/2, built from 16 x 16
//    blocks of v_mfma_f32_16x16x32_f16 (_bf16).  With one wave per SIMD a
//    wave may hold 512 registers: the 64 (or 56) accumulator quads live in
//    the AGPRs for the whole tile -- the matrix instructions are asm
//    statements whose accumulator operand is an AGPR tuple, so the compiler
//    never moves them -- and the operand fragments of the current and the
//    next slab in the VGPRs (two sets);
//  * K is walked in slabs of 32 (rows of 64 bytes, 4 chunks), with one
//    barrier per slab.  Rows at 16-byte addresses (DIRECT) are copied global
//    -> LDS with global_load_lds_dwordx4 into a ring of four LDS stages:
//    during slab s the copies of slab s + 4 and the fragment reads of slab
//    s + 1 are spread over the slab's 64 (56) matrix instructions, and the
//    barrier at the top of slab s waits for this wave's copies of slab s + 1
//    only (the two slabs after it stay in flight).  Rows at 2-byte addresses
//    are register-staged instead (the direct copies of such rows measured
//    slower): each thread loads 16-byte chunks with ordinary loads
//    (unaligned access is enabled on this target) and writes them to LDS one
//    slab later; during slab s the loads of slab s + 3, the LDS writes of
//    slab s + 2 and the fragment reads of slab s + 1 share the slab's matrix
//    instructions, with two LDS stages;
//  * chunk c of slab row r sits at position c ^ ((r >> 2) & 2).  Under the
//    measured ds_read_b128 bank model (64 banks of 4 bytes, 16 lanes served
//    per cycle in the groups {0-3, 12-15, 20-23, 24-27} and {4-7, 8-11,
//    16-19, 28-31}, and the same + 32) the fragment reads (lane l: row
//    l % 16, chunk l / 16) touch 16 distinct bank quads per group, and each
//    8-lane group of LDS writes covers 128 contiguous bytes;
//  * boundaries: a row past M or N re-reads the matrix's last row (its
//    products are never stored); in a slab that reaches past K each chunk is
//    loaded from a start clamped to K - 8 and shifted and zero-filled --
//    in registers before its LDS write, or (DIRECT) in LDS by the thread
//    whose copy wrote it, once the copy has landed and before the barrier
//    after which the slab is read -- so every chunk is always exactly one
//    load instruction;
//  * B is the first MFMA operand, so a lane's accumulator quad holds four
//    consecutive columns of one row; the epilogue applies the fused
//    write-back (bias, activation, residual in fp32) where asked, rounds
//    once, stages 16 rows at a time per wave through LDS and stores 16-byte
//    row segments (streaming stores), element by element where a segment
//    leaves the matrix, nothing past M or N, C at any alignment;
//  * tiles are persistent (one workgroup per CU walks its tiles as one
//    stream of slabs, so the next tile's first slabs load while the current
//    one finishes) and ordered per XCD (map_tile).
//
// Preconditions (checked by the host): M, N >= 1, K >= 8, leading dimensions
// below 2^23 elements (a chunk's 32-bit byte offset from its tile's first row
// stays below 2^32).
#include "hgemm_tile.hpp"

namespace mi355gemm {
namespace hstaged {

using hgemm::f4;
using hgemm::h4;
using hgemm::h8;
using hgemm::map_tile;
using hgemm::static_for;

template <int BN_, bool DIRECT_>
struct Cfg {
  static constexpr int BM = 256, BN = BN_, BK = 32;
  static constexpr int kThreads = 256;
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int kBM = WM / 16, kBN = WN / 16;        // blocks per wave
  static constexpr int kMfma = kBM * kBN;                    // per wave per slab
  static constexpr int kReads = kBM + kBN;                   // fragments per wave per slab
  static constexpr int kRow = 2 * BK;                        // bytes per slab row
  static constexpr int kStage = (BM + BN) * kRow;
  // thread t stages chunks t + 256 u: slab row (t >> 2) + 64 u, chunk t & 3
  static constexpr int kLoads = (BM + BN + 63) / 64;         // 8
  static constexpr int kLoadsA = BM / 64;                    // the first 4 are rows of A
  static constexpr int kOutRowBytes = 256;
  static constexpr int kOutBytes = 4 * 16 * kOutRowBytes;
  static constexpr int kStages = DIRECT_ ? 4 : 2;
  static constexpr int kLds = kStages * kStage + kOutBytes;
  static_assert(kLds <= 160 * 1024, "LDS");
};

// Position of chunk c (16 bytes) in slab row r.
__device__ __forceinline__ int swz(int r) { return (r >> 2) & 2; }

// acc += b * a^T on the matrix cores, the accumulator kept in AGPRs.
template <int FMT>
__device__ __forceinline__ void mma(f4& acc, const h8& b, const h8& a) {
  if constexpr (FMT == kFmtF16) {
    asm("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a));
  } else {
    asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a));
  }
}

// The 8 elements k .. k + 7 of a row, given the 8 elements loaded from
// kc = min(k, K - 8) .. kc + 7: elements shift down by k - kc and those at or
// past K become zero.  Done on the four 32-bit words of the chunk.
__device__ __forceinline__ h8 tail_fix(h8 x, int k, int K) {
  const int kc = k < K - 8 ? k : K - 8;
  const int s = k - kc;                      // 0 .. 7 while k < K
  const int nv = K - k;                      // valid elements (<= 0: none)
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  const u4 w = __builtin_bit_cast(u4, x);
  const int q = s >> 1;
  uint32_t y[5];
#pragma unroll
  for (int d = 0; d < 5; ++d) {
    const uint32_t w0 = d < 4 ? w[d] : 0u, w1 = d + 1 < 4 ? w[d + 1] : 0u;
    const uint32_t w2 = d + 2 < 4 ? w[d + 2] : 0u, w3 = d + 3 < 4 ? w[d + 3] : 0u;
    y[d] = q == 0 ? w0 : q == 1 ? w1 : q == 2 ? w2 : w3;
  }
  u4 z;
#pragma unroll
  for (int d = 0; d < 4; ++d)
    z[d] = (s & 1) ? __builtin_amdgcn_alignbyte(y[d + 1], y[d], 2) : y[d];
  h8 v = __builtin_bit_cast(h8, z);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (e >= nv) v[e] = (half_t)0;
  return v;
}

constexpr int kWaitLgkm0 = 0xC07F;      // s_waitcnt lgkmcnt(0)
constexpr int kWaitVmLgkm0 = 0x0070;    // s_waitcnt vmcnt(0) lgkmcnt(0)
// s_waitcnt vmcnt(vm) (vm < 64)
constexpr int wait_vm(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (15 << 8); }

struct Args {
  Args16 p;
  int64_t tiles;
};

template <int BN, int FMT, bool EPI, bool DIRECT>
__global__ __launch_bounds__(256, 1) void hgemm_staged_kernel(Args ta) {
  typedef Cfg<BN, DIRECT> C;
  constexpr int BM = C::BM, kBM = C::kBM, kBN = C::kBN;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[C::kLds];
  const Args16& p = ta.p;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = (wave >> 1) * C::WM, wn = (wave & 1) * C::WN;
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  const int64_t stride = gridDim.x;
  const int ntiles = (int)((ta.tiles - blockIdx.x + stride - 1) / stride);
  // slabs per tile, rounded up to an even count (slabs past K are zeros)
  const int nk = (p.K + 2 * C::BK - 1) / (2 * C::BK) * 2;
  auto origin = [&](int j, int& m0, int& n0) __attribute__((always_inline)) {
    int tm, tn;
    map_tile<8>(blockIdx.x + (int64_t)j * stride, tiles_m, tiles_n, tm, tn);
    m0 = tm * BM;
    n0 = tn * BN;
  };

  // ---- staging.  Thread t loads chunks t + 256 u: slab row R = (t >> 2) +
  // 64 u -- rows of A for u < 4, then of B -- chunk t & 3, and writes each
  // one to row R at position (t & 3) ^ swz(R), the same for every u since
  // 64 u keeps R's bits 2-3.  With BN = 224 the last chunk of threads
  // 128-255 lies past the slab (R >= 480): it re-reads the chunk 64 rows up
  // and is not written.  roff[u] is the byte offset of the chunk's row from
  // the tile's first row (re-computed per tile: rows past the matrix clamp
  // to its last row).
  const int lrow = tid >> 2, lchunk = tid & 3;
  const int lpos = 16 * (lchunk ^ swz(lrow));
  int cj = 0, ct = 0, cm0 = 0, cn0 = 0;        // the load target: slab ct of tile cj
  origin(0, cm0, cn0);
  uint32_t roff[C::kLoads];
  auto set_offsets = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < C::kLoads; ++u) {
      int R = lrow + 64 * u;
      if (R >= BM + BN) R -= 64;
      const bool isA = u < C::kLoadsA;
      const int row0 = isA ? cm0 : cn0, lim = isA ? p.M : p.N;
      int row = row0 + (isA ? R : R - BM);
      row = row < lim ? row : lim - 1;
      roff[u] = (uint32_t)((int64_t)(row - row0) * (isA ? p.lda : p.ldb) * 2);
    }
  };
  set_offsets();
  // koff: byte offset of this lane's chunk in its row for the load target
  // slab, the chunk start clamped to K - 8 (re-computed once per slab); each
  // load is then a wave-uniform row-0 base plus one 32-bit lane offset.  A
  // direct copy writes lane l's 16 bytes to position l & 3 of its row, so the
  // lane loads logical chunk kchunk = (l & 3) ^ swz(row) there.
  const int kchunk = DIRECT ? lchunk ^ swz(lrow) : lchunk;
  const int kmax = p.K - 8;
  uint32_t koff = 0;
  auto set_koff = [&]() __attribute__((always_inline)) {
    const int k = ct * C::BK + 8 * kchunk;
    koff = (uint32_t)(2 * (k < kmax ? k : kmax));
  };
  set_koff();
  // Past the end of the stream the target stays on the last slab of the last
  // tile, so that every slab issues the same loads (their data is not used).
  auto advance_load = [&]() __attribute__((always_inline)) {
    if (++ct == nk) {
      if (cj + 1 < ntiles) {
        ct = 0;
        origin(++cj, cm0, cn0);
        set_offsets();
      } else {
        ct = nk - 1;
      }
    }
    set_koff();
  };
  // DIRECT: copy u of this wave fills slab rows 16 w + 64 u .. + 15 (with
  // BN = 224, waves 2 and 3 have no eighth row group and repeat their seventh,
  // the same data to the same place, so that every wave issues the same
  // number of copies per slab and one wait count serves them all).
  auto copy_one = [&](int stage, int u) __attribute__((always_inline)) {
    const int uu = (C::kLoads * 64 > BM + BN && u == C::kLoads - 1 && 16 * wave + 64 * u >= BM + BN)
                       ? u - 1 : u;
    const char* base = uu < C::kLoadsA ? (const char*)(p.A + (int64_t)cm0 * p.lda)
                                       : (const char*)(p.B + (int64_t)cn0 * p.ldb);
    __builtin_amdgcn_global_load_lds(
        (hgemm::gbl_void_t*)(base + roff[uu] + koff),
        (hgemm::lds_void_t*)(lds + stage * C::kStage + (16 * wave + 64 * uu) * C::kRow), 16, 0, 0);
  };
  // DIRECT: slab ts of a tile reaches past K and has landed in `stage`: each
  // thread shifts and zero-fills the chunks its own copies wrote.
  auto fix_tail = [&](int stage, int ts) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < C::kLoads; ++u) {
      const int R = lrow + 64 * u;
      if (C::kLoads * 64 > BM + BN && u == C::kLoads - 1 && R >= BM + BN) continue;
      h8* q = (h8*)(lds + stage * C::kStage + R * C::kRow + 16 * lchunk);
      *q = tail_fix(*q, ts * C::BK + 8 * kchunk, p.K);
    }
  };
  h8 stg[2][C::kLoads];
  auto load_one = [&](int set, int u) __attribute__((always_inline)) {
    const bool isA = u < C::kLoadsA;
    const char* base = isA ? (const char*)(p.A + (int64_t)cm0 * p.lda)
                           : (const char*)(p.B + (int64_t)cn0 * p.ldb);
    const uint32_t off = roff[u] + koff;
    h8 v;
    __builtin_memcpy(&v, base + off, 16);
    if (set == 0) stg[0][u] = v;
    else stg[1][u] = v;
  };
  // wt: the slab (within its tile) whose chunks the LDS writes store
  int wt = 0;
  auto write_one = [&](int set, int stage, int u) __attribute__((always_inline)) {
    const int R = lrow + 64 * u;
    if (C::kLoads * 64 > BM + BN && u == C::kLoads - 1 && R >= BM + BN) return;
    h8 v = set == 0 ? stg[0][u] : stg[1][u];
    if (wt * C::BK + C::BK > p.K) v = tail_fix(v, wt * C::BK + 8 * lchunk, p.K);
    *(h8*)(lds + stage * C::kStage + R * C::kRow + lpos) = v;
  };

  // ---- fragment reads: lane l reads row (block base) + l % 16, chunk l / 16.
  const int r = lane & 15, g = lane >> 4;
  const int rpos = 16 * (g ^ swz(r));
  const int a_off = (wm + r) * C::kRow + rpos;
  const int b_off = (BM + wn + r) * C::kRow + rpos;
  h8 fa[2][kBM], fb[2][kBN];
  auto read_frag = [&](int set, int stage, int f) __attribute__((always_inline)) {
    const unsigned char* st = lds + stage * C::kStage;
    if (f < kBM) {
      const h8 v = *(const h8*)(st + a_off + f * 16 * C::kRow);
      if (set == 0) fa[0][f] = v;
      else fa[1][f] = v;
    } else {
      const int j = f - kBM;
      const h8 v = *(const h8*)(st + b_off + j * 16 * C::kRow);
      if (set == 0) fb[0][j] = v;
      else fb[1][j] = v;
    }
  };

  f4 acc[kBM][kBN];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kBM; ++i)
#pragma unroll
      for (int j = 0; j < kBN; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};
  };

  // One slab (index gs, of parity SET): its matrix instructions on fragment
  // set SET, with the fragment reads of slab gs + 1 into set 1 - SET, and
  // either (DIRECT) the copies of slab gs + 4 or the LDS writes of slab gs + 2
  // from staging set SET and the loads of slab gs + 3 into staging set
  // 1 - SET, spread over them.  Past the end of the
  // stream the reads, loads and writes still happen (on a stage or registers
  // nothing uses any more), so that every slab has the same instruction
  // stream; the compiler then waits for exactly the load each LDS write
  // needs.
  auto slab = [&](auto set_c, int gs) __attribute__((always_inline)) {
    constexpr int SET = decltype(set_c)::value;
    const int rstage = (gs + 1) & (C::kStages - 1), wstage = gs & (C::kStages - 1);
    static_for<C::kMfma>([&](auto qc) __attribute__((always_inline)) {
      constexpr int q = decltype(qc)::value;
      constexpr int i = q / kBN, j = q % kBN;
      mma<FMT>(acc[i][j], fb[SET][j], fa[SET][i]);
      // The next slab's fragments go to the other set, evenly spaced (a
      // single A set, each fragment reloaded right after its row's last
      // product, measured 4-5 % slower on 5000 x 3001 x 1537).
      static_for<C::kReads>([&](auto rc) __attribute__((always_inline)) {
        constexpr int f = decltype(rc)::value;
        if constexpr (q == f * (C::kMfma / C::kReads) + 2) read_frag(1 - SET, rstage, f);
      });
      static_for<C::kLoads>([&](auto uc) __attribute__((always_inline)) {
        constexpr int u = decltype(uc)::value;
        if constexpr (q == u * C::kMfma / C::kLoads + 2) {
          if constexpr (DIRECT) {
            copy_one(wstage, u);         // slab gs + 4, into slab gs's stage
          } else {
            write_one(SET, wstage, u);
            load_one(1 - SET, u);
          }
        }
      });
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (!DIRECT) {
      if (++wt == nk) wt = 0;
    }
    advance_load();
  };

  // Top of a slab: this wave's fragment reads of the slab and its LDS writes
  // of the next one are done (DIRECT: its copies of the next slab -- index ts
  // in its tile, in `stage` -- have landed, and are fixed if that slab
  // reaches past K); then the workgroup meets, after which the next slab is
  // complete in LDS and every read of the previous slab's stage is done.
  // Right after an epilogue (whose stores follow the loads in flight) every
  // memory operation is waited for.
  auto top = [&](bool after_epi, int stage, int ts) __attribute__((always_inline)) {
    if constexpr (DIRECT) {
      if (after_epi) __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0);
      else __builtin_amdgcn_s_waitcnt(wait_vm(2 * C::kLoads));
      if ((ts + 1) * C::BK > p.K) fix_tail(stage, ts);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    } else {
      (void)stage;
      (void)ts;
      if (after_epi) __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0);
      else __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    }
    asm volatile("s_barrier" ::: "memory");
  };

  // Epilogue of the tile at (m0, n0): acc[i][j][v] is
  // C[m0 + wm + 16 i + r][n0 + wn + 16 j + 4 g + v].  Row block i at a time,
  // the quads are rounded and written (8 bytes per lane) to this wave's
  // 16-row staging area, chunk c of staging row R at slot c ^ R, then row
  // segments of 8 are stored, element by element where a segment crosses N.
  unsigned char* stage_out = lds + C::kStages * C::kStage + wave * (16 * C::kOutRowBytes);
  auto epilogue = [&](int m0, int n0) __attribute__((always_inline)) {
    const int cc = lane & 15;
    h4 bq[kBN];
    if constexpr (EPI) {
#pragma unroll
      for (int j = 0; j < kBN; ++j) {
        const int n = n0 + wn + 16 * j + 4 * g;
        bq[j] = h4{};
        if (p.bias) {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (n + v < p.N) bq[j][v] = p.bias[n + v];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kBM; ++i) {
      const int64_t m = m0 + wm + 16 * i + r;
      h4 rq[kBN];
      if constexpr (EPI) {
#pragma unroll
        for (int j = 0; j < kBN; ++j) {
          const int n = n0 + wn + 16 * j + 4 * g;
          rq[j] = h4{};
          if (p.res && m < p.M) {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (n + v < p.N) rq[j][v] = p.res[m * p.ldr + n + v];
          }
        }
      }
#pragma unroll
      for (int j = 0; j < kBN; ++j) {
        h4 o;
        const f4 a = acc[i][j];
        if constexpr (EPI) {
          f4 x = a;
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
          for (int v = 0; v < 4; ++v) o[v] = f32_to_word<FMT>(x[v] + word_to_f32<FMT>(rq[j][v]));
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v) o[v] = f32_to_word<FMT>(a[v]);
        }
        const int c = 2 * j + (g >> 1);
        *(h4*)(stage_out + r * C::kOutRowBytes + 16 * (c ^ r) + 8 * (g & 1)) = o;
      }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int R = 4 * q + (lane >> 4);
        const h8 v = *(const h8*)(stage_out + R * C::kOutRowBytes + 16 * (cc ^ R));
        const int64_t mm = m0 + wm + 16 * i + R;
        const int n = n0 + wn + 8 * cc;
        if ((C::WN == 128 || cc < C::WN / 8) && mm < p.M && n < p.N) {
          half_t* dst = p.C + mm * p.ldc + n;
          if (n + 8 <= p.N) {
            // streaming store: 2-3 % faster than a plain one here (all CUs
            // store their tiles at about the same time in these products)
            __builtin_nontemporal_store(v, (h8*)dst);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (n + e < p.N) dst[e] = v[e];
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    }
  };

  typedef std::integral_constant<int, 0> S0;
  typedef std::integral_constant<int, 1> S1;

  // Prologue.  DIRECT: slabs 0-3 copied to stages 0-3, then slab 0 waited
  // for (and fixed if it reaches past K).  Otherwise slab 0 written to stage
  // 0 and slab 1 to stage 1, slab 2 loaded into staging set 0 (the stream has
  // at least two slabs).  Then slab 0's fragments are read into set 0.
  if constexpr (DIRECT) {
    for (int st = 0; st < C::kStages; ++st) {
#pragma unroll
      for (int u = 0; u < C::kLoads; ++u) copy_one(st, u);
      advance_load();
    }
    __builtin_amdgcn_s_waitcnt(wait_vm(3 * C::kLoads));
    if (C::BK > p.K) fix_tail(0, 0);
  } else {
#pragma unroll
    for (int u = 0; u < C::kLoads; ++u) load_one(0, u);
    advance_load();
#pragma unroll
    for (int u = 0; u < C::kLoads; ++u) load_one(1, u);
    advance_load();
#pragma unroll
    for (int u = 0; u < C::kLoads; ++u) write_one(0, 0, u);
    if (++wt == nk) wt = 0;
#pragma unroll
    for (int u = 0; u < C::kLoads; ++u) write_one(1, 1, u);
    if (++wt == nk) wt = 0;
#pragma unroll
    for (int u = 0; u < C::kLoads; ++u) load_one(0, u);
    advance_load();
  }
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  asm volatile("s_barrier" ::: "memory");
#pragma unroll
  for (int f = 0; f < C::kReads; ++f) read_frag(0, 0, f);
  zero_acc();

  int gs = 0;
  bool after_epi = false;
  for (int j = 0; j < ntiles; ++j) {
    int m0, n0;
    origin(j, m0, n0);
    for (int t = 0; t < nk; t += 2) {
      top(after_epi, (gs + 1) & (C::kStages - 1), t + 1);
      after_epi = false;
      slab(S0(), gs);
      ++gs;
      top(false, (gs + 1) & (C::kStages - 1), t + 2 == nk ? 0 : t + 2);
      slab(S1(), gs);
      ++gs;
    }
    epilogue(m0, n0);
    zero_acc();
    after_epi = true;
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0);
}

template <int BN, int FMT, bool EPI, bool DIRECT>
hipError_t launch_bn(const Args16& a, int cus, hipStream_t stream) {
  const int64_t tiles = (int64_t)((a.M + 255) / 256) * ((a.N + BN - 1) / BN);
  int64_t grid = tiles < cus ? tiles : cus;
  if (grid < 1) grid = 1;
  Args ta{a, tiles};
  void* args[] = {&ta};
  return hipLaunchKernel((const void*)hgemm_staged_kernel<BN, FMT, EPI, DIRECT>, dim3((unsigned)grid),
                         dim3(256), args, 0, stream);
}

// 256 x 256 or 256 x 224 tiles, whichever takes fewer rounds of persistent
// workgroups times tile width (5000 x 3001 on 256 CUs: 240 tiles of 256 x 256
// in one round, against 280 of 256 x 224 in two).
template <int FMT, bool EPI, bool DIRECT>
hipError_t launch_tiles(const Args16& a, int cus, hipStream_t stream) {
  const int64_t tm = (a.M + 255) / 256;
  const int64_t r256 = (tm * ((a.N + 255) / 256) + cus - 1) / cus;
  const int64_t r224 = (tm * ((a.N + 223) / 224) + cus - 1) / cus;
  if (r224 * 224 < r256 * 256) return launch_bn<224, FMT, EPI, DIRECT>(a, cus, stream);
  return launch_bn<256, FMT, EPI, DIRECT>(a, cus, stream);
}

// Direct copies when every row of A and B starts at a 16-byte address.
template <int FMT, bool EPI>
hipError_t launch_fmt(const Args16& a, int cus, hipStream_t stream) {
  const bool direct = aligned16(a.A) && aligned16(a.B) && a.lda % 8 == 0 && a.ldb % 8 == 0;
  return direct ? launch_tiles<FMT, EPI, true>(a, cus, stream)
                : launch_tiles<FMT, EPI, false>(a, cus, stream);
}

}  // namespace hstaged

bool f16_staged_fits(int M, int N, int K, int64_t lda, int64_t ldb) {
  constexpr int64_t kMaxLd = int64_t(1) << 23;
  return M >= 1 && N >= 1 && K >= 8 && lda < kMaxLd && ldb < kMaxLd;
}

hipError_t launch_f16_staged(const Args16& a, bool epi, int cus, hipStream_t stream) {
  if (a.fmt == kFmtBF16)
    return epi ? hstaged::launch_fmt<kFmtBF16, true>(a, cus, stream)
               : hstaged::launch_fmt<kFmtBF16, false>(a, cus, stream);
  return epi ? hstaged::launch_fmt<kFmtF16, true>(a, cus, stream)
             : hstaged::launch_fmt<kFmtF16, false>(a, cus, stream);
}

}  // namespace mi355gemm
