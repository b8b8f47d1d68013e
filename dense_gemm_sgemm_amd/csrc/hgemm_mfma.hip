// The 16-bit A * B^T fast path (fp16 and bf16): instances of the tile kernel
// template and the choice between them.
#include "hgemm_tile.hpp"

namespace mi355gemm {

namespace {
// Large tiles: 256 rows of C by 256 or 224 columns, 8 waves in a 4 x 2 grid
// of which waves 0-3 (one per SIMD) issue the slab copies, one persistent
// workgroup per CU.  Small tiles: 128 x 128, 4 waves in a 2 x 2 grid that all
// copy, two persistent workgroups per CU; or 128 x 192, the same 4 waves
// (64 x 96 each), one workgroup per CU (its two LDS stages take 80 KiB).  K
// slabs of 64; tiles grouped 8 tile-rows at a time per XCD.  The small tiles
// store C with streaming stores (OPT bit 0): they are chosen where all tiles
// fit in one round, so every CU stores at about the same time, and there the
// streaming stores measured 3-6 % faster (2048 x 2304 x 768: 16.5 against
// 17.5 us; 2048 x 2048 x 1024 and 1536 x 2560 x 2048 on 128 x 128); on the
// 256-row tiles they were even (4096^2 x 2048, one round) or 2.6 % slower
// (5376^2 x 2048, two rounds).
constexpr int BK = 64, GM = 8;

enum TileShape { kNone, k256x256, k256x224, k128x128, k128x192 };

// A launch takes about ceil(tiles / slots) tile-times.  A 256-row tile-time
// is proportional to its width (one workgroup per CU); a 128 x 128 tile
// shares its CU with a second workgroup, and its smaller operand reuse costs
// a fifth more time per output (measured: 1.20-1.21x on 5376^2 x 2048 and
// 8192^3), so its tile-time counts as 2 x 128 x 128 x 6/5 against 256 x BN.
// Ties go to the larger tile.  5376 x 5376 on 256 CUs: 256 wide -> 441
// tiles, 2 rounds x 65536; 224 wide -> 504 tiles, 2 rounds x 57344; 128 x 128
// -> 1764 tiles, 4 rounds x 39321.  2048 x 2304: 256 wide -> 72 tiles, 1 round
// x 65536; 128 x 128 -> 288 tiles, 1 round x 39321 (measured 1.44x faster);
// 128 x 192 -> 192 tiles, 1 round x 32768 (measured 1.19x faster than
// 128 x 128).  A 128 x 192 tile runs alone on its CU with 4 waves: a third
// more time per output than the 256-row tiles (tile-time 128 x 192 x 4/3).
// RAGGED: the same over ceil(M / bm) x ceil(N / bn) tiles (the ragged form),
// for the shapes at least one tile wide and tall.
TileShape choose(int M, int N, int cus, bool ragged = false, int64_t* cost_out = nullptr) {
  TileShape best = kNone;
  int64_t best_cost = 0;
  auto consider = [&](TileShape t, int bm, int bn, int slots, int64_t tile_time) {
    if (ragged ? (M < bm || N < bn) : (M % bm != 0 || N % bn != 0)) return;
    const int64_t tiles = ragged ? (int64_t)((M + bm - 1) / bm) * ((N + bn - 1) / bn)
                                 : (int64_t)(M / bm) * (N / bn);
    const int64_t cost = (tiles + slots - 1) / slots * tile_time;
    if (best == kNone || cost < best_cost) {
      best = t;
      best_cost = cost;
    }
  };
  consider(k256x256, 256, 256, cus, 256 * 256);
  consider(k256x224, 256, 224, cus, 256 * 224);
  consider(k128x128, 128, 128, 2 * cus, 2 * 128 * 128 * 6 / 5);
  consider(k128x192, 128, 192, cus, 128 * 192 * 4 / 3);
  if (cost_out) *cost_out = best_cost;
  return best;
}
}  // namespace

bool f16_mfma_fits(int M, int N, int K, const void* A, int64_t lda, const void* B, int64_t ldb,
                   const void* C, int64_t ldc) {
  return hgemm::fits<256, 256, BK>(M, N, K, A, lda, B, ldb, C, ldc) ||
         hgemm::fits<256, 224, BK>(M, N, K, A, lda, B, ldb, C, ldc) ||
         hgemm::fits<128, 128, BK>(M, N, K, A, lda, B, ldb, C, ldc) ||
         hgemm::fits<128, 192, BK>(M, N, K, A, lda, B, ldb, C, ldc);
}

template <bool EPI, int FMT>
hipError_t launch_shape(const Args16& a, int cus, hipStream_t stream) {
  switch (choose(a.M, a.N, cus)) {
    case k256x224:
      return hgemm::launch<256, 224, BK, 4, 2, GM, 1, 0, true, EPI, FMT, false>(a, cus,
                                                                                      stream);
    case k128x128:
      return hgemm::launch<128, 128, BK, 2, 2, GM, 0, 1, true, EPI, FMT, false>(a, 2 * cus,
                                                                                      stream);
    case k128x192:
      return hgemm::launch<128, 192, BK, 2, 2, GM, 0, 1, true, EPI, FMT, false>(a, cus,
                                                                                      stream);
    default:
      // 64 x 128 per wave: 128 accumulator registers leave room for one set
      // of B fragments only (OPT bit 1)
      return hgemm::launch<256, 256, BK, 4, 2, GM, 1, 2, true, EPI, FMT, false>(a, cus,
                                                                                      stream);
  }
}

// Products that are not whole tiles (RAG instances): the tile shape of the
// same cost model over ceil(M / bm) x ceil(N / bn) tiles.
template <bool EPI, int FMT>
hipError_t launch_ragged(const Args16& a, int cus, hipStream_t stream) {
  switch (choose(a.M, a.N, cus, true)) {
    case k256x224:
      return hgemm::launch<256, 224, BK, 4, 2, GM, 1, 0, true, EPI, FMT, false, true>(a, cus,
                                                                                      stream);
    case k128x128:
      return hgemm::launch<128, 128, BK, 2, 2, GM, 0, 1, true, EPI, FMT, false, true>(a, 2 * cus,
                                                                                      stream);
    case k128x192:
      return hgemm::launch<128, 192, BK, 2, 2, GM, 0, 1, true, EPI, FMT, false, true>(a, cus,
                                                                                      stream);
    default:
      return hgemm::launch<256, 256, BK, 4, 2, GM, 1, 2, true, EPI, FMT, false, true>(a, cus,
                                                                                      stream);
  }
}

bool f16_ragged_fits(int M, int N, int K, const void* A, int64_t lda, const void* B, int64_t ldb) {
  constexpr int64_t kMaxLd = int64_t(1) << 28;
  return M >= 128 && N >= 128 && K > BK && K % 8 == 0 && aligned16(A) && aligned16(B) &&
         lda % 8 == 0 && ldb % 8 == 0 && lda < kMaxLd && ldb < kMaxLd;
}

hipError_t launch_f16_mfma(const Args16& a, bool epi, int cus, hipStream_t stream) {
  if (!epi && f16_small_fits(a.M, a.N, a.K, a.A, a.lda, a.B, a.ldb, a.C, a.ldc, cus))
    return launch_f16_small(a, cus, stream);
  if (!f16_mfma_fits(a.M, a.N, a.K, a.A, a.lda, a.B, a.ldb, a.C, a.ldc) ||
      (epi && !hgemm::epi_fits(a.bias, a.res, a.ldr))) {
    if (a.fmt == kFmtBF16)
      return epi ? launch_ragged<true, kFmtBF16>(a, cus, stream)
                 : launch_ragged<false, kFmtBF16>(a, cus, stream);
    return epi ? launch_ragged<true, kFmtF16>(a, cus, stream)
               : launch_ragged<false, kFmtF16>(a, cus, stream);
  }
  if (a.fmt == kFmtBF16)
    return epi ? launch_shape<true, kFmtBF16>(a, cus, stream)
               : launch_shape<false, kFmtBF16>(a, cus, stream);
  return epi ? launch_shape<true, kFmtF16>(a, cus, stream)
             : launch_shape<false, kFmtF16>(a, cus, stream);
}


// Split-K partial products on 128 x 128 full tiles (two workgroups per CU):
// needs whole tiles and the fast path's alignment, and ranges of exactly
// per slabs each.
bool f16_partials_fit(const Args16& a) {
  return a.M % 128 == 0 && a.N % 128 == 0 &&
         hgemm::fits<128, 128, BK>(a.M, a.N, a.K, a.A, a.lda, a.B, a.ldb, a.C, a.ldc) &&
         (int64_t)a.sk.splits * a.sk.per == a.K / BK;
}

hipError_t launch_f16_partials_mfma(const Args16& a, int cus, hipStream_t stream) {
  if (a.fmt == kFmtBF16)
    return hgemm::launch<128, 128, BK, 2, 2, GM, 0, 0, true, false, kFmtBF16, true>(a, 2 * cus,
                                                                                     stream);
  return hgemm::launch<128, 128, BK, 2, 2, GM, 0, 0, true, false, kFmtF16, true>(a, 2 * cus, stream);
}

// NN (lay 1: B stored [K][N]), TT (lay 2: A stored [K][M]) and TN (lay 3:
// both) read in place by the full-tile kernels (their LAY instances), on
// whole tiles with K a multiple of 64 and the fast path's alignment.  Tile
// shapes, by the cost model of choose(): 224 x 256 for NN (waves of
// 112 x 64, the four B blocks per k-step through the transposing reads) or
// 256 x 224 for TT and TN (waves of 64 x 112), so that 5376 x 5376 still
// takes 504 tiles in two rounds; 256 x 256 (NN and TT), 128 x 128 (two
// workgroups per CU) and 128 x 192 (one) as for NT.
TileShape choose_kmajor(int lay, int M, int N, int cus, int64_t* cost_out = nullptr) {
  TileShape best = kNone;
  int64_t best_cost = 0;
  auto consider = [&](TileShape t, int bm, int bn, int slots, int64_t tile_time) {
    if (M % bm != 0 || N % bn != 0) return;
    const int64_t tiles = (int64_t)(M / bm) * (N / bn);
    const int64_t cost = (tiles + slots - 1) / slots * tile_time;
    if (best == kNone || cost < best_cost) {
      best = t;
      best_cost = cost;
    }
  };
  // TN on 256 x 256 (both operands transposed, one B set) spills 64
  // registers: 4096^3 took 142.5 us against 127.5 us through the copies
  if (lay != 3) consider(k256x256, 256, 256, cus, 256 * 256);
  if (lay == 1)
    consider(k256x224, 224, 256, cus, 224 * 256);   // NN: 224 rows x 256 columns
  else
    consider(k256x224, 256, 224, cus, 256 * 224);
  consider(k128x128, 128, 128, 2 * cus, 2 * 128 * 128 * 6 / 5);
  consider(k128x192, 128, 192, cus, 128 * 192 * 4 / 3);
  if (cost_out) *cost_out = best_cost;
  return best;
}

// Whether the K-major tiles take the product (whole tiles, the fast path's
// alignment and leading dimensions) at no more cost, in the model above, than
// the NT tiles would on transposed copies -- the copy's own time aside.  The
// choice is made when the call is planned, before any device query, for the
// chip's 256 CUs (the launch then picks the shape for the device's count).
// Measured: 4096^3 NN, TT, TN on 128 x 128 tiles (two rounds, against one
// of NT's 256 x 256) took 139-145 us in place against 119-129 us through the
// copies; with the 256 x 256 K-major tiles NN 117.0 against 118.1 us and TT
// 113.0 against 117.8 us; 2048^3 28-30 against 31-34 us, 2048 x 2304 x 768
// 16-17 against 20-22 us, 5376^2 x 2048 102-116 against 105-112 us.
bool f16_kmajor_fits(int lay, int M, int N, int K, const void* A, int64_t lda, const void* B,
                     int64_t ldb, const void* C, int64_t ldc) {
  constexpr int kPlanCus = 256;
  int64_t kcost = 0, ncost = 0;
  if (lay < 1 || lay > 3 || choose_kmajor(lay, M, N, kPlanCus, &kcost) == kNone) return false;
  if (choose(M, N, kPlanCus, false, &ncost) != kNone && ncost < kcost) return false;
  return hgemm::fits<64, 64, BK>(64, 64, K, A, lda, B, ldb, C, ldc);
}

template <int LAY, bool EPI, int FMT>
hipError_t launch_kmajor_lay(const Args16& a, int cus, hipStream_t stream) {
  switch (choose_kmajor(LAY, a.M, a.N, cus)) {
    case k128x128:
      return hgemm::launch<128, 128, BK, 2, 2, GM, 0, 1, true, EPI, FMT, false, false, LAY>(
          a, 2 * cus, stream);
    case k128x192:
      return hgemm::launch<128, 192, BK, 2, 2, GM, 0, 1, true, EPI, FMT, false, false, LAY>(
          a, cus, stream);
    case k256x256:
      // one set of B fragments, as for NT (OPT bit 1); never chosen for TN
      if constexpr (LAY != 3)
        return hgemm::launch<256, 256, BK, 4, 2, GM, 1, 2, true, EPI, FMT, false, false, LAY>(
            a, cus, stream);
      else
        return hipErrorInvalidValue;
    default:
      if constexpr (LAY == 1)
        return hgemm::launch<224, 256, BK, 2, 4, GM, 1, 0, true, EPI, FMT, false, false, 1>(
            a, cus, stream);
      else
        return hgemm::launch<256, 224, BK, 4, 2, GM, 1, 0, true, EPI, FMT, false, false, LAY>(
            a, cus, stream);
  }
}

template <bool EPI, int FMT>
hipError_t launch_kmajor(const Args16& a, int lay, int cus, hipStream_t stream) {
  if (lay == 1) return launch_kmajor_lay<1, EPI, FMT>(a, cus, stream);
  if (lay == 2) return launch_kmajor_lay<2, EPI, FMT>(a, cus, stream);
  return launch_kmajor_lay<3, EPI, FMT>(a, cus, stream);
}

hipError_t launch_f16_kmajor(const Args16& a, int lay, bool epi, int cus, hipStream_t stream) {
  if (a.fmt == kFmtBF16)
    return epi ? launch_kmajor<true, kFmtBF16>(a, lay, cus, stream)
               : launch_kmajor<false, kFmtBF16>(a, lay, cus, stream);
  return epi ? launch_kmajor<true, kFmtF16>(a, lay, cus, stream)
             : launch_kmajor<false, kFmtF16>(a, lay, cus, stream);
}

bool f16_epi_fits(const void* bias, const void* res, int64_t ldr) {
  return hgemm::epi_fits(bias, res, ldr);
}

}  // namespace mi355gemm
