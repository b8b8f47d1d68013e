// The 16-bit full-tile kernels with K-major operands read in place (gemm_ex
// NN, TT and TN): instances of the tile kernel template and the choice
// between them.
#include "hgemm_shapes.hpp"
#include "hgemm_tile.hpp"

namespace mi355gemm {

using namespace hshape;

// NN (lay 1: B stored [K][N]), TT (lay 2: A stored [K][M]) and TN (lay 3:
// both) read in place by the full-tile kernels (their LAY instances), with A
// and B rows at 16-byte addresses.  Tile shapes, by
// the cost model of choose(): 224 x 256 for NN (waves of
// 112 x 64, the four B blocks per k-step through the transposing reads) or
// 256 x 224 for TT and TN (waves of 64 x 112), so that 5376 x 5376 still
// takes 504 tiles in two rounds; 256 x 256 (NN and TT), 128 x 128 (two
// workgroups per CU) and 128 x 192 (one) as for NT.
//
// RAGGED: the same over ceil(M / bm) x ceil(N / bn) tiles (the ragged form:
// the last tile row and column shifted back to end at M and N, and a K tail
// taken by a last slab copied from K - 64), for shapes at least one tile wide
// and tall.
namespace {
TileShape choose_kmajor(int lay, int M, int N, int cus, bool ragged = false,
                        int64_t* cost_out = nullptr) {
  TileShape best = kNone;
  int64_t best_cost = 0;
  auto consider = [&](TileShape t, int bm, int bn, int slots, int64_t tile_time) {
    if (ragged ? (M < bm || N < bn) : (M % bm != 0 || N % bn != 0)) return;
    const int64_t tiles = ragged ? (int64_t)((M + bm - 1) / bm) * ((N + bn - 1) / bn)
                                 : (int64_t)(M / bm) * (N / bn);
    // 128 x 128 tiles that do not outnumber the CUs each get a CU to
    // themselves: about 0.8 of a 128 x 192 tile-time (see the model above)
    if (t == k128x128 && tiles <= cus) tile_time = 128 * 128 * 8 / 5;
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

// At least 2^30 multiply-adds: where the A * B^T path on copies would take
// its ragged form (smaller ragged products take the edge kernel there).
bool large(int M, int N, int K) { return (int64_t)M * N * K >= (int64_t(1) << 30); }
}  // namespace

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
//
// Ragged M or N, or K not a multiple of 64 (C at any 2-byte address): the
// ragged form of the K-major tiles, for large products at least 128 wide and
// tall, against the NT tiles -- whole, or ragged where K % 8 == 0 -- on the
// copies.  Its last slab is copied from K - 64 (K > 64), which keeps the
// K-contiguous operand's chunks at 16-byte addresses only for K % 8 == 0: NN
// and TT need that, TN (both operands K-major) takes any K.
bool f16_kmajor_fits(int lay, int M, int N, int K, const void* A, int64_t lda, const void* B,
                     int64_t ldb, const void* C, int64_t ldc) {
  constexpr int kPlanCus = 256;
  constexpr int64_t kMaxLd = int64_t(1) << 28;
  if (lay < 1 || lay > 3 || K <= 0 || !aligned16(A) || !aligned16(B) || lda % 8 != 0 ||
      ldb % 8 != 0 || lda >= kMaxLd || ldb >= kMaxLd)
    return false;
  const bool whole_k = K % BK == 0;
  if (!whole_k && (K < BK || (lay != 3 && K % 8 != 0))) return false;
  int64_t kcost = 0, ncost = 0;
  if (whole_k && choose_kmajor(lay, M, N, kPlanCus, false, &kcost) != kNone) {
    // whole tiles: C 16-byte aligned as well
    if (!aligned16(C) || ldc % 8 != 0) return false;
    return choose(M, N, kPlanCus, false, &ncost) == kNone || kcost <= ncost;
  }
  if (!large(M, N, K) || choose_kmajor(lay, M, N, kPlanCus, true, &kcost) == kNone) return false;
  if (whole_k && choose(M, N, kPlanCus, false, &ncost) != kNone) return kcost <= ncost;
  if (K % 8 == 0 && choose(M, N, kPlanCus, true, &ncost) != kNone) return kcost <= ncost;
  return true;
}

template <int LAY, bool EPI, int FMT, bool RAG>
hipError_t launch_kmajor_lay(const Args16& a, TileShape t, int cus, hipStream_t stream) {
  switch (t) {
    case k128x128:
      return hgemm::launch<128, 128, BK, 2, 2, GM, 0, 1, true, EPI, FMT, false, RAG, LAY>(
          a, 2 * cus, stream);
    case k128x192:
      return hgemm::launch<128, 192, BK, 2, 2, GM, 0, 1, true, EPI, FMT, false, RAG, LAY>(
          a, cus, stream);
    case k256x256:
      // one set of B fragments, as for NT (OPT bit 1); never chosen for TN
      if constexpr (LAY != 3)
        return hgemm::launch<256, 256, BK, 4, 2, GM, 1, 2, true, EPI, FMT, false, RAG, LAY>(
            a, cus, stream);
      else
        return hipErrorInvalidValue;
    case k256x224:
      if constexpr (LAY == 1)
        return hgemm::launch<224, 256, BK, 2, 4, GM, 1, 0, true, EPI, FMT, false, RAG, 1>(
            a, cus, stream);
      else
        return hgemm::launch<256, 224, BK, 4, 2, GM, 1, 0, true, EPI, FMT, false, RAG, LAY>(
            a, cus, stream);
    default:
      return hipErrorInvalidValue;
  }
}

// Whole tiles where they fit and K is a multiple of 64, else the ragged form.
template <int LAY, bool EPI, int FMT>
hipError_t launch_kmajor_any(const Args16& a, int cus, hipStream_t stream) {
  const TileShape whole = a.K % BK == 0 ? choose_kmajor(LAY, a.M, a.N, cus) : kNone;
  if (whole != kNone) return launch_kmajor_lay<LAY, EPI, FMT, false>(a, whole, cus, stream);
  return launch_kmajor_lay<LAY, EPI, FMT, true>(a, choose_kmajor(LAY, a.M, a.N, cus, true), cus,
                                                stream);
}

template <bool EPI, int FMT>
hipError_t launch_kmajor(const Args16& a, int lay, int cus, hipStream_t stream) {
  if (lay == 1) return launch_kmajor_any<1, EPI, FMT>(a, cus, stream);
  if (lay == 2) return launch_kmajor_any<2, EPI, FMT>(a, cus, stream);
  return launch_kmajor_any<3, EPI, FMT>(a, cus, stream);
}

hipError_t launch_f16_kmajor(const Args16& a, int lay, bool epi, int cus, hipStream_t stream) {
  if (a.fmt == kFmtBF16)
    return epi ? launch_kmajor<true, kFmtBF16>(a, lay, cus, stream)
               : launch_kmajor<false, kFmtBF16>(a, lay, cus, stream);
  return epi ? launch_kmajor<true, kFmtF16>(a, lay, cus, stream)
             : launch_kmajor<false, kFmtF16>(a, lay, cus, stream);
}

}  // namespace mi355gemm
