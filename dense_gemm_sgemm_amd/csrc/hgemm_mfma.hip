// The 16-bit A * B^T fast path (fp16 and bf16): instances of the tile kernel
// template and the choice between them.
#include "hgemm_shapes.hpp"
#include "hgemm_tile.hpp"

namespace mi355gemm {

using namespace hshape;

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

bool f16_epi_fits(const void* bias, const void* res, int64_t ldr) {
  return hgemm::epi_fits(bias, res, ldr);
}

}  // namespace mi355gemm
