// The fp16 A * B^T fast path: instances of the tile kernel template and the
// choice between them.
#include "hgemm_tile.hpp"

namespace mi355gemm {

namespace {
// Tiles are 256 rows of C by 256 or 224 columns, K slabs of 64, 8 waves in a
// 4 x 2 grid of which waves 0-3 (one per SIMD) issue the slab copies; tiles
// are grouped 8 tile-rows at a time per XCD; one persistent workgroup per CU.
constexpr int BM = 256, BK = 64, GM = 8;
}  // namespace

bool f16_mfma_fits(int M, int N, int K, const void* A, int64_t lda, const void* B, int64_t ldb,
                   const void* C, int64_t ldc) {
  return (hgemm::fits<BM, 256, BK>(M, N, K, A, lda, B, ldb, C, ldc) ||
          hgemm::fits<BM, 224, BK>(M, N, K, A, lda, B, ldb, C, ldc));
}

// With one workgroup per CU at a time, a launch takes about ceil(tiles / cus)
// tile-times, and a tile-time is proportional to the tile width: pick the
// width with the smaller product (256 on a tie).  5376 x 5376 on 256 CUs:
// 256 wide -> 441 tiles, 2 rounds x 256 = 512; 224 wide -> 504 tiles,
// 2 rounds x 224 = 448.
int f16_mfma_tile_n(int M, int N, int cus) {
  const bool w256 = N % 256 == 0, w224 = N % 224 == 0;
  if (!(w256 && w224)) return w256 ? 256 : 224;
  const int64_t t256 = (int64_t)(M / BM) * (N / 256), t224 = (int64_t)(M / BM) * (N / 224);
  const int64_t cost256 = (t256 + cus - 1) / cus * 256, cost224 = (t224 + cus - 1) / cus * 224;
  return cost224 < cost256 ? 224 : 256;
}

hipError_t launch_f16_mfma(const F16Args& a, bool epi, int cus, hipStream_t stream) {
  const bool w224 = f16_mfma_tile_n(a.M, a.N, cus) == 224;
  if (epi) {
    return w224 ? hgemm::launch<BM, 224, BK, 4, 2, GM, 1, 0, true, true>(a, cus, stream)
                : hgemm::launch<BM, 256, BK, 4, 2, GM, 1, 0, true, true>(a, cus, stream);
  }
  return w224 ? hgemm::launch<BM, 224, BK, 4, 2, GM, 1>(a, cus, stream)
              : hgemm::launch<BM, 256, BK, 4, 2, GM, 1>(a, cus, stream);
}

bool f16_epi_fits(const void* bias, const void* res, int64_t ldr) {
  return hgemm::epi_fits(bias, res, ldr);
}

}  // namespace mi355gemm
