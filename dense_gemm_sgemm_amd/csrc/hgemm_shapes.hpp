// The tile shapes of the 16-bit full-tile kernels and the cost model that
// chooses between them (shared by the A * B^T instances and the in-place
// layout instances).
#pragma once

#include <stdint.h>

namespace mi355gemm {
namespace hshape {

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
// 128 x 128 tiles that do not outnumber the CUs run one per CU, each with a
// CU to itself: tile-time 128 x 128 x 8/5, about 0.8 of a 128 x 192 tile
// (measured: 1536 x 2304 x 2048 24.7 against 27.6 us on 144 tiles of
// 128 x 192; 1536^2 x 4096 40.8 against 46.9 us; 1024 x 3072 x 2048 23.7
// against 26.6 us).
// RAGGED: the same over ceil(M / bm) x ceil(N / bn) tiles (the ragged form),
// for the shapes at least one tile wide and tall.
inline TileShape choose(int M, int N, int cus, bool ragged = false, int64_t* cost_out = nullptr) {
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
  consider(k256x256, 256, 256, cus, 256 * 256);
  consider(k256x224, 256, 224, cus, 256 * 224);
  consider(k128x128, 128, 128, 2 * cus, 2 * 128 * 128 * 6 / 5);
  consider(k128x192, 128, 192, cus, 128 * 192 * 4 / 3);
  if (cost_out) *cost_out = best_cost;
  return best;
}

}  // namespace hshape
}  // namespace mi355gemm
