// Launch planner of the GEMM family: tile, split-K and rows per tile for one
// product shape (pure host code; choices measured on MI355X).
#include "qr_device.h"
#include "qr_gemm.h"

namespace {

constexpr int kCUs = 256;  // MI355X compute units: the plan targets this chip

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

namespace qr {

GemmPlan make_plan(int64_t M, int64_t N, int64_t K, int qt, int force_tile, int force_splitk,
                   int force_rows) {
  GemmPlan p{};
  // Tile by token count (indices into the tile table; choices measured on
  // MI355X with graph-replayed launches). Up to 32 tokens the product is a
  // weight stream: 8-wave LDS-DMA tiles of 128 weight rows on wide layers,
  // 64 x 16 or 4-wave 128 x 32 tiles split along K on narrow ones. 256-token decode
  // uses 8-wave 192 x 128 tiles on wide layers (two waves per SIMD cover
  // each other's copy and LDS stalls: 9-12% faster than 4 waves; 256 x 256
  // on very wide ones, such as stacked gate and up projections), 128 x 128
  // with split K on long-K
  // ones and 128 x 64 / 128 x 32 tiles on narrow ones (more blocks); up to
  // 1024 tokens 256 x 256 tiles on wide layers, 256 x 128 with split K on
  // long-K ones, 128 x 128 on the others and 64 x 16 tiles on very narrow
  // ones (1024-row k / v projections: two rounds of small blocks beat one of
  // 128 x 32 tiles that own half their rows); large token counts use
  // 256 x 256 tiles, 256 x 128 below N = 7168.
  const int64_t nks = (K + 127) / 128;
  int tile;
  if (force_tile >= 0) {
    tile = force_tile;
  } else if (M <= 32) {
    // weight streaming; narrow layers (split K below) on 64 x 16 tiles up to
    // 16 tokens and 4-wave 128 x 32 tiles of 32 x 32 fragments up to 32
    tile = N >= 8192 ? 0 : (M <= 16 ? 7 : 6);
  } else if (M <= 64) {
    tile = 1;
  } else if (M <= 128) {
    tile = 2;
  } else if (M <= 256) {
    // Very wide layers: 128 x 256 tiles (every token in one block, so each
    // weight byte is copied once) while they fit one round of the CUs, as
    // for the 32B gate and up (27648 rows: 51 us against 76 us on 256 x 256
    // tiles with split K); wider ones, such as the stacked 7B gate and up
    // (37888 rows), 192 x 256 while those fit one round (INT8 45.0 us against
    // 54.3 on 256 x 256 tiles and 57.9 for gate and up as two GEMMs on
    // 192 x 128 tiles; FP8 49.3, 55.6 and 58.8), 256 x 256 beyond.
    if (N >= 24576)
      tile = (N + 127) / 128 <= kCUs ? 5 : ((N + 191) / 192 <= kCUs ? 10 : 4);
    else if (N >= 8192) tile = 8;
    else if (nks >= 64) tile = 2;
    else if (N >= 4096)
      // INT8: 80 x 64 tiles issue 20 copies per K step where 128 x 64 ones
      // issue 24 (7-8% faster on the 7B QKV), while their full-height grid
      // fits one round; past it (the 32B stacked QKV, 7168 rows) the
      // 128 x 64 tiles' single round wins (23.6 us against 36.3 us).
      tile = qt == kQInt8 && ((N + 79) / 80) * ((M + 63) / 64) <= kCUs ? 9 : 1;
    else tile = qt == kQFp8 ? 6 : 0;  // FP8: 32x32 fragments 8% faster here
  } else if (M <= 1024) {
    if (N >= 16384) tile = 4;
    else if (N <= 2048) tile = 7;
    else tile = nks >= 64 ? 3 : 2;
  } else {
    tile = N >= 7168 ? 4 : 3;
  }
  const TileDesc& d = tile_desc(tile);
  p.tile = tile;
  p.tiles_m = (M + d.BM - 1) / d.BM;
  p.nks = (K + d.BK - 1) / d.BK;
  const int64_t full = ((N + d.BN - 1) / d.BN) * p.tiles_m;  // blocks at full tile height
  // Balance the grid over the CUs: first by shrinking the weight rows per
  // tile (a multiple of 8, at least half the tile height) so that about one
  // block per CU remains; where even full-height tiles leave CUs idle, split
  // K (every split keeps four or more K steps, and the partial sums, 4 M N
  // bytes per split, stay within the weight bytes) and then rebalance the
  // rows.
  // The weight-streaming tiles (64 tokens or fewer) shrink, and so do tiles
  // of at most 128 rows up to 1024 tokens (a 512-token 5120-row projection
  // on 80-row tiles is 6% faster); the 256-row tiles of wider layers and
  // larger token counts are bound by the MFMA work of the full tile, which
  // does not shrink with the row count, and keep their height.
  // With more full-height blocks than CUs the rows shrink to fill whole
  // rounds of kCUs blocks instead of leaving a short last round.
  auto balanced_rows = [&](int64_t splits) -> int64_t {
    if (d.BM > 64 && (M > 1024 || d.BN > 128)) return d.BN;
    const int64_t base = ((N + d.BN - 1) / d.BN) * p.tiles_m * splits;
    const int64_t per = kCUs * ((base + kCUs - 1) / kCUs);  // blocks wanted
    // The fewest rows (a multiple of 8) whose tiles along N, rounded up,
    // fit: at most per / (tiles_m * splits) of them.
    const int64_t tn = per / (p.tiles_m * splits);
    const int64_t want = 8 * ((N + 8 * tn - 1) / (8 * tn));
    return (want >= d.BN / 2 && want < d.BN) ? want : d.BN;
  };
  int64_t s = 1;
  int64_t rows = d.BN;
  if (force_tile >= 0) {
    s = force_splitk > 0 ? force_splitk : 1;
    rows = force_rows > 0 ? force_rows : d.BN;
  } else if (full == 0) {
    // M = 0 or N = 0: nothing to launch
  } else if (full >= kCUs) {
    rows = balanced_rows(1);
  } else if (8 * ((N * p.tiles_m + 8 * kCUs - 1) / (8 * kCUs)) >= d.BN / 2) {
    rows = balanced_rows(1);
  } else if (M <= 32) {
    // Weight streaming on a narrow layer: the largest grid of at most kCUs
    // blocks over splits of K (up to 8, each keeping four or more K steps,
    // partial sums within the weight bytes) and rows per tile (a multiple
    // of 8, at least half the tile height); fewer splits on a tie. Measured
    // on the 7B QKV, O and down projections at 1 and 32 tokens: the best
    // plan or within 3% of it, 8-22% faster than at most 4 splits.
    const int64_t by_bytes = K / (4 * M);
    int64_t best = 0;
    for (int64_t ss = 1; ss <= 8 && ss <= by_bytes && p.nks / ss >= 4; ++ss) {
      for (int64_t r = ((d.BN / 2 + 7) / 8) * 8; r <= d.BN; r += 8) {
        const int64_t blocks = ((N + r - 1) / r) * p.tiles_m * ss;
        if (blocks <= kCUs) {
          if (blocks > best) {
            best = blocks;
            s = ss;
            rows = r;
          }
          break;
        }
      }
    }
  } else {
    // As many splits as keep the grid within one round of kCUs blocks (a
    // second, partial round costs more than the split saves).
    s = kCUs / full;
    const int64_t by_bytes = K / (4 * (M > 0 ? M : 1));
    const int64_t by_steps = p.nks / 4;
    if (s > by_bytes) s = by_bytes;
    if (s > by_steps) s = by_steps;
    if (s > 4) s = 4;
    if (s < 1) s = 1;
    rows = balanced_rows(s);
  }
  if (p.nks > 0 && s > p.nks) s = p.nks;
  if (s < 1) s = 1;
  p.rows = (int)rows;
  p.tiles_n = (N + p.rows - 1) / p.rows;
  p.splitk = (int)s;
  if (p.splitk > 1 && p.tiles_n * p.tiles_m > 0)
    p.part_bytes = align256((size_t)p.splitk * (size_t)M * (size_t)N * 4);
  return p;
}

}  // namespace qr
