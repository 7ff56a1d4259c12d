// The GEMM family's interface: tile table, launch plans and the launcher.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qr {

// Static description of one GEMM tile configuration.
struct TileDesc {
  const char* name;
  int T;   // MFMA tile edge (16 or 32)
  int BN;  // macro-tile extent along N (weight rows)
  int BM;  // macro-tile extent along M (tokens)
  int BK;  // bytes of K per pipeline stage
  int NT;  // threads per block
  int S;   // LDS-DMA ring slots (prefetch depth in K steps for the direct kernel)
};

int num_tiles();
const TileDesc& tile_desc(int tile);

// A launch plan for one product shape.
struct GemmPlan {
  int tile;
  int splitk;
  int rows;  // weight rows per tile (multiple of 8, <= the tile's BN)
  int64_t tiles_n, tiles_m, nks;
  size_t part_bytes;  // split-K partial sums [splitk][M][N] (0 without split)
  // Workspace qr_w8a8_gemm needs: the partial sums, none without split-K.
  size_t ws_bytes() const { return part_bytes; }
};

GemmPlan make_plan(int64_t M, int64_t N, int64_t K, int qt, int force_tile, int force_splitk,
                   int force_rows);

struct GemmArgs {
  const uint8_t* Xq;
  const float* sx;
  const uint8_t* Wq;
  const float* sw;
  int64_t M, N, K;
  void* Y;
  int64_t ldy;
  int out_raw;
  void* part;  // split-K partial sums (workspace)
};

hipError_t launch_gemm(const GemmPlan& plan, int qt, const GemmArgs& a, hipStream_t st);

}  // namespace qr
