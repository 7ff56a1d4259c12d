// Internal interface between the C-ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qr {

hipError_t launch_act_quant(const void* X, int64_t M, int64_t K, int64_t ldx, float act_mult,
                            int qt, void* Xq, float* scale_x, hipStream_t st);
hipError_t launch_weight_quant(const float* W, int64_t N, int64_t K, int64_t ldw, float s, int qt,
                               void* Wq, float* scale_w, float* Wsc, hipStream_t st);
hipError_t launch_fold_norm(float* gamma, float* beta, int64_t K, float s, hipStream_t st);
hipError_t launch_norm_quant(const void* H, int64_t M, int64_t K, int64_t ldh, int kind,
                             const float* gamma, const float* beta, float eps, int qt, void* Xq,
                             float* scale_x, hipStream_t st);
hipError_t launch_silu_mul_quant(const void* G, const void* U, int64_t M, int64_t N, int64_t ldg,
                                 int64_t ldu, float act_mult, int qt, void* Xq, float* scale_x,
                                 hipStream_t st);
hipError_t launch_requant(const float* Wp, int64_t N, int64_t K, int64_t ldw, int qt, void* Wq,
                          float* scale_w, uint32_t* row_flips, hipStream_t st);

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
