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
  int FU;  // 1: has a fused chain-epilogue instantiation
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

// With sum_splits = false a split plan only writes its partial sums to a.part.
hipError_t launch_gemm(const GemmPlan& plan, int qt, const GemmArgs& a, hipStream_t st,
                       bool sum_splits = true);

// The split-K sum of a.part ([splitk][M][N]) with the bf16 epilogue into Y,
// and the per-token quantization of Y's columns [q0, q0 + qn) into Xq
// ([M][qn]) and scale_x, in one launch (one block per token row); the same
// bits as the split-K sum kernel followed by the per-token quantizer. For
// 2-8 splits, N a multiple of 8 up to 16384 (splitk_reduce_quant_ok), ldy,
// q0 and qn multiples of 8.
bool splitk_reduce_quant_ok(int64_t N, int splitk);
hipError_t launch_splitk_reduce_quant(int splitk, int qt, const void* part, int64_t M, int64_t N,
                                      const float* sx, const float* sw, void* Y, int64_t ldy,
                                      int64_t q0, int64_t qn, float act_mult, void* Xq,
                                      float* scale_x, hipStream_t st);

// Fused chain epilogue: the split-K sum and the per-token quantization of
// Y[:, qc0 : qc0 + qcn] for the next linear inside the GEMM launch.
// Workspace: a header of kFuseHeaderBytes (barrier words at offset 0, the
// per-token absmax buffer [2][kFuseMaxM] at offset 256; zero before the first
// launch that uses it, left so by every launch), then the partial sums.
constexpr size_t kFuseHeaderBytes = (size_t)64 << 10;
constexpr int64_t kFuseMaxM = 4096;
constexpr int kFuseItems = 4;  // split-K sum items of 256 outputs per wave, at most

struct FuseArgs {
  void* header;
  void* part;
  uint8_t* xq2;  // [M][qcn]
  float* sx2;    // [M]
  int64_t qc0, qcn;
  float am2;
};

// Whether `plan` can run fused for this shape: the tile has a fused
// instantiation, every block of the grid can be resident at once on this
// device, M <= kFuseMaxM, and a split plan's sum fits kFuseItems items per
// wave. The shape's other conditions (N, ldy, qc0, qcn multiples of 4) are
// the caller's.
bool fused_ok(const GemmPlan& plan, int qt, int64_t M, int64_t N);

hipError_t launch_gemm_fused(const GemmPlan& plan, int qt, const GemmArgs& a, const FuseArgs& fa,
                             hipStream_t st);

}  // namespace qr
