// The tiled int8 product for many tokens on 32 x 32 x 32 matrix-core
// products: the 256-row x 192-token tile of the large tiling, as 4 waves of
// 128 rows x 96 tokens (4 x 3 tiles of 32 x 32 int32 sums per wave, 192
// registers, held in the accumulation registers).  The 32 x 32 products run
// near the chip's int8 peak per clock where the 16 x 16 ones reach about half
// of it; with 157 KB of LDS per workgroup the CU holds one workgroup, one wave
// per SIMD.  Weights: packed ternary blocks ("Sherry: Hardware-Efficient
// 1.25-Bit Ternary Quantization via Fine-grained Sparsification", Abstract)
// and the 2-bit comparator (same paper, Figure 2 caption).
#include "gemm_tile.h"

namespace sherry {
namespace {

#ifndef SHERRY_TILE32_WAVES
#define SHERRY_TILE32_WAVES 8
#endif
#if SHERRY_TILE32_WAVES == 4
using TileWide = TileCfg<2, 2, 6, 128, true, 1>;
#else
using TileWide = TileCfg<4, 2, 6, 64, true, 1>;
#endif
static_assert(TileWide::kRows == kGemmLargeRows && TileWide::kTok == kGemmLargeTok, "large tiling");

template <class Fmt>
__global__ __launch_bounds__(TileWide::kThreads) void gemm_tile32_kernel(GemmDesc d) {
  gemm_tile<Fmt, TileWide>(d, blockIdx.x, blockIdx.y);
}

template <class Fmt>
__global__ __launch_bounds__(TileWide::kThreads) void gemm_tile32_grouped_kernel(const char* plan) {
  const PlanHeader* h = reinterpret_cast<const PlanHeader*>(plan);
  const GemmDesc* descs = reinterpret_cast<const GemmDesc*>(plan + sizeof(PlanHeader));
  const GemmTile tl = reinterpret_cast<const GemmTile*>(descs + h->count)[blockIdx.x];
  const GemmDesc d = descs[tl.prob];
  gemm_tile<Fmt, TileWide>(d, tl.tile_n, tl.tile_m);
}

}  // namespace

hipError_t launch_gemm_tile32(const GemmDesc& d, int32_t format, hipStream_t stream) {
  const dim3 grid((d.n + TileWide::kRows - 1) / TileWide::kRows, (d.m + TileWide::kTok - 1) / TileWide::kTok);
  if (format == kFmtTern2)
    hipLaunchKernelGGL((gemm_tile32_kernel<Tern2>), grid, dim3(TileWide::kThreads), 0, stream, d);
  else
    hipLaunchKernelGGL((gemm_tile32_kernel<Sherry3of4>), grid, dim3(TileWide::kThreads), 0, stream, d);
  return hipGetLastError();
}

hipError_t launch_gemm_tile32_grouped(const char* plan, int32_t n_tiles, int32_t format, hipStream_t stream) {
  const dim3 grid(n_tiles);
  if (format == kFmtTern2)
    hipLaunchKernelGGL((gemm_tile32_grouped_kernel<Tern2>), grid, dim3(TileWide::kThreads), 0, stream, plan);
  else
    hipLaunchKernelGGL((gemm_tile32_grouped_kernel<Sherry3of4>), grid, dim3(TileWide::kThreads), 0, stream, plan);
  return hipGetLastError();
}

}  // namespace sherry
