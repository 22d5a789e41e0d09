// The tiled int8 product for many tokens on 32 x 32 x 32 matrix-core
// products: the 256-row x 128-token tile of the large tiling, as 4 waves of
// 64 rows x 128 tokens (2 x 4 tiles of 32 x 32 int32 sums per wave, 128
// registers) and, with 78 KB of LDS per workgroup, two workgroups per CU
// (two waves per SIMD).  Half the product instructions of the 16 x 16 x 64
// form for the same work, each at the same rate per operation.  Weights: packed
// ternary blocks ("Sherry: Hardware-Efficient 1.25-Bit Ternary Quantization
// via Fine-grained Sparsification", Abstract) and the 2-bit comparator (same
// paper, Figure 2 caption).
#include "gemm_tile.h"

namespace sherry {
namespace {

using TileWide = TileCfg<4, 1, kGemmLargeTok / 16, 64, true, 2>;
// two waves per SIMD: at most 256 registers per wave
#define SHERRY_T32_OCC __attribute__((amdgpu_waves_per_eu(2)))
static_assert(TileWide::kRows == kGemmLargeRows && TileWide::kTok == kGemmLargeTok, "large tiling");

template <class Fmt>
__global__ __launch_bounds__(TileWide::kThreads) SHERRY_T32_OCC void gemm_tile32_kernel(GemmDesc d) {
  gemm_tile<Fmt, TileWide>(d, blockIdx.x, blockIdx.y);
}

template <class Fmt>
__global__ __launch_bounds__(TileWide::kThreads) SHERRY_T32_OCC void gemm_tile32_grouped_kernel(const char* plan) {
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
