// Internal launcher interface between the C ABI (abi.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace sherry {

// Reduction-length classes with a register-resident (x-stationary) kernel.
// L = lanes that share one row, GPL = 128-weight groups per lane (L*GPL*128 = k).
enum KClass : int32_t { kGeneric = 0, k1024 = 1, k2048 = 2, k4096 = 3, k8192 = 4, k3072 = 5, kT3k2048 = 6, kT3k8192 = 7 };

inline int32_t kclass_of(int64_t k) {
  switch (k) {
    case 1024: return k1024;
    case 2048: return k2048;
    case 4096: return k4096;
    case 8192: return k8192;
    case 3072: return k3072;
    default: return kGeneric;
  }
}
// 1.67-bit rows (96-weight groups): 22 groups at k = 2048, 86 at k = 8192.
inline int32_t kclass_of_t3(int64_t k) { return k == 2048 ? kT3k2048 : (k == 8192 ? kT3k8192 : kGeneric); }
// Lanes per row for a class (64 for the generic kernel).
// Lanes per row of a k class: one group per lane (k = 3072: 24 of 32 lanes
// hold one), except bf16 x at k = 3072, which keeps 3 groups in each of 8.
inline int lanes_per_row(int32_t kc, bool bf16 = false) {
  switch (kc) {
    case k1024: return 8;
    case k2048: return 16;
    case k4096: return 32;
    case k8192: return 64;
    case k3072: return bf16 ? 8 : 32;
    case kT3k2048: return 32;
    case kT3k8192: return 64;
    default: return 64;
  }
}
#ifndef SHERRY_GROUPED_ITERS
#define SHERRY_GROUPED_ITERS 32
#endif
#ifndef SHERRY_GEMV_THREADS
#define SHERRY_GEMV_THREADS 256
#endif
constexpr int kGemvThreads = SHERRY_GEMV_THREADS;  // GEMV workgroup size (4 waves by default)
// Rows one GEMV workgroup advances per iteration.
inline int rows_per_iter(int32_t kc, bool bf16 = false) {
  return (kGemvThreads / kWave) * (kWave / lanes_per_row(kc, bf16));
}

enum Format : int32_t { kFmtSherry = 0, kFmtTern2 = 1, kFmtTern3 = 2 };

// bf16 x on the matrix cores (3:4 codes, every problem k <= kBf16MfmaMaxK),
// chosen by sherry_gemv_plan_mfma: 8-wave workgroups over tiles of
// max(256, the int8 grouped tile) rows, so a plan sized for the int8 tiling
// also holds this one.
constexpr int kBf16MfmaMaxK = 8192;
#ifndef SHERRY_BF16_MFMA_WAVES
#define SHERRY_BF16_MFMA_WAVES 8
#endif
constexpr int kBf16MfmaWaves = SHERRY_BF16_MFMA_WAVES;
__host__ __device__ constexpr int bf16_mfma_tile_rows(int32_t kc) {
  const int lanes = kc == k1024 ? 8 : (kc == k2048 ? 16 : (kc == k3072 || kc == k4096 ? 32 : 64));
  const int r = (kGemvThreads / kWave) * (kWave / lanes) * SHERRY_GROUPED_ITERS;
  return r > 256 ? r : 256;
}


struct PlanHeader {
  uint32_t magic;
  uint32_t version;
  int32_t count;
  int32_t n_tiles;
  int32_t s_dt;
  int32_t x_dt;
  int32_t y_dt;
  int32_t format;
  uint64_t bytes;
  uint64_t reserved[3];  // GEMV plans: reserved[0] nonzero if some problem has k = 3072, reserved[1] nonzero
                         // for bf16 x on the matrix cores; GEMM plans: reserved[0] = the tiling,
                         // reserved[1] nonzero if every problem's k suits the decode-once prefill kernel
};
static_assert(sizeof(PlanHeader) == 64, "plan header layout");
// Largest GEMV plan that sherry_gemv_grouped_noalloc takes (its static plan
// memory per device), and the device ordinals it serves.
constexpr size_t kNoAllocPlanBytes = size_t(1) << 20;
constexpr int kMaxDevices = 256;
constexpr uint32_t kPlanMagic = 0x53485950u;  // "PYHS"
constexpr uint32_t kPlanVersion = 1;
// Row iterations per grouped-GEMV tile and depth of the GEMV prefetch ring
// (build-time tunables; the defaults are the measured best on MI355X).
#ifndef SHERRY_RING
#define SHERRY_RING 4
#endif
constexpr int kGroupedIters = SHERRY_GROUPED_ITERS;
constexpr int kRing = SHERRY_RING;
// GEMV decode: bit p set = block pair p of a group is read from the pair
// table, clear = its two blocks from the 32-entry table.
#ifndef SHERRY_PAIR_MASK
#define SHERRY_PAIR_MASK 0x5555
#endif
constexpr unsigned kPairMask = SHERRY_PAIR_MASK;
// The two-token walk does twice the dot products per decoded code, so there
// the VALU-saving pair reads pay for every block pair.
#ifndef SHERRY_PAIR_MASK_TWO
#define SHERRY_PAIR_MASK_TWO 0xFFFF
#endif
constexpr unsigned kPairMaskTwo = SHERRY_PAIR_MASK_TWO;
// Independent v_dot4 accumulation chains per row step.
#ifndef SHERRY_DOT_CHAINS
#define SHERRY_DOT_CHAINS 1
#endif
constexpr int kDotChains = SHERRY_DOT_CHAINS;

struct PlanTile {
  int32_t prob;
  int32_t row0;
};

// GEMM (M tokens) problem; the grouped plan stores these verbatim.
struct GemmDesc {
  const uint32_t* codes;
  const void* w_scales;
  const int8_t* x;
  const float* x_scales;
  int32_t* acc;
  void* y;
  int64_t ldx;
  int64_t ldy;
  int32_t n;
  int32_t k;
  int32_t m;
  int32_t flags;
};
static_assert(sizeof(GemmDesc) == 80, "grouped GEMM plan record layout");

// Grouped GEMM plan: PlanHeader (magic kGemmPlanMagic; reserved[0] = the
// tiling, kGemmTiling*) | GemmDesc[count] | GemmTile[n_tiles].
constexpr uint32_t kGemmPlanMagic = 0x53484750u;  // "PGHS"
struct GemmTile {
  int32_t prob;
  int32_t tile_n;  // row tile index
  int32_t tile_m;  // token tile index
  int32_t pad;
};
static_assert(sizeof(GemmTile) == 16, "grouped GEMM tile record layout");
// Rows x tokens of the tilings of the tiled kernel: 128 x 128, 256 x 256,
// and 256 x 16 for plans whose problems all have m <= 16.
constexpr int64_t kGemmTilingSmall = 0, kGemmTilingLarge = 1, kGemmTilingSkinny = 2, kGemmTilingFew = 3,
                  kGemmTilingTwo = 4, kGemmTilingBf16 = 5;
constexpr int kGemmLargeRows = 256, kGemmLargeTok = 128;
constexpr int kGemmSmallRows = 128, kGemmSmallTok = 128;
constexpr int kGemmSkinnyRows = 256, kGemmSkinnyTok = 16;
// Few-token kernel (every problem m <= 16, k <= 8192): a row tile of
// R = kFewMaxTileRows rows with all of k, for every k; S = k slices of 512
// weights rounded up to a power of two (at most 16).  Each wave keeps its
// slices of x in registers for the whole tile, so the longer the tile, the
// less x is reread per row.
constexpr int kFewMaxTok = 16;
constexpr int kFewMaxGroups = 64;
constexpr int kFewWaves = 8;
inline constexpr int few_slices(int groups) {
  int s = 1;
  while (4 * s < groups) s *= 2;
  return s;
}
#ifndef SHERRY_FEW_TILE_ROWS
#define SHERRY_FEW_TILE_ROWS 512
#endif
constexpr int kFewMaxTileRows = SHERRY_FEW_TILE_ROWS;
inline constexpr int few_tile_rows(int) { return kFewMaxTileRows; }
// Large tiles are used when they give at least this many workgroups.
#ifndef SHERRY_LARGE_TILE_MIN_GROUPS
#define SHERRY_LARGE_TILE_MIN_GROUPS 256
#endif
constexpr int64_t kLargeTileMinGroups = SHERRY_LARGE_TILE_MIN_GROUPS;

hipError_t launch_pack(const void* w, int w_dt, int64_t n, int64_t k, int64_t ldw, uint32_t* codes,
                       void* scales, bool s_f16, bool tern2, hipStream_t stream);
hipError_t launch_gemv(const GemvDesc& d, bool bf16_x, int32_t format, hipStream_t stream);
hipError_t launch_gemv_grouped(const PlanHeader* host, const void* dev, hipStream_t stream);
// The same launch with the plan copied (h->bytes bytes, stream-ordered) into
// the library's static per-device plan memory of kNoAllocPlanBytes.
hipError_t launch_gemv_grouped_noalloc(const PlanHeader* host, const void* plan_host, hipStream_t stream);
hipError_t launch_gemv_xq(const GemvDesc& d, int xdt, float* sx_out, int32_t format, hipStream_t stream);
hipError_t launch_gemm(const GemmDesc& d, int32_t format, hipStream_t stream);
// Two-token products: m <= 2 and a register-class k run the batch-1 walk with
// both tokens' x in registers (kGemmTilingTwo), row tiles as in the grouped
// GEMV.
inline bool gemm2_fits(int64_t m, int64_t k) { return m <= 2 && kclass_of(k) != kGeneric; }
inline int gemm2_tile_rows(int64_t k) { return rows_per_iter(kclass_of(k)) * kGroupedIters; }
hipError_t launch_gemm2(const GemmDesc& d, int32_t format, hipStream_t stream);
hipError_t launch_gemm2_grouped(const char* plan, int32_t n_tiles, int32_t format, hipStream_t stream);
hipError_t launch_gemm_grouped(const PlanHeader* host, const void* dev, hipStream_t stream);
// bf16 x for a few tokens (m <= kBfFewMaxTok, k <= kBfFewMaxK) on the matrix
// cores, fp32 outputs: 16-wave workgroups, k split into S slices of 512
// weights (S = bf_few_slices, a power of two) and the rows into 16 / S row
// groups; grouped tiles of kBfFewMaxTileRows rows.
constexpr int kBfFewWaves = 16;
constexpr int kBfFewMaxTok = 16;
constexpr int64_t kBfFewMaxK = 8192;
#ifndef SHERRY_BF_FEW_TILE_ROWS
#define SHERRY_BF_FEW_TILE_ROWS 1024
#endif
constexpr int kBfFewMaxTileRows = SHERRY_BF_FEW_TILE_ROWS;  // a multiple of 256
__host__ __device__ constexpr int bf_few_slices(int groups) {
  int s = 1;
  while (4 * s < groups) s *= 2;
  return s;
}
hipError_t launch_gemm_bf16(const GemmDesc& d, hipStream_t stream);
// Many tokens with the large tiling (kGemmLargeRows x kGemmLargeTok), by the
// process-wide prefill kind: the general tiled kernel (16 x 16 products, 8
// waves), the same kernel on 32 x 32 products (4 waves of 128 x 96), or, on
// Sherry codes, the decode-once kernel (each group's codes decoded once per
// workgroup into an int8 A tile in LDS).
constexpr int kPrefillTiled = 0, kPrefillDecodeOnce = 1, kPrefillTiled32 = 2;
void set_prefill_kind(int kind);
int prefill_kind();
hipError_t launch_gemm_tile32(const GemmDesc& d, int32_t format, hipStream_t stream);
hipError_t launch_gemm_tile32_grouped(const char* plan, int32_t n_tiles, int32_t format, hipStream_t stream);
// The decode-once kernel steps through k in unrolled runs of this many groups
// (two code stages); other k take the general tiled kernel.
constexpr int kPrefillGroupMultiple = 8;
inline bool prefill_fits(int64_t k) { return (k / kGroupWeights) % kPrefillGroupMultiple == 0; }
hipError_t launch_gemm_prefill(const GemmDesc& d, hipStream_t stream);
hipError_t launch_gemm_prefill_grouped(const char* plan, int32_t n_tiles, hipStream_t stream);
hipError_t launch_gemm_bf16_grouped(const char* plan, int32_t n_tiles, hipStream_t stream);
// Activation quantization: input element types; the GEMV that quantizes its
// own x holds it in LDS, k <= kActMaxK.
constexpr int kActF32 = 0, kActF16 = 1, kActBf16 = 2;
constexpr int64_t kActMaxK = 8192;
hipError_t launch_act_quant(const void* x, int dt, int64_t m, int64_t k, int64_t ldx, int8_t* q, int64_t ldq,
                            float* scales, hipStream_t stream);
hipError_t launch_decode(const uint32_t* codes, int64_t n, int64_t k, int8_t* t, int64_t ldt, hipStream_t stream);
hipError_t launch_tern3_encode(const int8_t* t, int64_t n, int64_t k, int64_t ldt, uint32_t* codes,
                               hipStream_t stream);
hipError_t launch_tern2_encode(const int8_t* t, int64_t n, int64_t k, int64_t ldt, uint32_t* codes,
                               hipStream_t stream);

}  // namespace sherry
