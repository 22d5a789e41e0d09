// Products for a few tokens with bf16 activations, Y[m, r] = s_w[r] * sum_k
// T[r, k] X[m, k] in fp32, on packed ternary weights ("Sherry: Hardware-
// Efficient 1.25-Bit Ternary Quantization via Fine-grained Sparsification",
// Abstract: 3:4 sparse ternary blocks of four weights in five bits).
//
// With M <= 16 tokens the contraction is dense enough for the matrix cores:
// v_mfma_f32_16x16x32_bf16 multiplies 16 weight rows by 16 tokens over 32
// k.  Lane (q, i) = (lane / 16, lane % 16) supplies row i's weights and token
// i's x at eight k of its own; any assignment of k to (q, slot) is valid as
// long as A and B use the same one.  Here lane (q, i) of wave kw owns group
// g = 4 kw + q (128 weights) of every row it meets: MFMA u of a row block
// takes the lane's blocks 2u and 2u + 1 (eight weights, two 8-byte entries
// of the bf16 code table) against the same eight x values, and the 16 MFMAs
// of a block consume the lane's whole group.  x is stationary: each lane
// keeps its token's 128 values of its group in registers (64 VGPRs) for the
// whole row tile.
//
// A workgroup of 16 waves splits k into S slices of 512 weights (S a power
// of two, KW = S waves per row group) and the rows of its tile into RG =
// 16 / S row groups.  After each block of 16 rows every wave writes its
// 16 x 16 partial sums to LDS; after every fourth block one barrier, and the
// workgroup adds the KW partials of every output of those blocks in a fixed
// order (so results repeat bit for bit), scales them and stores them, while
// the next blocks' products run.  The partial buffers alternate between two
// LDS halves.
#include "formats.h"
#include "launch.h"

namespace sherry {
namespace {

typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

constexpr int kBfThreads = kBfFewWaves * kWave;
constexpr int kBfRing = 4;  // blocks of code words in flight per wave
// table reads issued together ahead of their products (in MFMAs): each
// batch of products then waits on one LDS round trip, not one each
constexpr int kBfBatch = 2;  // (4 made the compiler spill inside the block loop)
static_assert(16 % kBfBatch == 0, "whole batches per group");

// Row blocks whose partial sums are written before one barrier and added
// together after it (the partials of 4 blocks, double-buffered: 128 KB of
// LDS; the workgroup's 16 waves at 128 registers already fill the CU).
constexpr int kBfBps = 4;

struct BfFewShared {
  uint2 tab[32];                                   // code -> four bf16 weights
  float part[2][kBfBps][kBfFewWaves][4 * kWave];   // per wave and block: 16 rows x 16 tokens
  float sws[kBfFewMaxTileRows];                    // the tile's row scales
};

// Rows [row0, row0 + 16 RG NB) of d: row group rg walks NB blocks of 16 rows
// at row0 + 16 (rg NB + b).  NB is a compile-time constant (with a run-time
// block count the compiler spilled registers inside the block loop).
template <int S, int NB>
__device__ __forceinline__ void gemm_bf16_few_tile(const GemmDesc& d, int row0, BfFewShared& sh) {
  constexpr int nblk = NB;
  constexpr int KW = S;
  constexpr int RG = kBfFewWaves / S;
  constexpr int D = kBfRing;
  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int kw = wave % KW;
  const int rg = wave / KW;
  const int i = lane & 15;
  const int q = lane >> 4;
  const int G = d.k / kGroupWeights;
  const int g = 4 * kw + q;
  const int gc = min(g, G - 1);
  const int rt = 16 * RG * nblk;                   // tile rows
  const int rbase = row0 + 16 * rg * nblk;         // this row group's first row
  const int64_t row_words = static_cast<int64_t>(G) * kGroupWords;

  // x of token i for group g (zero past m and past k): issued first
  uint32_t xr[64];
  {
    const bool ok = i < d.m && g < G;
    const SHERRY_GLOBAL u32x4_t* xp = gmem(reinterpret_cast<const u32x4_t*>(
        reinterpret_cast<const uint16_t*>(d.x) + (ok ? static_cast<int64_t>(i) * d.ldx + 128 * g : 0)));
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const u32x4_t v = xp[u];
      xr[4 * u + 0] = ok ? v.x : 0u;
      xr[4 * u + 1] = ok ? v.y : 0u;
      xr[4 * u + 2] = ok ? v.z : 0u;
      xr[4 * u + 3] = ok ? v.w : 0u;
    }
  }
  // rows past n load the last row (results dropped); groups past k load the
  // last group (x is zero there)
  auto fetch = [&](uint32_t (&w)[kGroupWords], int blk) {
    const int row = min(rbase + 16 * blk + i, d.n - 1);
    Sherry3of4::load_cached(w, d.codes + row * row_words, G, gc);
  };
  uint32_t ring[D][kGroupWords];
#pragma unroll
  for (int b = 0; b + 1 < D; ++b) fetch(ring[b], min(b, nblk - 1));
  // the code table and the tile's row scales in LDS
  if (tid < 32) sh.tab[tid] = decode_bf16x4(static_cast<uint32_t>(tid));
  const bool s_f16 = d.flags & kFlagScaleF16;
  for (int t = tid; t < rt; t += kBfThreads) sh.sws[t] = load_scale(d.w_scales, min(row0 + t, d.n - 1), s_f16);
  __syncthreads();

  // The table reads of a batch of kBfBatch products go out before the
  // products of the batch before it, so each batch's reads are in flight
  // during the previous batch's products (scheduling barriers hold the
  // order).
  auto step = [&](const uint32_t (&w)[kGroupWords]) {
    f4_t c = {0.0f, 0.0f, 0.0f, 0.0f};
    uint2 a[2][2 * kBfBatch];
#pragma unroll
    for (int v = 0; v < 2 * kBfBatch; ++v) a[0][v] = lds_u64(sh.tab, code_offset<3>(w, v));
#pragma unroll
    for (int h = 0; h < 16 / kBfBatch; ++h) {
      if (h + 1 < 16 / kBfBatch) {
#pragma unroll
        for (int v = 0; v < 2 * kBfBatch; ++v)
          a[(h + 1) & 1][v] = lds_u64(sh.tab, code_offset<3>(w, 2 * kBfBatch * (h + 1) + v));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int v = 0; v < kBfBatch; ++v) {
        const int u = kBfBatch * h + v;  // blocks 2u, 2u + 1: k 8u .. 8u + 7 of the group
        const uint2* ah = a[h & 1];
        const u4_t av = {ah[2 * v].x, ah[2 * v].y, ah[2 * v + 1].x, ah[2 * v + 1].y};
        const u4_t bv = {xr[4 * u], xr[4 * u + 1], xr[4 * u + 2], xr[4 * u + 3]};
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8_t, av), __builtin_bit_cast(bf8_t, bv), c,
                                                     0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    return c;
  };
  const int ldy = static_cast<int>(d.ldy);
  float* y = static_cast<float*>(d.y);
  for (int b0 = 0; b0 < nblk; b0 += D) {
#pragma unroll
    for (int bb = 0; bb < D; ++bb) {
      const int blk = b0 + bb;
      fetch(ring[(bb + D - 1) % D], min(blk + D - 1, nblk - 1));
      if (blk < nblk) {
        // c[e] = C[4q + e][i]: row 4q + e of the block, token i
        const f4_t c = step(ring[bb]);
        const int sb = (blk / kBfBps) & 1;  // buffer of this run of blocks
        float* pw = sh.part[sb][blk % kBfBps][wave];
#pragma unroll
        for (int e = 0; e < 4; ++e) pw[64 * e + lane] = c[e];
        if ((blk + 1) % kBfBps == 0 || blk + 1 == nblk) {
          __syncthreads();
          // outputs of the run's blocks (row group, block, row r, token j):
          // the KW partials added in slice order; consecutive threads take
          // consecutive rows
          const int b1 = blk - blk % kBfBps;
          const int nb = blk + 1 - b1;
          for (int o = tid; o < RG * 256 * nb; o += kBfThreads) {
            const int og = o / (256 * nb);
            const int bi = (o >> 8) % nb;
            const int j = (o >> 4) & 15;
            const int r = o & 15;
            const int row = row0 + 16 * (og * nblk + b1 + bi) + r;
            if (row < d.n && j < d.m) {
              const float* pp = &sh.part[sb][bi][og * KW][64 * (r & 3) + 16 * (r >> 2) + j];
              float sum = pp[0];
#pragma unroll
              for (int w2 = 1; w2 < KW; ++w2) sum = __fadd_rn(sum, pp[w2 * 4 * kWave]);
              gmem(y)[static_cast<int64_t>(j) * ldy + row] = __fmul_rn(sum, sh.sws[row - row0]);
            }
          }
        }
      }
    }
  }
}

// Row tiles of three sizes, by `size`: 2 = full (kBfFewMaxTileRows rows,
// NB = F S blocks per row group), 1 = 256 rows (NB = S), 0 = one block per
// row group (16 RG rows).  NB stays a compile-time constant.
__host__ __device__ inline int bf_tile_rows(int k, int size) {
  const int S = bf_few_slices(k / kGroupWeights);
  return size == 2 ? kBfFewMaxTileRows : (size == 1 ? 256 : 16 * (kBfFewWaves / S));
}

template <int S>
__device__ __forceinline__ void gemm_bf16_few_sized(const GemmDesc& d, int row0, int size, BfFewShared& sh) {
  constexpr int F = kBfFewMaxTileRows / 256;
  if (size == 2)
    gemm_bf16_few_tile<S, F * S>(d, row0, sh);
  else if (size == 1 && F > 1)
    gemm_bf16_few_tile<S, S>(d, row0, sh);
  else
    gemm_bf16_few_tile<S, 1>(d, row0, sh);
}

__device__ __forceinline__ void gemm_bf16_few_dispatch(const GemmDesc& d, int tile, int size, BfFewShared& sh) {
  const int row0 = tile * bf_tile_rows(d.k, size);
  switch (bf_few_slices(d.k / kGroupWeights)) {
    case 1: gemm_bf16_few_sized<1>(d, row0, size, sh); break;
    case 2: gemm_bf16_few_sized<2>(d, row0, size, sh); break;
    case 4: gemm_bf16_few_sized<4>(d, row0, size, sh); break;
    case 8: gemm_bf16_few_sized<8>(d, row0, size, sh); break;
    default: gemm_bf16_few_sized<16>(d, row0, size, sh); break;
  }
}

// Single product: the largest tiles that still give every CU a workgroup.
__global__ __launch_bounds__(kBfThreads) void gemm_bf16_few_kernel(GemmDesc d, int size) {
  __shared__ BfFewShared sh;
  gemm_bf16_few_dispatch(d, static_cast<int>(blockIdx.x), size, sh);
}

// Grouped: one workgroup per plan tile {problem, row tile}; a tile is
// kBfFewMaxTileRows rows.
__global__ __launch_bounds__(kBfThreads) void gemm_bf16_few_grouped_kernel(const char* plan) {
  __shared__ BfFewShared sh;
  const PlanHeader* h = reinterpret_cast<const PlanHeader*>(plan);
  const GemmDesc* descs = reinterpret_cast<const GemmDesc*>(plan + sizeof(PlanHeader));
  const GemmTile tl = reinterpret_cast<const GemmTile*>(descs + h->count)[blockIdx.x];
  gemm_bf16_few_dispatch(descs[tl.prob], tl.tile_n, 2, sh);
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmDesc& d, hipStream_t stream) {
  int size = 2;
  while (size > 0 && (d.n + bf_tile_rows(d.k, size) - 1) / bf_tile_rows(d.k, size) < 256) --size;
  const int rows = bf_tile_rows(d.k, size);
  const dim3 grid(static_cast<unsigned>((d.n + rows - 1) / rows));
  hipLaunchKernelGGL(gemm_bf16_few_kernel, grid, dim3(kBfThreads), 0, stream, d, size);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16_grouped(const char* plan, int32_t n_tiles, hipStream_t stream) {
  hipLaunchKernelGGL(gemm_bf16_few_grouped_kernel, dim3(n_tiles), dim3(kBfThreads), 0, stream, plan);
  return hipGetLastError();
}

}  // namespace sherry
