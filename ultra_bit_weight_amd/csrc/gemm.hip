// Products for M tokens, Y[m, r] = s_x[m] * s_w[r] * sum_k X[m, k] T[r, k], on
// packed ternary weights ("Sherry: Hardware-Efficient 1.25-Bit Ternary
// Quantization via Fine-grained Sparsification", Abstract: 3:4 sparse
// ternary blocks in five bits; Figure 2 caption: 4-way blocks).
//
// Small M (decode with a few tokens): codes are expanded in registers straight
// into the A operand of v_mfma_i32_16x16x64_i8 (16 weight rows x 64 k), with
// the tokens as the B operand (16 columns, padded with zeros).  The A and B
// fragments of one lane cover the same 16 reduction indices, so any
// assignment of k to (lane group, byte) is valid as long as A and B use the
// same one: lane (i, q) = (lane % 16, lane / 16) takes its four blocks per
// MFMA from group 4w + q of the workgroup's wave w.  Each wave owns one
// 512-wide slice of k and keeps its tokens' x for that slice in registers
// (x-stationary); the waves' 16x16 partial tiles are summed through LDS.
#include "formats.h"
#include "launch.h"

namespace sherry {
namespace {


constexpr int kMaxKRanges = 16;  // waves per workgroup (k <= 8192 stays x-stationary)

template <class Fmt, bool kStationary>
__global__ __launch_bounds__(1024) void gemm_small_kernel(GemmDesc d, int n_tiles) {
  constexpr int NW = Fmt::kWords;
  __shared__ uint32_t tab[32];
  __shared__ int32_t part[2][kMaxKRanges][kWave * 4];
  Fmt::init_table(tab, threadIdx.x);

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nwaves = blockDim.x / kWave;
  const int i = lane & 15;
  const int q = lane >> 4;
  const int G = d.k / kGroupWeights;
  const int m0 = blockIdx.y * 16;
  const int tok = m0 + i;
  const bool tok_ok = tok < d.m;
  const bool s_f16 = d.flags & kFlagScaleF16;
  const bool y_f16 = d.flags & kFlagYF16;

  // Slices of k handled by this wave: groups 4 * (wave + nwaves * s) + q.
  const int n_slices = (G + 3) / 4;
  uint32_t xr[32];
  auto load_x = [&](int g) {
    const bool ok = tok_ok && g < G;
    const uint4* xp = reinterpret_cast<const uint4*>(d.x + static_cast<int64_t>(tok) * d.ldx +
                                                     static_cast<int64_t>(g) * kGroupWeights);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint4 v = ok ? xp[u] : make_uint4(0, 0, 0, 0);
      xr[4 * u + 0] = v.x;
      xr[4 * u + 1] = v.y;
      xr[4 * u + 2] = v.z;
      xr[4 * u + 3] = v.w;
    }
  };
  if (kStationary) load_x(4 * wave + q);
  __syncthreads();

  int buf = 0;
  for (int tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const int n0 = tile * 16;
    const int row = n0 + i;
    v4i acc = {0, 0, 0, 0};
    for (int s = wave; s < n_slices; s += nwaves) {
      const int g = 4 * s + q;
      if (!kStationary) load_x(g);
      uint32_t w[NW];
      const bool ok = row < d.n && g < G;
      if (ok) {
        Fmt::load(w, d.codes + static_cast<int64_t>(row) * (G * NW), G, g);
      } else {
#pragma unroll
        for (int t = 0; t < NW; ++t) w[t] = 0u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        v4i a, b;
        // A operand: weights of blocks 4u .. 4u+3 of this lane's group; a
        // missing row or group contributes zeros (x is zero there too).
        a[0] = ok ? static_cast<int>(Fmt::i8x4(w, 4 * u + 0, tab)) : 0;
        a[1] = ok ? static_cast<int>(Fmt::i8x4(w, 4 * u + 1, tab)) : 0;
        a[2] = ok ? static_cast<int>(Fmt::i8x4(w, 4 * u + 2, tab)) : 0;
        a[3] = ok ? static_cast<int>(Fmt::i8x4(w, 4 * u + 3, tab)) : 0;
        b[0] = static_cast<int>(xr[4 * u + 0]);
        b[1] = static_cast<int>(xr[4 * u + 1]);
        b[2] = static_cast<int>(xr[4 * u + 2]);
        b[3] = static_cast<int>(xr[4 * u + 3]);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc, 0, 0, 0);
      }
    }
    // acc[e] of lane l is D[4 * (l / 16) + e][l % 16]: weight row, token.
#pragma unroll
    for (int e = 0; e < 4; ++e) part[buf][wave][lane * 4 + e] = acc[e];
    __syncthreads();
    for (int t = threadIdx.x; t < kWave * 4; t += blockDim.x) {
      int sum = 0;
      for (int w2 = 0; w2 < nwaves; ++w2) sum += part[buf][w2][t];
      const int l = t >> 2;
      const int e = t & 3;
      const int r = n0 + 4 * (l >> 4) + e;
      const int m = m0 + (l & 15);
      if (r < d.n && m < d.m) {
        const int64_t o = static_cast<int64_t>(m) * d.n + r;
        if (d.acc) d.acc[o] = sum;
        if (d.y) {
          const float sx = d.x_scales ? d.x_scales[m] : 1.0f;
          store_y(d.y, static_cast<int64_t>(m) * d.ldy + r,
                  epilogue_i32(sum, load_scale(d.w_scales, r, s_f16), sx, d.x_scales != nullptr), y_f16);
        }
      }
    }
    buf ^= 1;
  }
}

// Tiled kernel for many tokens (prefill).  A 4-wave workgroup computes a
// 128 (weight rows) x 128 (tokens) tile of Y, stepping k by one 128-weight
// group.  Wave w owns the 64 x 64 quarter (rows 64 (w & 1), tokens 64 (w >> 1))
// as 4 x 4 MFMA tiles.  Per step:
//   * the tokens' int8 tile (128 x 128 bytes) sits in LDS (double-buffered,
//     one barrier per step; the next tile is loaded into registers first);
//   * lane (i, q) decodes, for each of its 4 row tiles t (row 16 t + i), part q
//     of the group (blocks 8q .. 8q+7, two code words) in registers straight
//     into two A fragments: half s takes blocks 8q + 4s .. 8q + 4s + 3, i.e. k
//     bytes 32q + 16s .. + 16, which is the B fragment it reads from LDS.
constexpr int kTileN = 128;
constexpr int kTileM = 128;

template <class Fmt>
__global__ __launch_bounds__(256) void gemm_tile_kernel(GemmDesc d) {
  __shared__ uint32_t tab[32];
  __shared__ uint4 xt[2][kTileM][9];  // 128 bytes of k per token + 16-byte pad
  Fmt::init_table(tab, threadIdx.x);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int i = lane & 15;
  const int q = lane >> 4;
  const int wn = wave & 1;
  const int wm = wave >> 1;
  const int n0 = blockIdx.x * kTileN;
  const int m0 = blockIdx.y * kTileM;
  const int G = d.k / kGroupWeights;
  const int lastn = d.n - 1;
  const int lastm = d.m - 1;

  // X tile loader: thread t moves token t / 2, bytes 64 (t & 1) .. + 64
  const int xtok = tid >> 1;
  const int xhalf = tid & 1;
  const u32x4_t* xrow =
      reinterpret_cast<const u32x4_t*>(d.x + static_cast<int64_t>(min(m0 + xtok, lastm)) * d.ldx + 64 * xhalf);
  u32x4_t* xdst0 = reinterpret_cast<u32x4_t*>(&xt[0][xtok][4 * xhalf]);
  u32x4_t* xdst1 = reinterpret_cast<u32x4_t*>(&xt[1][xtok][4 * xhalf]);
  // codes of this lane's four weight rows (rows past n read row n - 1)
  const uint32_t* crow[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
    crow[t] = d.codes + static_cast<int64_t>(min(n0 + 64 * wn + 16 * t + i, lastn)) * (G * Fmt::kWords);
  auto load_c = [&](uint32_t (&c)[4][2], int g) {
#pragma unroll
    for (int t = 0; t < 4; ++t) Fmt::part_load(c[t], crow[t], G, g, q);
  };

  v4i acc[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[t][u] = v4i{0, 0, 0, 0};

  u32x4_t x0, x1, x2, x3;
  uint32_t cc[4][2], cn[4][2];
  x0 = xrow[0];
  x1 = xrow[1];
  x2 = xrow[2];
  x3 = xrow[3];
  load_c(cc, 0);
  xdst0[0] = x0;
  xdst0[1] = x1;
  xdst0[2] = x2;
  xdst0[3] = x3;
  __syncthreads();
  for (int g = 0; g < G; ++g) {
    const int buf = g & 1;
    // next step (clamped to the last group: no branch around the loads)
    const int gn = min(g + 1, G - 1);
    {
      const u32x4_t* p = xrow + gn * (kGroupWeights / 16);
      x0 = p[0];
      x1 = p[1];
      x2 = p[2];
      x3 = p[3];
    }
    load_c(cn, gn);
    uint32_t off[4][8];
#pragma unroll
    for (int t = 0; t < 4; ++t) Fmt::part_decode(off[t], cc[t], q);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      v4i b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint4 v = xt[buf][64 * wm + 16 * u + i][2 * q + s];
        b[u] = v4i{static_cast<int>(v.x), static_cast<int>(v.y), static_cast<int>(v.z), static_cast<int>(v.w)};
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const v4i a = {static_cast<int>(Fmt::part_i8x4(off[t], cc[t], 4 * s + 0, tab)),
                       static_cast<int>(Fmt::part_i8x4(off[t], cc[t], 4 * s + 1, tab)),
                       static_cast<int>(Fmt::part_i8x4(off[t], cc[t], 4 * s + 2, tab)),
                       static_cast<int>(Fmt::part_i8x4(off[t], cc[t], 4 * s + 3, tab))};
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[t][u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b[u], acc[t][u], 0, 0, 0);
      }
    }
    u32x4_t* dst = buf ? xdst0 : xdst1;
    dst[0] = x0;
    dst[1] = x1;
    dst[2] = x2;
    dst[3] = x3;
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      cc[t][0] = cn[t][0];
      cc[t][1] = cn[t][1];
    }
  }

  // acc[t][u][e] of lane l is Y[token 16 u + l % 16][row 16 t + 4 (l / 16) + e] of the quarter
  const bool s_f16 = d.flags & kFlagScaleF16;
  const bool y_f16 = d.flags & kFlagYF16;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int m = m0 + 64 * wm + 16 * u + i;
      if (m >= d.m) continue;
      const float sx = d.x_scales ? d.x_scales[m] : 1.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = n0 + 64 * wn + 16 * t + 4 * q + e;
        if (r >= d.n) continue;
        const int32_t v = acc[t][u][e];
        if (d.acc) d.acc[static_cast<int64_t>(m) * d.n + r] = v;
        if (d.y)
          store_y(d.y, static_cast<int64_t>(m) * d.ldy + r,
                  epilogue_i32(v, load_scale(d.w_scales, r, s_f16), sx, d.x_scales != nullptr), y_f16);
      }
    }
  }
}

template <class Fmt>
hipError_t launch_tile(const GemmDesc& d, hipStream_t stream) {
  const dim3 grid((d.n + kTileN - 1) / kTileN, (d.m + kTileM - 1) / kTileM);
  hipLaunchKernelGGL(gemm_tile_kernel<Fmt>, grid, dim3(256), 0, stream, d);
  return hipGetLastError();
}

template <class Fmt>
hipError_t launch_small(const GemmDesc& d, hipStream_t stream) {
  const int G = d.k / kGroupWeights;
  const int n_slices = (G + 3) / 4;
  const bool stationary = n_slices <= kMaxKRanges;
  const int nwaves = stationary ? n_slices : kMaxKRanges;
  const int n_tiles = (d.n + 15) / 16;
  const int m_chunks = (d.m + 15) / 16;
  // Enough workgroups to fill the chip, each walking several row tiles.
  int grid_x = n_tiles;
  const int target = 2048 / (m_chunks > 0 ? m_chunks : 1);
  if (grid_x > target && target > 0) grid_x = target;
  if (grid_x < 1) grid_x = 1;
  dim3 grid(grid_x, m_chunks), block(nwaves * kWave);
  if (stationary)
    hipLaunchKernelGGL((gemm_small_kernel<Fmt, true>), grid, block, 0, stream, d, n_tiles);
  else
    hipLaunchKernelGGL((gemm_small_kernel<Fmt, false>), grid, block, 0, stream, d, n_tiles);
  return hipGetLastError();
}

}  // namespace

// Tokens per launch above which the tiled kernel is used.
constexpr int kTiledMinM = 64;

hipError_t launch_gemm(const GemmDesc& d, int32_t format, hipStream_t stream) {
  if (d.m >= kTiledMinM)
    return format == kFmtTern2 ? launch_tile<Tern2>(d, stream) : launch_tile<Sherry3of4>(d, stream);
  return format == kFmtTern2 ? launch_small<Tern2>(d, stream) : launch_small<Sherry3of4>(d, stream);
}

}  // namespace sherry
