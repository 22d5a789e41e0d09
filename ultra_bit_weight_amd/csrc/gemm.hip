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

typedef int v4i __attribute__((ext_vector_type(4)));

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

hipError_t launch_gemm(const GemmDesc& d, int32_t format, hipStream_t stream) {
  if (format == kFmtTern2) return launch_small<Tern2>(d, stream);
  return launch_small<Sherry3of4>(d, stream);
}

}  // namespace sherry
