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
// Steps of x and code words the tiled kernel keeps in flight (LDS ring depth).
#ifndef SHERRY_TILE_DEPTH
#define SHERRY_TILE_DEPTH 4
#endif
constexpr int kTileDepth = SHERRY_TILE_DEPTH;
static_assert(kTileDepth >= 2 && kTileDepth <= 4, "tile pipeline depth");
// Workgroups the 256 x 256 tiling must give before it is used.
#ifndef SHERRY_LARGE_TILE_MIN_GROUPS
#define SHERRY_LARGE_TILE_MIN_GROUPS 256
#endif
constexpr int64_t kLargeTileMinGroups = SHERRY_LARGE_TILE_MIN_GROUPS;
// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8; a field at its maximum means "do not wait").
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);

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

// Tiled kernel for many tokens (prefill).  A workgroup of WR x WC waves
// computes a (64 WR weight rows) x (16 UT WC tokens) tile of Y, stepping k by
// one 128-weight group.  Wave w owns rows 64 (w % WR) .. + 64 and tokens
// 16 UT (w / WR) .. + 16 UT as 4 x UT MFMA tiles.
//   * Everything a step reads from memory is copied by the memory system
//     straight into LDS (global_load_lds, no staging registers), kTileDepth
//     steps ahead, into a ring of LDS buffers: the tokens' int8 tile, and per
//     weight row of the tile the group's 16-byte head (words 0-3) and 4-byte
//     tail (word 4).  Within a token's 128 bytes the 16-byte chunk c sits at
//     position c ^ ((token >> 1) & 7), so the B-fragment reads of 16
//     consecutive tokens hit 16 different bank groups.
//   * Lane (i, q) decodes, for each of its 4 row tiles t (row 16 t + i), part q
//     of the group (blocks 8q .. 8q+7, two code words) straight into two A
//     fragments: half s takes blocks 8q + 4s .. 8q + 4s + 3, i.e. k bytes
//     32q + 16s .. + 16, which is the B fragment it reads from LDS.
//   * One barrier per step.  Every vector-memory operation in the loop is one
//     of these copies, a fixed number per wave and step, so before the
//     barrier each wave waits (vmcnt) for exactly its copies of the next
//     step; after it the whole step is in LDS and the buffers of the finished
//     step are free for the copies issued next.
template <int WR_, int WC_, int UT_>
struct TileCfg {
  static constexpr int WR = WR_, WC = WC_, UT = UT_;
  static constexpr int kWaves = WR * WC;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kRows = 64 * WR;
  static constexpr int kTok = 16 * UT * WC;
  static constexpr int kXBytes = kTok * kGroupWeights;            // one step's x tile
  static constexpr int kCopies = kXBytes / (16 * kWave) / kWaves;  // 1 KB x copies per wave per step
  static_assert(kCopies * 16 * kWave * kWaves == kXBytes, "x tile split");
  static constexpr int kRowGroups = kRows / 64;  // 64-row blocks (one copy each per kind)
  static constexpr int kWgPerCu = kWaves <= 4 ? 2 : 1;  // workgroups one CU is sized to hold
};
using TileSmall = TileCfg<2, 2, 4>;  // 128 x 128, 4 waves
using TileLarge = TileCfg<4, 2, 8>;  // 256 x 256, 8 waves

// Ring depth: kTileDepth, or fewer steps if a CU's share of the 160 KB of LDS
// cannot hold them (x tile + code chunks + tail words per step, plus 1 KB).
template <class Fmt, class C>
constexpr int tile_depth() {
  constexpr int slot = C::kXBytes + C::kRows * (16 * Fmt::kTileChunks + (Fmt::kTileTail ? 4 : 0));
  constexpr int fit = (160 * 1024 / C::kWgPerCu - 1024) / slot;
  return fit < kTileDepth ? fit : kTileDepth;
}

template <class Fmt, class C>
__global__ __launch_bounds__(C::kThreads) void gemm_tile_kernel(GemmDesc d) {
  // code copies per step: one per 64-row block and kind (16-byte chunks of
  // the format, then its 4-byte tail word), exactly one per wave
  constexpr int kKinds = Fmt::kTileChunks + (Fmt::kTileTail ? 1 : 0);
  static_assert(kKinds * C::kRowGroups == C::kWaves, "one code copy per wave");
  constexpr int D = tile_depth<Fmt, C>();
  static_assert(D >= 2, "tile ring depth");
  constexpr int UT = C::UT;
  constexpr int NC = C::kCopies;
  constexpr int kOpsPerStep = NC + 1;  // copies per wave and step
  constexpr int XV = C::kXBytes / 16;
  constexpr int R = C::kRows;
  // the code table first in LDS (largest alignment): its address then fits
  // the 16-bit offset field of the lookups
  __shared__ __attribute__((aligned(1024))) uint32_t tab[32];
  // one LDS array per ring slot and kind: distinct objects let the compiler
  // see that reading one slot does not depend on the copies to the others
  __shared__ u32x4_t xt0[XV], xt1[XV], xt2[D > 2 ? XV : 1], xt3[D > 3 ? XV : 1];
  constexpr int HV = R * Fmt::kTileChunks;
  constexpr int TV = Fmt::kTileTail ? R : 1;
  __shared__ u32x4_t hd0[HV], hd1[HV], hd2[D > 2 ? HV : 1], hd3[D > 3 ? HV : 1];
  __shared__ uint32_t tl0[TV], tl1[TV], tl2[D > 2 ? TV : 1], tl3[D > 3 ? TV : 1];
  auto xbuf = [&](int slot) -> u32x4_t* {
    return slot == 0 ? xt0 : slot == 1 ? xt1 : slot == 2 ? xt2 : xt3;
  };
  auto hbuf = [&](int slot) -> u32x4_t* {
    return slot == 0 ? hd0 : slot == 1 ? hd1 : slot == 2 ? hd2 : hd3;
  };
  auto tbuf = [&](int slot) -> uint32_t* {
    return slot == 0 ? tl0 : slot == 1 ? tl1 : slot == 2 ? tl2 : tl3;
  };
  Fmt::init_table(tab, threadIdx.x);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int i = lane & 15;
  const int q = lane >> 4;
  const int wn = wave % C::WR;
  const int wm = wave / C::WR;
  const int n0 = blockIdx.x * R;
  const int m0 = blockIdx.y * C::kTok;
  const int G = d.k / kGroupWeights;
  const int lastn = d.n - 1;
  const int lastm = d.m - 1;
  typedef __attribute__((address_space(3))) void* lds_ptr;

  // x copies: copy j of wave w fills 16-byte slots 64 (NC w + j) + lane of
  // the buffer; slot s holds chunk (s % 8) ^ ((token >> 1) & 7) of token s / 8.
  const SHERRY_GLOBAL int8_t* xsrc[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int slot = 64 * (NC * wave + j) + lane;
    const int tok = slot >> 3;
    const int chunk = (slot & 7) ^ ((tok >> 1) & 7);
    xsrc[j] = gmem(d.x + static_cast<int64_t>(min(m0 + tok, lastm)) * d.ldx + 16 * chunk);
  }
  // code copy of this wave: kind wave / (R / 64) (a 16-byte chunk, or the
  // tail word) of rows 64 c + lane, c = wave % (R / 64); rows past n read row
  // n - 1
  const int cblk = wave % C::kRowGroups;
  const int kind = wave / C::kRowGroups;
  const bool is_chunk = kind < Fmt::kTileChunks;
  const uint32_t* crow = d.codes + static_cast<int64_t>(min(n0 + 64 * cblk + lane, lastn)) * (G * Fmt::kWords);
  auto fetch = [&](int step, int slot) {
    const int g = min(step, G - 1);  // past the end: a valid group, never used
#pragma unroll
    for (int j = 0; j < NC; ++j)
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const SHERRY_GLOBAL void*>(xsrc[j] + static_cast<int64_t>(g) * kGroupWeights),
          (lds_ptr)(xbuf(slot) + 64 * (NC * wave + j)), 16, 0, 0);
    const SHERRY_GLOBAL uint32_t* src = gmem(Fmt::tile_src(crow, G, g, kind));
    if (is_chunk)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const SHERRY_GLOBAL void*>(src),
                                       (lds_ptr)(hbuf(slot) + R * kind + 64 * cblk), 16, 0, 0);
    else
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const SHERRY_GLOBAL void*>(src),
                                       (lds_ptr)(tbuf(slot) + 64 * cblk), 4, 0, 0);
  };

  v4i acc[4][UT];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int u = 0; u < UT; ++u) acc[t][u] = v4i{0, 0, 0, 0};

  auto compute = [&](int slot) {
    const u32x4_t* xb = xbuf(slot);
    const uint32_t* hb = reinterpret_cast<const uint32_t*>(hbuf(slot));
    const uint32_t* tb = tbuf(slot);
    // this lane's two code words of each row tile
    uint32_t w[4][2];
#pragma unroll
    for (int t = 0; t < 4; ++t) Fmt::tile_words(w[t], hb, tb, R, 64 * wn + 16 * t + i, q);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      v4i a[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        uint32_t off[8];
        Fmt::part_decode(off, w[t], q);
        a[t] = v4i{static_cast<int>(Fmt::part_i8x4(off, w[t], 4 * s + 0, tab)),
                   static_cast<int>(Fmt::part_i8x4(off, w[t], 4 * s + 1, tab)),
                   static_cast<int>(Fmt::part_i8x4(off, w[t], 4 * s + 2, tab)),
                   static_cast<int>(Fmt::part_i8x4(off, w[t], 4 * s + 3, tab))};
      }
#pragma unroll
      for (int u = 0; u < UT; ++u) {
        const int tok = 16 * UT * wm + 16 * u + i;
        const u32x4_t v = xb[8 * tok + ((2 * q + s) ^ ((tok >> 1) & 7))];
        const v4i b = {static_cast<int>(v.x), static_cast<int>(v.y), static_cast<int>(v.z), static_cast<int>(v.w)};
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t][u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t], b, acc[t][u], 0, 0, 0);
      }
    }
  };
  // Wait until this wave's copies of step k landed (the copies of the D - 2
  // younger steps may still be in flight), then the barrier.  The empty asm
  // statements keep the compiler from moving memory accesses across.
  auto step_barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(kOpsPerStep * (D - 2)));
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

#pragma unroll
  for (int b = 0; b + 1 < D; ++b) fetch(b, b);
  __syncthreads();  // code table
  for (int g = 0; g < G; g += D) {
#pragma unroll
    for (int b = 0; b < D; ++b) {
      // step g + b: its data sits in slot b; the slot of the previous step
      // ((b + D - 1) % D) is refilled with step g + b + D - 1 after the barrier
      step_barrier();
      fetch(g + b + D - 1, (b + D - 1) % D);
      if (g + b < G) compute(b);
    }
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // no copy may outlive the workgroup

  // acc[t][u][e] of lane l is Y[token 16 u + l % 16][row 16 t + 4 (l / 16) + e]
  // of the wave's sub-tile.  Four consecutive rows of one token are stored
  // together where the layout allows it.
  const bool s_f16 = d.flags & kFlagScaleF16;
  const bool y_f16 = d.flags & kFlagYF16;
  const bool has_sx = d.x_scales != nullptr;
  const bool vec_acc = d.acc && (d.n % 4 == 0) && ((reinterpret_cast<uintptr_t>(d.acc) & 15) == 0);
  const bool vec_y = d.y && (d.ldy % 4 == 0) && ((reinterpret_cast<uintptr_t>(d.y) & 15) == 0);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int r0 = n0 + 64 * wn + 16 * t + 4 * q;
    if (r0 >= d.n) continue;
    const bool full = r0 + 3 < d.n;
    float sw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) sw[e] = load_scale(d.w_scales, min(r0 + e, lastn), s_f16);
#pragma unroll
    for (int u = 0; u < UT; ++u) {
      const int m = m0 + 16 * UT * wm + 16 * u + i;
      if (m >= d.m) continue;
      const float sx = has_sx ? gmem(d.x_scales)[m] : 1.0f;
      const v4i v = acc[t][u];
      if (d.acc) {
        const int64_t o = static_cast<int64_t>(m) * d.n + r0;
        if (vec_acc && full) {
          *gmem(reinterpret_cast<v4i*>(d.acc + o)) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (r0 + e < d.n) gmem(d.acc)[o + e] = v[e];
        }
      }
      if (d.y) {
        const int64_t o = static_cast<int64_t>(m) * d.ldy + r0;
        float f[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = epilogue_i32(v[e], sw[e], sx, has_sx);
        if (vec_y && full) {
          if (y_f16) {
            typedef _Float16 h4 __attribute__((ext_vector_type(4)));
            const h4 hv = {static_cast<_Float16>(f[0]), static_cast<_Float16>(f[1]), static_cast<_Float16>(f[2]),
                           static_cast<_Float16>(f[3])};
            *gmem(reinterpret_cast<h4*>(static_cast<_Float16*>(d.y) + o)) = hv;
          } else {
            typedef float f4 __attribute__((ext_vector_type(4)));
            const f4 fv = {f[0], f[1], f[2], f[3]};
            *gmem(reinterpret_cast<f4*>(static_cast<float*>(d.y) + o)) = fv;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (r0 + e < d.n) store_y(d.y, o + e, f[e], y_f16);
        }
      }
    }
  }
}

// The 256 x 256 tiles when they still give every CU a workgroup, else the
// 128 x 128 tiles.
template <class Fmt>
hipError_t launch_tile(const GemmDesc& d, hipStream_t stream) {
  const int64_t large = ((d.n + TileLarge::kRows - 1) / TileLarge::kRows) *
                        ((d.m + TileLarge::kTok - 1) / TileLarge::kTok);
  if (large >= kLargeTileMinGroups) {
    const dim3 grid((d.n + TileLarge::kRows - 1) / TileLarge::kRows, (d.m + TileLarge::kTok - 1) / TileLarge::kTok);
    hipLaunchKernelGGL((gemm_tile_kernel<Fmt, TileLarge>), grid, dim3(TileLarge::kThreads), 0, stream, d);
  } else {
    const dim3 grid((d.n + TileSmall::kRows - 1) / TileSmall::kRows, (d.m + TileSmall::kTok - 1) / TileSmall::kTok);
    hipLaunchKernelGGL((gemm_tile_kernel<Fmt, TileSmall>), grid, dim3(TileSmall::kThreads), 0, stream, d);
  }
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
