// Output stage of the tiled int8 products: a wave's 64-row x 16 UT-token
// block of int32 sums (v_mfma_i32_16x16x64_i8 tiles) to Y = s_w s_x acc
// (and the raw sums to acc when asked).
#pragma once

#include "common.h"
#include "launch.h"

namespace sherry {

// Scales of the output stage, staged through LDS.  When its tile starts,
// thread t loads the scale of row n0 + t and of token m0 + t (t past the
// tile: the tile's last; rows and tokens clamped to the matrix).  After the k
// loop, stage() writes them to LDS (R row scales, then T token scales, as
// fp32) for the output stage.  By then the loads have long completed, so the
// waves do not stall on them at the end of the tile, when nothing else keeps
// the CU busy.
struct EpiScales {
  uint32_t w;  // the row scale's bits: fp16 in the low half, or fp32
  float x;     // the token scale (1 without token scales)
  __device__ __forceinline__ void load(const GemmDesc& d, int n0, int m0, int R, int T, int tid) {
    const int r = min(n0 + min(tid, R - 1), d.n - 1);
    if (d.flags & kFlagScaleF16)
      w = gmem(static_cast<const uint16_t*>(d.w_scales))[r];
    else
      w = gmem(static_cast<const uint32_t*>(d.w_scales))[r];
    x = d.x_scales ? gmem(d.x_scales)[min(m0 + min(tid, T - 1), d.m - 1)] : 1.0f;
  }
  // Call between two barriers, after every wave's last LDS read of `lds`.
  __device__ __forceinline__ void stage(const GemmDesc& d, float* lds, int R, int T, int tid) const {
    if (tid < R)
      lds[tid] = (d.flags & kFlagScaleF16) ? static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w)))
                                           : __builtin_bit_cast(float, w);
    if (tid < T) lds[R + tid] = x;
  }
};

// acc[t][u] holds the 16 x 16 tile of rows row0 + 16 t .., tokens tok0 + 16 u ..
// sw / sx: the LDS scales of rows row0 .. and tokens tok0 .. (EpiScales).
template <int UT>
__device__ __forceinline__ void tile_store(const GemmDesc& d, const v4i (&acc)[4][UT], int row0, int tok0, int i,
                                           int q, const float* sw_l, const float* sx_l) {
  // acc[t][u][e] of lane l is Y[token 16 u + l % 16][row 16 t + 4 (l / 16) + e]
  // of the wave's sub-tile.  Four consecutive rows of one token are stored
  // together where the layout allows it.
  const bool y_f16 = d.flags & kFlagYF16;
  const bool has_sx = d.x_scales != nullptr;
  const bool vec_acc = d.acc && (d.n % 4 == 0) && ((reinterpret_cast<uintptr_t>(d.acc) & 15) == 0);
  const bool vec_y = d.y && (d.ldy % 4 == 0) && ((reinterpret_cast<uintptr_t>(d.y) & 15) == 0);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int r0 = row0 + 16 * t + 4 * q;
    if (r0 >= d.n) continue;
    const bool full = r0 + 3 < d.n;
    float sw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) sw[e] = sw_l[16 * t + 4 * q + e];
#pragma unroll
    for (int u = 0; u < UT; ++u) {
      const int m = tok0 + 16 * u + i;
      if (m >= d.m) continue;
      const float sx = sx_l[16 * u + i];
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

// 32 x 32 tiles (v_mfma_i32_32x32x32_i8): element 4 j + e of acc[t][u] in
// lane l is row row0 + 32 t + 8 j + 4 (l / 32) + e, token tok0 + 32 u + l % 32.
template <int RT, int U>
__device__ __forceinline__ void tile_store32(const GemmDesc& d, const v16i (&acc)[RT][U], int row0, int tok0,
                                             int lane, const float* sw_l, const float* sx_l) {
  const bool y_f16 = d.flags & kFlagYF16;
  const bool has_sx = d.x_scales != nullptr;
  const bool vec_acc = d.acc && (d.n % 4 == 0) && ((reinterpret_cast<uintptr_t>(d.acc) & 15) == 0);
  const bool vec_y = d.y && (d.ldy % 4 == 0) && ((reinterpret_cast<uintptr_t>(d.y) & 15) == 0);
  const int h = lane >> 5;
  const int c = lane & 31;
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r0 = row0 + 32 * t + 8 * j + 4 * h;
      if (r0 >= d.n) continue;
      const bool full = r0 + 3 < d.n;
      float sw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) sw[e] = sw_l[32 * t + 8 * j + 4 * h + e];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int m = tok0 + 32 * u + c;
        if (m >= d.m) continue;
        const float sx = sx_l[32 * u + c];
        const v4i v = {acc[t][u][4 * j], acc[t][u][4 * j + 1], acc[t][u][4 * j + 2], acc[t][u][4 * j + 3]};
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

}  // namespace sherry
