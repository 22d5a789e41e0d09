// Output stage of the tiled int8 products: a wave's 64-row x 16 UT-token
// block of int32 sums (v_mfma_i32_16x16x64_i8 tiles) to Y = s_w s_x acc
// (and the raw sums to acc when asked).
#pragma once

#include "common.h"
#include "launch.h"

namespace sherry {

// acc[t][u] holds the 16 x 16 tile of rows row0 + 16 t .., tokens tok0 + 16 u ..
template <int UT>
__device__ __forceinline__ void tile_store(const GemmDesc& d, const v4i (&acc)[4][UT], int row0, int tok0, int i,
                                           int q) {
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
    const int r0 = row0 + 16 * t + 4 * q;
    if (r0 >= d.n) continue;
    const bool full = r0 + 3 < d.n;
    float sw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) sw[e] = load_scale(d.w_scales, min(r0 + e, d.n - 1), s_f16);
#pragma unroll
    for (int u = 0; u < UT; ++u) {
      const int m = tok0 + 16 * u + i;
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

}  // namespace sherry
