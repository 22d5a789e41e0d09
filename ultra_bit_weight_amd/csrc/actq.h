// Device helpers of the per-token absmax int8 activation quantization (the
// symmetric rule the int8 products take: scale = absmax / 127 by one IEEE
// division, 1 for an all-zero token; each value one IEEE division, round
// half to even, clip to 127), shared by the stand-alone kernel and the
// GEMV that quantizes its x itself.
#pragma once

#include "launch.h"  // kActF32, kActF16, kActBf16

namespace sherry {

constexpr int kActThreads = 256;  // workgroup size of both users

__device__ __forceinline__ float act_value(const void* x, int dt, int64_t i) {
  if (dt == kActF32) return gmem(static_cast<const float*>(x))[i];
  if (dt == kActF16) return static_cast<float>(gmem(static_cast<const _Float16*>(x))[i]);
  return __uint_as_float(static_cast<uint32_t>(gmem(static_cast<const uint16_t*>(x))[i]) << 16);
}

// v combined with the DPP move CTRL of v (rows outside ROWS keep v).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_max(float v) {
  const int b = __float_as_int(v);
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(b, b, CTRL, ROWS, 0xF, false)));
}

// Max over the workgroup (kActThreads threads; every thread gets it).  The
// wave max uses DPP only (no LDS round trips): quad_perm and row mirrors
// inside 16-lane rows, then row broadcasts, so lane 63 holds it.
__device__ __forceinline__ float block_max(float v, float* wmax) {
  v = dpp_max<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_max<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_max<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_max<0x140, 0xF>(v);  // row_mirror
  v = dpp_max<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_max<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  if ((threadIdx.x & (kWave - 1)) == kWave - 1) wmax[threadIdx.x / kWave] = v;
  __syncthreads();
  v = wmax[0];
#pragma unroll
  for (int w = 1; w < kActThreads / kWave; ++w) v = fmaxf(v, wmax[w]);
  return v;
}

__device__ __forceinline__ float act_scale(float amax) { return amax == 0.0f ? 1.0f : __fdiv_rn(amax, 127.0f); }

__device__ __forceinline__ int8_t act_code(float v, float s) {
  const float r = __builtin_rintf(__fdiv_rn(v, s));
  return static_cast<int8_t>(static_cast<int>(fminf(fmaxf(r, -127.0f), 127.0f)));
}

// Tokens of up to kActRegs * kActThreads values: every thread loads its
// values (j = thread + kActThreads i) at once into registers.
constexpr int kActRegs = 32;
constexpr int kActMaxRegK = kActRegs * kActThreads;
static_assert(kActMaxRegK == kActMaxK, "the in-kernel quantization covers every k it accepts");

// The token's values as raw bits, every load issued before any is used:
// indices past k are clamped to the last value (an unconditional load; a
// conditional one, or a conversion next to the load, made the compiler wait
// for each load before issuing the next), and act_raw_value converts them
// afterwards (zero past k).  XB = 4: 32-bit values, kept as bits; XB = 2:
// 16-bit values, zero-extended.  (A compile-time width: with a run-time
// branch between the two kinds of load, the compiler drained every load in
// flight on entry to one of them.)  NR values per thread (NR * kActThreads
// >= k; k fits 32 bits here).
template <int NR, int XB>
__device__ __forceinline__ void act_issue_raw(const void* x, int64_t base, int64_t k, uint32_t (&raw)[NR]) {
  static_assert(XB == 2 || XB == 4, "16- or 32-bit values");
  const int last = static_cast<int>(k) - 1;
  const int t = static_cast<int>(threadIdx.x);
  if constexpr (XB == 4) {
    const SHERRY_GLOBAL uint32_t* p = gmem(static_cast<const uint32_t*>(x)) + base;
#pragma unroll
    for (int i = 0; i < NR; ++i) raw[i] = p[min(t + i * kActThreads, last)];
  } else {
    const SHERRY_GLOBAL uint16_t* p = gmem(static_cast<const uint16_t*>(x)) + base;
#pragma unroll
    for (int i = 0; i < NR; ++i) raw[i] = p[min(t + i * kActThreads, last)];
  }
}

__device__ __forceinline__ float act_raw_value(uint32_t r, int dt, bool valid) {
  const float v = dt == kActF32 ? __uint_as_float(r)
                                : (dt == kActF16 ? static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(r)))
                                                 : __uint_as_float(r << 16));
  return valid ? v : 0.0f;
}

__device__ __forceinline__ float act_load_token(const void* x, int dt, int64_t base, int64_t k, float (&v)[kActRegs]) {
  uint32_t raw[kActRegs];
  if (dt == kActF32)
    act_issue_raw<kActRegs, 4>(x, base, k, raw);
  else
    act_issue_raw<kActRegs, 2>(x, base, k, raw);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kActRegs; ++i) {
    v[i] = act_raw_value(raw[i], dt, static_cast<int>(threadIdx.x) + i * kActThreads < k);
    amax = fmaxf(amax, fabsf(v[i]));
  }
  return amax;
}

}  // namespace sherry
