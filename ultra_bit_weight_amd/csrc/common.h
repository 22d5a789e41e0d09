// Device helpers shared by the libsherry kernels (gfx950, wave64).
//
// Format: "Sherry: Hardware-Efficient 1.25-Bit Ternary Quantization via
// Fine-grained Sparsification", Abstract and Figure 2 caption: ternary
// weights, one zero per block of four, a block packed in five bits.  The bit
// layout (code = z | n0<<2 | n1<<3 | n2<<4, 32 codes per LSB-first 5-word
// group) is documented in include/sherry.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sherry.h"

namespace sherry {

constexpr int kGroupWeights = 128;  // weights per group
constexpr int kGroupCodes = 32;     // 4-weight blocks per group
constexpr int kGroupWords = 5;      // uint32 words per group (160 bits)
constexpr int kWave = 64;

// Per-problem record shared by the single and grouped GEMV launches.  The
// grouped plan stores these verbatim, so the layout is fixed (64 bytes).
struct GemvDesc {
  const uint32_t* codes;
  const void* w_scales;
  const void* x;
  const float* x_scale;
  int32_t* acc;
  void* y;
  int32_t n;
  int32_t k;
  int32_t flags;  // kFlag* bits below
  int32_t kclass;
};
static_assert(sizeof(GemvDesc) == 64, "plan record layout");

constexpr int32_t kFlagScaleF16 = 1;  // w_scales are fp16 (else fp32)
constexpr int32_t kFlagYF16 = 2;      // y is fp16 (else fp32)

// Decoded block of one code, as four int8 lanes (slot 0 in the low byte).
// Rule: slot z = code & 3 holds 0; the remaining slots, in ascending order,
// take -1 if their sign bit (code bits 2, 3, 4 in turn) is set, else +1.
__device__ __forceinline__ uint32_t decode_i8x4(uint32_t c) {
  const uint32_t z = c & 3u;
  uint32_t out = 0;
  uint32_t sbit = 2;
#pragma unroll
  for (uint32_t slot = 0; slot < 4; ++slot) {
    if (slot == z) continue;
    const uint32_t byte = ((c >> sbit) & 1u) ? 0xFFu : 0x01u;
    out |= byte << (8 * slot);
    ++sbit;
  }
  return out;
}

// Same block as four bf16 values (0x0000, 0x3F80 = +1, 0xBF80 = -1).
__device__ __forceinline__ uint2 decode_bf16x4(uint32_t c) {
  const uint32_t b = decode_i8x4(c);
  uint32_t h[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t v = (b >> (8 * s)) & 0xFFu;
    h[s] = v == 0 ? 0u : (v == 1 ? 0x3F80u : 0xBF80u);
  }
  return make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
}

// Byte offset (code * SCALE) of code j of a 5-word group held in registers.
// For a code inside one word a shift and a mask suffice; the four codes that
// straddle two words (j = 6, 12, 19, 25) take a funnel shift first.
template <int SCALE_LOG2>
__device__ __forceinline__ uint32_t code_offset(const uint32_t* w, int j) {
  const int bit = 5 * j;
  const int i = bit >> 5;
  const int o = bit & 31;
  const uint32_t mask = 31u << SCALE_LOG2;
  if (o <= 27) {
    if (o >= SCALE_LOG2) return (w[i] >> (o - SCALE_LOG2)) & mask;
    return (w[i] << (SCALE_LOG2 - o)) & mask;
  }
  return __builtin_amdgcn_alignbit(w[i + 1], w[i], o - SCALE_LOG2) & mask;
}

// Row layout: a row of G groups is 5G words; words 0-3 of group g sit at
// 4g (16 bytes, aligned when the row is), word 4 of group g at 4G + g.  So
// the lanes reading consecutive groups issue one contiguous 16-byte-per-lane
// load and one contiguous 4-byte-per-lane load.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));  // MFMA int8 operands / int32 accumulators
typedef int v16i __attribute__((ext_vector_type(16)));  // 32 x 32 MFMA int32 accumulators

// Pointers read from a grouped plan are generic to the compiler, which then
// emits FLAT accesses; those also count against the LDS wait counter, so an
// LDS wait would drain the prefetched loads too.  Every device-memory access
// goes through gmem(), which states the global address space.
#define SHERRY_GLOBAL __attribute__((address_space(1)))
template <class T>
__device__ __forceinline__ const SHERRY_GLOBAL T* gmem(const T* p) {
  return (const SHERRY_GLOBAL T*)p;
}
template <class T>
__device__ __forceinline__ SHERRY_GLOBAL T* gmem(T* p) {
  return (SHERRY_GLOBAL T*)p;
}

__device__ __forceinline__ void load_group(uint32_t* w, const uint32_t* row, int G, int g) {
  const u32x4_t h = __builtin_nontemporal_load(gmem(reinterpret_cast<const u32x4_t*>(row + 4 * g)));
  w[0] = h.x;
  w[1] = h.y;
  w[2] = h.z;
  w[3] = h.w;
  w[4] = __builtin_nontemporal_load(gmem(row + 4 * G + g));
}

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8; a field at its maximum means "do not wait").
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);

// Direct global->LDS copies (global_load_lds_dword{,x4}, saddr form): lane l
// copies 4 or 16 bytes from base + voff to LDS byte address lds + l * size.
// Written as asm so that the compiler does not track them: its wait-count
// pass cannot tell which LDS buffer such a copy writes and would wait for all
// of them before every LDS read.  The kernel waits for them explicitly.  The
// instructions write no register (the address VGPR is read at issue); the
// s_nop covers the M0-write-to-LDS-DMA hazard.
__device__ __forceinline__ void lds_copy16(const SHERRY_GLOBAL void* base, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(lds), "v"(voff), "s"(base)
      : "memory", "m0");
}
__device__ __forceinline__ void lds_copy4(const SHERRY_GLOBAL void* base, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, %2"
      :
      : "s"(lds), "v"(voff), "s"(base)
      : "memory", "m0");
}
// A pointer the caller knows to be the same in every lane, in scalar
// registers (a descriptor read with vector loads is not known uniform to the
// compiler; the copies above take their base from scalar registers).
template <class T>
__device__ __forceinline__ const SHERRY_GLOBAL T* uniform_ptr(const SHERRY_GLOBAL T* p) {
  const uint64_t v = reinterpret_cast<uintptr_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const SHERRY_GLOBAL T*>(static_cast<uintptr_t>((static_cast<uint64_t>(hi) << 32) | lo));
}
template <class T>
__device__ __forceinline__ uint32_t lds_addr(const T* p) {
  return __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) T*)p)));
}

__device__ __forceinline__ uint32_t lds_u32(const uint32_t* base, uint32_t byte_off) {
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(base) + byte_off);
}
__device__ __forceinline__ uint2 lds_u64(const uint2* base, uint32_t byte_off) {
  return *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(base) + byte_off);
}

// ---- wave reductions over aligned lane groups of width W (power of two) ----

// Sum over the group, valid in its LAST lane (in every lane for W <= 16):
// DPP quad_perm and row mirrors inside 16-lane rows, then DPP row broadcasts
// across rows (row_bcast:15 into rows 1 and 3, then row_bcast:31 into rows 2
// and 3), so no LDS round trip.
template <int W>
__device__ __forceinline__ int reduce_add_i32_last(int v) {
  if (W >= 2) v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  if (W >= 4) v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  if (W >= 8) v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  if (W >= 16) v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false); // row_mirror
  if (W >= 32) v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false); // row_bcast:15, rows 1 and 3
  if (W >= 64) v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false); // row_bcast:31, rows 2 and 3
  return v;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// fp32 sum valid in the last lane of each group of W lanes, as
// reduce_add_i32_last (a fixed order, so results repeat bit for bit).
template <int W>
__device__ __forceinline__ float reduce_add_f32_last(float v) {
  if (W >= 2) v += dpp_f32<0xB1>(v);
  if (W >= 4) v += dpp_f32<0x4E>(v);
  if (W >= 8) v += dpp_f32<0x141>(v);
  if (W >= 16) v += dpp_f32<0x140>(v);
  if (W >= 32) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
  if (W >= 64) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
  return v;
}

// ---- epilogue: y = ydt((fp32(acc) * s_w) * s_x), each product IEEE RNE ----
__device__ __forceinline__ float load_scale(const void* s, int r, bool f16) {
  return f16 ? static_cast<float>(gmem(reinterpret_cast<const _Float16*>(s))[r])
             : gmem(reinterpret_cast<const float*>(s))[r];
}

__device__ __forceinline__ void store_y(void* y, int64_t idx, float v, bool f16) {
  if (f16)
    gmem(reinterpret_cast<_Float16*>(y))[idx] = static_cast<_Float16>(v);
  else
    gmem(reinterpret_cast<float*>(y))[idx] = v;
}

__device__ __forceinline__ float epilogue_i32(int32_t acc, float sw, float sx, bool has_sx) {
  float t = __fmul_rn(static_cast<float>(acc), sw);
  if (has_sx) t = __fmul_rn(t, sx);
  return t;
}

}  // namespace sherry
