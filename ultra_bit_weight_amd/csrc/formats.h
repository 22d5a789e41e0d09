// Decoders for the two weight formats handled by the GEMV / GEMM kernels.
//
// Both expose the same interface so one kernel template serves both:
//   kWords            uint32 words per 128-weight group of one row
//   init_table(lds)   fill the workgroup's lookup table (call from 32 lanes)
//   load(w, row, G, g) load group g of a row (row points at the row's words)
//   i8x4(w, j, tab)   int8x4 dword of weights 4j .. 4j+3 of the group
//
// Sherry3of4: 3:4-sparse ternary, 5-bit block codes ("Sherry: Hardware-
//   Efficient 1.25-Bit Ternary Quantization via Fine-grained Sparsification",
//   Abstract; Figure 2 caption: four weights packed in five bits).  A code is
//   expanded through a 32-entry table in LDS: one shift-and-mask gives the
//   table byte offset, one LDS read the four int8 weights.  The 32 entries sit
//   in 32 distinct banks, so lookups never conflict.
// Tern2: the 2-bit aligned comparator (same paper, Figure 2 caption, left).
//   Weight 4q+p of a word sits at bits 8p+2q, so (w >> 2q) & 0x03030303 holds
//   four 2-bit fields, one per byte, and v_perm_b32 with the constant
//   0xFF000100 maps field values 0, 1, 3 to bytes 0x00, 0x01, 0xFF.
#pragma once

#include "common.h"

namespace sherry {

struct Sherry3of4 {
  static constexpr int kWords = kGroupWords;
  __device__ static void init_table(uint32_t* tab, int t) {
    if (t < 32) tab[t] = decode_i8x4(static_cast<uint32_t>(t));
  }
  __device__ __forceinline__ static void load(uint32_t* w, const uint32_t* row, int G, int g) {
    load_group(w, row, G, g);
  }
  __device__ __forceinline__ static uint32_t i8x4(const uint32_t* w, int j, const uint32_t* tab) {
    return lds_u32(tab, code_offset<2>(w, j));
  }
  // group g of a row held in LDS (same layout as in memory)
  __device__ __forceinline__ static void lds_load(uint32_t* w, const uint32_t* row, int G, int g) {
    const uint4 h = *reinterpret_cast<const uint4*>(row + 4 * g);
    w[0] = h.x;
    w[1] = h.y;
    w[2] = h.z;
    w[3] = h.w;
    w[4] = row[4 * G + g];
  }
};

struct Tern2 {
  static constexpr int kWords = 8;  // 128 weights * 2 bits
  __device__ static void init_table(uint32_t*, int) {}
  __device__ __forceinline__ static void load(uint32_t* w, const uint32_t* row, int, int g) {
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(row + 8 * g);
    const u32x4_t a = __builtin_nontemporal_load(p);
    const u32x4_t b = __builtin_nontemporal_load(p + 1);
    w[0] = a.x;
    w[1] = a.y;
    w[2] = a.z;
    w[3] = a.w;
    w[4] = b.x;
    w[5] = b.y;
    w[6] = b.z;
    w[7] = b.w;
  }
  __device__ __forceinline__ static uint32_t i8x4(const uint32_t* w, int j, const uint32_t*) {
    const uint32_t sel = (w[j >> 2] >> (2 * (j & 3))) & 0x03030303u;
    return __builtin_amdgcn_perm(0u, 0xFF000100u, sel);
  }
  __device__ __forceinline__ static void lds_load(uint32_t* w, const uint32_t* row, int, int g) {
    const uint4 a = *reinterpret_cast<const uint4*>(row + 8 * g);
    const uint4 b = *reinterpret_cast<const uint4*>(row + 8 * g + 4);
    w[0] = a.x;
    w[1] = a.y;
    w[2] = a.z;
    w[3] = a.w;
    w[4] = b.x;
    w[5] = b.y;
    w[6] = b.z;
    w[7] = b.w;
  }
};

}  // namespace sherry
