// Decoders for the two weight formats handled by the GEMV / GEMM kernels.
//
// Both expose the same interface so one kernel template serves both:
//   kWords            uint32 words per 128-weight group of one row
//   init_table(lds)   fill the workgroup's lookup table (call from 32 lanes)
//   load(w, row, G, g) load group g of a row (row points at the row's words)
//   i8x4(w, j, tab)   int8x4 dword of weights 4j .. 4j+3 of the group
//   i8x8(w, p, pairs) the eight weights 8p .. 8p+7 (GEMV; pair table in LDS)
//
// Sherry3of4: 3:4-sparse ternary, 5-bit block codes ("Sherry: Hardware-
//   Efficient 1.25-Bit Ternary Quantization via Fine-grained Sparsification",
//   Abstract; Figure 2 caption: four weights packed in five bits).  A code is
//   expanded through a 32-entry table in LDS: one shift-and-mask gives the
//   table byte offset, one LDS read the four int8 weights.  The 32 entries sit
//   in 32 distinct banks, so lookups never conflict.  The GEMV reads two codes
//   at once from a 1024-entry table of eight weights (8 KB): one extraction
//   and one 8-byte LDS read per two blocks.
// Tern2: the 2-bit aligned comparator (same paper, Figure 2 caption, left).
//   Weight 4q+p of a word sits at bits 8p+2q, so (w >> 2q) & 0x03030303 holds
//   four 2-bit fields, one per byte, and v_perm_b32 with the constant
//   0xFF000100 maps field values 0, 1, 3 to bytes 0x00, 0x01, 0xFF.
#pragma once

#include "common.h"

namespace sherry {

struct Sherry3of4 {
  static constexpr int kWords = kGroupWords;
  static constexpr int kPairEntries = 1024;  // GEMV table: two codes per entry
  __device__ static void init_table(uint32_t* tab, int t) {
    if (t < 32) tab[t] = decode_i8x4(static_cast<uint32_t>(t));
  }
  // Pair table for the GEMV: entry c0 | c1 << 5 holds the eight int8 weights
  // of codes c0 (low dword) and c1, i.e. of two consecutive blocks.  Built
  // from the 32-entry table tab32 (filled and synchronised before the call).
  __device__ static void init_pair_table(uint2* pairs, const uint32_t* tab32, int t, int nthreads) {
    for (int e = t; e < kPairEntries; e += nthreads) pairs[e] = make_uint2(tab32[e & 31], tab32[e >> 5]);
  }
  // Weights of blocks 2p and 2p + 1 of a group: the two codes form the 10-bit
  // field at bit 10p of the stream, which is the pair-table index.
  __device__ __forceinline__ static uint2 i8x8(const uint32_t* w, int p, const uint2* pairs) {
    const int bit = 10 * p;
    const int i = bit >> 5;
    const int o = bit & 31;
    constexpr uint32_t mask = 0x3FFu << 3;  // index * 8 = byte offset
    uint32_t off;
    if (o <= 22)
      off = (o >= 3 ? (w[i] >> (o - 3)) : (w[i] << (3 - o))) & mask;
    else
      off = __builtin_amdgcn_alignbit(w[i + 1], w[i], o - 3) & mask;
    return lds_u64(pairs, off);
  }
  __device__ __forceinline__ static void load(uint32_t* w, const uint32_t* row, int G, int g) {
    load_group(w, row, G, g);
  }
  __device__ __forceinline__ static uint32_t i8x4(const uint32_t* w, int j, const uint32_t* tab) {
    return lds_u32(tab, code_offset<2>(w, j));
  }
  // Tiled GEMM: lane part q (0..3) of a group is blocks 8q .. 8q+7, bits
  // [40q, 40q + 40) of the 160-bit stream, which lie in words q and q + 1.
  // part_words returns the word offsets of those two words for group g:
  // word i < 4 sits at 4g + i, word 4 at 4G + g.
  __device__ __forceinline__ static void part_load(uint32_t* w, const uint32_t* row, int G, int g, int q) {
    w[0] = __builtin_nontemporal_load(gmem(row + 4 * g + q));
    w[1] = __builtin_nontemporal_load(gmem(row + (q < 3 ? 4 * g + q + 1 : 4 * G + g)));
  }
  // the 8 codes of part q as table offsets (code * 4)
  __device__ __forceinline__ static void part_decode(uint32_t (&o)[8], const uint32_t* w, int q) {
    const uint32_t sh = (8u * static_cast<uint32_t>(q)) & 31u;  // 40q mod 32
    const uint32_t lo = __builtin_amdgcn_alignbit(w[1], w[0], sh);  // window bits 0..31
    const uint32_t hi = w[1] >> sh;                                 // window bits 32..
#pragma unroll
    for (int e = 0; e < 6; ++e) o[e] = e == 0 ? (lo << 2) & 0x7Cu : (lo >> (5 * e - 2)) & 0x7Cu;
    o[6] = __builtin_amdgcn_alignbit(hi, lo, 28) & 0x7Cu;  // window bits 30..34
    o[7] = (hi >> 1) & 0x7Cu;                              // window bits 35..39
  }
  __device__ __forceinline__ static uint32_t part_i8x4(const uint32_t (&o)[8], const uint32_t* w, int b,
                                                       const uint32_t* tab) {
    (void)w;
    return lds_u32(tab, o[b]);
  }
  // Tiled GEMM copies a step's words of a row into LDS as kTileChunks 16-byte
  // chunks (chunk-major, rows contiguous) and, with kTileTail, one 4-byte word:
  // here words 0-3 of group g (at 4g) and word 4 (at 4G + g).
  static constexpr int kTileChunks = 1;
  static constexpr bool kTileTail = true;
  __device__ __forceinline__ static const uint32_t* tile_src(const uint32_t* row, int G, int g, int kind) {
    return kind < kTileChunks ? row + 4 * g : row + 4 * G + g;
  }
  // the two words of part q of row r from those LDS copies (R rows per chunk)
  __device__ __forceinline__ static void tile_words(uint32_t* w, const uint32_t* chunks, const uint32_t* tail, int R,
                                                    int r, int q) {
    (void)R;
    w[0] = chunks[4 * r + q];
    w[1] = q < 3 ? chunks[4 * r + q + 1] : tail[r];
  }
};

struct Tern2 {
  static constexpr int kWords = 8;  // 128 weights * 2 bits
  static constexpr int kPairEntries = 1;
  __device__ static void init_table(uint32_t*, int) {}
  __device__ static void init_pair_table(uint2*, const uint32_t*, int, int) {}
  __device__ __forceinline__ static void load(uint32_t* w, const uint32_t* row, int, int g) {
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(row + 8 * g);
    const u32x4_t a = __builtin_nontemporal_load(gmem(p));
    const u32x4_t b = __builtin_nontemporal_load(gmem(p + 1));
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
  __device__ __forceinline__ static uint2 i8x8(const uint32_t* w, int p, const uint2*) {
    return make_uint2(i8x4(w, 2 * p, nullptr), i8x4(w, 2 * p + 1, nullptr));
  }
  // Tiled GEMM: lane part q of a group is weights 32q .. 32q + 31, words 2q
  // and 2q + 1 of the group; block b (0..7) of the part is quarter b & 3 of
  // word 2q + (b >> 2).
  __device__ __forceinline__ static void part_load(uint32_t* w, const uint32_t* row, int, int g, int q) {
    const u32x2_t v = *gmem(reinterpret_cast<const u32x2_t*>(row + 8 * g + 2 * q));
    w[0] = v.x;
    w[1] = v.y;
  }
  __device__ __forceinline__ static void part_decode(uint32_t (&)[8], const uint32_t*, int) {}
  __device__ __forceinline__ static uint32_t part_i8x4(const uint32_t (&)[8], const uint32_t* w, int b,
                                                       const uint32_t*) {
    const uint32_t sel = (w[b >> 2] >> (2 * (b & 3))) & 0x03030303u;
    return __builtin_amdgcn_perm(0u, 0xFF000100u, sel);
  }
  // Tiled GEMM copies: the group's 8 words as two 16-byte chunks, no tail.
  static constexpr int kTileChunks = 2;
  static constexpr bool kTileTail = false;
  __device__ __forceinline__ static const uint32_t* tile_src(const uint32_t* row, int, int g, int kind) {
    return row + 8 * g + 4 * kind;
  }
  __device__ __forceinline__ static void tile_words(uint32_t* w, const uint32_t* chunks, const uint32_t*, int R,
                                                    int r, int q) {
    const uint32_t* h = chunks + 4 * ((q >> 1) * R + r) + 2 * (q & 1);
    w[0] = h[0];
    w[1] = h[1];
  }
};

}  // namespace sherry
