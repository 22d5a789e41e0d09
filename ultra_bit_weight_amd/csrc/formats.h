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
  static constexpr int kGroupW = kGroupWeights;  // weights per group
  static constexpr bool kTableDecode = true;  // decoding reads LDS
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
  // The same words of the row at byte offset ro from a uniform base: 32-bit
  // lane offsets (one matrix's codes stay below 4 GiB), so the loads take the
  // base from scalar registers and need no 64-bit address arithmetic.
  __device__ __forceinline__ static void load_at(uint32_t* w, const SHERRY_GLOBAL char* base, uint32_t ro, int G,
                                                 int g) {
    const u32x4_t h = __builtin_nontemporal_load(
        reinterpret_cast<const SHERRY_GLOBAL u32x4_t*>(base + (ro + 16u * static_cast<uint32_t>(g))));
    w[0] = h.x;
    w[1] = h.y;
    w[2] = h.z;
    w[3] = h.w;
    // word 4 with an ordinary (cached) load: the row's run of tail words
    // shares cache lines with the next row's head run (non-temporal as well,
    // the grouped launch measured about 1 % slower)
    w[4] = *reinterpret_cast<const SHERRY_GLOBAL uint32_t*>(base + (ro + 4u * static_cast<uint32_t>(4 * G + g)));
  }
  // Same words with ordinary (cached) loads, for kernels whose waves share
  // the cache lines of a row.
  __device__ __forceinline__ static void load_cached(uint32_t* w, const uint32_t* row, int G, int g) {
    const u32x4_t h = *gmem(reinterpret_cast<const u32x4_t*>(row + 4 * g));
    w[0] = h.x;
    w[1] = h.y;
    w[2] = h.z;
    w[3] = h.w;
    w[4] = *gmem(row + 4 * G + g);
  }
  __device__ __forceinline__ static uint32_t i8x4(const uint32_t* w, int j, const uint32_t* tab) {
    return lds_u32(tab, code_offset<2>(w, j));
  }
  // Tiled GEMM: lane part q (0..3) of a group is blocks 8q .. 8q+7, bits
  // [40q, 40q + 40) of the 160-bit stream, which lie in words q and q + 1
  // (w[0], w[1]).  frag returns half s of the part (blocks 8q + 4s .. + 4) as
  // an MFMA int8 fragment: four table lookups.
  __device__ __forceinline__ static v4i frag(const uint32_t* w, int q, int s, const uint32_t* tab) {
    const uint32_t sh = (8u * static_cast<uint32_t>(q)) & 31u;     // 40q mod 32
    const uint32_t lo = __builtin_amdgcn_alignbit(w[1], w[0], sh);  // window bits 0..31
    uint32_t o[4];
    if (s == 0) {
      o[0] = (lo << 2) & 0x7Cu;
      o[1] = (lo >> 3) & 0x7Cu;
      o[2] = (lo >> 8) & 0x7Cu;
      o[3] = (lo >> 13) & 0x7Cu;
    } else {
      const uint32_t hi = w[1] >> sh;  // window bits 32..
      o[0] = (lo >> 18) & 0x7Cu;
      o[1] = (lo >> 23) & 0x7Cu;
      o[2] = __builtin_amdgcn_alignbit(hi, lo, 28) & 0x7Cu;  // window bits 30..34
      o[3] = (hi >> 1) & 0x7Cu;                              // window bits 35..39
    }
    return v4i{static_cast<int>(lds_u32(tab, o[0])), static_cast<int>(lds_u32(tab, o[1])),
               static_cast<int>(lds_u32(tab, o[2])), static_cast<int>(lds_u32(tab, o[3]))};
  }
  // Tiled GEMM: codes reach LDS in stages of kTileP groups per row, as
  // kTileHC 16-byte head chunks (words 0-3 of each group, contiguous in the
  // row) and, with kTileTail, kTileP tail words (word 4 of each group).
  static constexpr int kTileP = 4;
  static constexpr int kTileHC = 4;
  static constexpr bool kTileTail = true;
  // Head chunk c of the stage of groups 0 .. P-1 is bytes 16 c of the row;
  // the next stage's heads start kTileP kTileHeadBytes further, its tails
  // 4 kTileP bytes further.
  static constexpr int kTileHeadBytes = 16;  // head bytes per group (words 0-3)
  __device__ __forceinline__ static uint32_t tile_tail_byte(int G, int j) { return 16u * G + 4u * j; }
  // Part q of group j of a stage from the LDS copy.  heads / tails point at
  // the first row of the lane's row tile; lh / lt are the lane's byte
  // offsets from there (its row), and chunk c of a row sits at position
  // c ^ swz.  The next head word, or for part 3 the group's tail word,
  // completes the part.
  __device__ __forceinline__ static void stage_words(uint32_t* w, const char* heads, const char* tails,
                                                     uint32_t lh, uint32_t lt, int swz, int j, int q) {
    const char* c = heads + lh + 16 * (j ^ swz);
    w[0] = *reinterpret_cast<const uint32_t*>(c + 4 * q);
    const uint32_t nxt = *reinterpret_cast<const uint32_t*>(c + 4 * min(q + 1, 3));
    const uint32_t tail = *reinterpret_cast<const uint32_t*>(tails + lt + 4 * j);
    w[1] = q < 3 ? nxt : tail;
  }
  // 32 x 32 tiles: in substep s (of four) lane half h of a row takes blocks
  // 8 s + 4 h .. + 3 of a group (k bytes 32 s + 16 h .. + 16, x chunk
  // 2 s + h).  window32 shifts the 160-bit group down by 20 h bits (a
  // per-lane funnel-shift amount, no select between the halves), so those
  // blocks sit at window bits 40 s .. 40 s + 19 for either half; frag32
  // expands them with four table lookups.
  static constexpr int kWin = 5;
  __device__ __forceinline__ static int x_chunk32(int h, int s) { return 2 * s + h; }
  __device__ __forceinline__ static void window32(uint32_t (&win)[kWin], const char* heads, const char* tails,
                                                  uint32_t lh, uint32_t lt, int swz, int j, int h) {
    const u32x4_t c = *reinterpret_cast<const u32x4_t*>(heads + lh + 16 * (j ^ swz));
    const uint32_t tail = *reinterpret_cast<const uint32_t*>(tails + lt + 4 * j);
    const uint32_t sh = 20u * static_cast<uint32_t>(h);
    win[0] = __builtin_amdgcn_alignbit(c.y, c.x, sh);
    win[1] = __builtin_amdgcn_alignbit(c.z, c.y, sh);
    win[2] = __builtin_amdgcn_alignbit(c.w, c.z, sh);
    win[3] = __builtin_amdgcn_alignbit(tail, c.w, sh);
    win[4] = tail >> sh;
  }
  __device__ __forceinline__ static v4i frag32(const uint32_t (&win)[kWin], int s, const uint32_t* tab) {
    return v4i{static_cast<int>(i8x4(win, 8 * s, tab)), static_cast<int>(i8x4(win, 8 * s + 1, tab)),
               static_cast<int>(i8x4(win, 8 * s + 2, tab)), static_cast<int>(i8x4(win, 8 * s + 3, tab))};
  }
};

struct Tern2 {
  static constexpr int kWords = 8;  // 128 weights * 2 bits
  static constexpr int kGroupW = kGroupWeights;
  static constexpr bool kTableDecode = false;
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
  __device__ __forceinline__ static void load_at(uint32_t* w, const SHERRY_GLOBAL char* base, uint32_t ro, int,
                                                 int g) {
    const SHERRY_GLOBAL u32x4_t* p =
        reinterpret_cast<const SHERRY_GLOBAL u32x4_t*>(base + (ro + 32u * static_cast<uint32_t>(g)));
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
  __device__ __forceinline__ static void load_cached(uint32_t* w, const uint32_t* row, int, int g) {
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(row + 8 * g);
    const u32x4_t a = *gmem(p);
    const u32x4_t b = *gmem(p + 1);
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
  // and 2q + 1 of the group (w[0], w[1]); block b (0..7) of the part is
  // quarter b & 3 of word b >> 2.  frag returns half s (blocks 4s .. 4s + 3).
  __device__ __forceinline__ static v4i frag(const uint32_t* w, int, int s, const uint32_t*) {
    const uint32_t x = w[s];
    return v4i{static_cast<int>(__builtin_amdgcn_perm(0u, 0xFF000100u, x & 0x03030303u)),
               static_cast<int>(__builtin_amdgcn_perm(0u, 0xFF000100u, (x >> 2) & 0x03030303u)),
               static_cast<int>(__builtin_amdgcn_perm(0u, 0xFF000100u, (x >> 4) & 0x03030303u)),
               static_cast<int>(__builtin_amdgcn_perm(0u, 0xFF000100u, (x >> 6) & 0x03030303u))};
  }
  // Tiled GEMM stages: 2 groups per row (4 chunks of 16 bytes), no tail.
  static constexpr int kTileP = 2;
  static constexpr int kTileHC = 4;
  static constexpr bool kTileTail = false;
  // Head chunk c of the stage of groups 0 .. P-1 is bytes 16 c of the row
  // (group c / 2, half c % 2); the next stage starts kTileP groups further.
  static constexpr int kTileHeadBytes = 32;  // bytes per group
  __device__ __forceinline__ static uint32_t tile_tail_byte(int, int) { return 0; }
  __device__ __forceinline__ static void stage_words(uint32_t* w, const char* heads, const char*, uint32_t lh,
                                                     uint32_t, int swz, int j, int q) {
    const uint32_t* c =
        reinterpret_cast<const uint32_t*>(heads + lh + 16 * ((2 * j + (q >> 1)) ^ swz) + 8 * (q & 1));
    w[0] = c[0];
    w[1] = c[1];
  }
  // 32 x 32 tiles: lane half h takes words 4 h .. 4 h + 3 of a group (chunk
  // 2 j + h of the stage); word 4 h + s holds k bytes 64 h + 16 s .. + 16
  // (x chunk 4 h + s).
  static constexpr int kWin = 4;
  __device__ __forceinline__ static int x_chunk32(int h, int s) { return 4 * h + s; }
  __device__ __forceinline__ static void window32(uint32_t (&win)[kWin], const char* heads, const char*, uint32_t lh,
                                                  uint32_t, int swz, int j, int h) {
    const u32x4_t c = *reinterpret_cast<const u32x4_t*>(heads + lh + 16 * ((2 * j + h) ^ swz));
    win[0] = c.x;
    win[1] = c.y;
    win[2] = c.z;
    win[3] = c.w;
  }
  __device__ __forceinline__ static v4i frag32(const uint32_t (&win)[kWin], int s, const uint32_t* tab) {
    return frag(win, 0, s, tab);  // word s of the window
  }
};

// Tern3: the 1.67-bit comparator, three ternary weights per 5-bit code
// (base 3: c = (t0 + 1) + 3 (t1 + 1) + 9 (t2 + 1); same paper, Figure 2
// caption, middle), 32 codes per group of 96 weights in the stream and
// two-part row layout of Sherry3of4, rows zero-padded to whole groups.  A
// code expands to a dword of three int8 weights and a zero byte, so the
// code extraction, tables and GEMV of Sherry3of4 serve it unchanged; only the
// table differs, and x is taken 3 bytes per code (repacked per lane).
__device__ __forceinline__ uint32_t decode_t3_i8x3(uint32_t c) {
  if (c >= 27) return 0u;  // not a code
  const uint32_t t0 = c % 3u, t1 = (c / 3u) % 3u, t2 = c / 9u;  // digit 0, 1, 2 = weight -1, 0, +1
  auto b = [](uint32_t d) { return d == 0u ? 0xFFu : (d == 1u ? 0x00u : 0x01u); };
  return b(t0) | (b(t1) << 8) | (b(t2) << 16);
}

struct Tern3 : Sherry3of4 {
  static constexpr int kGroupW = 96;
  __device__ static void init_table(uint32_t* tab, int t) {
    if (t < 32) tab[t] = decode_t3_i8x3(static_cast<uint32_t>(t));
  }
};

// Byte offsets code * 8 of the 32 codes of a group (8-byte table entries)
// with one bit-field extraction for most codes.  Code j sits at bit
// o = 5j mod 32 of word 5j / 32; its offset is the 8-bit field
// [o - 3, o + 5) once the three bits under the code -- the top three bits of
// code j - 1 -- are zero.  Two masked copies of the words provide that: m[0..4]
// with bits 2-4 of every odd code cleared (for even j), m[5..9] with those of
// every even code (odd j).  The copies pass through an empty asm statement,
// or the compiler folds the cleared bits back into a shift and a mask.
constexpr uint32_t top3_bits(int word, int parity) {
  uint32_t m = 0;
  for (int j = parity; j < 32; j += 2)
    for (int b = 5 * j + 2; b <= 5 * j + 4; ++b)
      if (b >= 32 * word && b < 32 * word + 32) m |= 1u << (b - 32 * word);
  return m;
}

__device__ __forceinline__ void masked_words8(const uint32_t* w, uint32_t* m) {
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    m[i] = w[i] & ~top3_bits(i, 1);
    m[5 + i] = w[i] & ~top3_bits(i, 0);
    asm volatile("" : "+v"(m[i]), "+v"(m[5 + i]));
  }
}

__device__ __forceinline__ uint32_t code_offset8(const uint32_t* w, const uint32_t* m, int j) {
  const int bit = 5 * j;
  const int i = bit >> 5;
  const int o = bit & 31;
  const uint32_t* c = m + 5 * (j & 1);
  if (o < 3) return (w[i] << (3 - o)) & 0xF8u;                       // j = 0, 13, 26
  if (o <= 27) return (c[i] >> (o - 3)) & 0xFFu;                    // one v_bfe_u32
  return __builtin_amdgcn_alignbit(w[i + 1], c[i], o - 3) & 0xFFu;  // j = 6, 12, 19, 25
}

// Groups per row of a format (Tern3 pads rows to whole groups).
template <class Fmt>
__host__ __device__ constexpr int groups_of(int64_t k) {
  return static_cast<int>((k + Fmt::kGroupW - 1) / Fmt::kGroupW);
}

}  // namespace sherry
