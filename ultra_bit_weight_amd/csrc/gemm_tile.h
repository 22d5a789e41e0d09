// The tiled int8 product for many tokens (prefill), shared by the files that
// instantiate its tile configurations.  Products on packed ternary weights
// ("Sherry: Hardware-Efficient 1.25-Bit Ternary Quantization via Fine-grained
// Sparsification", Abstract: 3:4 sparse ternary blocks in five bits) and on the
// 2-bit comparator.
#pragma once

#include <type_traits>

#include "formats.h"
#include "gemm_epi.h"
#include "launch.h"

namespace sherry {
namespace {

// Tiled kernel for many tokens.  A workgroup of WR x WC waves computes a
// (64 WR weight rows) x (16 UT WC tokens) tile of Y, stepping k by one
// 128-weight group.  Wave w owns rows 64 (w % WR) .. + 64 and tokens
// 16 UT (w / WR) .. + 16 UT as 4 x UT MFMA tiles.
//   * Everything the loop reads from memory is copied by the memory system
//     straight into LDS (global_load_lds, no staging registers):
//       - the tokens' int8 tile of a step, one step ahead, into a ring of 2
//         buffers.  Within a token's 128 bytes the 16-byte chunk c sits at
//         position c ^ ((token >> 1) & 7), so the B-fragment reads of 16
//         consecutive tokens hit 16 different bank groups;
//       - the codes in stages of P groups, one stage ahead, into a ring of 2
//         buffers: per row the P groups' HC 16-byte head chunks (contiguous
//         in the row, a 64-byte run) and their tail words (a 4 P-byte run).
//         Chunk c of a row sits at position c ^ ((row >> 2) & (HC - 1)),
//         which spreads the word reads of consecutive rows over the banks.
//         A stage's copies are issued in the first P / 2 steps of the stage
//         before it.  Long runs per row matter: a copy instruction reads
//         64 lanes x 16 (or 4) bytes, and the rows of a tile are a row of
//         codes apart, so the instruction touches as many cache lines as
//         rows -- 16 here, against 32 for stages of 2 groups.
//   * Lane (i, q) decodes, for each of its 4 row tiles t (row 16 t + i), part q
//     of the group (blocks 8q .. 8q+7, two code words) straight into two A
//     fragments: half s takes blocks 8q + 4s .. 8q + 4s + 3, i.e. k bytes
//     32q + 16s .. + 16, which is the B fragment it reads from LDS.  The
//     next step's A fragments are expanded while the step's products run.
//   * One barrier per step, after each wave has waited for all of its copies
//     (vmcnt(0)).  A copy issued in step s has then landed by the barrier of
//     step s + 1: the x tile of step s + 1 is read in step s + 1, and a code
//     stage, whose copies end P / 2 steps before its first step, is first
//     read in the step before its first (to expand that step's fragments).
//     A copy only ever goes to the buffer of a step or stage whose last
//     read came before the barrier it follows.
//
// With M32 the products run as v_mfma_i32_32x32x32_i8 instead: lane (r, h) = (l % 32, l / 32) of a wave takes row or token r of a
// 32-wide tile and, in substep s of four, the 16 k bytes of x chunk
// Fmt::x_chunk32(h, s) of the group (the format's decoder expands the same
// weights); each wave holds (WROWS / 32) x (UT / 2) tiles of 32 x 32 sums, and the A and B
// fragments of substep s + 1 are read while the products of substep s run.
template <int WR_, int WC_, int UT_, int WROWS_ = 64, bool M32_ = false, int WGCU_ = (WR_ * WC_ > 4 ? 1 : 2)>
struct TileCfg {
  static constexpr int WR = WR_, WC = WC_, UT = UT_;
  static constexpr int kWaveRows = WROWS_;
  static constexpr bool kM32 = M32_;
  static_assert(M32_ ? (WROWS_ % 32 == 0 && UT_ % 2 == 0) : WROWS_ == 64, "wave tile");
  static constexpr int kWaves = WR * WC;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kRows = WROWS_ * WR;
  static constexpr int kTok = 16 * UT * WC;
  static constexpr int kXBytes = kTok * kGroupWeights;  // one step's x tile
  static constexpr int kXCopies = kXBytes / (16 * kWave);  // 1 KB copies of it per step
  static_assert(kXCopies * 16 * kWave == kXBytes, "x tile split");
  // workgroups one CU is sized to hold (sets the x ring depth)
  static constexpr int kWgPerCu = WGCU_;
};
using TileSmall = TileCfg<2, 2, 4>;   // 128 x 128, 4 waves
using TileLarge = TileCfg<4, 1, 8, 64, false, 2>;  // 256 x 128, 4 waves, two workgroups per CU
using TileSkinny = TileCfg<4, 1, 1>;  // 256 x 16, 4 waves (a few tokens: HBM-bound)
static_assert(TileSmall::kRows == kGemmSmallRows && TileSmall::kTok == kGemmSmallTok, "small tiling");
static_assert(TileLarge::kRows == kGemmLargeRows && TileLarge::kTok == kGemmLargeTok, "large tiling");
static_assert(TileSkinny::kRows == kGemmSkinnyRows && TileSkinny::kTok == kGemmSkinnyTok, "skinny tiling");

constexpr int kCodeSlots = 2;  // code stages in LDS: in use, next
constexpr int kTileDepth = 2;  // x steps in LDS: in use, next
constexpr int kTileUnroll = 8;
#ifndef SHERRY_TILE_BPREF
#define SHERRY_TILE_BPREF 0
#endif
#ifndef SHERRY_TILE_SPLIT
#define SHERRY_TILE_SPLIT 0
#endif  // steps per loop iteration: two stages of 4 (3:4 codes) or four of 2 (2-bit)

// Code bytes of one stage; the rings must fit the CU's share of the LDS.
template <class Fmt, class C>
constexpr int code_stage_bytes() {
  return C::kRows * (16 * Fmt::kTileHC + (Fmt::kTileTail ? 4 * Fmt::kTileP : 0));
}
template <class Fmt, class C>
constexpr bool tile_lds_fits() {
  return 128 + kTileDepth * C::kXBytes + kCodeSlots * code_stage_bytes<Fmt, C>() <=
         160 * 1024 / C::kWgPerCu;
}

template <class Fmt, class C>
__device__ __forceinline__ void gemm_tile(const GemmDesc& d, int tile_n, int tile_m) {
  constexpr int D = kTileDepth;
  static_assert(tile_lds_fits<Fmt, C>(), "LDS rings");
  constexpr int P = Fmt::kTileP;
  constexpr int HC = Fmt::kTileHC;
  static_assert(P % 2 == 0 && kTileUnroll % (kCodeSlots * P) == 0 && kTileUnroll % D == 0, "code stage cadence");
  constexpr int UT = C::UT;
  constexpr int W = C::kWaves;
  constexpr int R = C::kRows;
  // x copies per step: TX, wave w issues NX w .. (those that exist)
  constexpr int TX = C::kXCopies;
  constexpr int NX = (TX + W - 1) / W;
  // code copies per stage: head copies (64 chunk slots each) then tail copies
  // (64 words each); every wave issues CPW of them in each of the first P / 2
  // steps of the stage before
  constexpr int TH = R * HC / 64;
  constexpr int TT = Fmt::kTileTail ? R * P / 64 : 0;
  constexpr int CPW = (TH + TT) / ((P / 2) * W);
  static_assert(CPW * (P / 2) * W == TH + TT && CPW >= 1, "code copies per wave and step");
  constexpr int XV = C::kXBytes / 16;
  constexpr int HV = R * HC;
  constexpr int TV = Fmt::kTileTail ? R * P : 1;
  // the code table first in LDS (largest alignment): its address then fits
  // the 16-bit offset field of the lookups
  __shared__ __attribute__((aligned(1024))) uint32_t tab[32];
  // one LDS array per ring slot and kind: distinct objects let the compiler
  // see that reading one slot does not depend on the copies to the others
  __shared__ u32x4_t xt0[XV], xt1[XV];
  __shared__ u32x4_t hd0[HV], hd1[HV];
  __shared__ uint32_t tl0[TV], tl1[TV];
  auto xbuf = [&](int slot) -> u32x4_t* { return slot == 0 ? xt0 : xt1; };
  auto hbuf = [&](int slot) -> u32x4_t* { return slot == 0 ? hd0 : hd1; };
  auto tbuf = [&](int slot) -> uint32_t* { return slot == 0 ? tl0 : tl1; };
  // LDS byte addresses of the slots (copy destinations are these plus a
  // constant, so no generic pointer is live across the loop)
  const uint32_t xlds[2] = {lds_addr(xt0), lds_addr(xt1)};
  const uint32_t hlds[2] = {lds_addr(hd0), lds_addr(hd1)};
  const uint32_t tlds[2] = {lds_addr(tl0), lds_addr(tl1)};
  Fmt::init_table(tab, threadIdx.x);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int i = lane & 15;
  const int q = lane >> 4;
  const int wn = wave % C::WR;
  const int wm = wave / C::WR;
  const int n0 = tile_n * R;
  const int m0 = tile_m * C::kTok;
  const int G = d.k / kGroupWeights;
  const int lastn = d.n - 1;
  const int lastm = d.m - 1;
  // Copy sources are a uniform base plus a 32-bit per-lane byte offset (the
  // caller keeps each matrix's codes and x below 4 GiB).
  const uint32_t row_words = static_cast<uint32_t>(G) * Fmt::kWords;
  const SHERRY_GLOBAL char* cbase = uniform_ptr(gmem(reinterpret_cast<const char*>(d.codes)));
  const SHERRY_GLOBAL char* xbase = uniform_ptr(gmem(reinterpret_cast<const char*>(d.x)));

  EpiScales es;
  es.load(d, n0, m0, R, C::kTok, tid);
  static_assert((R + C::kTok) * 4 <= C::kXBytes, "output-stage scales fit an x slot");
  static_assert(R <= C::kThreads && C::kTok <= C::kThreads, "one row and one token scale per thread");

  // x copy c fills 16-byte slots 64 c + lane of the buffer; slot s holds
  // chunk (s % 8) ^ ((token >> 1) & 7) of token s / 8.
  uint32_t xoff[NX];
#pragma unroll
  for (int j = 0; j < NX; ++j) {
    const int slot = 64 * min(NX * wave + j, TX - 1) + lane;
    const int tok = slot >> 3;
    const int chunk = (slot & 7) ^ ((tok >> 1) & 7);
    xoff[j] = static_cast<uint32_t>(min(m0 + tok, lastm)) * static_cast<uint32_t>(d.ldx) + 16u * chunk;
  }
  // Per-lane copy offsets are recomputed in every step from values passed
  // through an empty asm statement: otherwise the compiler keeps the offsets
  // of all unrolled steps live at once.
  auto opaque = [](uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
  };
  auto copy_x = [&](int step, int slot) {
    const uint32_t g = static_cast<uint32_t>(min(step, G - 1));  // past the end: a valid group, never used
#pragma unroll
    for (int j = 0; j < NX; ++j) {
      const int c = NX * wave + j;
      if (c < TX) lds_copy16(xbase, opaque(xoff[j]) + g * kGroupWeights, xlds[slot] + 1024u * c);
    }
  };
  // Code copies: in each of the first P / 2 steps of a stage (part p), wave
  // w issues copies c = p CPW W + CPW w + j (j < CPW) of the next stage:
  // head copies (c < TH) take 64 16-byte chunk slots of the stage buffer,
  // tail copies 64 words.  The lane's source offsets for stage 0 are fixed
  // for the whole tile (rows past the matrix clamp to its last row); stage s
  // adds s times a stage's run per row.  A stage that reaches past the row's
  // last group reads the row's tail words or the next row instead (copied,
  // never used), and every offset is clamped to the last chunk or word of
  // the matrix, so no copy leaves it.
  constexpr int CC = (P / 2) * CPW;  // a wave's copies of one stage
  static_assert(TH % (CPW * W) == 0, "a part's copies are all head or all tail copies");
  const uint32_t row_bytes = 4u * row_words;
  uint32_t coff[CC];
#pragma unroll
  for (int p = 0; p < P / 2; ++p)
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const int c = p * (CPW * W) + CPW * wave + j;
      if (p * (CPW * W) < TH) {
        const int sl = 64 * c + lane;  // chunk slot of the stage buffer
        const int r = sl / HC;
        const int chunk = (sl % HC) ^ ((r >> 2) & (HC - 1));
        coff[p * CPW + j] = static_cast<uint32_t>(min(n0 + r, lastn)) * row_bytes + 16u * chunk;
      } else {
        const int sl = 64 * (c - TH) + lane;  // word slot of the stage's tails
        coff[p * CPW + j] =
            static_cast<uint32_t>(min(n0 + sl / P, lastn)) * row_bytes + Fmt::tile_tail_byte(G, sl % P);
      }
    }
  const uint32_t end_bytes = static_cast<uint32_t>(d.n) * row_bytes;
  // copy (p, j) of stage `stage` (groups P stage ..), into code slot `slot`
  auto copy_code = [&](int stage, int slot, int p, int j) {
    const int c = p * (CPW * W) + CPW * wave + j;
    if (p * (CPW * W) < TH) {
      const uint32_t o = coff[p * CPW + j] + static_cast<uint32_t>(stage) * (P * Fmt::kTileHeadBytes);
      lds_copy16(cbase, min(o, end_bytes - 16u), hlds[slot] + 1024u * c);
    } else {
      const uint32_t o = coff[p * CPW + j] + static_cast<uint32_t>(stage) * (4 * P);
      lds_copy4(cbase, min(o, end_bytes - 4u), tlds[slot] + 256u * (c - TH));
    }
  };
  // in step s (unrolled position b): in the first P / 2 steps of a stage,
  // this wave's share (part s % P) of the copies of stage s / P + 1
  auto copy_code_part = [&](int s, int b) {
    if (b % P < P / 2) {
#pragma unroll
      for (int j = 0; j < CPW; ++j) copy_code(s / P + 1, (b / P + 1) % kCodeSlots, b % P, j);
    }
  };

  constexpr bool M32 = C::kM32;
  constexpr int WROWS = C::kWaveRows;
  constexpr int RT32 = WROWS / 32;  // 32-row tiles per wave
  constexpr int U32 = M32 ? UT / 2 : 1;
  v4i acc[M32 ? 1 : 4][M32 ? 1 : UT];
  v16i acc32[M32 ? RT32 : 1][U32];
  if constexpr (M32) {
#pragma unroll
    for (int t = 0; t < RT32; ++t)
#pragma unroll
      for (int u = 0; u < U32; ++u) acc32[t][u] = v16i{};
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int u = 0; u < UT; ++u) acc[t][u] = v4i{0, 0, 0, 0};
  }

  // The lane's code byte offsets pass through opaque() in every step, so the
  // addresses are rebuilt from them there (the slot and row-tile parts are
  // constants the LDS reads take as offsets); otherwise the compiler keeps an
  // address register for every slot, row tile and group of the unrolled loop.
  // 16 x 16 products: lane (i, q) has rows 16 t + i of the wave's rows;
  // 32 x 32: lane (r32, h) has rows 32 t + r32.  Either way the stage
  // swizzle of the lane's rows is (row >> 2) & (HC - 1) of its row index.
  const int lr = M32 ? (lane & 31) : i;
  const int h32 = lane >> 5;
  const uint32_t lane_h = static_cast<uint32_t>(16 * HC * (WROWS * wn + lr));
  const uint32_t lane_t = static_cast<uint32_t>(4 * P * (WROWS * wn + lr));
  const int swz = (lr >> 2) & (HC - 1);
  // A fragments of the next step: a step's codes are in LDS one step early
  // (their copies are older than the step's x copies, which the barrier
  // before it waits for), so each step expands the next step's codes while
  // its own products run.  an[s][t]: substep (half) s, row tile t.
  constexpr int AS = M32 ? 4 : 2;
  constexpr int AT = M32 ? RT32 : 4;
  v4i an[AS][AT];
  auto decode = [&](int cs, int j) {
    const char* hb = reinterpret_cast<const char*>(hbuf(cs));
    const char* tb = reinterpret_cast<const char*>(tbuf(cs));
    const uint32_t lh = opaque(lane_h);
    const uint32_t lt = opaque(lane_t);
    if constexpr (M32) {
      uint32_t win[RT32][Fmt::kWin];
#pragma unroll
      for (int t = 0; t < RT32; ++t)
        Fmt::window32(win[t], hb + 16 * HC * 32 * t, tb + 4 * P * 32 * t, lh, lt, swz, j, h32);
#pragma unroll
      for (int s = 0; s < AS; ++s)
#pragma unroll
        for (int t = 0; t < RT32; ++t) an[s][t] = Fmt::frag32(win[t], s, tab);
    } else {
      uint32_t w[4][2];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        Fmt::stage_words(w[t], hb + 16 * HC * 16 * t, tb + 4 * P * 16 * t, lh, lt, swz, j, q);
#pragma unroll
      for (int s = 0; s < AS; ++s)
#pragma unroll
        for (int t = 0; t < 4; ++t) an[s][t] = Fmt::frag(w[t], q, s, tab);
    }
  };
  // the products of a step: A from an[][], B from x slot xs.  16 x 16:
  // each B fragment is read one fragment ahead of the four products that
  // use it (scheduling barriers keep that order: left alone, the compiler
  // reused one register pair and waited on every read).
  auto products = [&](int xs) {
    const u32x4_t* xb = xbuf(xs);
    auto bfrag = [&](int tok, int chunk) {
      const u32x4_t v = xb[8 * tok + (chunk ^ ((tok >> 1) & 7))];
      return v4i{static_cast<int>(v.x), static_cast<int>(v.y), static_cast<int>(v.z), static_cast<int>(v.w)};
    };
    if constexpr (M32) {
#pragma unroll
      for (int s = 0; s < AS; ++s)
#pragma unroll
        for (int u = 0; u < U32; ++u) {
          const v4i b = bfrag(16 * UT * wm + 32 * u + lr, Fmt::x_chunk32(h32, s));
#pragma unroll
          for (int t = 0; t < RT32; ++t)
            acc32[t][u] = __builtin_amdgcn_mfma_i32_32x32x32_i8(an[s][t], b, acc32[t][u], 0, 0, 0);
        }
    } else {
      constexpr int NK = AS * UT;  // fragment k: half k / UT, token tile k % UT
      auto bk = [&](int k) { return bfrag(16 * UT * wm + 16 * (k % UT) + i, 2 * q + k / UT); };
      v4i bb[2];
      bb[0] = bk(0);
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        if (k + 1 < NK) bb[(k + 1) & 1] = bk(k + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[t][k % UT] =
              __builtin_amdgcn_mfma_i32_16x16x64_i8(an[k / UT][t], bb[k & 1], acc[t][k % UT], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Wait until all of this wave's copies landed, then the barrier.  The empty
  // asm statements keep the compiler from moving memory accesses across.
  auto step_barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // prologue: code stage 0 and the x tile of step 0, landed and published
  // before the first decode (the barrier also covers the code table)
#pragma unroll
  for (int p = 0; p < P / 2; ++p)
#pragma unroll
    for (int j = 0; j < CPW; ++j) copy_code(0, 0, p, j);
  copy_x(0, 0);
  step_barrier();
  decode(0, 0);
  for (int g = 0; g < G; g += kTileUnroll) {
#pragma unroll
    for (int b = 0; b < kTileUnroll; ++b) {
      // step g + b: x in slot b % 2, codes of stage (g + b) / P in code slot
      // (b / P) % 2; after the barrier the finished step's x slot is refilled
      // with step g + b + 1, and part of stage (g + b) / P + 1 is copied
      step_barrier();
      copy_x(g + b + 1, (b + 1) % D);
      copy_code_part(g + b, b);
      if (g + b < G) {
        products(b % D);
        decode(((b + 1) / P) % kCodeSlots, (b + 1) % P);  // step g + b + 1 (kTileUnroll is a multiple of 2 P)
      }
    }
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // no copy may outlive the workgroup
  // the scales go to x slot 0 once every wave is past its last step
  float* sl = reinterpret_cast<float*>(xt0);
  __syncthreads();
  es.stage(d, sl, R, C::kTok, tid);
  __syncthreads();
  if constexpr (M32)
    tile_store32<RT32, U32>(d, acc32, n0 + WROWS * wn, m0 + 16 * UT * wm, lane, sl + WROWS * wn,
                            sl + R + 16 * UT * wm);
  else
    tile_store<UT>(d, acc, n0 + 64 * wn, m0 + 16 * UT * wm, i, q, sl + 64 * wn, sl + R + 16 * UT * wm);
}

template <class Fmt, class C>
__global__ __launch_bounds__(C::kThreads) void gemm_tile_kernel(GemmDesc d) {
  gemm_tile<Fmt, C>(d, blockIdx.x, blockIdx.y);
}

// Grouped: one workgroup per plan tile {problem, row tile, token tile}.
template <class Fmt, class C>
__global__ __launch_bounds__(C::kThreads) void gemm_tile_grouped_kernel(const char* plan) {
  const PlanHeader* h = reinterpret_cast<const PlanHeader*>(plan);
  const GemmDesc* descs = reinterpret_cast<const GemmDesc*>(plan + sizeof(PlanHeader));
  const GemmTile tl = reinterpret_cast<const GemmTile*>(descs + h->count)[blockIdx.x];
  const GemmDesc d = descs[tl.prob];
  gemm_tile<Fmt, C>(d, tl.tile_n, tl.tile_m);
}

}  // namespace
}  // namespace sherry
