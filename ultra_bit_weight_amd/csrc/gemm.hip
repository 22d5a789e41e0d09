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
#include <type_traits>

#include "formats.h"
#include "gemm_epi.h"
#include "launch.h"

namespace sherry {
namespace {

constexpr int kMaxKRanges = 16;  // waves per workgroup (k <= 8192 stays x-stationary)
// Steps of x and code words the tiled kernel keeps in flight (LDS ring depth;
// 3 measured faster than 4 on the 1B layer at M = 2048).
#ifndef SHERRY_TILE_DEPTH
#define SHERRY_TILE_DEPTH 3
#endif
constexpr int kTileDepth = SHERRY_TILE_DEPTH;
static_assert(kTileDepth >= 2 && kTileDepth <= 4, "tile pipeline depth");

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

// Tiled kernel for many tokens.  A workgroup of WR x WC waves computes a
// (64 WR weight rows) x (16 UT WC tokens) tile of Y, stepping k by one
// 128-weight group.  Wave w owns rows 64 (w % WR) .. + 64 and tokens
// 16 UT (w / WR) .. + 16 UT as 4 x UT MFMA tiles.
//   * Everything the loop reads from memory is copied by the memory system
//     straight into LDS (global_load_lds, no staging registers):
//       - the tokens' int8 tile of a step, D steps ahead, into a ring of D
//         buffers.  Within a token's 128 bytes the 16-byte chunk c sits at
//         position c ^ ((token >> 1) & 7), so the B-fragment reads of 16
//         consecutive tokens hit 16 different bank groups;
//       - the codes in stages of P groups, two stages ahead, into a ring of 3
//         buffers: per row the P groups' head words (contiguous in the row,
//         so four lanes read 64 contiguous bytes) and tail words.  Chunk c of
//         a row sits at position c ^ ((row >> 2) & 3): the word reads of 16
//         consecutive rows then hit 64 different banks.  A stage's copies
//         are spread evenly over the P steps of the stage two earlier.
//   * Lane (i, q) decodes, for each of its 4 row tiles t (row 16 t + i), part q
//     of the group (blocks 8q .. 8q+7, two code words) straight into two A
//     fragments: half s takes blocks 8q + 4s .. 8q + 4s + 3, i.e. k bytes
//     32q + 16s .. + 16, which is the B fragment it reads from LDS.
//   * One barrier per step.  Every vector-memory operation in the loop is one
//     of these copies, a fixed number per wave and step, so before the
//     barrier each wave waits (vmcnt) for its copies of the step's x tile;
//     the copies of the step's code stage are older, so they have landed
//     too.  After the barrier the whole step is in LDS, and the buffers of
//     the finished step (and, at a stage start, stage) are free for the
//     copies issued next.
template <int WR_, int WC_, int UT_>
struct TileCfg {
  static constexpr int WR = WR_, WC = WC_, UT = UT_;
  static constexpr int kWaves = WR * WC;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kRows = 64 * WR;
  static constexpr int kTok = 16 * UT * WC;
  static constexpr int kXBytes = kTok * kGroupWeights;  // one step's x tile
  static constexpr int kXCopies = kXBytes / (16 * kWave);  // 1 KB copies of it per step
  static_assert(kXCopies * 16 * kWave == kXBytes, "x tile split");
  // workgroups one CU is sized to hold (sets the x ring depth)
  static constexpr int kWgPerCu = kWaves > 4 ? 1 : 2;
};
using TileSmall = TileCfg<2, 2, 4>;   // 128 x 128, 4 waves
using TileLarge = TileCfg<4, 2, 6>;   // 256 x 192, 8 waves
using TileSkinny = TileCfg<4, 1, 1>;  // 256 x 16, 4 waves (a few tokens: HBM-bound)
static_assert(TileSmall::kRows == kGemmSmallRows && TileSmall::kTok == kGemmSmallTok, "small tiling");
static_assert(TileLarge::kRows == kGemmLargeRows && TileLarge::kTok == kGemmLargeTok, "large tiling");
static_assert(TileSkinny::kRows == kGemmSkinnyRows && TileSkinny::kTok == kGemmSkinnyTok, "skinny tiling");

constexpr int kCodeSlots = 3;  // code stages in LDS: in use, next, in flight
constexpr int kTileUnroll = 12;  // steps per loop iteration: a multiple of D and of 3 P

// Code bytes of one stage and x-ring depth: kTileDepth, or fewer steps if the
// CU's share of the 160 KB of LDS cannot hold them next to the code ring.
template <class Fmt, class C>
constexpr int code_stage_bytes() {
  return C::kRows * (16 * Fmt::kTileHC + (Fmt::kTileTail ? 4 * Fmt::kTileP : 0));
}
// The depth is also at most P + 1: a stage's last copies are then issued
// before the x copies of its first step, so waiting for those covers them.
template <class Fmt, class C>
constexpr int tile_depth() {
  constexpr int fit = (160 * 1024 / C::kWgPerCu - 1024 - kCodeSlots * code_stage_bytes<Fmt, C>()) / C::kXBytes;
  constexpr int cap = kTileDepth < Fmt::kTileP + 1 ? kTileDepth : Fmt::kTileP + 1;
  return fit < cap ? fit : cap;
}

template <class Fmt, class C>
__device__ __forceinline__ void gemm_tile(const GemmDesc& d, int tile_n, int tile_m) {
  constexpr int D = tile_depth<Fmt, C>();
  static_assert(D >= 2 && kTileUnroll % D == 0, "x ring depth");
  constexpr int P = Fmt::kTileP;
  constexpr int HC = Fmt::kTileHC;
  static_assert(kTileUnroll % (kCodeSlots * P) == 0 && D <= P + 1, "code stage cadence");
  constexpr int UT = C::UT;
  constexpr int W = C::kWaves;
  constexpr int R = C::kRows;
  // x copies per step: TX, wave w issues NX w .. (those that exist)
  constexpr int TX = C::kXCopies;
  constexpr int NX = (TX + W - 1) / W;
  // code copies per stage: head copies (64 chunk slots each) then tail copies
  // (64 words each); every wave issues CPW of them in every step
  constexpr int TH = R * HC / 64;
  constexpr int TT = Fmt::kTileTail ? R * P / 64 : 0;
  constexpr int CPW = (TH + TT) / (P * W);
  static_assert(CPW * P * W == TH + TT && CPW >= 1, "code copies per wave and step");
  constexpr int kOpsPerStep = TX / W + CPW;  // vector-memory operations per wave and step, at least
  constexpr int XV = C::kXBytes / 16;
  constexpr int HV = R * HC;
  constexpr int TV = Fmt::kTileTail ? R * P : 1;
  // the code table first in LDS (largest alignment): its address then fits
  // the 16-bit offset field of the lookups
  __shared__ __attribute__((aligned(1024))) uint32_t tab[32];
  // one LDS array per ring slot and kind: distinct objects let the compiler
  // see that reading one slot does not depend on the copies to the others
  __shared__ u32x4_t xt0[XV], xt1[XV], xt2[D > 2 ? XV : 1], xt3[D > 3 ? XV : 1];
  __shared__ u32x4_t hd0[HV], hd1[HV], hd2[HV];
  __shared__ uint32_t tl0[TV], tl1[TV], tl2[TV];
  auto xbuf = [&](int slot) -> u32x4_t* {
    return slot == 0 ? xt0 : slot == 1 ? xt1 : slot == 2 ? xt2 : xt3;
  };
  auto hbuf = [&](int slot) -> u32x4_t* { return slot == 0 ? hd0 : slot == 1 ? hd1 : hd2; };
  auto tbuf = [&](int slot) -> uint32_t* { return slot == 0 ? tl0 : slot == 1 ? tl1 : tl2; };
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
  const SHERRY_GLOBAL char* cbase = gmem(reinterpret_cast<const char*>(d.codes));
  const SHERRY_GLOBAL char* xbase = gmem(reinterpret_cast<const char*>(d.x));

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
      if (c < TX) lds_copy16(xbase, opaque(xoff[j]) + g * kGroupWeights, lds_addr(xbuf(slot) + 64 * c));
    }
  };
  // code copy c of stage `stage` (groups P stage ..), into code slot `slot`
  auto copy_code = [&](int stage, int slot, int c) {
    const int g0 = P * stage;
    const int ln = static_cast<int>(opaque(static_cast<uint32_t>(lane)));
    if (c < TH) {
      const int sl = 64 * c + ln;  // chunk slot of the stage buffer
      const int r = sl / HC;
      const int chunk = (sl % HC) ^ ((r >> 2) & 3);
      const uint32_t w = static_cast<uint32_t>(min(n0 + r, lastn)) * row_words + Fmt::head_word(G, g0, chunk);
      lds_copy16(cbase, 4u * w, lds_addr(hbuf(slot) + 64 * c));
    } else {
      const int sl = 64 * (c - TH) + ln;  // word slot of the stage's tails
      const uint32_t w = static_cast<uint32_t>(min(n0 + sl / P, lastn)) * row_words + Fmt::tail_word(G, g0, sl % P);
      lds_copy4(cbase, 4u * w, lds_addr(tbuf(slot) + 64 * (c - TH)));
    }
  };
  // in step s: this wave's share (part s % P) of the copies of stage s / P + 2
  auto copy_code_part = [&](int s, int b) {
#pragma unroll
    for (int j = 0; j < CPW; ++j)
      copy_code(s / P + 2, (b / P + 2) % kCodeSlots, (b % P) * (CPW * W) + CPW * wave + j);
  };

  v4i acc[4][UT];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int u = 0; u < UT; ++u) acc[t][u] = v4i{0, 0, 0, 0};

  // step with x in x slot xs, codes in code slot cs, group j of its stage
  // The lane's code byte offsets pass through opaque() in every step, so the
  // addresses are rebuilt from them there (the slot and row-tile parts are
  // constants the LDS reads take as offsets); otherwise the compiler keeps an
  // address register for every slot, row tile and group of the unrolled loop.
  const uint32_t lane_h = static_cast<uint32_t>(16 * HC * (64 * wn + i));
  const uint32_t lane_t = static_cast<uint32_t>(4 * P * (64 * wn + i));
  const int swz = (i >> 2) & 3;  // = (row >> 2) & 3 for the lane's rows
  auto compute = [&](int xs, int cs, int j) {
    const u32x4_t* xb = xbuf(xs);
    const char* hb = reinterpret_cast<const char*>(hbuf(cs));
    const char* tb = reinterpret_cast<const char*>(tbuf(cs));
    const uint32_t lh = opaque(lane_h);
    const uint32_t lt = opaque(lane_t);
    uint32_t w[4][2];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      Fmt::stage_words(w[t], hb + 16 * HC * 16 * t, tb + 4 * P * 16 * t, lh, lt, swz, j, q);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      v4i a[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) a[t] = Fmt::frag(w[t], q, s, tab);
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
  // Wait until this wave's x copies of step k landed (the copies of the D - 2
  // younger steps may still be in flight), then the barrier.  The empty asm
  // statements keep the compiler from moving memory accesses across.
  auto step_barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(kOpsPerStep * (D - 2)));
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // prologue: code stages 0 and 1, x steps 0 .. D - 2.  As in the loop, CPW
  // code copies follow the x copies of each step, so that the wait count of
  // the barriers holds from step 0 on: after a step's x copies every wave has
  // issued at least kOpsPerStep * (D - 2) + CPW more operations by the
  // barrier that needs them.  A wave's copies of one stage are copies
  // wave + W t, t < P CPW.
  constexpr int PC = P * CPW;
  constexpr int late = (D - 1) * CPW;  // stage-1 copies after the x copies
  static_assert(late <= PC, "prologue code copies");
#pragma unroll
  for (int t = 0; t < PC; ++t) copy_code(0, 0, wave + W * t);
#pragma unroll
  for (int t = 0; t < PC - late; ++t) copy_code(1, 1, wave + W * t);
#pragma unroll
  for (int b = 0; b + 1 < D; ++b) {
    copy_x(b, b);
#pragma unroll
    for (int j = 0; j < CPW; ++j) copy_code(1, 1, wave + W * (PC - late + CPW * b + j));
  }
  __syncthreads();  // code table, and all of the above
  for (int g = 0; g < G; g += kTileUnroll) {
#pragma unroll
    for (int b = 0; b < kTileUnroll; ++b) {
      // step g + b: x in slot b % D, codes of stage (g + b) / P in code slot
      // (b / P) % 3; after the barrier the finished step's x slot is refilled
      // with step g + b + D - 1, and part of stage (g + b) / P + 2 is copied
      step_barrier();
      copy_x(g + b + D - 1, (b + D - 1) % D);
      copy_code_part(g + b, b);
      if (g + b < G) compute(b % D, (b / P) % kCodeSlots, b % P);
    }
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // no copy may outlive the workgroup

  tile_store<UT>(d, acc, n0 + 64 * wn, m0 + 16 * UT * wm, i, q);
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

// ------------------------------------------------------- few tokens ---
// m <= 16 (decode with a handful of sequences): HBM-bound, so the codes
// stream once through registers, GEMV-like, and only the products use the
// matrix cores.  v_mfma_i32_16x16x64_i8 contracts over the four quarter-
// waves and 16 bytes per lane, so lane (q, i) = (lane / 16, lane % 16) takes
// weight row i and group 4 c + q of a k slice c of 512 weights: one slice of
// 16 rows is eight instructions with the decoded group as A and the 16
// tokens' x for the same group as B (token i in lane (q, i)).
//
// A workgroup of kFewWaves waves owns a tile of rows with all of k.  The S
// slices of k (a power of two) are split over KW = min(S, 8) waves (SPW
// slices each), so each wave keeps its x in registers; the 8 / KW row groups
// of KW waves walk NBLK blocks of 16 rows each, with a ring of code
// registers kept D blocks ahead.  Each wave adds its 16 x 16 partial sums of
// a block into the tile's int32 sums in LDS (exact, so the order of the
// additions does not matter); one barrier at the end, then the epilogue
// writes the tile.
//
// Sums of block row (4 q + e) and token t sit at LDS word 256 blk +
// 16 (4 e + q) + t: the four quarter-waves' adds then hit distinct banks.
#ifndef SHERRY_FEW_RING
#define SHERRY_FEW_RING 4
#endif
constexpr int kFewRing = SHERRY_FEW_RING;  // blocks of codes in flight per wave (5-word groups)

template <class Fmt, int S>
struct FewShape {
  static constexpr int KW = S < kFewWaves ? S : kFewWaves;  // waves per row group
  static constexpr int SPW = S / KW;                         // slices per wave
  static constexpr int RG = kFewWaves / KW;                  // row groups
  static constexpr int RT = few_tile_rows(4 * S);
  static constexpr int NBLK = RT / (16 * RG);                // blocks per row group
  // ring depth (blocks): kFewRing words-of-a-5-word-group budget
  static constexpr int DW = kFewRing * 5 / (SPW * Fmt::kWords);
  static constexpr int D = DW < 2 ? 2 : (DW > NBLK ? NBLK : DW);
  static_assert(NBLK * 16 * RG == RT, "few-token tile shape");
};

// LDS word of the sum for row 16 b + 4 q + e of a tile and token i.  Blocks
// are 257 words apart, so the bank is (b + 16 q + i) mod 64: the MFMA lanes
// (q, i) of one block and e, and the epilogue's 64 consecutive quads (b, q)
// of one token, each fall in 64 different banks.
constexpr int kFewSumStride = 257;
constexpr int kFewSumWords = kFewMaxTileRows / 16 * kFewSumStride;
static_assert(kFewSumWords % 4 == 0, "sums are cleared as int4");
__device__ __forceinline__ int few_sum_word(int b, int q, int e, int i) {
  return kFewSumStride * b + 64 * e + 16 * q + i;
}

// `setup` builds the tile's LDS state (tables, zeroed sums, staged scales)
// and meets the barriers; it runs after this wave's x loads and first code
// loads are issued, which stay in flight across the barriers (they wait for
// LDS operations only).
// x staged in LDS (tiles with several row groups, k <= 2048): token rows of
// k / 16 + 1 chunks of 16 bytes (one pad chunk, so that the four quarters'
// reads of one group fall in different banks).
constexpr int kFewXChunks = kFewMaxTok * (4 * kGroupWeights * 4 / 16 + 1);
#ifndef SHERRY_FEW_STAGE_MIN_TOK
#define SHERRY_FEW_STAGE_MIN_TOK 8
#endif
constexpr int kFewStageMinTok = SHERRY_FEW_STAGE_MIN_TOK;

template <class Fmt, int S, class Setup>
__device__ __forceinline__ void gemm_few(const GemmDesc& d, int tile, const uint32_t* tab32, const uint2* pairs,
                                         int32_t* sums, u32x4_t* xst, const Setup& setup) {
  using Sh = FewShape<Fmt, S>;
  constexpr int NW = Fmt::kWords;
  constexpr int KW = Sh::KW, SPW = Sh::SPW, NBLK = Sh::NBLK, D = Sh::D;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int kw = wave % KW;
  const int rg = wave / KW;
  const int i = lane & 15;
  const int q = lane >> 4;
  const int G = d.k / kGroupWeights;
  const int row0 = tile * Sh::RT + rg * (NBLK * 16);
  const int64_t row_words = static_cast<int64_t>(G) * NW;

  // x of token i for this lane's groups (zero past m and past k).  With
  // several row groups every one of them needs all of x: the workgroup then
  // copies x once into LDS with contiguous loads (issued first, written
  // before the set-up's barrier) and the lanes read their slices there.
  constexpr bool kCanStage = Sh::RG > 1;
  static_assert(!kCanStage || (S <= 4 && SPW == 1), "staged x: k <= 2048, one slice per wave");
  // only worth its extra LDS round trip with several tokens
  const bool stage = kCanStage && d.m >= kFewStageMinTok;
  constexpr int kThreads = kFewWaves * kWave;
  constexpr int kStageLoads = kFewXChunks / kThreads + 1;  // 16-byte loads per thread, upper bound
  const int cpt = d.k / 16;  // chunks per token
  uint32_t xr[SPW][32];
  u32x4_t xsv[kCanStage ? kStageLoads : 1];
  auto set_xr = [&](int sp, int u, const u32x4_t& v, bool ok) {
    xr[sp][4 * u + 0] = ok ? v.x : 0u;
    xr[sp][4 * u + 1] = ok ? v.y : 0u;
    xr[sp][4 * u + 2] = ok ? v.z : 0u;
    xr[sp][4 * u + 3] = ok ? v.w : 0u;
  };
  if (stage) {
#pragma unroll
    for (int j = 0; j < (kCanStage ? kStageLoads : 0); ++j) {
      const int c = static_cast<int>(threadIdx.x) + kThreads * j;
      const int tok = c / cpt;
      if (tok < d.m)
        xsv[j] = *gmem(reinterpret_cast<const u32x4_t*>(d.x + static_cast<int64_t>(tok) * d.ldx + 16 * (c % cpt)));
    }
  } else {
#pragma unroll
    for (int sp = 0; sp < SPW; ++sp) {
      const int g = 4 * (kw + KW * sp) + q;
      const bool ok = i < d.m && g < G;
      const SHERRY_GLOBAL u32x4_t* xp = gmem(reinterpret_cast<const u32x4_t*>(
          d.x + static_cast<int64_t>(ok ? i : 0) * d.ldx + static_cast<int64_t>(ok ? g : 0) * kGroupWeights));
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const u32x4_t v = xp[u];
        set_xr(sp, u, v, ok);
      }
    }
  }
  // rows past n and groups past k load valid words (clamped) whose products
  // are never stored or meet zero x
  auto fetch = [&](uint32_t (&buf)[SPW][NW], int blk) {
    const int row = min(row0 + 16 * blk + i, d.n - 1);
#pragma unroll
    for (int sp = 0; sp < SPW; ++sp)
      Fmt::load_cached(buf[sp], d.codes + row * row_words, G, min(4 * (kw + KW * sp) + q, G - 1));
  };
  // With table decoding, the lookups of half a group are issued before its
  // four products, so the products wait on one LDS round trip per half, not
  // one each (decoding in registers needs no batching).
  constexpr int HB = Fmt::kTableDecode ? 2 : 8;  // batches per group
  auto step = [&](const uint32_t (&buf)[SPW][NW], int blk) {
    v4i c = {0, 0, 0, 0};
#pragma unroll
    for (int sp = 0; sp < SPW; ++sp) {
#pragma unroll
      for (int hf = 0; hf < HB; ++hf) {
        uint32_t a[32 / HB];
#pragma unroll
        for (int pp = 0; pp < 16 / HB; ++pp) {
          const int p = (16 / HB) * hf + pp;
          const uint2 v = ((kPairMask >> p) & 1)
                              ? Fmt::i8x8(buf[sp], p, pairs)
                              : make_uint2(Fmt::i8x4(buf[sp], 2 * p, tab32), Fmt::i8x4(buf[sp], 2 * p + 1, tab32));
          a[2 * pp] = v.x;
          a[2 * pp + 1] = v.y;
        }
#pragma unroll
        for (int uu = 0; uu < 8 / HB; ++uu) {
          const int u = (8 / HB) * hf + uu;
          const v4i av = {static_cast<int>(a[4 * uu]), static_cast<int>(a[4 * uu + 1]),
                          static_cast<int>(a[4 * uu + 2]), static_cast<int>(a[4 * uu + 3])};
          const v4i bv = {static_cast<int>(xr[sp][4 * u]), static_cast<int>(xr[sp][4 * u + 1]),
                          static_cast<int>(xr[sp][4 * u + 2]), static_cast<int>(xr[sp][4 * u + 3])};
          c = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, c, 0, 0, 0);
        }
      }
    }
    const int b = rg * NBLK + blk;
    int32_t* dst = sums + few_sum_word(b, q, 0, i);
#pragma unroll
    for (int e = 0; e < 4; ++e) atomicAdd(dst + 64 * e, c[e]);
  };
  uint32_t ring[D][SPW][NW];
#pragma unroll
  for (int b = 0; b + 1 < D; ++b) fetch(ring[b], b);
  if (stage) {
#pragma unroll
    for (int j = 0; j < (kCanStage ? kStageLoads : 0); ++j) {
      const int c = static_cast<int>(threadIdx.x) + kThreads * j;
      const int tok = c / cpt;
      if (tok < d.m) xst[tok * (cpt + 1) + c % cpt] = xsv[j];
    }
  }
  setup();
  if (stage) {
    const int g = 4 * kw + q;
    const bool ok = i < d.m && g < G;
    const u32x4_t* xp = xst + (ok ? i * (cpt + 1) + 8 * g : 0);
#pragma unroll
    for (int u = 0; u < 8; ++u) set_xr(0, u, xp[u], ok);
  }
  for (int b0 = 0; b0 < NBLK; b0 += D) {
#pragma unroll
    for (int b = 0; b < D; ++b) {
      fetch(ring[(b + D - 1) % D], min(b0 + b + D - 1, NBLK - 1));
      if (NBLK % D == 0 || b0 + b < NBLK) step(ring[b], b0 + b);
    }
  }
}

// Zero the tile's sums, build the tables, run the row groups, write the tile.
// Thread t writes the four rows 4Q .. 4Q + 3 of quad Q = t % (rt / 4) for
// tokens t / (rt / 4), + 2048 / rt, ...: consecutive threads hold consecutive
// quads of one token, so a wave stores 64 x 4 consecutive outputs at once
// (8 bytes per lane in fp16), and its LDS reads of the sums hit 64 banks
// (few_sum_word).  The tile's weight scales and the token scales are staged
// in LDS before the main loop, so the epilogue waits on no global load.
template <class Fmt>
__device__ __forceinline__ void gemm_few_tile(const GemmDesc& d, int tile) {
  constexpr int kThreads = kFewWaves * kWave;
  static_assert(kThreads % (kFewMaxTileRows / 4) == 0 && kFewMaxTileRows % 64 == 0, "epilogue mapping");
  __shared__ uint32_t tab32[32];
  __shared__ uint2 pairs[kPairMask != 0 ? Fmt::kPairEntries : 1];
  __shared__ __attribute__((aligned(16))) int32_t sums[kFewSumWords];
  __shared__ float sxs[kFewMaxTok];
  __shared__ float sws[kFewMaxTileRows];
  __shared__ u32x4_t xst[kFewXChunks];
  const int G = d.k / kGroupWeights;
  const int rt = few_tile_rows(G);
  const int tid = static_cast<int>(threadIdx.x);
  const bool s_f16 = d.flags & kFlagScaleF16;
  const bool has_sx = d.x_scales != nullptr;
  auto setup = [&]() {
    for (int t = tid; t < rt; t += kThreads)
      sws[t] = d.y ? load_scale(d.w_scales, min(tile * rt + t, d.n - 1), s_f16) : 0.0f;
    if (tid < kFewMaxTok) sxs[tid] = has_sx && tid < d.m ? gmem(d.x_scales)[tid] : 1.0f;
    for (int t = tid; t < kFewSumWords / 4; t += kThreads) reinterpret_cast<v4i*>(sums)[t] = v4i{0, 0, 0, 0};
    Fmt::init_table(tab32, threadIdx.x);
    __syncthreads();
    if constexpr (kPairMask != 0) {
      Fmt::init_pair_table(pairs, tab32, threadIdx.x, kThreads);
      __syncthreads();
    }
  };
  switch (few_slices(G)) {
    case 1: gemm_few<Fmt, 1>(d, tile, tab32, pairs, sums, xst, setup); break;
    case 2: gemm_few<Fmt, 2>(d, tile, tab32, pairs, sums, xst, setup); break;
    case 4: gemm_few<Fmt, 4>(d, tile, tab32, pairs, sums, xst, setup); break;
    case 8: gemm_few<Fmt, 8>(d, tile, tab32, pairs, sums, xst, setup); break;
    default: gemm_few<Fmt, 16>(d, tile, tab32, pairs, sums, xst, setup); break;
  }
  __syncthreads();
  const int nq = rt / 4;                // quads of the tile (32, 64 or 128)
  const int quad = tid % nq;
  const int m0 = tid / nq;              // first token; then + kThreads / nq
  const int mstep = kThreads / nq;
  const int n4 = tile * rt + 4 * quad;  // the quad's first row
  if (n4 >= d.n) return;
  const bool y_f16 = d.flags & kFlagYF16;
  const bool full = n4 + 3 < d.n;
  const int b = quad >> 2;
  const int q = quad & 3;
  // whole quads go out as one 8- (fp16) or 16-byte (fp32, int32) store
  const bool vec_acc = d.acc && full && d.n % 4 == 0 && (reinterpret_cast<uintptr_t>(d.acc) & 15) == 0;
  const bool vec_y = d.y && full && d.ldy % 4 == 0 &&
                     (reinterpret_cast<uintptr_t>(d.y) & (y_f16 ? 7 : 15)) == 0;
  float sw[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) sw[e] = sws[4 * quad + e];
  for (int m = m0; m < d.m; m += mstep) {
    const int32_t* col = sums + few_sum_word(b, q, 0, m);
    v4i v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = col[64 * e];
    if (d.acc) {
      const int64_t o = static_cast<int64_t>(m) * d.n + n4;
      if (vec_acc) {
        *gmem(reinterpret_cast<v4i*>(d.acc + o)) = v;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n4 + e < d.n) gmem(d.acc)[o + e] = v[e];
      }
    }
    if (d.y) {
      const int64_t o = static_cast<int64_t>(m) * d.ldy + n4;
      float f[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) f[e] = epilogue_i32(v[e], sw[e], sxs[m], has_sx);
      if (vec_y && y_f16) {
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        const h4 hv = {static_cast<_Float16>(f[0]), static_cast<_Float16>(f[1]), static_cast<_Float16>(f[2]),
                       static_cast<_Float16>(f[3])};
        *gmem(reinterpret_cast<h4*>(static_cast<_Float16*>(d.y) + o)) = hv;
      } else if (vec_y) {
        typedef float f4 __attribute__((ext_vector_type(4)));
        *gmem(reinterpret_cast<f4*>(static_cast<float*>(d.y) + o)) = f4{f[0], f[1], f[2], f[3]};
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n4 + e < d.n) store_y(d.y, o + e, f[e], y_f16);
      }
    }
  }
}

// Two workgroups per CU (four waves per SIMD) is the occupancy aimed at: the
// compiler may then use up to 128 VGPRs for overlapping the lookups.
template <class Fmt>
__global__ __launch_bounds__(kFewWaves * kWave) __attribute__((amdgpu_waves_per_eu(4, 4))) void gemm_few_kernel(
    GemmDesc d) {
  gemm_few_tile<Fmt>(d, blockIdx.x);
}

template <class Fmt>
__global__ __launch_bounds__(kFewWaves * kWave) __attribute__((amdgpu_waves_per_eu(4, 4))) void
gemm_few_grouped_kernel(const char* plan) {
  const PlanHeader* h = reinterpret_cast<const PlanHeader*>(plan);
  const GemmDesc* descs = reinterpret_cast<const GemmDesc*>(plan + sizeof(PlanHeader));
  const GemmTile tl = reinterpret_cast<const GemmTile*>(descs + h->count)[blockIdx.x];
  gemm_few_tile<Fmt>(descs[tl.prob], tl.tile_n);
}

// The 256 x 256 tiles when they still give every CU a workgroup, else the
// 128 x 128 tiles.
template <class Fmt>
hipError_t launch_tile(const GemmDesc& d, hipStream_t stream) {
  const int64_t large = ((d.n + TileLarge::kRows - 1) / TileLarge::kRows) *
                        ((d.m + TileLarge::kTok - 1) / TileLarge::kTok);
  if (large >= kLargeTileMinGroups) {
    if (std::is_same<Fmt, Sherry3of4>::value && prefill_decode_once() && prefill_fits(d.k))
      return launch_gemm_prefill(d, stream);
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

hipError_t launch_gemm_grouped(const PlanHeader* h, const void* dev, hipStream_t stream) {
  if (h->n_tiles == 0) return hipSuccess;
  const char* plan = static_cast<const char*>(dev);
  const int64_t tiling = h->reserved[0];
  const dim3 grid(h->n_tiles);
  const bool t2 = h->format == kFmtTern2;
  if (tiling == kGemmTilingTwo) return launch_gemm2_grouped(plan, h->n_tiles, h->format, stream);
  if (tiling == kGemmTilingBf16) return launch_gemm_bf16_grouped(plan, h->n_tiles, stream);
  if (tiling == kGemmTilingFew) {
    if (t2)
      hipLaunchKernelGGL((gemm_few_grouped_kernel<Tern2>), grid, dim3(kFewWaves * kWave), 0, stream, plan);
    else
      hipLaunchKernelGGL((gemm_few_grouped_kernel<Sherry3of4>), grid, dim3(kFewWaves * kWave), 0, stream, plan);
  } else if (tiling == kGemmTilingLarge) {
    if (!t2 && prefill_decode_once() && h->reserved[1] != 0)
      return launch_gemm_prefill_grouped(plan, h->n_tiles, stream);
    if (t2)
      hipLaunchKernelGGL((gemm_tile_grouped_kernel<Tern2, TileLarge>), grid, dim3(TileLarge::kThreads), 0, stream,
                         plan);
    else
      hipLaunchKernelGGL((gemm_tile_grouped_kernel<Sherry3of4, TileLarge>), grid, dim3(TileLarge::kThreads), 0,
                         stream, plan);
  } else if (tiling == kGemmTilingSkinny) {
    if (t2)
      hipLaunchKernelGGL((gemm_tile_grouped_kernel<Tern2, TileSkinny>), grid, dim3(TileSkinny::kThreads), 0, stream,
                         plan);
    else
      hipLaunchKernelGGL((gemm_tile_grouped_kernel<Sherry3of4, TileSkinny>), grid, dim3(TileSkinny::kThreads), 0,
                         stream, plan);
  } else {
    if (t2)
      hipLaunchKernelGGL((gemm_tile_grouped_kernel<Tern2, TileSmall>), grid, dim3(TileSmall::kThreads), 0, stream,
                         plan);
    else
      hipLaunchKernelGGL((gemm_tile_grouped_kernel<Sherry3of4, TileSmall>), grid, dim3(TileSmall::kThreads), 0,
                         stream, plan);
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmDesc& d, int32_t format, hipStream_t stream) {
  if (gemm2_fits(d.m, d.k)) return launch_gemm2(d, format, stream);
  const int G = d.k / kGroupWeights;
  if (d.m <= kFewMaxTok && G <= kFewMaxGroups) {
    const int rt = few_tile_rows(G);
    const dim3 grid((d.n + rt - 1) / rt);
    if (format == kFmtTern2)
      hipLaunchKernelGGL((gemm_few_kernel<Tern2>), grid, dim3(kFewWaves * kWave), 0, stream, d);
    else
      hipLaunchKernelGGL((gemm_few_kernel<Sherry3of4>), grid, dim3(kFewWaves * kWave), 0, stream, d);
    return hipGetLastError();
  }
  if (d.m >= kTiledMinM)
    return format == kFmtTern2 ? launch_tile<Tern2>(d, stream) : launch_tile<Sherry3of4>(d, stream);
  return format == kFmtTern2 ? launch_small<Tern2>(d, stream) : launch_small<Sherry3of4>(d, stream);
}

}  // namespace sherry
