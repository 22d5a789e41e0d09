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
#include "gemm_tile.h"
#include "launch.h"

namespace sherry {
namespace {

constexpr int kMaxKRanges = 16;  // waves per workgroup (k <= 8192 stays x-stationary)

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
  // the tables first in LDS (largest alignments): their addresses then fit
  // the 16-bit offset field of the lookups, which need no base add
  __shared__ __attribute__((aligned(4096))) uint32_t tab32[32];
  __shared__ __attribute__((aligned(4096))) uint2 pairs[kPairMask != 0 ? Fmt::kPairEntries : 1];
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
    const int kind = prefill_kind();
    if (std::is_same<Fmt, Sherry3of4>::value && kind == kPrefillDecodeOnce && prefill_fits(d.k))
      return launch_gemm_prefill(d, stream);
    if (kind == kPrefillTiled32)
      return launch_gemm_tile32(d, std::is_same<Fmt, Tern2>::value ? kFmtTern2 : kFmtSherry, stream);
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
    const int kind = prefill_kind();
    if (!t2 && kind == kPrefillDecodeOnce && h->reserved[1] != 0)
      return launch_gemm_prefill_grouped(plan, h->n_tiles, stream);
    if (kind == kPrefillTiled32) return launch_gemm_tile32_grouped(plan, h->n_tiles, h->format, stream);
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
