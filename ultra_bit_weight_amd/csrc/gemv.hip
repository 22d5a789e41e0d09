// Batch-1 products y = diag(s_w) * T * x on packed ternary weights
// (decode-phase GEMV; "Sherry: Hardware-Efficient 1.25-Bit Ternary
// Quantization via Fine-grained Sparsification", Abstract: 3:4 sparse ternary
// blocks, four weights in five bits).
//
// The kernels stream the packed rows once from HBM and never materialise the
// weights: each lane keeps its slice of x in registers (x-stationary) and
// walks down the rows; per 4-weight block it expands the code to four int8
// (or bf16) weights and accumulates with v_dot4_i32_i8 (or two
// v_dot2_f32_bf16).  L lanes share one row and combine their partial sums
// with DPP row operations; the lane that owns the row applies the scale.
//
// Row-to-lane mapping for L lanes per row and GPL groups per lane: lane
// (row r, position p) owns groups p, p + L, ..., p + (GPL-1) L.  With the row
// layout (words 0-3 of every group, then word 4 of every group) the L lanes
// of a row read 16 L contiguous bytes with one 16-byte load each and 4 L
// contiguous bytes with one 4-byte load each.
#include <atomic>
#include <mutex>

#include "actq.h"
#include "formats.h"
#include "launch.h"

// Plan memory of sherry_gemv_grouped_noalloc: one copy on every GPU the
// library runs on, held until the process ends.  Host code never passes this
// name to a kernel or a copy (on the host it is only a stand-in); it looks up
// the device address once per device (scratch_plan) and uses that.
static __device__ __align__(256) unsigned char scratch[sherry::kNoAllocPlanBytes];

namespace sherry {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b),
                                         c, false);
}

// ---------------------------------------------------------------- int8 x ---
// The 32-entry code table, then the pair table built from it.  Ends with a
// barrier, so the tables are ready to read.
template <class Fmt, bool kPairs = true>
__device__ __forceinline__ void init_tables(uint32_t* tab32, uint2* pairs) {
  Fmt::init_table(tab32, threadIdx.x);
  __syncthreads();
  if constexpr (kPairs) {
    Fmt::init_pair_table(pairs, tab32, threadIdx.x, blockDim.x);
    __syncthreads();
  }
}

// Fused-quantization products (single calls, latency-bound) read every block
// pair from the 32-entry table: no pair table to build, one barrier fewer
// per workgroup (measured faster there; the grouped walks keep the pairs).
constexpr bool kXqSingles = true;

// x quantized by the workgroup itself (XQ): all threads load the token's fp
// values (kActRegs each), take the absmax over the workgroup, and write the
// int8 codes to xl in LDS; the scale goes to *sx.  Ends with a barrier.
// In two phases, so that other start-up work can run while the loads of x
// are in flight: xq_issue loads the token (kActRegs values per thread),
// xq_finish takes the absmax over the workgroup, writes the int8 codes to xl
// and the scale to *sx, and ends with a barrier.
template <int NR, int XB>
__device__ __forceinline__ void xq_issue(const GemvDesc& d, uint32_t (&raw)[NR]) {
  act_issue_raw<NR, XB>(d.x, 0, d.k, raw);
}

template <int NR>
__device__ __forceinline__ void xq_finish(const GemvDesc& d, int dt, const uint32_t (&raw)[NR], int8_t* xl,
                                          float* sx, float* wmax) {
  float v[NR];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    v[i] = act_raw_value(raw[i], dt, static_cast<int>(threadIdx.x) + i * kActThreads < d.k);
    amax = fmaxf(amax, fabsf(v[i]));
  }
  const float s = act_scale(block_max(amax, wmax));
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int j = threadIdx.x + i * kActThreads;
    if (j < d.k) xl[j] = act_code(v[i], s);
  }
  if (threadIdx.x == 0) *sx = s;
  __syncthreads();
}

template <int XB>
__device__ __forceinline__ void quantize_x_lds(const GemvDesc& d, int dt, int8_t* xl, float* sx, float* wmax) {
  uint32_t raw[kActRegs];
  xq_issue<kActRegs, XB>(d, raw);
  xq_finish(d, dt, raw, xl, sx, wmax);
}

// XQ: d.x holds fp values of type xdt; the workgroup quantizes them into xl
// (LDS, scale to *sx) right after issuing its first code loads, and the
// lanes take their x from there.
struct XQuant {
  int dt;
  int8_t* xl;
  float* sx;
  float* wmax;
  uint2* swb;  // (class walks) the two half words of the scale of row row_begin + thread, loaded with the codes
};

// The 32 x dwords a lane multiplies with group g's 32 decoded dwords: for
// 128-weight groups the group's 128 bytes as they are; for 96-weight groups
// (three weights per code) bytes 3j .. 3j + 2 in dword j, top byte zero.
// Bytes at or past k read as zero.
template <class Fmt>
__device__ __forceinline__ void load_x_group(const void* x, int k, int g, uint32_t* xr) {
  const int8_t* xb = static_cast<const int8_t*>(x);
  if constexpr (Fmt::kGroupW == 128) {
    const SHERRY_GLOBAL u32x4_t* xp = gmem(reinterpret_cast<const u32x4_t*>(xb + static_cast<int64_t>(g) * 128));
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const u32x4_t v = xp[q];
      xr[4 * q + 0] = v.x;
      xr[4 * q + 1] = v.y;
      xr[4 * q + 2] = v.z;
      xr[4 * q + 3] = v.w;
    }
  } else {
    static_assert(Fmt::kGroupW == 96, "x layout of the format");
    const int base = 96 * g;
    const SHERRY_GLOBAL u32x4_t* xp = gmem(reinterpret_cast<const u32x4_t*>(xb + base));
    uint32_t raw[24];
#pragma unroll
    for (int q = 0; q < 6; ++q) {
      const u32x4_t v = base + 16 * q < k ? xp[q] : u32x4_t{0u, 0u, 0u, 0u};
      raw[4 * q + 0] = v.x;
      raw[4 * q + 1] = v.y;
      raw[4 * q + 2] = v.z;
      raw[4 * q + 3] = v.w;
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int i = (3 * j) >> 2;
      xr[j] = __builtin_amdgcn_alignbyte(raw[i + 1 < 24 ? i + 1 : 23], raw[i], (3 * j) & 3) & 0x00FFFFFFu;
    }
  }
}

// int8 x staged once per workgroup in LDS: 16-byte chunk c at slot c + c / 8
// (one pad chunk after each group's 128 bytes, so that the 16 lanes reading
// 16 group slices hit 16 disjoint sets of four banks).
constexpr int kMaxStagedKI8 = 8192;  // largest k of the register-resident classes
constexpr int kXsChunks = kMaxStagedKI8 / 16 * 9 / 8;
constexpr int kXsPerThread = kMaxStagedKI8 / 16 / kGemvThreads;
static_assert(kXsPerThread * 16 * kGemvThreads == kMaxStagedKI8, "x staging split");

// XM tokens per walk (1, or 2 for two-token products): token t's x row is
// d.x + min(t, m - 1) * ldx, and its row results go to out[t * out_stride + ..];
// the decoded codes serve every token.
template <class Fmt, int L, int GPL, int GR = GPL * L, int XQ = 0, int XM = 1>
__device__ __forceinline__ void gemv_i8_rows(const GemvDesc& d, int row_begin, int row_end, uint32_t* tab32,
                                             uint2* tab, int32_t* out, u32x4_t* xs, XQuant xq = XQuant{},
                                             int64_t ldx = 0, int m = 1, int out_stride = 0) {
  constexpr int RPW = kWave / L;
  constexpr int RPI = (kGemvThreads / kWave) * RPW;
  constexpr int NW = Fmt::kWords;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int lp = lane % L;
  const int rs = lane / L;
  constexpr int G = GR;  // groups per row (lanes t L + lp >= G hold none: x = 0)

  // Start-up order keeps the memory pipe busy: x (shared by every row, so
  // cache-resident after the first workgroup), then the first kRing - 1 ring
  // entries, and only then the LDS writes, tables and barriers.  x comes
  // either as the lane's own 128-byte slice straight from global memory, or
  // (XS) as one or two 16-byte chunks per thread staged through LDS, which
  // replaces eight loads per lane with at most two per thread.
  constexpr bool XS = !XQ && Fmt::kGroupW == 128;
  static_assert(XM == 1 || XS, "several tokens: x staged in LDS");
  uint32_t xr[XM][GPL][32];
  u32x4_t xv[XS ? XM * kXsPerThread : 1];
  const int nchunks = d.k / 16;
  if constexpr (XS) {
#pragma unroll
    for (int tk = 0; tk < XM; ++tk) {
      const SHERRY_GLOBAL u32x4_t* xg = gmem(reinterpret_cast<const u32x4_t*>(
          static_cast<const int8_t*>(d.x) + static_cast<int64_t>(min(tk, m - 1)) * ldx));
#pragma unroll
      for (int j = 0; j < kXsPerThread; ++j) {
        const int c = static_cast<int>(threadIdx.x) + kGemvThreads * j;
        if (c < nchunks) xv[tk * kXsPerThread + j] = xg[c];
      }
    }
  }
  auto load_x = [&]() {
#pragma unroll
    for (int t = 0; t < GPL; ++t) {
      if constexpr (XQ) {
        static_assert(Fmt::kGroupW == 128, "in-kernel quantization: 128-weight groups");
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const u32x4_t v = reinterpret_cast<const u32x4_t*>(xq.xl + min(t * L + lp, G - 1) * kGroupWeights)[q];
          xr[0][t][4 * q + 0] = v.x;
          xr[0][t][4 * q + 1] = v.y;
          xr[0][t][4 * q + 2] = v.z;
          xr[0][t][4 * q + 3] = v.w;
        }
      } else {
        load_x_group<Fmt>(d.x, d.k, min(t * L + lp, G - 1), xr[0][t]);
      }
      if (G < GPL * L && t * L + lp >= G) {
#pragma unroll
        for (int j = 0; j < 32; ++j) xr[0][t][j] = 0u;
      }
    }
  };
  if constexpr (!XQ && !XS) load_x();
  // Rows past the tile load the tile's last row instead (results discarded).
  // A ring of kRing register buffers (the loop is unrolled by kRing): while
  // one row is decoded, the words of the next kRing - 1 rows are in flight.
  const int last = row_end - 1;
  // Rows are addressed by 32-bit byte offsets from the matrix base (the host
  // keeps one matrix's codes below 4 GiB).  A fetch takes the unclamped
  // offset of its row, advanced by additions, and clamps it to the tile's
  // last row: no multiply per row.
  constexpr uint32_t kRowBytes = G * NW * 4;
  const SHERRY_GLOBAL char* cbase = gmem(reinterpret_cast<const char*>(d.codes));
  const uint32_t ro_last = static_cast<uint32_t>(last) * kRowBytes;
  auto fetch = [&](uint32_t (&buf)[GPL][NW], uint32_t ro_unclamped) {
    const uint32_t ro = min(ro_unclamped, ro_last);
#pragma unroll
    for (int t = 0; t < GPL; ++t) Fmt::load_at(buf[t], cbase, ro, G, min(t * L + lp, G - 1));
  };
  auto step = [&](const uint32_t (&buf)[GPL][NW], int row) {
    constexpr int C = kDotChains;  // independent dot4 accumulation chains
    int a4[XM][C] = {};
#pragma unroll
    for (int t = 0; t < GPL; ++t) {
#pragma unroll
      for (int p = 0; p < 16; ++p) {
        // block pairs in the mask (kPairMask, kPairMaskTwo for two tokens):
        // one pair-table read; the others: two reads of the 32-entry table
        // (balances VALU against LDS bank conflicts)
        constexpr unsigned PM = XM > 1 ? kPairMaskTwo : (XQ && kXqSingles ? 0u : kPairMask);
        const uint2 v = ((PM >> p) & 1) ? Fmt::i8x8(buf[t], p, tab)
                                        : make_uint2(Fmt::i8x4(buf[t], 2 * p, tab32),
                                                     Fmt::i8x4(buf[t], 2 * p + 1, tab32));
#pragma unroll
        for (int tk = 0; tk < XM; ++tk) {
          a4[tk][(2 * p) % C] = __builtin_amdgcn_sdot4(static_cast<int>(v.x), static_cast<int>(xr[tk][t][2 * p]),
                                                       a4[tk][(2 * p) % C], false);
          a4[tk][(2 * p + 1) % C] = __builtin_amdgcn_sdot4(
              static_cast<int>(v.y), static_cast<int>(xr[tk][t][2 * p + 1]), a4[tk][(2 * p + 1) % C], false);
        }
      }
    }
#pragma unroll
    for (int tk = 0; tk < XM; ++tk) {
      int sum = a4[tk][0];
#pragma unroll
      for (int c = 1; c < C; ++c) sum += a4[tk][c];
      const int acc = reduce_add_i32_last<L>(sum);  // valid in lane L - 1 of the row
      if (lp == L - 1 && row < row_end) out[tk * out_stride + row - row_begin] = acc;
    }
  };
  constexpr int NR = GPL > 1 ? 2 : kRing;  // several groups per lane: two buffers (registers)
  uint32_t ring[NR][GPL][NW];
  const int r0 = row_begin + wave * RPW + rs;
  // XQ: the token's loads go first (the loads complete in order, and the
  // token, cache-resident, is needed first), then every row of the tile --
  // one ring round (the launch sizes it so), all of it in flight while the
  // token is quantized -- then the first output row's scale
  // a class kernel's k is 128 GR: GR / 2 values per thread
  static_assert(!XQ || (GR % 2 == 0 && GR / 2 <= kActRegs), "x of the class fits the quantizing threads");
  static_assert(!XQ || NR == kRing, "single calls: one group per lane");
  uint32_t xqv[XQ ? GR / 2 : 1];
  if constexpr (XQ) xq_issue<GR / 2, XQ>(d, xqv);
#pragma unroll
  for (int b = 0; b + 1 < NR; ++b) fetch(ring[b], static_cast<uint32_t>(r0 + b * RPI) * kRowBytes);
  if constexpr (XQ) {
    fetch(ring[NR - 1], static_cast<uint32_t>(r0 + (NR - 1) * RPI) * kRowBytes);
    // two half-word loads on either path (fp16: the element twice; fp32:
    // its halves): a fixed count keeps the compiler's waits exact
    const int sr = min(row_begin + static_cast<int>(threadIdx.x), last);
    const bool f16 = d.flags & kFlagScaleF16;
    const SHERRY_GLOBAL uint16_t* sp = gmem(static_cast<const uint16_t*>(d.w_scales));
    // (combined in the epilogue: an operation on them here would wait for them)
    xq.swb->x = sp[f16 ? sr : 2 * sr];
    xq.swb->y = sp[f16 ? sr : 2 * sr + 1];
  }
  if constexpr (XS) {
#pragma unroll
    for (int tk = 0; tk < XM; ++tk)
#pragma unroll
      for (int j = 0; j < kXsPerThread; ++j) {
        const int c = static_cast<int>(threadIdx.x) + kGemvThreads * j;
        if (c < nchunks) xs[tk * kXsChunks + c + c / 8] = xv[tk * kXsPerThread + j];
      }
  }
  init_tables<Fmt, !(XQ && kXqSingles)>(tab32, tab);  // its barriers also publish the staged x
  if constexpr (XQ) {
    xq_finish(d, xq.dt, xqv, xq.xl, xq.sx, xq.wmax);
    load_x();
  }
  if constexpr (XS) {
#pragma unroll
    for (int tk = 0; tk < XM; ++tk)
#pragma unroll
      for (int t = 0; t < GPL; ++t) {
        const bool has = t * L + lp < G;
        const u32x4_t* xp = xs + tk * kXsChunks + 9 * min(t * L + lp, G - 1);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const u32x4_t v = xp[q];
          xr[tk][t][4 * q + 0] = has ? v.x : 0u;
          xr[tk][t][4 * q + 1] = has ? v.y : 0u;
          xr[tk][t][4 * q + 2] = has ? v.z : 0u;
          xr[tk][t][4 * q + 3] = has ? v.w : 0u;
        }
      }
  }
  if constexpr (XQ) {
#pragma unroll
    for (int b = 0; b < NR; ++b) step(ring[b], r0 + b * RPI);
    return;
  }
  // Every round runs all NR steps; rows past the tile end are clamped loads
  // whose results are never stored (no branch inside the ring).  The last
  // round fetches only its own last row: nothing follows it.
  int base = row_begin, r = r0;
  uint32_t ro_r = static_cast<uint32_t>(r0) * kRowBytes;  // offset of row r
  for (; base + NR * RPI < row_end; base += NR * RPI, r += NR * RPI, ro_r += NR * RPI * kRowBytes) {
#pragma unroll
    for (int b = 0; b < NR; ++b) {
      fetch(ring[(b + NR - 1) % NR], ro_r + (b + NR - 1) * RPI * kRowBytes);
      step(ring[b], r + b * RPI);
    }
  }
  fetch(ring[NR - 1], ro_r + (NR - 1) * RPI * kRowBytes);
#pragma unroll
  for (int b = 0; b < NR; ++b) step(ring[b], r + b * RPI);
}

// Any k % 128 == 0: 64 lanes per row, x read per group (not register-resident).
template <class Fmt, int XQ = 0>
__device__ __forceinline__ void gemv_i8_rows_generic(const GemvDesc& d, int row_begin, int row_end,
                                                     uint32_t* tab32, uint2* tab, int32_t* out,
                                                     XQuant xq = XQuant{}) {
  constexpr int NW = Fmt::kWords;
  if constexpr (XQ != 0) quantize_x_lds<XQ>(d, xq.dt, xq.xl, xq.sx, xq.wmax);
  init_tables<Fmt>(tab32, tab);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int G = groups_of<Fmt>(d.k);
  const int8_t* x = static_cast<const int8_t*>(d.x);
  for (int r = row_begin + wave; r < row_end; r += kGemvThreads / kWave) {
    int acc = 0;
    for (int g = lane; g < G; g += kWave) {
      uint32_t w[NW];
      Fmt::load(w, d.codes + static_cast<int64_t>(r) * (G * NW), G, g);
      if constexpr (Fmt::kGroupW != 128) {  // three weights per code
        uint32_t xv[32];
        load_x_group<Fmt>(d.x, d.k, g, xv);
#pragma unroll
        for (int p = 0; p < 16; ++p) {
          const uint2 v = kPairMask != 0 ? Fmt::i8x8(w, p, tab)
                                         : make_uint2(Fmt::i8x4(w, 2 * p, tab32), Fmt::i8x4(w, 2 * p + 1, tab32));
          acc = __builtin_amdgcn_sdot4(static_cast<int>(v.x), static_cast<int>(xv[2 * p]), acc, false);
          acc = __builtin_amdgcn_sdot4(static_cast<int>(v.y), static_cast<int>(xv[2 * p + 1]), acc, false);
        }
        continue;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const u32x4_t v = xq.xl ? reinterpret_cast<const u32x4_t*>(xq.xl + g * kGroupWeights)[q]
                                : gmem(reinterpret_cast<const u32x4_t*>(x + static_cast<int64_t>(g) * kGroupWeights))[q];
        const uint2 w0 = kPairMask != 0 ? Fmt::i8x8(w, 2 * q, tab)
                                        : make_uint2(Fmt::i8x4(w, 4 * q, tab32), Fmt::i8x4(w, 4 * q + 1, tab32));
        const uint2 w1 = kPairMask != 0 ? Fmt::i8x8(w, 2 * q + 1, tab)
                                        : make_uint2(Fmt::i8x4(w, 4 * q + 2, tab32), Fmt::i8x4(w, 4 * q + 3, tab32));
        acc = __builtin_amdgcn_sdot4(static_cast<int>(w0.x), static_cast<int>(v.x), acc, false);
        acc = __builtin_amdgcn_sdot4(static_cast<int>(w0.y), static_cast<int>(v.y), acc, false);
        acc = __builtin_amdgcn_sdot4(static_cast<int>(w1.x), static_cast<int>(v.z), acc, false);
        acc = __builtin_amdgcn_sdot4(static_cast<int>(w1.y), static_cast<int>(v.w), acc, false);
      }
    }
    acc = reduce_add_i32_last<64>(acc);
    if (lane == kWave - 1) out[r - row_begin] = acc;
  }
}

// ---------------------------------------------------------------- bf16 x ---
// Weights expanded to four bf16 (one 8-byte table entry) per code, two
// v_dot2_f32_bf16 per block; fp32 accumulation, then y = acc * s_w.
// bf16 x is staged once per workgroup into LDS with contiguous 16-byte
// loads; the register-resident classes then read their slices from LDS.  One
// 16-byte pad follows every group slice (16 chunks) so that lanes reading
// different slices hit different banks.
constexpr int kMaxStagedK = 8192;
constexpr int kStagedChunksBf16 = kMaxStagedK * 2 / 16 * 17 / 16;

template <int L, int GPL, int GR = GPL * L>
__device__ __forceinline__ void gemv_bf16_rows(const GemvDesc& d, int row_begin, int row_end, const uint2* tab,
                                               uint4* xs, float* out) {
  constexpr int RPW = kWave / L;
  constexpr int RPI = (kGemvThreads / kWave) * RPW;
  constexpr int NW = kGroupWords;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int lp = lane % L;
  const int rs = lane / L;
  constexpr int G = GR;  // groups per row (lanes t L + lp >= G hold none: x = 0)

  // Start-up order as in the int8 walk: x's 16-byte chunks into registers,
  // then the first ring fetches, then the LDS copy of x (one pad chunk per
  // 256 bytes) and one barrier (which also publishes the code table), then
  // the lane's slices into registers.
  constexpr int kXsPer = (kMaxStagedK * 2 / 16 + kGemvThreads - 1) / kGemvThreads;
  const int nx = 2 * d.k / 16;
  u32x4_t xv[kXsPer];
  {
    const SHERRY_GLOBAL u32x4_t* src = gmem(static_cast<const u32x4_t*>(d.x));
#pragma unroll
    for (int j = 0; j < kXsPer; ++j) {
      const int c = static_cast<int>(threadIdx.x) + kGemvThreads * j;
      if (c < nx) xv[j] = src[c];
    }
  }
  uint32_t xr[GPL][64];
  const int last = row_end - 1;
  // row offsets as in the int8 walk: 32-bit, advanced by additions, clamped
  constexpr uint32_t kRowBytes = G * NW * 4;
  const SHERRY_GLOBAL char* cbase = gmem(reinterpret_cast<const char*>(d.codes));
  const uint32_t ro_last = static_cast<uint32_t>(last) * kRowBytes;
  auto fetch = [&](uint32_t (&buf)[GPL][NW], uint32_t ro_unclamped) {
    const uint32_t ro = min(ro_unclamped, ro_last);
#pragma unroll
    for (int t = 0; t < GPL; ++t) Sherry3of4::load_at(buf[t], cbase, ro, G, min(t * L + lp, G - 1));
  };
  auto step = [&](const uint32_t (&buf)[GPL][NW], int row) {
    float a2[2] = {0.0f, 0.0f};  // two chains: slot pairs (0,1) and (2,3)
#pragma unroll
    for (int t = 0; t < GPL; ++t) {
      uint32_t m[10];
      masked_words8(buf[t], m);
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const uint2 wv = lds_u64(tab, code_offset8(buf[t], m, j));
        a2[0] = dot2_bf16(wv.x, xr[t][2 * j], a2[0]);
        a2[1] = dot2_bf16(wv.y, xr[t][2 * j + 1], a2[1]);
      }
    }
    const float acc = reduce_add_f32_last<L>(a2[0] + a2[1]);  // valid in lane L - 1 of the row
    if (lp == L - 1 && row < row_end) out[row - row_begin] = acc;
  };
  constexpr int NR = GPL > 1 ? 2 : kRing;  // several groups per lane: two buffers (registers)
  uint32_t ring[NR][GPL][NW];
  const int r0 = row_begin + wave * RPW + rs;
#pragma unroll
  for (int b = 0; b + 1 < NR; ++b) fetch(ring[b], static_cast<uint32_t>(r0 + b * RPI) * kRowBytes);
#pragma unroll
  for (int j = 0; j < kXsPer; ++j) {
    const int c = static_cast<int>(threadIdx.x) + kGemvThreads * j;
    if (c < nx) reinterpret_cast<u32x4_t*>(xs)[c + c / 16] = xv[j];
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < GPL; ++t) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      uint4 v = xs[min(t * L + lp, G - 1) * 17 + q];
      if (G < GPL * L && t * L + lp >= G) v = make_uint4(0u, 0u, 0u, 0u);
      xr[t][4 * q + 0] = v.x;
      xr[t][4 * q + 1] = v.y;
      xr[t][4 * q + 2] = v.z;
      xr[t][4 * q + 3] = v.w;
    }
  }
  // All NR steps of every round run (rows past the tile end are clamped
  // loads).  Peeling the last round's surplus fetches, as the int8 walk
  // does, measured 6 % slower here.
  uint32_t ro_r = static_cast<uint32_t>(r0) * kRowBytes;  // offset of row r
  for (int base = row_begin, r = r0; base < row_end;
       base += NR * RPI, r += NR * RPI, ro_r += NR * RPI * kRowBytes) {
#pragma unroll
    for (int b = 0; b < NR; ++b) {
      fetch(ring[(b + NR - 1) % NR], ro_r + (b + NR - 1) * RPI * kRowBytes);
      step(ring[b], r + b * RPI);
    }
  }
}

__device__ __forceinline__ void gemv_bf16_rows_generic(const GemvDesc& d, int row_begin, int row_end,
                                                       const uint2* tab, float* out) {
  __syncthreads();  // the code table
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int G = d.k / kGroupWeights;
  const uint16_t* x = static_cast<const uint16_t*>(d.x);
  for (int r = row_begin + wave; r < row_end; r += kGemvThreads / kWave) {
    float acc = 0.0f;
    for (int g = lane; g < G; g += kWave) {
      uint32_t w[kGroupWords];
      load_group(w, d.codes + static_cast<int64_t>(r) * (G * kGroupWords), G, g);
      const SHERRY_GLOBAL u32x4_t* xp =
          gmem(reinterpret_cast<const u32x4_t*>(x + static_cast<int64_t>(g) * kGroupWeights));
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const u32x4_t v = xp[q];
        const uint2 w0 = lds_u64(tab, code_offset<3>(w, 2 * q));
        const uint2 w1 = lds_u64(tab, code_offset<3>(w, 2 * q + 1));
        acc = dot2_bf16(w0.x, v.x, acc);
        acc = dot2_bf16(w0.y, v.y, acc);
        acc = dot2_bf16(w1.x, v.z, acc);
        acc = dot2_bf16(w1.y, v.w, acc);
      }
    }
    acc = reduce_add_f32_last<64>(acc);
    if (lane == kWave - 1) out[r - row_begin] = acc;
  }
}

// ---------------------------------------------------------------- kernels ---
// Row results go to LDS during the row loop; after it the workgroup applies
// the epilogue and writes the tile's outputs in one coalesced pass.  Keeping
// global stores out of the loop keeps the prefetched loads in flight.
constexpr int kMaxTileRows = 2048;

__device__ __forceinline__ void finalize_i8(const GemvDesc& d, int row0, int row1, const int32_t* res,
                                            bool has_sx, float sx) {
  const bool s_f16 = d.flags & kFlagScaleF16;
  const bool y_f16 = d.flags & kFlagYF16;
  for (int i = threadIdx.x; i < row1 - row0; i += blockDim.x) {
    const int r = row0 + i;
    if (d.acc) gmem(d.acc)[r] = res[i];
    if (d.y) store_y(d.y, r, epilogue_i32(res[i], load_scale(d.w_scales, r, s_f16), sx, has_sx), y_f16);
  }
}

__device__ __forceinline__ void finalize_bf16(const GemvDesc& d, int row0, int row1, const float* res) {
  const bool s_f16 = d.flags & kFlagScaleF16;
  for (int i = threadIdx.x; i < row1 - row0; i += blockDim.x) {
    const int r = row0 + i;
    gmem(reinterpret_cast<float*>(d.y))[r] = __fmul_rn(res[i], load_scale(d.w_scales, r, s_f16));
  }
}

// Single problem: one kernel per class, so each keeps its own register count.
// The row walkers build the LDS tables themselves (after their first loads).
template <class Fmt, int L, int GPL, int GR>
__global__ __launch_bounds__(kGemvThreads) void gemv_i8_kernel(GemvDesc d, int tile_rows) {
  __shared__ uint32_t tab32[32];
  __shared__ uint2 tab[Fmt::kPairEntries];
  __shared__ int32_t res[kMaxTileRows];
  __shared__ u32x4_t xs[L > 0 && Fmt::kGroupW == 128 ? kXsChunks : 1];
  const int row0 = blockIdx.x * tile_rows;
  const int row1 = min(row0 + tile_rows, d.n);
  if (L == 0)
    gemv_i8_rows_generic<Fmt>(d, row0, row1, tab32, tab, res);
  else
    gemv_i8_rows<Fmt, (L > 0 ? L : 64), GPL, (L > 0 ? GR : 64)>(d, row0, row1, tab32, tab, res, xs);
  __syncthreads();
  finalize_i8(d, row0, row1, res, d.x_scale != nullptr, d.x_scale ? *gmem(d.x_scale) : 1.0f);
}

// fp x quantized per token inside the workgroup (k <= kActMaxRegK), then
// the int8 product; block 0 writes the scale to sx_out if given.
static_assert(kGemvThreads == kActThreads, "the workgroup quantizes x with every thread");
// XB: bytes per x value (4: fp32, 2: fp16 or bf16).
template <class Fmt, int L, int GPL, int GR, int XB>
__global__ __launch_bounds__(kGemvThreads) void gemv_i8_xq_kernel(GemvDesc d, int tile_rows, int xdt,
                                                                  float* sx_out) {
  __shared__ uint32_t tab32[32];
  __shared__ uint2 tab[kPairMask != 0 ? Fmt::kPairEntries : 1];
  __shared__ int32_t res[kMaxTileRows];
  __shared__ __attribute__((aligned(16))) int8_t xl[kActMaxRegK];
  __shared__ float sx;
  __shared__ float wmax[kGemvThreads / kWave];
  // class walks load the scale of this thread's first output row with the
  // codes, so that the epilogue does not wait for it (raw bits: a
  // conversion there would wait for the load at once)
  uint2 swb = make_uint2(0u, 0u);
  const XQuant xq{xdt, xl, &sx, wmax, &swb};
  const int row0 = blockIdx.x * tile_rows;
  const int row1 = min(row0 + tile_rows, d.n);
  const bool s_f16 = d.flags & kFlagScaleF16;
  if constexpr (L == 0)
    gemv_i8_rows_generic<Fmt, XB>(d, row0, row1, tab32, tab, res, xq);
  else
    gemv_i8_rows<Fmt, L, GPL, GR, XB>(d, row0, row1, tab32, tab, res, nullptr, xq);
  __syncthreads();
  const bool y_f16 = d.flags & kFlagYF16;
  for (int i = threadIdx.x; i < row1 - row0; i += blockDim.x) {
    const int r = row0 + i;
    const float sw = L != 0 && i < kGemvThreads
                         ? (s_f16 ? static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(swb.x)))
                                  : __uint_as_float(swb.x | swb.y << 16))
                         : load_scale(d.w_scales, r, s_f16);
    if (d.acc) gmem(d.acc)[r] = res[i];
    if (d.y) store_y(d.y, r, epilogue_i32(res[i], sw, sx, true), y_f16);
  }
  if (sx_out && blockIdx.x == 0 && threadIdx.x == 0) *gmem(sx_out) = sx;
}

template <int L, int GPL, int GR>
__global__ __launch_bounds__(kGemvThreads) void gemv_bf16_kernel(GemvDesc d, int tile_rows) {
  __shared__ uint2 tab[32];
  __shared__ float res[kMaxTileRows];
  __shared__ uint4 xs[L == 0 ? 1 : kStagedChunksBf16];
  const int row0 = blockIdx.x * tile_rows;
  const int row1 = min(row0 + tile_rows, d.n);
  if (threadIdx.x < 32) tab[threadIdx.x] = decode_bf16x4(threadIdx.x);
  if (L == 0)
    gemv_bf16_rows_generic(d, row0, row1, tab, res);
  else
    gemv_bf16_rows<(L > 0 ? L : 64), GPL, (L > 0 ? GR : 64)>(d, row0, row1, tab, xs, res);
  __syncthreads();
  finalize_bf16(d, row0, row1, res);
}

// Grouped: one workgroup per plan tile {problem, first row}; a tile spans
// kGroupedIters row iterations of its problem's class.  The int8 classes
// keep one group per lane (k = 3072: 24 of 32 lanes), so one register
// budget serves all of them.  The bf16 path is bound by its VALU work, where
// idle lanes cost more than occupancy gains: its k = 3072 class keeps 3
// groups in each of 8 lanes, in the WIDE kernel family (more registers),
// used only by plans that hold such a problem.
__device__ __forceinline__ int tile_rows_of(int32_t kc, bool bf16) {
  int lanes = 64;
  switch (kc) {
    case k1024: lanes = 8; break;
    case k2048: lanes = 16; break;
    case k4096: lanes = 32; break;
    case k8192: lanes = 64; break;
    case k3072: lanes = bf16 ? 8 : 32; break;
    case kT3k2048: lanes = 32; break;
    case kT3k8192: lanes = 64; break;
    default: lanes = 64; break;
  }
  return (kGemvThreads / kWave) * (kWave / lanes) * kGroupedIters;
}
constexpr int kMaxGroupedTileRows = (kGemvThreads / kWave) * (kWave / 8) * kGroupedIters;

template <class Fmt>
__global__ __launch_bounds__(kGemvThreads) void gemv_i8_grouped_kernel(const char* plan) {
  __shared__ uint32_t tab32[32];
  __shared__ uint2 tab[Fmt::kPairEntries];
  __shared__ int32_t res[kMaxGroupedTileRows];
  __shared__ u32x4_t xs[Fmt::kGroupW == 128 ? kXsChunks : 1];
  const PlanHeader* h = reinterpret_cast<const PlanHeader*>(plan);
  const GemvDesc* descs = reinterpret_cast<const GemvDesc*>(plan + sizeof(PlanHeader));
  const PlanTile* tiles = reinterpret_cast<const PlanTile*>(descs + h->count);
  const PlanTile tl = tiles[blockIdx.x];
  const GemvDesc d = descs[tl.prob];
  const int row0 = tl.row0;
  const int row1 = min(row0 + tile_rows_of(d.kclass, false), d.n);
  if constexpr (Fmt::kGroupW != 128) {
    switch (d.kclass) {
      case kT3k2048: gemv_i8_rows<Fmt, 32, 1, 22>(d, row0, row1, tab32, tab, res, nullptr); break;
      case kT3k8192: gemv_i8_rows<Fmt, 64, 2, 86>(d, row0, row1, tab32, tab, res, nullptr); break;
      default: gemv_i8_rows_generic<Fmt>(d, row0, row1, tab32, tab, res); break;
    }
  } else switch (d.kclass) {
    case k1024: gemv_i8_rows<Fmt, 8, 1>(d, row0, row1, tab32, tab, res, xs); break;
    case k2048: gemv_i8_rows<Fmt, 16, 1>(d, row0, row1, tab32, tab, res, xs); break;
    case k4096: gemv_i8_rows<Fmt, 32, 1>(d, row0, row1, tab32, tab, res, xs); break;
    case k8192: gemv_i8_rows<Fmt, 64, 1>(d, row0, row1, tab32, tab, res, xs); break;
    case k3072: gemv_i8_rows<Fmt, 32, 1, 24>(d, row0, row1, tab32, tab, res, xs); break;
    default: gemv_i8_rows_generic<Fmt>(d, row0, row1, tab32, tab, res); break;
  }
  __syncthreads();
  finalize_i8(d, row0, row1, res, d.x_scale != nullptr, d.x_scale ? *gmem(d.x_scale) : 1.0f);
}

// Two-token products (GEMM with m <= 2 and a register-class k): the batch-1
// walk with both tokens' x in registers, so each decoded code feeds two
// v_dot4; tiles as in the grouped GEMV.  m = 1 walks token 0 twice and
// stores it once.
__device__ __forceinline__ int32_t kclass_dev(int k) {
  return k == 1024 ? k1024 : k == 2048 ? k2048 : k == 4096 ? k4096 : k == 8192 ? k8192 : k == 3072 ? k3072 : kGeneric;
}

// rows: the tile's row count (a whole number of row iterations, at most
// kMaxGroupedTileRows); 0 = the grouped GEMV tile of the class.
template <class Fmt>
__device__ __forceinline__ void gemm2_tile(const GemmDesc& g, int tile_n, int rows, uint32_t* tab32, uint2* tab,
                                           int32_t* res, u32x4_t* xs) {
  const int32_t kc = kclass_dev(g.k);
  if (kc == kGeneric) return;  // the host routes only the register classes here
  if (rows == 0) rows = tile_rows_of(kc, false);
  const int row0 = tile_n * rows;
  const int row1 = min(row0 + rows, g.n);
  GemvDesc d{};
  d.codes = g.codes;
  d.x = g.x;
  d.n = g.n;
  d.k = g.k;
  d.kclass = kc;
  constexpr int S = kMaxGroupedTileRows;  // res stride between the two tokens
  const XQuant none{};
  switch (kc) {
    case k1024: gemv_i8_rows<Fmt, 8, 1, 8, false, 2>(d, row0, row1, tab32, tab, res, xs, none, g.ldx, g.m, S); break;
    case k2048: gemv_i8_rows<Fmt, 16, 1, 16, false, 2>(d, row0, row1, tab32, tab, res, xs, none, g.ldx, g.m, S); break;
    case k4096: gemv_i8_rows<Fmt, 32, 1, 32, false, 2>(d, row0, row1, tab32, tab, res, xs, none, g.ldx, g.m, S); break;
    case k8192: gemv_i8_rows<Fmt, 64, 1, 64, false, 2>(d, row0, row1, tab32, tab, res, xs, none, g.ldx, g.m, S); break;
    default: gemv_i8_rows<Fmt, 32, 1, 24, false, 2>(d, row0, row1, tab32, tab, res, xs, none, g.ldx, g.m, S); break;
  }
  __syncthreads();
  const bool s_f16 = g.flags & kFlagScaleF16;
  const bool y_f16 = g.flags & kFlagYF16;
  const bool has_sx = g.x_scales != nullptr;
  const int nr = row1 - row0;
  for (int i = threadIdx.x; i < g.m * nr; i += kGemvThreads) {
    const int tk = i / nr;
    const int r = row0 + (i - tk * nr);
    const int32_t v = res[tk * S + (r - row0)];
    if (g.acc) gmem(g.acc)[static_cast<int64_t>(tk) * g.n + r] = v;
    if (g.y) {
      const float sx = has_sx ? gmem(g.x_scales)[tk] : 1.0f;
      store_y(g.y, static_cast<int64_t>(tk) * g.ldy + r, epilogue_i32(v, load_scale(g.w_scales, r, s_f16), sx, has_sx),
              y_f16);
    }
  }
}

template <class Fmt>
__global__ __launch_bounds__(kGemvThreads) void gemm2_kernel(GemmDesc d, int tile_rows) {
  __shared__ uint32_t tab32[32];
  __shared__ uint2 tab[Fmt::kPairEntries];
  __shared__ int32_t res[2 * kMaxGroupedTileRows];
  __shared__ u32x4_t xs[2 * kXsChunks];
  gemm2_tile<Fmt>(d, blockIdx.x, tile_rows, tab32, tab, res, xs);
}

template <class Fmt>
__global__ __launch_bounds__(kGemvThreads) void gemm2_grouped_kernel(const char* plan) {
  __shared__ uint32_t tab32[32];
  __shared__ uint2 tab[Fmt::kPairEntries];
  __shared__ int32_t res[2 * kMaxGroupedTileRows];
  __shared__ u32x4_t xs[2 * kXsChunks];
  const PlanHeader* h = reinterpret_cast<const PlanHeader*>(plan);
  const GemmDesc* descs = reinterpret_cast<const GemmDesc*>(plan + sizeof(PlanHeader));
  const GemmTile* tiles = reinterpret_cast<const GemmTile*>(descs + h->count);
  const GemmTile tl = tiles[blockIdx.x];
  gemm2_tile<Fmt>(descs[tl.prob], tl.tile_n, 0, tab32, tab, res, xs);
}

template <bool WIDE>
__global__ __launch_bounds__(kGemvThreads) void gemv_bf16_grouped_kernel(const char* plan) {
  __shared__ uint2 tab[32];
  __shared__ float res[kMaxGroupedTileRows];
  __shared__ uint4 xs[kStagedChunksBf16];
  if (threadIdx.x < 32) tab[threadIdx.x] = decode_bf16x4(threadIdx.x);
  const PlanHeader* h = reinterpret_cast<const PlanHeader*>(plan);
  const GemvDesc* descs = reinterpret_cast<const GemvDesc*>(plan + sizeof(PlanHeader));
  const PlanTile* tiles = reinterpret_cast<const PlanTile*>(descs + h->count);
  const PlanTile tl = tiles[blockIdx.x];
  const GemvDesc d = descs[tl.prob];
  const int row0 = tl.row0;
  const int row1 = min(row0 + tile_rows_of(d.kclass, true), d.n);
  switch (d.kclass) {
    case k1024: gemv_bf16_rows<8, 1>(d, row0, row1, tab, xs, res); break;
    case k2048: gemv_bf16_rows<16, 1>(d, row0, row1, tab, xs, res); break;
    case k4096: gemv_bf16_rows<32, 1>(d, row0, row1, tab, xs, res); break;
    case k8192: gemv_bf16_rows<64, 1>(d, row0, row1, tab, xs, res); break;
    case k3072:
      if (WIDE) {
        gemv_bf16_rows<8, 3>(d, row0, row1, tab, xs, res);
        break;
      }
      [[fallthrough]];
    default: gemv_bf16_rows_generic(d, row0, row1, tab, res); break;
  }
  __syncthreads();
  finalize_bf16(d, row0, row1, res);
}

// ----------------------------------------------- bf16 x on the matrix cores ---
// v_mfma_f32_16x16x32_bf16 multiplies A (16 x 32) by B (32 x 16): lane
// (q, i) = (lane / 16, lane % 16) holds 8 bf16 of row i of A and the same 8 k
// of column i of B, and C[4q + e][i] lands in register e.  Only the diagonal
// is used: C[i][i] = sum over q of lane (q, i)'s 8 weights times its own 8 x
// values, so each lane may take any k positions as long as its A and B
// agree, and the four lanes of column i add up.  Here lane (q, i) owns one
// 128-weight group of one row (its 32 codes feed 16 products, two blocks
// each, and the group's 128 x values stay in 64 registers), and the four
// lanes of a column belong to the same row: a row of G groups takes
// P = ceil(G / 4) columns (group 4p + q in column p of the row), and a wave
// walks R = 16 / P rows at a time.  A row's codes are therefore read by
// consecutive lanes as in the VALU kernel, whole lines per instruction; the
// multiply-adds and the 4-lane sum run on the matrix cores, and the VALU
// keeps only the code extraction.  The P diagonal values of a row go to LDS
// and are added in column order after the walk, so the result does not
// depend on timing.  Columns past R P, and groups past G, repeat the loads
// of an active lane (same addresses) with x = 0.
// x is staged in LDS once per tile (a 16-byte pad after every group); the
// first code loads are issued before the staging barrier and the epilogue's
// scales are loaded with them.
typedef __bf16 v8bf_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));
typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));
constexpr int kBfThreads = kBf16MfmaWaves * kWave;
constexpr int kBfResFloats = 4096;  // tile rows * P: 256 * 16 (k = 8192), 1024 * 2 (k = 1024)
constexpr int kBfMaxTileRows = 1024;
constexpr int kBfRowsPerThread = (kBfMaxTileRows + kBfThreads - 1) / kBfThreads;
constexpr int kBfStagedChunks = kBf16MfmaMaxK / 8 * 17 / 16;  // 16-byte chunks of x with one pad per group
// Codes whose table reads are issued before their products; independent
// accumulators (back-to-back products into one accumulator wait for each
// other's results); depth of the code prefetch ring.
#ifndef SHERRY_BF_BATCH
#define SHERRY_BF_BATCH 8
#endif
#ifndef SHERRY_BF_ACC
#define SHERRY_BF_ACC 1
#endif
#ifndef SHERRY_BF_RING
#define SHERRY_BF_RING 4
#endif
constexpr int kBfBatch = SHERRY_BF_BATCH;
constexpr int kBfAcc = SHERRY_BF_ACC;
constexpr int kBfRing = SHERRY_BF_RING;

struct BfShared {
  uint2 tab[32];
  float res[kBfResFloats];
  u32x4_t xs[kBfStagedChunks];
};

__device__ __forceinline__ void gemv_bf16_mfma_tile(const GemvDesc& d, int row0, int rt, BfShared& sh) {
  constexpr int D = kBfRing;
  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int i = lane & 15;
  const int q = lane >> 4;
  const int G = d.k / kGroupWeights;
  const int P = (G + 3) / 4;  // columns per row
  const int R = 16 / P;       // rows per step
  const int RW = rt / kBf16MfmaWaves;
  const int steps = (RW + R - 1) / R;
  const int wrow0 = wave * RW;  // the wave's first row in the tile
  const int nrows = min(rt, d.n - row0);
  const int ie = i % (R * P);  // idle columns load what column ie loads
  const int rho = ie / P;
  const int g = 4 * (ie % P) + q;
  const bool active = i < R * P && g < G;
  const int gc = min(g, G - 1);
  const int64_t row_words = static_cast<int64_t>(G) * kGroupWords;
  auto fetch = [&](uint32_t (&w)[kGroupWords], int t) {
    const int row = min(row0 + wrow0 + min(t, steps - 1) * R + rho, d.n - 1);
    Sherry3of4::load(w, d.codes + row * row_words, G, gc);
  };
  uint32_t ring[D][kGroupWords];
#pragma unroll
  for (int r = 0; r + 1 < D; ++r) fetch(ring[r], r);
  // epilogue scales, x staged in LDS, the table
  const bool s_f16 = d.flags & kFlagScaleF16;
  float sw[kBfRowsPerThread];
#pragma unroll
  for (int u = 0; u < kBfRowsPerThread; ++u) {
    const int t = tid + u * kBfThreads;
    sw[u] = t < nrows ? load_scale(d.w_scales, row0 + t, s_f16) : 0.0f;
  }
  const SHERRY_GLOBAL u32x4_t* xg = gmem(static_cast<const u32x4_t*>(d.x));
  for (int c = tid; c < d.k / 8; c += kBfThreads) sh.xs[c + c / 16] = xg[c];
  if (tid < 32) sh.tab[tid] = decode_bf16x4(tid);
  __syncthreads();
  uint32_t xr[64];
  {
    const u32x4_t* xp = sh.xs + 17 * gc;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const u32x4_t v = xp[u];
      xr[4 * u + 0] = active ? v.x : 0u;
      xr[4 * u + 1] = active ? v.y : 0u;
      xr[4 * u + 2] = active ? v.z : 0u;
      xr[4 * u + 3] = active ? v.w : 0u;
    }
  }
  // C[i][i] sits in lane (i / 4, i), register i % 4
  const bool diag = q == (i >> 2) && i < R * P;
  auto step = [&](const uint32_t (&w)[kGroupWords], int t) {
    uint32_t m[10];
    masked_words8(w, m);
    v4f_t c[kBfAcc];
#pragma unroll
    for (int r = 0; r < kBfAcc; ++r) c[r] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int h = 0; h < 32 / kBfBatch; ++h) {
      uint2 a[kBfBatch];
#pragma unroll
      for (int u = 0; u < kBfBatch; ++u) a[u] = lds_u64(sh.tab, code_offset8(w, m, kBfBatch * h + u));
      // the batch's table reads all go out before its products (left to
      // itself the scheduler pairs each product with its own two reads, and
      // every product waits on an LDS round trip)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kBfBatch / 2; ++u) {
        const int p = (kBfBatch / 2) * h + u;  // blocks 2p, 2p + 1: x values 8p .. 8p + 7
        const v4u_t av = {a[2 * u].x, a[2 * u].y, a[2 * u + 1].x, a[2 * u + 1].y};
        const v4u_t bv = {xr[4 * p], xr[4 * p + 1], xr[4 * p + 2], xr[4 * p + 3]};
        c[p % kBfAcc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(v8bf_t, av), __builtin_bit_cast(v8bf_t, bv), c[p % kBfAcc], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int r = 1; r < kBfAcc; ++r) c[0] += c[r];
    const int e = i & 3;
    const float v = e == 0 ? c[0][0] : (e == 1 ? c[0][1] : (e == 2 ? c[0][2] : c[0][3]));
    const int rl = t * R + rho;
    if (diag && rl < RW) sh.res[(wrow0 + rl) * P + ie % P] = v;
  };
  for (int t0 = 0; t0 < steps; t0 += D) {
#pragma unroll
    for (int r = 0; r < D; ++r) {
      fetch(ring[(r + D - 1) % D], t0 + r + D - 1);
      if (t0 + r < steps) step(ring[r], t0 + r);
    }
  }
  __syncthreads();
  // y[row] = (sum over the row's columns, in order) * s_w[row], fp32
#pragma unroll
  for (int u = 0; u < kBfRowsPerThread; ++u) {
    const int t = tid + u * kBfThreads;
    if (t < nrows) {
      float acc = sh.res[t * P];
      for (int p = 1; p < P; ++p) acc = __fadd_rn(acc, sh.res[t * P + p]);
      gmem(reinterpret_cast<float*>(d.y))[row0 + t] = __fmul_rn(acc, sw[u]);
    }
  }
}

__global__ __launch_bounds__(kBfThreads) void gemv_bf16_mfma_grouped_kernel(const char* plan) {
  __shared__ BfShared sh;
  const PlanHeader* h = reinterpret_cast<const PlanHeader*>(plan);
  const GemvDesc* descs = reinterpret_cast<const GemvDesc*>(plan + sizeof(PlanHeader));
  const PlanTile tl = reinterpret_cast<const PlanTile*>(descs + h->count)[blockIdx.x];
  const GemvDesc d = descs[tl.prob];
  gemv_bf16_mfma_tile(d, tl.row0, bf16_mfma_tile_rows(d.kclass), sh);
}

// ---------------------------------------------------------- tern3 encode ---
// One thread per (row, group): the group's 96 weights (zero past k; values
// taken by sign) -> 32 base-3 codes -> the 5-word stream, words 0-3 at 4g and
// word 4 at 4G + g of the row.
__global__ __launch_bounds__(256) void tern3_encode_kernel(const int8_t* t, int64_t n, int64_t k, int64_t ldt,
                                                           uint32_t* codes) {
  const int64_t G = (k + 95) / 96;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= n * G) return;
  const int64_t r = idx / G;
  const int64_t g = idx % G;
  uint32_t raw[24];
  const int64_t base = 96 * g;
#pragma unroll
  for (int q = 0; q < 6; ++q) {
    const u32x4_t v = base + 16 * q < k ? *gmem(reinterpret_cast<const u32x4_t*>(t + r * ldt + base + 16 * q))
                                        : u32x4_t{0u, 0u, 0u, 0u};
    raw[4 * q + 0] = v.x;
    raw[4 * q + 1] = v.y;
    raw[4 * q + 2] = v.z;
    raw[4 * q + 3] = v.w;
  }
  uint32_t w[5] = {0u, 0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    uint32_t c = 0;
#pragma unroll
    for (int i = 2; i >= 0; --i) {
      const int b = 3 * j + i;
      const int8_t v = static_cast<int8_t>((raw[b >> 2] >> (8 * (b & 3))) & 0xFFu);
      c = 3u * c + (v < 0 ? 0u : (v == 0 ? 1u : 2u));
    }
    const int bit = 5 * j;
    w[bit >> 5] |= c << (bit & 31);
    if ((bit & 31) > 27) w[(bit >> 5) + 1] |= c >> (32 - (bit & 31));
  }
  uint32_t* row = codes + r * 5 * G;
#pragma unroll
  for (int i = 0; i < 4; ++i) gmem(row)[4 * g + i] = w[i];
  gmem(row)[4 * G + g] = w[4];
}

// ---------------------------------------------------------- tern2 encode ---
// One thread per output word: 16 int8 weights -> 2-bit fields at 8p + 2q.
__global__ __launch_bounds__(256) void tern2_encode_kernel(const int8_t* t, int64_t n, int64_t k, int64_t ldt,
                                                           uint32_t* codes) {
  const int64_t wpr = k / 16;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= n * wpr) return;
  const int64_t r = idx / wpr;
  const int64_t c = idx % wpr;
  const uint4 v = *reinterpret_cast<const uint4*>(t + r * ldt + c * 16);
  const uint32_t b[4] = {v.x, v.y, v.z, v.w};
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int8_t val = static_cast<int8_t>((b[i >> 2] >> (8 * (i & 3))) & 0xFF);
    const uint32_t f = val < 0 ? 3u : static_cast<uint32_t>(val);
    w |= (f & 3u) << (8 * (i & 3) + 2 * (i >> 2));
  }
  codes[idx] = w;
}

}  // namespace

int tile_iters_for(int64_t n, int rpi) {
  // Up to 1024 workgroups, each at least four row iterations long (a
  // workgroup's start-up -- tables, x -- costs about as much as a few
  // iterations, and single calls are latency-bound: measured faster than
  // one iteration per workgroup); a tile never exceeds kMaxTileRows rows
  // (its scales are staged in LDS).
  constexpr int64_t kMinIters = 4;
  const int64_t per = (n + rpi - 1) / rpi;
  int64_t iters = (per + 1023) / 1024;
  if (iters < kMinIters) iters = kMinIters;
  if (iters * rpi > n) iters = (n + rpi - 1) / rpi;  // no tile longer than the matrix
  if (iters < 1) iters = 1;
  if (iters * rpi > kMaxTileRows) iters = kMaxTileRows / rpi;
  return static_cast<int>(iters);
}

namespace {

template <class Fmt, int L, int GPL, int GR = GPL * L>
void launch_i8(const GemvDesc& d, unsigned grid, int tile_rows, hipStream_t stream) {
  hipLaunchKernelGGL((gemv_i8_kernel<Fmt, L, GPL, GR>), dim3(grid), dim3(kGemvThreads), 0, stream, d, tile_rows);
}

template <class Fmt>
void launch_i8_class(const GemvDesc& d, unsigned grid, int tile_rows, hipStream_t stream) {
  if constexpr (Fmt::kGroupW != 128) {  // 1.67-bit rows: 22 or 86 groups, else the generic walk
    switch (d.kclass) {
      case kT3k2048: launch_i8<Fmt, 32, 1, 22>(d, grid, tile_rows, stream); break;
      case kT3k8192: launch_i8<Fmt, 64, 2, 86>(d, grid, tile_rows, stream); break;
      default: launch_i8<Fmt, 0, 1>(d, grid, tile_rows, stream); break;
    }
  } else {
    switch (d.kclass) {
      case k1024: launch_i8<Fmt, 8, 1>(d, grid, tile_rows, stream); break;
      case k2048: launch_i8<Fmt, 16, 1>(d, grid, tile_rows, stream); break;
      case k4096: launch_i8<Fmt, 32, 1>(d, grid, tile_rows, stream); break;
      case k8192: launch_i8<Fmt, 64, 1>(d, grid, tile_rows, stream); break;
      case k3072: launch_i8<Fmt, 32, 1, 24>(d, grid, tile_rows, stream); break;
      default: launch_i8<Fmt, 0, 1>(d, grid, tile_rows, stream); break;
    }
  }
}

template <class Fmt, int L, int GPL, int GR = GPL * L>
void launch_xq(const GemvDesc& d, unsigned grid, int tile_rows, int xdt, float* sx_out, hipStream_t stream) {
  if (xdt == kActF32)
    hipLaunchKernelGGL((gemv_i8_xq_kernel<Fmt, L, GPL, GR, 4>), dim3(grid), dim3(kGemvThreads), 0, stream, d, tile_rows,
                       xdt, sx_out);
  else
    hipLaunchKernelGGL((gemv_i8_xq_kernel<Fmt, L, GPL, GR, 2>), dim3(grid), dim3(kGemvThreads), 0, stream, d, tile_rows,
                       xdt, sx_out);
}

template <class Fmt>
void launch_xq_class(const GemvDesc& d, unsigned grid, int tile_rows, int xdt, float* sx_out, hipStream_t stream) {
  switch (d.kclass) {
    case k1024: launch_xq<Fmt, 8, 1>(d, grid, tile_rows, xdt, sx_out, stream); break;
    case k2048: launch_xq<Fmt, 16, 1>(d, grid, tile_rows, xdt, sx_out, stream); break;
    case k4096: launch_xq<Fmt, 32, 1>(d, grid, tile_rows, xdt, sx_out, stream); break;
    case k8192: launch_xq<Fmt, 64, 1>(d, grid, tile_rows, xdt, sx_out, stream); break;
    case k3072: launch_xq<Fmt, 32, 1, 24>(d, grid, tile_rows, xdt, sx_out, stream); break;
    default: launch_xq<Fmt, 0, 1>(d, grid, tile_rows, xdt, sx_out, stream); break;
  }
}

template <int L, int GPL, int GR = GPL * L>
void launch_bf16(const GemvDesc& d, unsigned grid, int tile_rows, hipStream_t stream) {
  hipLaunchKernelGGL((gemv_bf16_kernel<L, GPL, GR>), dim3(grid), dim3(kGemvThreads), 0, stream, d, tile_rows);
}

void launch_bf16_class(const GemvDesc& d, unsigned grid, int tile_rows, hipStream_t stream) {
  switch (d.kclass) {
    case k1024: launch_bf16<8, 1>(d, grid, tile_rows, stream); break;
    case k2048: launch_bf16<16, 1>(d, grid, tile_rows, stream); break;
    case k4096: launch_bf16<32, 1>(d, grid, tile_rows, stream); break;
    case k8192: launch_bf16<64, 1>(d, grid, tile_rows, stream); break;
    case k3072: launch_bf16<8, 3>(d, grid, tile_rows, stream); break;
    default: launch_bf16<0, 1>(d, grid, tile_rows, stream); break;
  }
}

}  // namespace

hipError_t launch_gemv(const GemvDesc& d, bool bf16_x, int32_t format, hipStream_t stream) {
  const int rpi = rows_per_iter(d.kclass, bf16_x);
  const int tile_rows = rpi * tile_iters_for(d.n, rpi);
  const unsigned grid = static_cast<unsigned>((d.n + tile_rows - 1) / tile_rows);
  if (bf16_x)
    launch_bf16_class(d, grid, tile_rows, stream);
  else if (format == kFmtTern2)
    launch_i8_class<Tern2>(d, grid, tile_rows, stream);
  else if (format == kFmtTern3)
    launch_i8_class<Tern3>(d, grid, tile_rows, stream);
  else
    launch_i8_class<Sherry3of4>(d, grid, tile_rows, stream);
  return hipGetLastError();
}

hipError_t launch_gemv_xq(const GemvDesc& d, int xdt, float* sx_out, int32_t format, hipStream_t stream) {
  // class kernels walk exactly one ring round per workgroup (kRing row
  // iterations, all fetched at start-up); the generic walk takes any tile
  const int rpi = rows_per_iter(d.kclass);
  const int tile_rows = d.kclass == kGeneric ? rpi * tile_iters_for(d.n, rpi) : rpi * kRing;
  const unsigned grid = static_cast<unsigned>((d.n + tile_rows - 1) / tile_rows);
  if (format == kFmtTern2)
    launch_xq_class<Tern2>(d, grid, tile_rows, xdt, sx_out, stream);
  else
    launch_xq_class<Sherry3of4>(d, grid, tile_rows, xdt, sx_out, stream);
  return hipGetLastError();
}

hipError_t launch_gemm2(const GemmDesc& d, int32_t format, hipStream_t stream) {
  // a single call: tiles as for a single GEMV call (enough workgroups to
  // cover the chip), not the grouped ones, at most kMaxGroupedTileRows rows (the LDS results)
  const int rpi = rows_per_iter(kclass_of(d.k));
  const int iters = tile_iters_for(d.n, rpi);
  const int rows = rpi * (iters * rpi > kMaxGroupedTileRows ? kMaxGroupedTileRows / rpi : iters);
  const dim3 grid(static_cast<unsigned>((d.n + rows - 1) / rows));
  if (format == kFmtTern2)
    hipLaunchKernelGGL((gemm2_kernel<Tern2>), grid, dim3(kGemvThreads), 0, stream, d, rows);
  else
    hipLaunchKernelGGL((gemm2_kernel<Sherry3of4>), grid, dim3(kGemvThreads), 0, stream, d, rows);
  return hipGetLastError();
}

hipError_t launch_gemm2_grouped(const char* plan, int32_t n_tiles, int32_t format, hipStream_t stream) {
  if (format == kFmtTern2)
    hipLaunchKernelGGL((gemm2_grouped_kernel<Tern2>), dim3(n_tiles), dim3(kGemvThreads), 0, stream, plan);
  else
    hipLaunchKernelGGL((gemm2_grouped_kernel<Sherry3of4>), dim3(n_tiles), dim3(kGemvThreads), 0, stream, plan);
  return hipGetLastError();
}

hipError_t launch_gemv_grouped(const PlanHeader* h, const void* dev, hipStream_t stream) {
  if (h->n_tiles == 0) return hipSuccess;
  const char* plan = static_cast<const char*>(dev);
  const dim3 grid(h->n_tiles), block(kGemvThreads);
  if (h->x_dt == SHERRY_BF16 && h->reserved[1] != 0)  // matrix-core tiling
    hipLaunchKernelGGL(gemv_bf16_mfma_grouped_kernel, grid, dim3(kBfThreads), 0, stream, plan);
  else if (h->x_dt == SHERRY_BF16 && h->reserved[0] != 0)  // some problem has k = 3072
    hipLaunchKernelGGL((gemv_bf16_grouped_kernel<true>), grid, block, 0, stream, plan);
  else if (h->x_dt == SHERRY_BF16)
    hipLaunchKernelGGL((gemv_bf16_grouped_kernel<false>), grid, block, 0, stream, plan);
  else if (h->format == kFmtTern2)
    hipLaunchKernelGGL((gemv_i8_grouped_kernel<Tern2>), grid, block, 0, stream, plan);
  else if (h->format == kFmtTern3)
    hipLaunchKernelGGL((gemv_i8_grouped_kernel<Tern3>), grid, block, 0, stream, plan);
  else
    hipLaunchKernelGGL((gemv_i8_grouped_kernel<Sherry3of4>), grid, block, 0, stream, plan);
  return hipGetLastError();
}

namespace {
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_dev[kMaxDevices];  // device address of `scratch`, per device
}  // namespace

hipError_t scratch_plan(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_dev[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_dev[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_dev[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_gemv_grouped_noalloc(const PlanHeader* h, const void* plan_host, hipStream_t stream) {
  void* dev = nullptr;
  hipError_t e = scratch_plan(&dev);
  if (e != hipSuccess) return e;
  // stream-ordered: the copy waits for the previous launch on this stream
  // that reads the plan memory, and the kernel waits for the copy
  e = hipMemcpyAsync(dev, plan_host, h->bytes, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return e;
  return launch_gemv_grouped(h, dev, stream);
}

hipError_t launch_tern3_encode(const int8_t* t, int64_t n, int64_t k, int64_t ldt, uint32_t* codes,
                               hipStream_t stream) {
  const int64_t items = n * ((k + 95) / 96);
  const unsigned grid = static_cast<unsigned>((items + 255) / 256);
  hipLaunchKernelGGL(tern3_encode_kernel, dim3(grid), dim3(256), 0, stream, t, n, k, ldt, codes);
  return hipGetLastError();
}

hipError_t launch_tern2_encode(const int8_t* t, int64_t n, int64_t k, int64_t ldt, uint32_t* codes,
                               hipStream_t stream) {
  const int64_t words = n * (k / 16);
  const unsigned grid = static_cast<unsigned>((words + 255) / 256);
  hipLaunchKernelGGL(tern2_encode_kernel, dim3(grid), dim3(256), 0, stream, t, n, k, ldt, codes);
  return hipGetLastError();
}

}  // namespace sherry
