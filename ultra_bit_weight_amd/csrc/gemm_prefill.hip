// Prefill products (many tokens) on Sherry 3:4 codes, Y[m, r] = s_x[m] s_w[r]
// sum_k X[m, k] T[r, k], with every code of a tile decoded once per workgroup
// ("Sherry: Hardware-Efficient 1.25-Bit Ternary Quantization via Fine-grained
// Sparsification", Abstract: 3:4 sparse ternary blocks in five bits; Figure 2
// caption: four-weight blocks).
//
// A workgroup of 16 waves computes a 256-row x 128-token tile of Y (the large
// tiling), stepping k by one 128-weight group.  In the step of group g:
//   * every wave multiplies its 64-row x 32-token sub-tile for group g: A and B
//     fragments read from the LDS tiles of g, 16 v_mfma_i32_16x16x64_i8;
//   * the 1024 threads decode the tile's weights of group g + 1 once: thread
//     (row r, quarter j) expands blocks 8 j .. 8 j + 7 of row r (eight reads of
//     the 32-entry table, 32 int8 weights) into the int8 A tile of g + 1 in
//     LDS;
//   * they copy the x tile of g + 1 (128 tokens x 128 bytes) from registers to
//     its LDS tile; x of g + 2 is loaded into registers meanwhile.
// Codes come in stages of four groups: the four threads of a row (a quad)
// load the row's 64-byte run of the four group heads (16 bytes each) and its
// 16-byte run of the four tails with ordinary loads a stage ahead, so one
// request serves four groups of a row; in each step the quad's owner of the
// group broadcasts its five words to the quad (DPP quad_perm).  The compiler
// counts the waits of these loads.  A and x tiles are double-buffered: the
// tiles of g + 1 are written while the tiles of g are read, and one barrier
// per step separates the two.  The decode and copies do not feed the step's
// products, so they overlap with the matrix cores.
//
// Within a 128-byte line (a row of A, a token of x), 16-byte chunk c sits at
// position c ^ (line & 7), so the fragment reads of 8 consecutive lines fall
// in distinct banks (measured fewer bank conflicts than c ^ ((line >> 1) & 7)).  Fragment k-order: lane (i, q) takes bytes
// 32 q + 16 s .. + 16 of the group as half s of its A (row i) and B (token
// i) operands; any assignment is valid when A and B share it.
#include <atomic>
#include <type_traits>

#include "formats.h"
#include "gemm_epi.h"
#include "launch.h"

namespace sherry {
namespace {

constexpr int kPfRows = kGemmLargeRows;  // 256
constexpr int kPfTok = kGemmLargeTok;    // 128
constexpr int kPfWaves = 16;
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kPfWR = 4;                                  // waves along the rows (64 rows each)
constexpr int kPfUT = kPfTok / (16 * (kPfWaves / kPfWR));  // 16-token tiles per wave: 2
constexpr int kPfXChunks = kPfTok * 8;                    // 16-byte chunks of one group's x tile
constexpr int kPfXPer = (kPfXChunks + kPfThreads - 1) / kPfThreads;  // per thread: 1
constexpr int kPfStage = 4;                               // groups per code stage (one per quad lane)
constexpr int kPfRowsPer = kPfRows * kPfStage / kPfThreads;  // rows per thread: 1
constexpr int kPfUnroll = 2 * kPfStage;                   // two stages: register slots are compile-time
static_assert(kPfXChunks % kWave == 0, "x tile split: whole waves");
static_assert(kPfRowsPer * kPfThreads == kPfRows * kPfStage, "decode split");

struct PfShared {
  uint32_t tab32[32];
  u32x4_t a[2][kPfRows * 8];  // decoded A tiles (int8), 32 KB each
  u32x4_t x[2][kPfXChunks];   // x tiles (int8), 24 KB each
};

__device__ __forceinline__ int pf_swz(int line) { return line & 7; }

// v of quad lane J, in every lane of the quad
template <int J>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), J * 0x55, 0xF, 0xF, false));
}

__device__ __forceinline__ void gemm_pf_tile(const GemmDesc& d, int tile_n, int tile_m, PfShared& sh) {
  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int i = lane & 15;
  const int q = lane >> 4;
  const int wn = wave % kPfWR;
  const int wm = wave / kPfWR;
  const int n0 = tile_n * kPfRows;
  const int m0 = tile_m * kPfTok;
  const int G = d.k / kGroupWeights;

  // decoding role: quad lane j (the group of a stage it loads, the quarter of
  // a group it expands), rows dr + 128 e
  const int j = tid & 3;
  const int dr = tid >> 2;
  // Offsets from uniform bases are 32-bit (the host keeps one matrix's codes
  // and x below 4 GiB).
  const uint32_t row_bytes = static_cast<uint32_t>(G) * (kGroupWords * 4);
  uint32_t cro[kPfRowsPer];
#pragma unroll
  for (int e = 0; e < kPfRowsPer; ++e)
    cro[e] = static_cast<uint32_t>(min(n0 + dr + (kPfRows / kPfRowsPer) * e, d.n - 1)) * row_bytes;
  const SHERRY_GLOBAL char* cbase = gmem(reinterpret_cast<const char*>(d.codes));
  // copying role: chunks tid + 512 j of the x tile (token c / 8, chunk c % 8);
  // tokens past m read the last token (their outputs are not stored)
  const SHERRY_GLOBAL char* xbase = gmem(reinterpret_cast<const char*>(d.x));
  uint32_t xoff[kPfXPer];
  int xdst[kPfXPer];
#pragma unroll
  for (int c0 = 0; c0 < kPfXPer; ++c0) {
    const int c = min(tid + kPfThreads * c0, kPfXChunks - 1);  // (chunks past the tile are not copied)
    const int tok = c >> 3;
    xoff[c0] = static_cast<uint32_t>(min(m0 + tok, d.m - 1)) * static_cast<uint32_t>(d.ldx) + 16u * (c & 7);
    xdst[c0] = 8 * tok + ((c & 7) ^ pf_swz(tok));
  }
  // groups past the end load the last group (a valid address; never used)
  // chunk tid + kPfThreads c0 exists for c0 = 0 and, for the first waves, 1
  const bool x2 = __builtin_amdgcn_readfirstlane(tid / kWave) * kWave + kPfThreads < kPfXChunks;
  auto load_x = [&](u32x4_t (&v)[kPfXPer], int g) {
    const uint32_t go = static_cast<uint32_t>(min(g, G - 1)) * kGroupWeights;
#pragma unroll
    for (int c0 = 0; c0 < kPfXPer; ++c0)
      v[c0] = *reinterpret_cast<const SHERRY_GLOBAL u32x4_t*>(xbase + (xoff[c0] + go));
  };
  // stage st: this lane's group 4 st + j of each of its rows
  auto load_stage = [&](uint32_t (&w)[kPfRowsPer][kGroupWords], int st) {
#pragma unroll
    for (int e = 0; e < kPfRowsPer; ++e) Sherry3of4::load_at(w[e], cbase, cro[e], G, min(kPfStage * st + j, G - 1));
  };
  auto store_x = [&](const u32x4_t (&v)[kPfXPer], int b) {
#pragma unroll
    for (int c0 = 0; c0 < kPfXPer; ++c0)
      if (c0 == 0 || x2) sh.x[b][xdst[c0]] = v[c0];
  };
  // group J of the stage in w (held by quad lane J) into A tile b: lane j
  // expands blocks 8 j .. 8 j + 7 (words j and j + 1) as chunks 2 j, 2 j + 1
  auto decode = [&](const uint32_t (&w)[kPfRowsPer][kGroupWords], auto jc, int b) {
    constexpr int J = decltype(jc)::value;
#pragma unroll
    for (int e = 0; e < kPfRowsPer; ++e) {
      uint32_t v[kGroupWords];
#pragma unroll
      for (int c = 0; c < kGroupWords; ++c) v[c] = quad_bcast<J>(w[e][c]);
      const uint32_t pw[2] = {j == 0 ? v[0] : j == 1 ? v[1] : j == 2 ? v[2] : v[3],
                              j == 0 ? v[1] : j == 1 ? v[2] : j == 2 ? v[3] : v[4]};
      const int r = dr + (kPfRows / kPfRowsPer) * e;
      u32x4_t* line = sh.a[b] + 8 * r;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const v4i f = Sherry3of4::frag(pw, j, s2, sh.tab32);
        line[(2 * j + s2) ^ pf_swz(r)] =
            u32x4_t{static_cast<uint32_t>(f[0]), static_cast<uint32_t>(f[1]), static_cast<uint32_t>(f[2]),
                    static_cast<uint32_t>(f[3])};
      }
    }
  };

  v4i acc[4][kPfUT];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int u = 0; u < kPfUT; ++u) acc[t][u] = v4i{0, 0, 0, 0};
  // Fragment addresses: row 64 wn + 16 t + i and token 16 kPfUT wm + 16 u + i
  // both have swizzle i & 7, so one lane offset per half s serves every tile
  // t, u and buffer (immediate offsets).
  const int swi = i & 7;
  const int ca[2] = {(2 * q) ^ swi, (2 * q + 1) ^ swi};
  const u32x4_t* a_lane = &sh.a[0][8 * (64 * wn + i)];
  const u32x4_t* x_lane = &sh.x[0][8 * (16 * kPfUT * wm + i)];
  auto compute = [&](int b) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      v4i a[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const u32x4_t v = a_lane[b * (kPfRows * 8) + 128 * t + ca[s]];
        a[t] = v4i{static_cast<int>(v.x), static_cast<int>(v.y), static_cast<int>(v.z), static_cast<int>(v.w)};
      }
#pragma unroll
      for (int u = 0; u < kPfUT; ++u) {
        const u32x4_t v = x_lane[b * kPfXChunks + 128 * u + ca[s]];
        const v4i bv = {static_cast<int>(v.x), static_cast<int>(v.y), static_cast<int>(v.z), static_cast<int>(v.w)};
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t][u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t], bv, acc[t][u], 0, 0, 0);
      }
    }
  };

  EpiScales es;
  es.load(d, n0, m0, kPfRows, kPfTok, tid);

  // prologue: table, x of groups 0 and 1, code stage 0; the tiles of group 0
  u32x4_t xr[2][kPfXPer];
  uint32_t cw[2][kPfRowsPer][kGroupWords];
  load_x(xr[0], 0);
  load_x(xr[1], 1);
  load_stage(cw[0], 0);
  Sherry3of4::init_table(sh.tab32, tid);
  __syncthreads();
  store_x(xr[0], 0);
  decode(cw[0], std::integral_constant<int, 0>{}, 0);
  __syncthreads();

  // G is a multiple of kPfUnroll (the host sends other k to the general
  // tiled kernel), so no step is conditional; the last step decodes and
  // copies a group past the end (clamped loads) into tiles never read.
  auto step = [&](int g0, auto bbc) {
    constexpr int bb = decltype(bbc)::value;
    const int g = g0 + bb;
    // stage of g: slot (bb / 4) & 1; at a stage start the next stage's codes
    // go to the other slot (its groups were decoded by the step before last).
    // x of g + 2 goes to the slot of x of g (stored a step ago).
    if constexpr (bb % kPfStage == 0) load_stage(cw[(bb / kPfStage + 1) & 1], g / kPfStage + 1);
    load_x(xr[bb & 1], g + 2);
    compute(bb & 1);
    store_x(xr[(bb + 1) & 1], (bb + 1) & 1);
    // group g + 1 is group (bb + 1) % 4 of its stage
    decode(cw[((bb + 1) / kPfStage) & 1], std::integral_constant<int, (bb + 1) % kPfStage>{}, (bb + 1) & 1);
    __syncthreads();
  };
  static_assert(kPfUnroll == 8, "the loop body below lists its eight steps");
  for (int g0 = 0; g0 < G; g0 += kPfUnroll) {
    step(g0, std::integral_constant<int, 0>{});
    step(g0, std::integral_constant<int, 1>{});
    step(g0, std::integral_constant<int, 2>{});
    step(g0, std::integral_constant<int, 3>{});
    step(g0, std::integral_constant<int, 4>{});
    step(g0, std::integral_constant<int, 5>{});
    step(g0, std::integral_constant<int, 6>{});
    step(g0, std::integral_constant<int, 7>{});
  }
  // the loop ends with a barrier after the last reads of the x tiles: the
  // output-stage scales go to x slot 0
  static_assert((kPfRows + kPfTok) * 4 <= sizeof(sh.x[0]), "output-stage scales fit an x slot");
  float* sl = reinterpret_cast<float*>(sh.x[0]);
  es.stage(d, sl, kPfRows, kPfTok, tid);
  __syncthreads();
  tile_store<kPfUT>(d, acc, n0 + 64 * wn, m0 + 16 * kPfUT * wm, i, q, sl + 64 * wn, sl + kPfRows + 16 * kPfUT * wm);
}

__global__ __launch_bounds__(kPfThreads) void gemm_prefill_kernel(GemmDesc d) {
  __shared__ PfShared sh;
  gemm_pf_tile(d, blockIdx.x, blockIdx.y, sh);
}

// Grouped: one workgroup per plan tile {problem, row tile, token tile}.
__global__ __launch_bounds__(kPfThreads) void gemm_prefill_grouped_kernel(const char* plan) {
  __shared__ PfShared sh;
  const PlanHeader* h = reinterpret_cast<const PlanHeader*>(plan);
  const GemmDesc* descs = reinterpret_cast<const GemmDesc*>(plan + sizeof(PlanHeader));
  const GemmTile tl = reinterpret_cast<const GemmTile*>(descs + h->count)[blockIdx.x];
  gemm_pf_tile(descs[tl.prob], tl.tile_n, tl.tile_m, sh);
}

std::atomic<int> g_prefill_kind{kPrefillTiled};

}  // namespace

void set_prefill_kind(int kind) { g_prefill_kind.store(kind, std::memory_order_relaxed); }
int prefill_kind() { return g_prefill_kind.load(std::memory_order_relaxed); }

hipError_t launch_gemm_prefill(const GemmDesc& d, hipStream_t stream) {
  const dim3 grid((d.n + kPfRows - 1) / kPfRows, (d.m + kPfTok - 1) / kPfTok);
  hipLaunchKernelGGL(gemm_prefill_kernel, grid, dim3(kPfThreads), 0, stream, d);
  return hipGetLastError();
}

hipError_t launch_gemm_prefill_grouped(const char* plan, int32_t n_tiles, hipStream_t stream) {
  hipLaunchKernelGGL(gemm_prefill_grouped_kernel, dim3(n_tiles), dim3(kPfThreads), 0, stream, plan);
  return hipGetLastError();
}

}  // namespace sherry
