// C ABI of libsherry.so: argument validation, device check and dispatch.
//
// Every argument check runs on the host before the first HIP call, so an
// invalid call returns a status without touching the device (and can be
// tested without a GPU).  Contracts are documented in include/sherry.h.
#include <algorithm>
#include <atomic>
#include <cstring>
#include <limits>
#include <vector>

#include "launch.h"
#include "sherry.h"

using namespace sherry;

namespace {

constexpr int64_t kMaxDim = std::numeric_limits<int32_t>::max();

// Enum arguments arrive from C callers as plain integers, which may lie
// outside the enumerators (a C enum is an int).  They are read through their
// bytes into int32 and validated as integers: loading an out-of-range value
// as the C++ enum type would itself be undefined.
using dt_t = int32_t;
template <class E>
int32_t raw(const E& e) {  // by reference: no load of the enum value
  static_assert(sizeof(E) == sizeof(int32_t), "enum arguments are 32-bit");
  int32_t v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t dt_size(dt_t d) {
  switch (d) {
    case SHERRY_I8: return 1;
    case SHERRY_F16:
    case SHERRY_BF16: return 2;
    case SHERRY_I32:
    case SHERRY_F32: return 4;
  }
  return 0;
}

bool is_scale_dt(dt_t d) { return d == SHERRY_F32 || d == SHERRY_F16; }

// n x k packed matrix shape: positive, k % 128 == 0, every index fits int32
// rows and int64 words.
sherry_status check_nk(int64_t n, int64_t k) {
  if (n <= 0 || k <= 0) return SHERRY_EINVAL;
  if (k % kGroupWeights != 0) return SHERRY_ESHAPE;
  if (n > kMaxDim || k > kMaxDim) return SHERRY_ESHAPE;
  const int64_t g = k / kGroupWeights;
  if (n > std::numeric_limits<int64_t>::max() / (g * 32)) return SHERRY_ESHAPE;
  return SHERRY_OK;
}

// The kernels address one matrix's codes with 32-bit byte offsets from its
// base pointer, so the codes of every matrix stay below 4 GiB.
bool codes_fit_32(int32_t format, int64_t n, int64_t k) {
  const uint64_t groups = format == kFmtTern3 ? static_cast<uint64_t>((k + 95) / 96)
                                              : static_cast<uint64_t>(k / kGroupWeights);
  const uint64_t words = format == kFmtTern2 ? 8 : kGroupWords;
  return static_cast<uint64_t>(n) * groups * words * 4 <= 0xFFFFFFFFull;
}

std::atomic<int> g_dev_state[256];  // 0 unknown, 1 gfx950, 2 other

sherry_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return SHERRY_EDEVICE;
  if (dev < 256) {
    const int s = g_dev_state[dev].load(std::memory_order_relaxed);
    if (s == 1) return SHERRY_OK;
    if (s == 2) return SHERRY_EDEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SHERRY_EDEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 256) g_dev_state[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? SHERRY_OK : SHERRY_EDEVICE;
}

sherry_status launched(hipError_t e) { return e == hipSuccess ? SHERRY_OK : SHERRY_ELAUNCH; }

// Shared validation of a batch-1 product (every format).
sherry_status check_gemv(int32_t format, const uint32_t* codes, const void* w_scales, dt_t s_dt, int64_t n,
                         int64_t k, const void* x, dt_t x_dt, const float* x_scale, const int32_t* acc,
                         const void* y, dt_t y_dt) {
  const bool allow_bf16 = format == kFmtSherry;
  if (!codes || !w_scales || !x || (!acc && !y)) return SHERRY_EINVAL;
  if (sherry_status s = check_nk(n, k)) return s;
  if (!codes_fit_32(format, n, k)) return SHERRY_ESHAPE;
  if (!is_scale_dt(s_dt)) return SHERRY_EDTYPE;
  if (x_dt == SHERRY_I8) {
    if (y && y_dt != SHERRY_F32 && y_dt != SHERRY_F16) return SHERRY_EDTYPE;
  } else if (x_dt == SHERRY_BF16 && allow_bf16) {
    if (acc || x_scale || !y || y_dt != SHERRY_F32) return SHERRY_EDTYPE;
  } else {
    return SHERRY_EDTYPE;
  }
  if (!aligned(codes, 4) || !aligned(x, 16) || !aligned(w_scales, dt_size(s_dt)) || (acc && !aligned(acc, 4)) ||
      (x_scale && !aligned(x_scale, 4)) || (y && !aligned(y, dt_size(y_dt))))
    return SHERRY_EALIGN;
  return SHERRY_OK;
}

GemvDesc make_desc(int32_t format, const uint32_t* codes, const void* w_scales, dt_t s_dt, int64_t n,
                   int64_t k, const void* x, const float* x_scale, int32_t* acc, void* y, dt_t y_dt) {
  GemvDesc d;
  d.codes = codes;
  d.w_scales = w_scales;
  d.x = x;
  d.x_scale = x_scale;
  d.acc = acc;
  d.y = y;
  d.n = static_cast<int32_t>(n);
  d.k = static_cast<int32_t>(k);
  d.flags = (s_dt == SHERRY_F16 ? kFlagScaleF16 : 0) | (y && y_dt == SHERRY_F16 ? kFlagYF16 : 0);
  d.kclass = format == kFmtTern3 ? kclass_of_t3(k) : kclass_of(k);
  return d;
}

sherry_status gemv_impl(int32_t format, const uint32_t* codes, const void* w_scales, dt_t s_dt, int64_t n,
                        int64_t k, const void* x, dt_t x_dt, const float* x_scale, int32_t* acc, void* y,
                        dt_t y_dt, hipStream_t stream) {
  if (sherry_status s = check_gemv(format, codes, w_scales, s_dt, n, k, x, x_dt, x_scale, acc, y, y_dt))
    return s;
  if (sherry_status s = check_device()) return s;
  const GemvDesc d = make_desc(format, codes, w_scales, s_dt, n, k, x, x_scale, acc, y, y_dt);
  return launched(launch_gemv(d, x_dt == SHERRY_BF16, format, stream));
}

// Batch-1 product of fp activations quantized per token inside the kernel.
sherry_status gemv_quant_impl(int32_t format, const uint32_t* codes, const void* w_scales, dt_t s_dt,
                              int64_t n, int64_t k, const void* x, dt_t x_dt, float* x_scale_out,
                              int32_t* acc, void* y, dt_t y_dt, hipStream_t stream) {
  if (!codes || !w_scales || !x || (!acc && !y)) return SHERRY_EINVAL;
  if (sherry_status s = check_nk(n, k)) return s;
  if (k > kActMaxK || !codes_fit_32(format, n, k)) return SHERRY_ESHAPE;
  int dt = 0;
  switch (x_dt) {
    case SHERRY_F32: dt = kActF32; break;
    case SHERRY_F16: dt = kActF16; break;
    case SHERRY_BF16: dt = kActBf16; break;
    default: return SHERRY_EDTYPE;
  }
  if (!is_scale_dt(s_dt) || (y && y_dt != SHERRY_F32 && y_dt != SHERRY_F16)) return SHERRY_EDTYPE;
  if (!aligned(codes, 4) || !aligned(x, dt_size(x_dt)) || !aligned(w_scales, dt_size(s_dt)) ||
      (acc && !aligned(acc, 4)) || (x_scale_out && !aligned(x_scale_out, 4)) || (y && !aligned(y, dt_size(y_dt))))
    return SHERRY_EALIGN;
  if (sherry_status s = check_device()) return s;
  const GemvDesc d = make_desc(format, codes, w_scales, s_dt, n, k, x, nullptr, acc, y, y_dt);
  return launched(launch_gemv_xq(d, dt, x_scale_out, format, stream));
}

// Validation of one product for M tokens; fills the kernel record.
sherry_status check_gemm(int32_t format, const uint32_t* codes, const void* w_scales, dt_t s_dt, int64_t n,
                         int64_t k,
                         const void* x, dt_t x_dt, int64_t m, int64_t ldx, const float* x_scales, int32_t* acc,
                         void* y, dt_t y_dt, int64_t ldy, GemmDesc* out) {
  if (!codes || !w_scales || !x || (!acc && !y)) return SHERRY_EINVAL;
  if (m <= 0) return SHERRY_EINVAL;
  if (sherry_status s = check_nk(n, k)) return s;
  // bf16 X (3:4 codes only): a few tokens on the matrix cores, fp32 Y only;
  // row stride ldx in elements, 16-byte rows
  const bool bf16 = x_dt == SHERRY_BF16;
  if (bf16 && format != kFmtSherry) return SHERRY_EDTYPE;
  if (bf16 && (acc || x_scales || !y || y_dt != SHERRY_F32)) return SHERRY_EDTYPE;
  if (bf16 && (m > kBfFewMaxTok || k > kBfFewMaxK)) return SHERRY_ESHAPE;
  const int64_t row_align = bf16 ? 8 : 16;  // elements per 16 bytes
  if (m > 16 * 65535 || ldx < k || ldx % row_align != 0 || (y && ldy < n)) return SHERRY_ESHAPE;
  if (ldx > std::numeric_limits<int64_t>::max() / (2 * m) || (y && ldy > std::numeric_limits<int64_t>::max() / m))
    return SHERRY_ESHAPE;
  // the tiled kernel addresses one matrix's codes and x with 32-bit offsets
  if (!codes_fit_32(format, n, k) ||
      static_cast<uint64_t>(m) * static_cast<uint64_t>(ldx) * (bf16 ? 2u : 1u) > 0xFFFFFFFFull)
    return SHERRY_ESHAPE;
  if (!is_scale_dt(s_dt) || (x_dt != SHERRY_I8 && !bf16)) return SHERRY_EDTYPE;
  if (y && y_dt != SHERRY_F32 && y_dt != SHERRY_F16) return SHERRY_EDTYPE;
  if (!aligned(codes, 4) || !aligned(x, 16) || !aligned(w_scales, dt_size(s_dt)) || (acc && !aligned(acc, 4)) ||
      (x_scales && !aligned(x_scales, 4)) || (y && !aligned(y, dt_size(y_dt))))
    return SHERRY_EALIGN;
  GemmDesc& d = *out;
  d.codes = codes;
  d.w_scales = w_scales;
  d.x = static_cast<const int8_t*>(x);
  d.x_scales = x_scales;
  d.acc = acc;
  d.y = y;
  d.ldx = ldx;
  d.ldy = y ? ldy : n;
  d.n = static_cast<int32_t>(n);
  d.k = static_cast<int32_t>(k);
  d.m = static_cast<int32_t>(m);
  d.flags = (s_dt == SHERRY_F16 ? kFlagScaleF16 : 0) | (y && y_dt == SHERRY_F16 ? kFlagYF16 : 0);
  return SHERRY_OK;
}

sherry_status gemm_impl(int32_t format, const uint32_t* codes, const void* w_scales, dt_t s_dt, int64_t n,
                        int64_t k, const void* x, dt_t x_dt, int64_t m, int64_t ldx, const float* x_scales,
                        int32_t* acc, void* y, dt_t y_dt, int64_t ldy, hipStream_t stream) {
  GemmDesc d;
  if (sherry_status s =
          check_gemm(format, codes, w_scales, s_dt, n, k, x, x_dt, m, ldx, x_scales, acc, y, y_dt, ldy, &d))
    return s;
  if (sherry_status s = check_device()) return s;
  if (x_dt == SHERRY_BF16) return launched(launch_gemm_bf16(d, stream));
  return launched(launch_gemm(d, format, stream));
}

// Grouped GEMM plan: header | GemmDesc[count] | GemmTile[n_tiles].  Tiling:
// the few-token kernel when every problem has m <= 16 and k <= 8192 (row
// tiles of few_tile_rows(k / 128) rows, all tokens); else 256 x 16 when every
// problem has m <= 16; else 256 x 128 when that gives at least
// kLargeTileMinGroups tiles; else 128 x 128.
struct GemmTiling {
  int64_t kind;
  int rows, tok;
  int64_t rows_of(const sherry_gemm_problem& p) const {
    if (kind == kGemmTilingBf16) return kBfFewMaxTileRows;
    if (kind == kGemmTilingTwo) return gemm2_tile_rows(p.k);
    return kind == kGemmTilingFew ? few_tile_rows(static_cast<int>(p.k / kGroupWeights)) : rows;
  }
};

int64_t gemm_tiles(const sherry_gemm_problem* probs, int32_t count, const GemmTiling& t) {
  int64_t tiles = 0;
  for (int32_t i = 0; i < count; ++i) {
    const int64_t rows = t.rows_of(probs[i]);
    tiles += ((probs[i].n + rows - 1) / rows) * ((probs[i].m + t.tok - 1) / t.tok);
  }
  return tiles;
}

GemmTiling gemm_tiling(const sherry_gemm_problem* probs, int32_t count, dt_t x_dt = SHERRY_I8) {
  if (x_dt == SHERRY_BF16) return GemmTiling{kGemmTilingBf16, kBfFewMaxTileRows, kBfFewMaxTok};
  bool two = true, few = true, skinny = true;
  for (int32_t i = 0; i < count; ++i) {
    two = two && gemm2_fits(probs[i].m, probs[i].k);
    skinny = skinny && probs[i].m <= kGemmSkinnyTok;
    few = few && probs[i].m <= kFewMaxTok && probs[i].k <= kFewMaxGroups * kGroupWeights;
  }
  if (two) return GemmTiling{kGemmTilingTwo, 0, 2};
  if (few) return GemmTiling{kGemmTilingFew, 0, kFewMaxTok};
  if (skinny) return GemmTiling{kGemmTilingSkinny, kGemmSkinnyRows, kGemmSkinnyTok};
  const GemmTiling large{kGemmTilingLarge, kGemmLargeRows, kGemmLargeTok};
  if (gemm_tiles(probs, count, large) >= kLargeTileMinGroups) return large;
  return GemmTiling{kGemmTilingSmall, kGemmSmallRows, kGemmSmallTok};
}

size_t gemm_plan_bytes_impl(const sherry_gemm_problem* probs, int32_t count) {
  if (!probs || count <= 0) return 0;
  for (int32_t i = 0; i < count; ++i) {
    if (check_nk(probs[i].n, probs[i].k) != SHERRY_OK) return 0;
    if (probs[i].m <= 0 || probs[i].m > 16 * 65535) return 0;
  }
  // the plan holds the tiles of the int8 tiling or, if every problem allows
  // bf16 x, of the bf16 one (the caller's x type decides): room for the larger
  bool bf16_fits = true;
  for (int32_t i = 0; i < count; ++i)
    bf16_fits = bf16_fits && probs[i].m <= kBfFewMaxTok && probs[i].k <= kBfFewMaxK;
  int64_t tiles = gemm_tiles(probs, count, gemm_tiling(probs, count));
  if (bf16_fits) tiles = std::max(tiles, gemm_tiles(probs, count, gemm_tiling(probs, count, SHERRY_BF16)));
  if (tiles > kMaxDim) return 0;
  return sizeof(PlanHeader) + sizeof(GemmDesc) * static_cast<size_t>(count) + sizeof(GemmTile) * tiles;
}

// Tile order of the tiled kernels (many tokens).  The workgroups of a launch
// go to the chip's eight XCDs in turn (workgroup w to XCD w mod 8), each XCD
// with an L2 of its own, so the plan holds eight interleaved lists, one per
// XCD.  Each problem's tiles, listed token tile by token tile (the row tiles
// of one token tile together), are cut into eight contiguous shares of equal
// count (the remainders of all problems dealt in turn, so that the lists
// differ in length by at most one and only the first ones are longer), and
// XCD c takes share c of every problem, longest rows first.  Every XCD then
// does an equal part of each problem's work, and the workgroups one XCD
// holds at once read few distinct x tiles, which its L2 serves.
constexpr int kXcds = 8;
bool xcd_order(const sherry_gemm_problem* probs, const std::vector<int32_t>& order, const GemmTiling& tiling,
               GemmTile* tiles, int64_t n_tiles) {
  std::vector<std::vector<GemmTile>> lists(kXcds);
  int next = 0;  // XCD that takes the next remainder tile
  for (const int32_t i : order) {
    const int64_t rows = tiling.rows_of(probs[i]);
    const int64_t tn = (probs[i].n + rows - 1) / rows, tm = (probs[i].m + tiling.tok - 1) / tiling.tok;
    const int64_t n = tn * tm, q = n / kXcds, r = n % kXcds;
    int64_t u = 0;
    for (int c = 0; c < kXcds; ++c) {
      const int64_t share = q + ((c - next + kXcds) % kXcds < r ? 1 : 0);
      for (int64_t e = 0; e < share; ++e, ++u)
        lists[static_cast<size_t>(c)].push_back(
            GemmTile{i, static_cast<int32_t>(u % tn), static_cast<int32_t>(u / tn), 0});
    }
    next = static_cast<int>((next + r) % kXcds);
  }
  for (int c = 0; c < kXcds; ++c)
    if (static_cast<int64_t>(lists[static_cast<size_t>(c)].size()) != (n_tiles - c + kXcds - 1) / kXcds) return false;
  for (int64_t w = 0; w < n_tiles; ++w)
    tiles[w] = lists[static_cast<size_t>(w % kXcds)][static_cast<size_t>(w / kXcds)];
  return true;
}

sherry_status gemm_plan_impl(int32_t format, const sherry_gemm_problem* probs, int32_t count, dt_t s_dt,
                             dt_t x_dt, dt_t y_dt, void* plan, size_t plan_bytes) {
  if (!probs || count <= 0 || !plan) return SHERRY_EINVAL;
  std::vector<GemmDesc> descs(static_cast<size_t>(count));
  for (int32_t i = 0; i < count; ++i) {
    const sherry_gemm_problem& p = probs[i];
    if (sherry_status s = check_gemm(format, p.codes, p.w_scales, s_dt, p.n, p.k, p.x, x_dt, p.m, p.ldx, p.x_scales, p.acc,
                                     p.y, y_dt, p.ldy, &descs[static_cast<size_t>(i)]))
      return s;
  }
  const size_t need = gemm_plan_bytes_impl(probs, count);
  if (need == 0) return SHERRY_ESHAPE;
  if (plan_bytes < need) return SHERRY_EINVAL;
  if (!aligned(plan, 8)) return SHERRY_EALIGN;
  const GemmTiling tiling = gemm_tiling(probs, count, x_dt);
  char* out = static_cast<char*>(plan);
  PlanHeader h;
  std::memset(&h, 0, sizeof(h));
  h.magic = kGemmPlanMagic;
  h.version = kPlanVersion;
  h.count = count;
  h.n_tiles = static_cast<int32_t>(gemm_tiles(probs, count, tiling));
  if (gemm_tiles(probs, count, tiling) > kMaxDim) return SHERRY_ESHAPE;
  h.s_dt = s_dt;
  h.x_dt = x_dt;
  h.y_dt = y_dt;
  h.format = format;
  h.bytes = need;
  h.reserved[0] = static_cast<uint64_t>(tiling.kind);
  bool fits = true;
  for (int32_t i = 0; i < count; ++i) fits = fits && prefill_fits(probs[i].k);
  h.reserved[1] = fits ? 1u : 0u;
  std::memcpy(out, &h, sizeof(h));
  std::memcpy(out + sizeof(PlanHeader), descs.data(), sizeof(GemmDesc) * descs.size());
  GemmTile* tiles = reinterpret_cast<GemmTile*>(out + sizeof(PlanHeader) + sizeof(GemmDesc) * descs.size());
  // longest rows (most k steps) first
  std::vector<int32_t> order(static_cast<size_t>(count));
  for (int32_t i = 0; i < count; ++i) order[static_cast<size_t>(i)] = i;
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return probs[a].k > probs[b].k; });
  if (tiling.kind == kGemmTilingLarge || tiling.kind == kGemmTilingSmall) {
    return xcd_order(probs, order, tiling, tiles, h.n_tiles) ? SHERRY_OK : SHERRY_ESHAPE;
  }
  int64_t t = 0;
  for (const int32_t i : order) {
    const int64_t rows = tiling.rows_of(probs[i]);
    const int64_t tn = (probs[i].n + rows - 1) / rows, tm = (probs[i].m + tiling.tok - 1) / tiling.tok;
    for (int64_t a = 0; a < tn; ++a)
      for (int64_t b = 0; b < tm; ++b)
        tiles[t++] = GemmTile{i, static_cast<int32_t>(a), static_cast<int32_t>(b), 0};
  }
  return SHERRY_OK;
}

// Grouped plan: header | GemvDesc[count] | PlanTile[n_tiles].  Tile rows
// depend on the k class and the x type (bf16 x on the matrix cores: at
// least 256 rows); the int8 tiling has at least as many tiles, so plan sizes
// are computed for it.
int64_t tile_rows_for(const sherry_gemv_problem& p, bool bf16, int32_t format, bool mfma = false) {
  const int32_t kc = format == kFmtTern3 ? kclass_of_t3(p.k) : kclass_of(p.k);
  if (mfma) return bf16_mfma_tile_rows(kc);
  return static_cast<int64_t>(rows_per_iter(kc, bf16)) * kGroupedIters;
}

int64_t plan_tiles(const sherry_gemv_problem* probs, int32_t count, bool bf16, int32_t format, bool mfma = false) {
  int64_t tiles = 0;
  for (int32_t i = 0; i < count; ++i) {
    const int64_t rows = tile_rows_for(probs[i], bf16, format, mfma);
    tiles += (probs[i].n + rows - 1) / rows;
  }
  return tiles;
}

size_t plan_bytes_impl(const sherry_gemv_problem* probs, int32_t count, int32_t format) {
  if (!probs || count <= 0) return 0;
  for (int32_t i = 0; i < count; ++i)
    if (check_nk(probs[i].n, probs[i].k) != SHERRY_OK) return 0;
  const int64_t tiles = plan_tiles(probs, count, false, format);
  if (tiles > kMaxDim) return 0;
  return sizeof(PlanHeader) + sizeof(GemvDesc) * static_cast<size_t>(count) + sizeof(PlanTile) * tiles;
}

sherry_status plan_impl(int32_t format, const sherry_gemv_problem* probs, int32_t count, dt_t s_dt,
                        dt_t x_dt, dt_t y_dt, void* plan, size_t plan_bytes, bool mfma = false) {
  if (!probs || count <= 0 || !plan) return SHERRY_EINVAL;
  for (int32_t i = 0; i < count; ++i) {
    const sherry_gemv_problem& p = probs[i];
    if (sherry_status s = check_gemv(format, p.codes, p.w_scales, s_dt, p.n, p.k, p.x, x_dt, p.x_scale, p.acc, p.y,
                                     y_dt))
      return s;
  }
  if (mfma) {
    if (x_dt != SHERRY_BF16) return SHERRY_EDTYPE;
    for (int32_t i = 0; i < count; ++i)
      if (probs[i].k > kBf16MfmaMaxK) return SHERRY_ESHAPE;
  }
  const size_t need = plan_bytes_impl(probs, count, format);
  if (need == 0) return SHERRY_ESHAPE;
  if (plan_bytes < need) return SHERRY_EINVAL;
  if (!aligned(plan, 8)) return SHERRY_EALIGN;
  char* out = static_cast<char*>(plan);
  PlanHeader h;
  std::memset(&h, 0, sizeof(h));
  h.magic = kPlanMagic;
  h.version = kPlanVersion;
  h.count = count;
  const bool bf16 = x_dt == SHERRY_BF16;
  h.n_tiles = static_cast<int32_t>(plan_tiles(probs, count, bf16, format, mfma));
  h.s_dt = s_dt;
  h.x_dt = x_dt;
  h.y_dt = y_dt;
  h.format = format;
  h.bytes = need;
  for (int32_t i = 0; i < count; ++i)
    if (bf16 && kclass_of(probs[i].k) == k3072) h.reserved[0] = 1;  // the bf16 kernel family with 3 groups per lane
  h.reserved[1] = mfma ? 1 : 0;
  std::memcpy(out, &h, sizeof(h));
  GemvDesc* descs = reinterpret_cast<GemvDesc*>(out + sizeof(PlanHeader));
  PlanTile* tiles = reinterpret_cast<PlanTile*>(descs + count);
  for (int32_t i = 0; i < count; ++i) {
    const sherry_gemv_problem& p = probs[i];
    descs[i] = make_desc(format, p.codes, p.w_scales, s_dt, p.n, p.k, p.x, p.x_scale, p.acc, p.y, y_dt);
  }
  // Tiles of the longest rows first: the workgroups are dispatched in tile
  // order, so the large tiles start early and the small ones fill the tail.
  std::vector<int32_t> order(static_cast<size_t>(count));
  for (int32_t i = 0; i < count; ++i) order[static_cast<size_t>(i)] = i;
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return probs[a].k > probs[b].k; });
  int64_t t = 0;
  for (const int32_t i : order) {
    const sherry_gemv_problem& p = probs[i];
    const int64_t rows = tile_rows_for(p, bf16, format, mfma);
    for (int64_t r0 = 0; r0 < p.n; r0 += rows) tiles[t++] = PlanTile{i, static_cast<int32_t>(r0)};
  }
  return SHERRY_OK;
}

sherry_status pack_impl(const void* w, dt_t w_dt, int64_t n, int64_t k, int64_t ldw, uint32_t* codes,
                        void* scales, dt_t s_dt, bool tern2, hipStream_t stream) {
  if (!w || !codes || !scales) return SHERRY_EINVAL;
  if (sherry_status s = check_nk(n, k)) return s;
  if (ldw < k || ldw > std::numeric_limits<int64_t>::max() / n) return SHERRY_ESHAPE;
  if (w_dt != SHERRY_F32 && w_dt != SHERRY_F16 && w_dt != SHERRY_BF16) return SHERRY_EDTYPE;
  if (!is_scale_dt(s_dt)) return SHERRY_EDTYPE;
  if (!aligned(w, 4 * dt_size(w_dt)) || ldw % 4 != 0 || !aligned(codes, 4) || !aligned(scales, dt_size(s_dt)))
    return SHERRY_EALIGN;
  if (sherry_status s = check_device()) return s;
  return launched(launch_pack(w, w_dt, n, k, ldw, codes, scales, s_dt == SHERRY_F16, tern2, stream));
}

}  // namespace

extern "C" {

const char* sherry_version(void) { return "0.1.0"; }

sherry_status sherry_set_prefill_kernel(sherry_prefill_kernel kind) {
  const dt_t v = raw(kind);
  if (v != SHERRY_PREFILL_TILED && v != SHERRY_PREFILL_DECODE_ONCE && v != SHERRY_PREFILL_TILED32)
    return SHERRY_EINVAL;
  set_prefill_kind(v == SHERRY_PREFILL_DECODE_ONCE ? kPrefillDecodeOnce
                   : v == SHERRY_PREFILL_TILED32   ? kPrefillTiled32
                                                   : kPrefillTiled);
  return SHERRY_OK;
}

const char* sherry_status_str(sherry_status s) {
  switch (raw(s)) {
    case SHERRY_OK: return "SHERRY_OK";
    case SHERRY_EINVAL: return "SHERRY_EINVAL: null pointer, non-positive size or bad argument";
    case SHERRY_ESHAPE: return "SHERRY_ESHAPE: k % 128 != 0, leading dimension too small or size overflow";
    case SHERRY_EDTYPE: return "SHERRY_EDTYPE: unsupported dtype combination";
    case SHERRY_EALIGN: return "SHERRY_EALIGN: pointer or leading dimension misaligned";
    case SHERRY_EDEVICE: return "SHERRY_EDEVICE: no HIP device or the current device is not gfx950";
    case SHERRY_ELAUNCH: return "SHERRY_ELAUNCH: kernel launch failed";
    case SHERRY_ESCRATCH: return "SHERRY_ESCRATCH: plan larger than the library's static plan memory (1 MiB)";
  }
  return "SHERRY_UNKNOWN_STATUS";
}

size_t sherry_packed_bytes(int64_t n, int64_t k) {
  if (check_nk(n, k) != SHERRY_OK) return 0;
  return static_cast<size_t>(n) * static_cast<size_t>(k / kGroupWeights) * kGroupWords * 4;
}

sherry_status sherry_pack(const void* w, sherry_dtype w_dt, int64_t n, int64_t k, int64_t ldw, uint32_t* codes,
                          void* scales, sherry_dtype s_dt, hipStream_t stream) {
  return pack_impl(w, raw(w_dt), n, k, ldw, codes, scales, raw(s_dt), false, stream);
}

sherry_status tern2_pack(const void* w, sherry_dtype w_dt, int64_t n, int64_t k, int64_t ldw, uint32_t* codes,
                         void* scales, sherry_dtype s_dt, hipStream_t stream) {
  return pack_impl(w, raw(w_dt), n, k, ldw, codes, scales, raw(s_dt), true, stream);
}

sherry_status sherry_act_quant(const void* x, sherry_dtype x_dt, int64_t m, int64_t k, int64_t ldx, int8_t* xq,
                               int64_t ldq, float* scales, hipStream_t stream) {
  if (!x || !xq || !scales) return SHERRY_EINVAL;
  if (m <= 0 || k <= 0) return SHERRY_EINVAL;
  int dt = 0;
  const dt_t xd = raw(x_dt);
  switch (xd) {
    case SHERRY_F32: dt = kActF32; break;
    case SHERRY_F16: dt = kActF16; break;
    case SHERRY_BF16: dt = kActBf16; break;
    default: return SHERRY_EDTYPE;
  }
  if (m > kMaxDim || ldx < k || ldq < k) return SHERRY_ESHAPE;
  if (ldx > std::numeric_limits<int64_t>::max() / m || ldq > std::numeric_limits<int64_t>::max() / m)
    return SHERRY_ESHAPE;
  if (!aligned(x, dt_size(xd)) || !aligned(scales, 4)) return SHERRY_EALIGN;
  if (sherry_status s = check_device()) return s;
  return launched(launch_act_quant(x, dt, m, k, ldx, xq, ldq, scales, stream));
}

sherry_status sherry_decode(const uint32_t* codes, int64_t n, int64_t k, int8_t* t, int64_t ldt,
                            hipStream_t stream) {
  if (!codes || !t) return SHERRY_EINVAL;
  if (sherry_status s = check_nk(n, k)) return s;
  if (ldt < k || ldt > std::numeric_limits<int64_t>::max() / n) return SHERRY_ESHAPE;
  if (!aligned(codes, 4) || !aligned(t, 16) || ldt % 16 != 0) return SHERRY_EALIGN;
  if (sherry_status s = check_device()) return s;
  return launched(launch_decode(codes, n, k, t, ldt, stream));
}

sherry_status sherry_gemv_quant(const uint32_t* codes, const void* w_scales, sherry_dtype s_dt, int64_t n, int64_t k,
                                const void* x, sherry_dtype x_dt, float* x_scale_out, int32_t* acc, void* y,
                                sherry_dtype y_dt, hipStream_t stream) {
  return gemv_quant_impl(kFmtSherry, codes, w_scales, raw(s_dt), n, k, x, raw(x_dt),
                         x_scale_out, acc, y, raw(y_dt), stream);
}

sherry_status sherry_gemv(const uint32_t* codes, const void* w_scales, sherry_dtype s_dt, int64_t n, int64_t k,
                          const void* x, sherry_dtype x_dt, const float* x_scale, int32_t* acc, void* y,
                          sherry_dtype y_dt, hipStream_t stream) {
  return gemv_impl(kFmtSherry, codes, w_scales, raw(s_dt), n, k, x, raw(x_dt), x_scale, acc, y, raw(y_dt), stream);
}

size_t sherry_gemv_plan_bytes(const sherry_gemv_problem* probs, int32_t count) {
  return plan_bytes_impl(probs, count, kFmtSherry);
}

sherry_status sherry_gemv_plan(const sherry_gemv_problem* probs, int32_t count, sherry_dtype s_dt,
                               sherry_dtype x_dt, sherry_dtype y_dt, void* plan, size_t plan_bytes) {
  return plan_impl(kFmtSherry, probs, count, raw(s_dt), raw(x_dt), raw(y_dt), plan, plan_bytes);
}

sherry_status sherry_gemv_plan_mfma(const sherry_gemv_problem* probs, int32_t count, sherry_dtype s_dt,
                                    sherry_dtype x_dt, sherry_dtype y_dt, void* plan, size_t plan_bytes) {
  return plan_impl(kFmtSherry, probs, count, raw(s_dt), raw(x_dt), raw(y_dt), plan, plan_bytes, true);
}

sherry_status sherry_gemv_grouped(const void* plan_host, const void* plan_dev, hipStream_t stream) {
  if (!plan_host || !plan_dev) return SHERRY_EINVAL;
  if (!aligned(plan_host, 8) || !aligned(plan_dev, 8)) return SHERRY_EALIGN;
  PlanHeader h;
  std::memcpy(&h, plan_host, sizeof(h));
  if (h.magic != kPlanMagic || h.version != kPlanVersion || h.count <= 0 || h.n_tiles < 0 ||
      (h.format != kFmtSherry && h.format != kFmtTern2 && h.format != kFmtTern3))
    return SHERRY_EINVAL;
  if (sherry_status s = check_device()) return s;
  return launched(launch_gemv_grouped(&h, plan_dev, stream));
}

sherry_status sherry_gemv_grouped_noalloc(const void* plan_host, hipStream_t stream) {
  if (!plan_host) return SHERRY_EINVAL;
  if (!aligned(plan_host, 8)) return SHERRY_EALIGN;
  PlanHeader h;
  std::memcpy(&h, plan_host, sizeof(h));
  if (h.magic != kPlanMagic || h.version != kPlanVersion || h.count <= 0 || h.n_tiles < 0 ||
      (h.format != kFmtSherry && h.format != kFmtTern2 && h.format != kFmtTern3))
    return SHERRY_EINVAL;
  // the records the kernel reads must lie inside the bytes that are copied
  const uint64_t used = sizeof(PlanHeader) + sizeof(GemvDesc) * static_cast<uint64_t>(h.count) +
                        sizeof(PlanTile) * static_cast<uint64_t>(h.n_tiles);
  if (h.bytes < used) return SHERRY_EINVAL;
  if (h.bytes > kNoAllocPlanBytes) return SHERRY_ESCRATCH;
  if (sherry_status s = check_device()) return s;
  return launched(launch_gemv_grouped_noalloc(&h, plan_host, stream));
}

size_t sherry_gemm_plan_bytes(const sherry_gemm_problem* probs, int32_t count) {
  return gemm_plan_bytes_impl(probs, count);
}

sherry_status sherry_gemm_plan(const sherry_gemm_problem* probs, int32_t count, sherry_dtype s_dt, sherry_dtype x_dt,
                               sherry_dtype y_dt, void* plan, size_t plan_bytes) {
  return gemm_plan_impl(kFmtSherry, probs, count, raw(s_dt), raw(x_dt), raw(y_dt), plan, plan_bytes);
}

sherry_status tern2_gemm_plan(const sherry_gemm_problem* probs, int32_t count, sherry_dtype s_dt, sherry_dtype x_dt,
                              sherry_dtype y_dt, void* plan, size_t plan_bytes) {
  return gemm_plan_impl(kFmtTern2, probs, count, raw(s_dt), raw(x_dt), raw(y_dt), plan, plan_bytes);
}

sherry_status sherry_gemm_grouped(const void* plan_host, const void* plan_dev, hipStream_t stream) {
  if (!plan_host || !plan_dev) return SHERRY_EINVAL;
  if (!aligned(plan_host, 8) || !aligned(plan_dev, 8)) return SHERRY_EALIGN;
  PlanHeader h;
  std::memcpy(&h, plan_host, sizeof(h));
  if (h.magic != kGemmPlanMagic || h.version != kPlanVersion || h.count <= 0 || h.n_tiles < 0 ||
      (h.format != kFmtSherry && h.format != kFmtTern2))
    return SHERRY_EINVAL;
  if (sherry_status s = check_device()) return s;
  return launched(launch_gemm_grouped(&h, plan_dev, stream));
}

sherry_status sherry_gemm(const uint32_t* codes, const void* w_scales, sherry_dtype s_dt, int64_t n, int64_t k,
                          const void* x, sherry_dtype x_dt, int64_t m, int64_t ldx, const float* x_scales,
                          int32_t* acc, void* y, sherry_dtype y_dt, int64_t ldy, hipStream_t stream) {
  return gemm_impl(kFmtSherry, codes, w_scales, raw(s_dt), n, k, x, raw(x_dt),
                   m, ldx, x_scales, acc, y, raw(y_dt), ldy, stream);
}

size_t tern2_packed_bytes(int64_t n, int64_t k) {
  if (check_nk(n, k) != SHERRY_OK) return 0;
  return static_cast<size_t>(n) * static_cast<size_t>(k) / 4;
}

sherry_status tern2_encode(const int8_t* t, int64_t n, int64_t k, int64_t ldt, uint32_t* codes, hipStream_t stream) {
  if (!t || !codes) return SHERRY_EINVAL;
  if (sherry_status s = check_nk(n, k)) return s;
  if (ldt < k || ldt > std::numeric_limits<int64_t>::max() / n) return SHERRY_ESHAPE;
  if (!aligned(t, 16) || ldt % 16 != 0 || !aligned(codes, 4)) return SHERRY_EALIGN;
  if (sherry_status s = check_device()) return s;
  return launched(launch_tern2_encode(t, n, k, ldt, codes, stream));
}

sherry_status tern2_gemv(const uint32_t* codes, const void* w_scales, sherry_dtype s_dt, int64_t n, int64_t k,
                         const void* x, sherry_dtype x_dt, const float* x_scale, int32_t* acc, void* y,
                         sherry_dtype y_dt, hipStream_t stream) {
  return gemv_impl(kFmtTern2, codes, w_scales, raw(s_dt), n, k, x, raw(x_dt), x_scale, acc, y, raw(y_dt), stream);
}

sherry_status tern2_gemv_plan(const sherry_gemv_problem* probs, int32_t count, sherry_dtype s_dt,
                              sherry_dtype x_dt, sherry_dtype y_dt, void* plan, size_t plan_bytes) {
  return plan_impl(kFmtTern2, probs, count, raw(s_dt), raw(x_dt), raw(y_dt), plan, plan_bytes);
}

size_t tern3_packed_bytes(int64_t n, int64_t k) {
  if (check_nk(n, k) != SHERRY_OK) return 0;
  return static_cast<size_t>(n) * static_cast<size_t>((k + 95) / 96) * 20;
}

sherry_status tern3_encode(const int8_t* t, int64_t n, int64_t k, int64_t ldt, uint32_t* codes, hipStream_t stream) {
  if (!t || !codes) return SHERRY_EINVAL;
  if (sherry_status s = check_nk(n, k)) return s;
  if (ldt < k || ldt > std::numeric_limits<int64_t>::max() / n) return SHERRY_ESHAPE;
  if (!aligned(t, 16) || ldt % 16 != 0 || !aligned(codes, 4)) return SHERRY_EALIGN;
  if (sherry_status s = check_device()) return s;
  return launched(launch_tern3_encode(t, n, k, ldt, codes, stream));
}

sherry_status tern3_gemv(const uint32_t* codes, const void* w_scales, sherry_dtype s_dt, int64_t n, int64_t k,
                         const void* x, sherry_dtype x_dt, const float* x_scale, int32_t* acc, void* y,
                         sherry_dtype y_dt, hipStream_t stream) {
  return gemv_impl(kFmtTern3, codes, w_scales, raw(s_dt), n, k, x, raw(x_dt), x_scale, acc, y, raw(y_dt), stream);
}

size_t tern3_gemv_plan_bytes(const sherry_gemv_problem* probs, int32_t count) {
  return plan_bytes_impl(probs, count, kFmtTern3);
}

sherry_status tern3_gemv_plan(const sherry_gemv_problem* probs, int32_t count, sherry_dtype s_dt,
                              sherry_dtype x_dt, sherry_dtype y_dt, void* plan, size_t plan_bytes) {
  return plan_impl(kFmtTern3, probs, count, raw(s_dt), raw(x_dt), raw(y_dt), plan, plan_bytes);
}

sherry_status tern2_gemm(const uint32_t* codes, const void* w_scales, sherry_dtype s_dt, int64_t n, int64_t k,
                         const void* x, sherry_dtype x_dt, int64_t m, int64_t ldx, const float* x_scales,
                         int32_t* acc, void* y, sherry_dtype y_dt, int64_t ldy, hipStream_t stream) {
  return gemm_impl(kFmtTern2, codes, w_scales, raw(s_dt), n, k, x, raw(x_dt),
                   m, ldx, x_scales, acc, y, raw(y_dt), ldy, stream);
}

}  // extern "C"
