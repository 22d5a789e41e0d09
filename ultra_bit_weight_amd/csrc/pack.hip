// Packer: real weights -> 5-bit 3:4 ternary codes + one scale per row
// ("Sherry: Hardware-Efficient 1.25-Bit Ternary Quantization via Fine-grained
// Sparsification", Abstract: ternary {-1, 0, +1} weights with 3:4
// fine-grained sparsity, four weights packed in five bits).
//
// Per block of four: the zero goes to the slot with the smallest |w| (lowest
// slot on ties), the other three keep their signs (w < 0 -> -1).  This is the
// least-squares projection for any positive scale.  Per row the scale is the
// least-squares value for the chosen pattern, (sum of kept |w|) / (3k/4); the
// sum runs in double-double so the rounded fp64 result is the correctly
// rounded exact sum, then one fp64 division and one RNE rounding to the scale
// type.
//
// One workgroup per row; a half-wave (32 lanes) owns one 128-weight group,
// lane j encodes block j and the group's five words are assembled with an
// OR-butterfly across the half-wave.  The same decisions can instead be
// stored as 2-bit fields (the dense-ternary comparator: 00 = 0, 01 = +1,
// 11 = -1, weight 4q + p of each 16-weight word at bits 8p + 2q), so both
// formats hold one matrix with the same scales.
#include "launch.h"

namespace sherry {
namespace {

struct DD {
  double hi, lo;
};

__device__ __forceinline__ DD two_sum(double a, double b) {
  const double s = a + b;
  const double bb = s - a;
  const double e = (a - (s - bb)) + (b - bb);
  return {s, e};
}

__device__ __forceinline__ DD dd_add(DD a, DD b) {
  DD s = two_sum(a.hi, b.hi);
  const double e = s.lo + (a.lo + b.lo);
  const double h = s.hi + e;
  return {h, e - (h - s.hi)};
}

__device__ __forceinline__ DD dd_shfl_xor(DD v, int m) {
  return {__shfl_xor(v.hi, m), __shfl_xor(v.lo, m)};
}

// Round a finite non-negative double to the nearest fp16 (ties to even),
// directly from its bits (one rounding).
__device__ __forceinline__ uint16_t f64_to_f16_rne(double x) {
  const uint64_t b = __double_as_longlong(x);
  const uint32_t sign = static_cast<uint32_t>(b >> 63) << 15;
  const int e = static_cast<int>((b >> 52) & 0x7FF) - 1023;
  uint64_t m = b & ((1ull << 52) - 1);
  if (((b >> 52) & 0x7FF) == 0x7FF) return static_cast<uint16_t>(sign | 0x7C00 | (m ? 0x200 : 0));
  if (((b >> 52) & 0x7FF) == 0) return static_cast<uint16_t>(sign);  // fp64 subnormal: far below fp16
  m |= 1ull << 52;                                                    // 53-bit significand
  if (e > 15) return static_cast<uint16_t>(sign | 0x7C00);           // overflow
  int shift;  // bits of m dropped to reach the fp16 significand
  uint32_t base;
  if (e >= -14) {
    shift = 42;  // keep 11 bits (hidden + 10)
    base = static_cast<uint32_t>(e + 14) << 10;
  } else {
    shift = 42 + (-14 - e);  // subnormal fp16
    base = 0;
    if (shift > 54) return static_cast<uint16_t>(sign);
  }
  const uint64_t q = m >> shift;
  const uint64_t rem = m & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  uint64_t r = q + ((rem > half || (rem == half && (q & 1))) ? 1 : 0);
  // base + r: the hidden bit of r carries into the exponent field naturally
  // (r in [1024, 2048] for normals, a carry to 2048 bumps the exponent).
  const uint32_t h = base + static_cast<uint32_t>(r);
  if (h >= 0x7C00) return static_cast<uint16_t>(sign | 0x7C00);
  return static_cast<uint16_t>(sign | h);
}

__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4(const _Float16* p) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  const _Float16* h = reinterpret_cast<const _Float16*>(&v);
  return make_float4(static_cast<float>(h[0]), static_cast<float>(h[1]), static_cast<float>(h[2]),
                     static_cast<float>(h[3]));
}
__device__ __forceinline__ float4 load4_bf16(const uint16_t* p) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u), __uint_as_float(v.y << 16),
                     __uint_as_float(v.y & 0xFFFF0000u));
}

template <typename T>
__device__ __forceinline__ float4 load_block(const T* p) {
  if constexpr (__is_same(T, uint16_t))
    return load4_bf16(p);
  else
    return load4(p);
}

template <typename T, bool TERN2>
__global__ __launch_bounds__(256) void pack_kernel(const T* w, int64_t ldw, int k, uint32_t* codes, void* scales,
                                                   int s_f16) {
  __shared__ double red_hi[4], red_lo[4];
  const int r = blockIdx.x;
  const T* row = w + static_cast<int64_t>(r) * ldw;
  const int G = k / kGroupWeights;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int j = lane & 31;  // block inside the group
  DD sum = {0.0, 0.0};
  for (int g = wave * 2 + (lane >> 5); g < G; g += 8) {
    const float4 v = load_block(row + g * kGroupWeights + 4 * j);
    const float val[4] = {v.x, v.y, v.z, v.w};
    float mag[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) mag[s] = fabsf(val[s]);
    int z = 0;
    float mz = mag[0];
#pragma unroll
    for (int s = 1; s < 4; ++s)
      if (mag[s] < mz) {
        z = s;
        mz = mag[s];
      }
    uint32_t code = static_cast<uint32_t>(z);
    int sb = 2;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s == z) continue;
      if (val[s] < 0.0f) code |= 1u << sb;
      sum = dd_add(sum, DD{static_cast<double>(mag[s]), 0.0});
      ++sb;
    }
    if constexpr (TERN2) {
      // block j = weights 4j .. 4j + 3 of the group: word j / 4 of the
      // group's eight, weight 4 (j % 4) + p of it at bits 8p + 2 (j % 4)
      uint32_t f = 0;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if (s != z) f |= (val[s] < 0.0f ? 3u : 1u) << (8 * s + 2 * (j & 3));
      f |= __shfl_xor(f, 1);
      f |= __shfl_xor(f, 2);
      if ((j & 3) == 0) codes[static_cast<int64_t>(r) * (k / 16) + 8 * g + (j >> 2)] = f;
      continue;
    }
    // contributions of code j to the group's five words
    const int bit = 5 * j;
    const int wi = bit >> 5;
    const int sh = bit & 31;
    const uint32_t lo = code << sh;
    const uint32_t hi = sh > 27 ? code >> (32 - sh) : 0u;
    uint32_t word[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) word[i] = (i == wi ? lo : 0u) | (i == wi + 1 ? hi : 0u);
#pragma unroll
    for (int m = 1; m < 32; m <<= 1)
#pragma unroll
      for (int i = 0; i < 5; ++i) word[i] |= __shfl_xor(word[i], m);
    uint32_t out = word[0];
    out = j == 1 ? word[1] : out;
    out = j == 2 ? word[2] : out;
    out = j == 3 ? word[3] : out;
    out = j == 4 ? word[4] : out;
    // row layout: words 0-3 of group g at 4g, word 4 at 4G + g
    uint32_t* rowc = codes + static_cast<int64_t>(r) * G * kGroupWords;
    if (j < 4) rowc[4 * g + j] = out;
    if (j == 4) rowc[4 * G + g] = out;
  }
  // row sum of kept magnitudes: wave butterfly, then across the 4 waves
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) sum = dd_add(sum, dd_shfl_xor(sum, m));
  if (lane == 0) {
    red_hi[wave] = sum.hi;
    red_lo[wave] = sum.lo;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    DD t = {red_hi[0], red_lo[0]};
    for (int i = 1; i < 4; ++i) t = dd_add(t, DD{red_hi[i], red_lo[i]});
    const double kept = static_cast<double>(3 * (k / 4));
    const double alpha = t.hi / kept;
    if (s_f16)
      reinterpret_cast<uint16_t*>(scales)[r] = f64_to_f16_rne(alpha);
    else
      reinterpret_cast<float*>(scales)[r] = static_cast<float>(alpha);
  }
}

// Decode: one thread per 128-weight group; the five words are expanded
// through the same per-block rule as the GEMV table and written as 8 x 16 B.
__global__ __launch_bounds__(256) void decode_kernel(const uint32_t* codes, int64_t n, int G, int8_t* t,
                                                     int64_t ldt) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= n * G) return;
  const int64_t r = idx / G;
  const int g = static_cast<int>(idx % G);
  uint32_t w[kGroupWords];
  load_group(w, codes + r * G * kGroupWords, G, g);
  uint4* out = reinterpret_cast<uint4*>(t + r * ldt + static_cast<int64_t>(g) * kGroupWeights);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    uint32_t v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = decode_i8x4(code_offset<0>(w, 4 * q + e));
    out[q] = make_uint4(v[0], v[1], v[2], v[3]);
  }
}

}  // namespace

hipError_t launch_decode(const uint32_t* codes, int64_t n, int64_t k, int8_t* t, int64_t ldt, hipStream_t stream) {
  const int G = static_cast<int>(k / kGroupWeights);
  const int64_t groups = n * G;
  const unsigned grid = static_cast<unsigned>((groups + 255) / 256);
  hipLaunchKernelGGL(decode_kernel, dim3(grid), dim3(256), 0, stream, codes, n, G, t, ldt);
  return hipGetLastError();
}

template <bool TERN2>
void launch_pack_fmt(const void* w, int w_dt, int64_t n, int64_t k, int64_t ldw, uint32_t* codes, void* scales,
                     bool s_f16, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(n)), block(256);
  const int kk = static_cast<int>(k);
  switch (w_dt) {
    case SHERRY_F32:
      hipLaunchKernelGGL((pack_kernel<float, TERN2>), grid, block, 0, stream, static_cast<const float*>(w), ldw, kk, codes,
                         scales, s_f16 ? 1 : 0);
      break;
    case SHERRY_F16:
      hipLaunchKernelGGL((pack_kernel<_Float16, TERN2>), grid, block, 0, stream, static_cast<const _Float16*>(w), ldw, kk,
                         codes, scales, s_f16 ? 1 : 0);
      break;
    default:
      hipLaunchKernelGGL((pack_kernel<uint16_t, TERN2>), grid, block, 0, stream, static_cast<const uint16_t*>(w), ldw, kk,
                         codes, scales, s_f16 ? 1 : 0);
      break;
  }
}

hipError_t launch_pack(const void* w, int w_dt, int64_t n, int64_t k, int64_t ldw, uint32_t* codes, void* scales,
                       bool s_f16, bool tern2, hipStream_t stream) {
  if (tern2)
    launch_pack_fmt<true>(w, w_dt, n, k, ldw, codes, scales, s_f16, stream);
  else
    launch_pack_fmt<false>(w, w_dt, n, k, ldw, codes, scales, s_f16, stream);
  return hipGetLastError();
}

}  // namespace sherry
