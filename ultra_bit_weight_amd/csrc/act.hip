// Per-token absmax int8 quantization of activations: the int8 products
// take x as int8 with one fp32 scale per token.  (The Sherry paper,
// "Sherry: Hardware-Efficient 1.25-Bit Ternary Quantization via Fine-grained
// Sparsification", quantizes the weights; the activation rule is the
// symmetric absmax one.)
//
// One workgroup per token.  The absmax of the token's fp32 values (fp16 and
// bf16 convert exactly) comes from a max over the workgroup; the scale is
// absmax / 127 by one IEEE division (1 for an all-zero token), and every
// element is x / s by one IEEE division, rounded to an integer with ties to
// even (v_rndne_f32) and clipped to [-127, 127].
#include "launch.h"

namespace sherry {
namespace {

constexpr int kActThreads = 256;

template <int DT>
__device__ __forceinline__ float act_value(const void* x, int64_t i) {
  if constexpr (DT == kActF32) {
    return gmem(static_cast<const float*>(x))[i];
  } else if constexpr (DT == kActF16) {
    return static_cast<float>(gmem(static_cast<const _Float16*>(x))[i]);
  } else {
    return __uint_as_float(static_cast<uint32_t>(gmem(static_cast<const uint16_t*>(x))[i]) << 16);
  }
}

template <int DT>
__global__ __launch_bounds__(kActThreads) void act_quant_kernel(const void* x, int64_t k, int64_t ldx, int8_t* q,
                                                                int64_t ldq, float* scales) {
  __shared__ float wmax[kActThreads / kWave];
  const int64_t row = blockIdx.x;
  const int64_t base = row * ldx;
  float amax = 0.0f;
  for (int64_t j = threadIdx.x; j < k; j += kActThreads) amax = fmaxf(amax, fabsf(act_value<DT>(x, base + j)));
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((threadIdx.x & (kWave - 1)) == 0) wmax[threadIdx.x / kWave] = amax;
  __syncthreads();
  amax = wmax[0];
#pragma unroll
  for (int w = 1; w < kActThreads / kWave; ++w) amax = fmaxf(amax, wmax[w]);
  const float s = amax == 0.0f ? 1.0f : __fdiv_rn(amax, 127.0f);
  if (threadIdx.x == 0) gmem(scales)[row] = s;
  int8_t* out = q + row * ldq;
  for (int64_t j = threadIdx.x; j < k; j += kActThreads) {
    const float v = __builtin_rintf(__fdiv_rn(act_value<DT>(x, base + j), s));
    gmem(out)[j] = static_cast<int8_t>(static_cast<int>(fminf(fmaxf(v, -127.0f), 127.0f)));
  }
}

}  // namespace

hipError_t launch_act_quant(const void* x, int dt, int64_t m, int64_t k, int64_t ldx, int8_t* q, int64_t ldq,
                            float* scales, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(m));
  switch (dt) {
    case kActF32:
      hipLaunchKernelGGL((act_quant_kernel<kActF32>), grid, dim3(kActThreads), 0, stream, x, k, ldx, q, ldq, scales);
      break;
    case kActF16:
      hipLaunchKernelGGL((act_quant_kernel<kActF16>), grid, dim3(kActThreads), 0, stream, x, k, ldx, q, ldq, scales);
      break;
    default:
      hipLaunchKernelGGL((act_quant_kernel<kActBf16>), grid, dim3(kActThreads), 0, stream, x, k, ldx, q, ldq, scales);
      break;
  }
  return hipGetLastError();
}

}  // namespace sherry
