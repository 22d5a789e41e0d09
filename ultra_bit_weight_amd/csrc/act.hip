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
#include "actq.h"
#include "launch.h"

namespace sherry {
namespace {

template <int DT>
__global__ __launch_bounds__(kActThreads) void act_quant_kernel(const void* x, int64_t k, int64_t ldx, int8_t* q,
                                                                int64_t ldq, float* scales) {
  __shared__ float wmax[kActThreads / kWave];
  const int64_t row = blockIdx.x;
  const int64_t base = row * ldx;
  int8_t* out = q + row * ldq;
  if (k <= kActMaxRegK) {
    float v[kActRegs];
    const float s = act_scale(block_max(act_load_token(x, DT, base, k, v), wmax));
    if (threadIdx.x == 0) gmem(scales)[row] = s;
#pragma unroll
    for (int i = 0; i < kActRegs; ++i) {
      const int64_t j = threadIdx.x + static_cast<int64_t>(i) * kActThreads;
      if (j < k) gmem(out)[j] = act_code(v[i], s);
    }
    return;
  }
  float amax = 0.0f;
  for (int64_t j = threadIdx.x; j < k; j += kActThreads) amax = fmaxf(amax, fabsf(act_value(x, DT, base + j)));
  const float s = act_scale(block_max(amax, wmax));
  if (threadIdx.x == 0) gmem(scales)[row] = s;
  for (int64_t j = threadIdx.x; j < k; j += kActThreads) gmem(out)[j] = act_code(act_value(x, DT, base + j), s);
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
