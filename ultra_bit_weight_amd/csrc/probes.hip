// Measured ceilings beside the published peaks of the rooflines: a streaming
// read of a large buffer (HBM), the int8 matrix-core rate, the v_dot4 rate,
// and the two together -- in the same wave, or in alternate waves -- which
// shows whether matrix-core and VALU work overlap.
#include "launch.h"
#include "sherry_probes.h"

namespace sherry {
namespace {

typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kProbeThreads = 256;
constexpr uint32_t kNever = 0x9E3779B9u;  // a result no probe produces in practice: its store keeps the work
constexpr int kReadUnroll = 4;            // 16-byte loads in flight per thread
constexpr int kReadWgPerCu = 64;

// Each workgroup streams one contiguous chunk of the buffer.  (Grid-stride
// order, where neighbouring workgroups read neighbouring 4 KB at the same
// time, measured 13 % slower on MI355X: 6.0-6.3 against 7.1 TB/s.)
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4_t* src, int64_t n16, uint32_t* sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t len = lo + per < n16 ? per : (n16 > lo ? n16 - lo : 0);
  const u32x4_t* q = src + lo;
  uint32_t acc = 0;
  int64_t i = threadIdx.x;
  for (; i + (kReadUnroll - 1) * kProbeThreads < len; i += kReadUnroll * kProbeThreads) {
    u32x4_t v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(gmem(q + i + u * kProbeThreads));
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < len; i += kProbeThreads) {
    const u32x4_t v = __builtin_nontemporal_load(gmem(q + i));
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == kNever) gmem(sink)[threadIdx.x] = acc;
}

// Per iteration and wave: 4 independent v_mfma_i32_16x16x64_i8 (4 x 32768
// int8 ops) and/or 16 independent v_dot4_i32_i8 (16 x 512 ops); in the
// MFMA32 mode 2 independent v_mfma_i32_32x32x32_i8 (the same 2 x 65536 ops);
// in the ALU modes 16 independent chains of a shift, a mask and an add (48
// plain 32-bit VALU operations, the kind a table decode issues).
// With ticks: thread 0 of workgroup b records the shader-clock counter
// (s_memtime) and the constant 100 MHz counter (s_memrealtime) before and
// after its wave's loop in ticks[4 b .. 4 b + 3].
template <int MODE>
__global__ __launch_bounds__(kProbeThreads) void probe_rate_kernel(int iters, uint32_t* sink, uint64_t* ticks) {
  uint64_t t0 = 0, r0 = 0;
  if (ticks && threadIdx.x == 0) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const bool alt = MODE == SHERRY_PROBE_ALT_WAVES;
  const bool do_mfma = MODE == SHERRY_PROBE_MFMA || MODE == SHERRY_PROBE_SAME_WAVE || MODE == SHERRY_PROBE_SAME_ALU ||
                       (alt && (wave & 1) == 0);
  const bool do_valu = MODE == SHERRY_PROBE_DOT4 || MODE == SHERRY_PROBE_SAME_WAVE || (alt && (wave & 1) == 1);
  const bool do_alu = MODE == SHERRY_PROBE_ALU || MODE == SHERRY_PROBE_SAME_ALU;
  v4i a = {lane, 3 * lane + 1, 5 * lane + 2, 7 * lane + 3};
  v4i b = {lane ^ 5, lane ^ 9, lane ^ 17, lane ^ 33};
  asm volatile("" : "+v"(a), "+v"(b));
  v4i c[4];
  v16i c32[2] = {};
  int d[16];
#pragma unroll
  for (int r = 0; r < 4; ++r) c[r] = v4i{0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < 16; ++j) d[j] = j;
  for (int it = 0; it < iters; ++it) {
    if (MODE == SHERRY_PROBE_MFMA32) {
#pragma unroll
      for (int r = 0; r < 2; ++r) c32[r] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c32[r], 0, 0, 0);
    }
    if (do_mfma) {
#pragma unroll
      for (int r = 0; r < 4; ++r) c[r] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c[r], 0, 0, 0);
    }
    if (do_valu) {
#pragma unroll
      for (int j = 0; j < 16; ++j) d[j] = __builtin_amdgcn_sdot4(a[j & 3], b[(j + 1) & 3], d[j], false);
    }
    if (do_alu) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        d[j] = static_cast<int>(((static_cast<uint32_t>(d[j]) >> (j + 1)) & 0x7Cu) + static_cast<uint32_t>(a[j & 3]));
    }
  }
  uint32_t h = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) h ^= static_cast<uint32_t>(c[r][0] ^ c[r][1] ^ c[r][2] ^ c[r][3]);
#pragma unroll
  for (int j = 0; j < 16; ++j) h ^= static_cast<uint32_t>(d[j]);
#pragma unroll
  for (int r = 0; r < 2; ++r) h ^= static_cast<uint32_t>(c32[r][0] ^ c32[r][15]);
  if (h == kNever) gmem(sink)[threadIdx.x] = h;
  if (ticks && threadIdx.x == 0) {
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    SHERRY_GLOBAL uint64_t* out = gmem(ticks) + 4 * static_cast<int64_t>(blockIdx.x);
    out[0] = t0;
    out[1] = t1;
    out[2] = r0;
    out[3] = r1;
  }
}

sherry_status launch_rates(int32_t mode, int32_t iters, int32_t blocks, uint32_t* sink, uint64_t* ticks,
                           hipStream_t stream) {
  if (!sink) return SHERRY_EINVAL;
  if (mode < SHERRY_PROBE_MFMA || mode > SHERRY_PROBE_SAME_ALU || iters <= 0 || iters > (1 << 24) || blocks <= 0 ||
      blocks > (1 << 20))
    return SHERRY_EINVAL;
  if (reinterpret_cast<uintptr_t>(sink) % 4 != 0 || reinterpret_cast<uintptr_t>(ticks) % 8 != 0) return SHERRY_EALIGN;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SHERRY_EDEVICE;
  const dim3 grid(static_cast<unsigned>(blocks)), block(kProbeThreads);
  switch (mode) {
    case SHERRY_PROBE_MFMA:
      hipLaunchKernelGGL(probe_rate_kernel<SHERRY_PROBE_MFMA>, grid, block, 0, stream, iters, sink, ticks);
      break;
    case SHERRY_PROBE_DOT4:
      hipLaunchKernelGGL(probe_rate_kernel<SHERRY_PROBE_DOT4>, grid, block, 0, stream, iters, sink, ticks);
      break;
    case SHERRY_PROBE_SAME_WAVE:
      hipLaunchKernelGGL(probe_rate_kernel<SHERRY_PROBE_SAME_WAVE>, grid, block, 0, stream, iters, sink, ticks);
      break;
    case SHERRY_PROBE_ALT_WAVES:
      hipLaunchKernelGGL(probe_rate_kernel<SHERRY_PROBE_ALT_WAVES>, grid, block, 0, stream, iters, sink, ticks);
      break;
    case SHERRY_PROBE_MFMA32:
      hipLaunchKernelGGL(probe_rate_kernel<SHERRY_PROBE_MFMA32>, grid, block, 0, stream, iters, sink, ticks);
      break;
    case SHERRY_PROBE_ALU:
      hipLaunchKernelGGL(probe_rate_kernel<SHERRY_PROBE_ALU>, grid, block, 0, stream, iters, sink, ticks);
      break;
    default:
      hipLaunchKernelGGL(probe_rate_kernel<SHERRY_PROBE_SAME_ALU>, grid, block, 0, stream, iters, sink, ticks);
      break;
  }
  return hipGetLastError() == hipSuccess ? SHERRY_OK : SHERRY_ELAUNCH;
}

}  // namespace
}  // namespace sherry

using namespace sherry;

extern "C" {

sherry_status sherry_probe_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!src || !sink || bytes == 0) return SHERRY_EINVAL;
  if (bytes % 16 != 0 || bytes / 16 > static_cast<size_t>(INT64_MAX / 4)) return SHERRY_ESHAPE;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 4 != 0) return SHERRY_EALIGN;
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) return SHERRY_EDEVICE;
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  // kReadWgPerCu workgroups per CU, each thread at least kReadUnroll loads when the buffer allows
  const int64_t want = (n16 + kReadUnroll * kProbeThreads - 1) / (kReadUnroll * kProbeThreads);
  const int64_t cap = static_cast<int64_t>(kReadWgPerCu) * prop.multiProcessorCount;
  const unsigned grid = static_cast<unsigned>(want < cap ? want : cap);
  hipLaunchKernelGGL(probe_read_kernel, dim3(grid), dim3(kProbeThreads), 0, stream,
                     static_cast<const u32x4_t*>(src), n16, sink);
  return hipGetLastError() == hipSuccess ? SHERRY_OK : SHERRY_ELAUNCH;
}

sherry_status sherry_probe_rates(int32_t mode, int32_t iters, int32_t blocks, uint32_t* sink, hipStream_t stream) {
  return launch_rates(mode, iters, blocks, sink, nullptr, stream);
}

sherry_status sherry_probe_clock(int32_t mode, int32_t iters, int32_t blocks, uint32_t* sink, uint64_t* ticks,
                                 hipStream_t stream) {
  if (!ticks) return SHERRY_EINVAL;
  return launch_rates(mode, iters, blocks, sink, ticks, stream);
}

}  // extern "C"
