// Calibration kernels for roofline reporting, not part of the method: a plain
// device copy (the achievable HBM rate, and the known traffic that scales the
// HBM byte counters) and a loop of bf16 MFMAs on independent accumulator
// chains (the achievable matrix-core rate under sustained load).
#include "casgd_internal.h"

namespace casgd {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kChains = 4;  // independent accumulators per wave

// 16-byte words, grid-stride, four loads in flight per thread before the
// stores, all marked nontemporal (streamed data: no reuse to cache).  On
// MI355X this form on 64 workgroups per CU measured fastest among grid sizes
// of 8 to 64 per CU, 2 to 8 loads in flight and contiguous per-workgroup
// spans, and above hipMemcpy's device-to-device copy.
__global__ __launch_bounds__(kThreads) void peak_copy_kernel(const u32x4_t* __restrict__ src,
                                                             u32x4_t* __restrict__ dst, int64_t n16) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4_t a = __builtin_nontemporal_load(&src[i]);
    const u32x4_t b = __builtin_nontemporal_load(&src[i + stride]);
    const u32x4_t c = __builtin_nontemporal_load(&src[i + 2 * stride]);
    const u32x4_t d = __builtin_nontemporal_load(&src[i + 3 * stride]);
    __builtin_nontemporal_store(a, &dst[i]);
    __builtin_nontemporal_store(b, &dst[i + stride]);
    __builtin_nontemporal_store(c, &dst[i + 2 * stride]);
    __builtin_nontemporal_store(d, &dst[i + 3 * stride]);
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

// iters x kChains dependent v_mfma_f32_32x32x16_bf16 per wave; each lane
// writes the sum of its accumulators so that nothing is optimised away
__global__ __launch_bounds__(kThreads) void peak_mfma_kernel(int iters, float* __restrict__ out) {
  bf16x8_t a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(static_cast<float>((threadIdx.x + e) & 7) * 0.125f);
    b[e] = static_cast<__bf16>(static_cast<float>((threadIdx.x * 3 + e) & 7) * 0.0625f);
  }
  f32x16_t c[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) c[k] = f32x16_t{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < kChains; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
  }
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < kChains; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) sum += c[k][e];
  out[static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x] = sum;
}

}  // namespace

hipError_t launch_peak_copy(const void* src, void* dst, int64_t bytes, int cus, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  if (n16 <= 0) return hipSuccess;
  int64_t grid = static_cast<int64_t>(cus) * 64;
  const int64_t need = (n16 + kThreads - 1) / kThreads;
  if (grid > need) grid = need;
  hipLaunchKernelGGL(peak_copy_kernel, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, stream,
                     static_cast<const u32x4_t*>(src), static_cast<u32x4_t*>(dst), n16);
  return hipGetLastError();
}

hipError_t launch_peak_mfma(float* out, int workgroups, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(peak_mfma_kernel, dim3(workgroups), dim3(kThreads), 0, stream, iters, out);
  return hipGetLastError();
}

}  // namespace casgd
