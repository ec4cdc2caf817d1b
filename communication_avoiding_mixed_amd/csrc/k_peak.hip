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

typedef __attribute__((address_space(3))) void lds_void;

// Read-only streaming: workgroup w reads its slice of src with direct-to-LDS
// loads (no register results, so every wave keeps its loads in flight) into
// an 8 KB ring, then writes the first word of each ring slot it holds, so
// the data is checked and nothing is optimised away.
__global__ __launch_bounds__(kThreads) void peak_read_kernel(const u32x4_t* __restrict__ src, int64_t n16,
                                                             float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) u32x4_t ring[8][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t b1 = b0 + per < n16 ? b0 + per : n16;
  int k = 0;
  for (int64_t c0 = b0 + static_cast<int64_t>(wave) * 64; c0 < b1; c0 += 64 * (kThreads / 64), ++k)
    if (c0 + lane < b1)
      __builtin_amdgcn_global_load_lds(src + c0 + lane, (lds_void*)(&ring[(2 * wave + (k & 1)) & 7][0]), 16, 0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x < 8) out[static_cast<int64_t>(blockIdx.x) * 8 + threadIdx.x] = __uint_as_float(ring[threadIdx.x][0].x);
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

hipError_t launch_peak_read(const void* src, int64_t bytes, float* out, int workgroups, hipStream_t stream) {
  hipLaunchKernelGGL(peak_read_kernel, dim3(workgroups), dim3(kThreads), 0, stream,
                     static_cast<const u32x4_t*>(src), bytes / 16, out);
  return hipGetLastError();
}

hipError_t launch_peak_mfma(float* out, int workgroups, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(peak_mfma_kernel, dim3(workgroups), dim3(kThreads), 0, stream, iters, out);
  return hipGetLastError();
}

}  // namespace casgd
