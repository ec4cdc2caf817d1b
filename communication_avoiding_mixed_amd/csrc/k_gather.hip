// Storage conversion (at create) and the per-step sample + gather kernel.
// The data matrix is kept in low precision, as the Abstract of "Mixed-
// Precision Communication-Avoiding SGD for Generalized Linear Models on GPUs"
// prescribes; rows are padded to ld (a multiple of 32 elements) so every row
// is a whole number of 16-byte chunks.
#include "casgd_device.h"
#include "casgd_gather.h"
#include "casgd_internal.h"

namespace casgd {
namespace {

// ---------------------------------------------------------------------------
// X (float32, m x n) -> Xs (m x ld).  One thread per 16-byte output chunk
// (8 elements), kSU chunks per thread per pass with every load issued before
// the first conversion.  VEC (n a multiple of 4, so every row starts on a
// 16-byte boundary): two 16-byte loads per chunk; the second half of a chunk
// that ends past n reads the chunk's first half again and is zeroed.
// Otherwise element loads with clamped addresses.
// ---------------------------------------------------------------------------
constexpr int kSU = 4;

template <bool VEC>
__global__ __launch_bounds__(256) void store_bf16_kernel(const float* __restrict__ X,
                                                         uint16_t* __restrict__ Xs, int64_t m,
                                                         int64_t n, int64_t ld) {
  const int64_t cpr = ld / 8;  // chunks per row
  const int64_t total = m * cpr;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t g0 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g0 < total;
       g0 += stride * kSU) {
    float v[kSU][8];
#pragma unroll
    for (int u = 0; u < kSU; ++u) {
      const int64_t g = g0 + stride * u < total ? g0 + stride * u : g0;
      const int64_t row = g / cpr;
      const int64_t c0 = (g - row * cpr) * 8;
      const float* src = X + row * n;
      if constexpr (VEC) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(src + (c0 < n ? c0 : 0));
        const f32x4 b = *reinterpret_cast<const f32x4*>(src + (c0 + 4 < n ? c0 + 4 : 0));
        v[u][0] = a.x; v[u][1] = a.y; v[u][2] = a.z; v[u][3] = a.w;
        v[u][4] = b.x; v[u][5] = b.y; v[u][6] = b.z; v[u][7] = b.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[u][e] = src[c0 + e < n ? c0 + e : n - 1];
      }
    }
#pragma unroll
    for (int u = 0; u < kSU; ++u) {
      const int64_t g = g0 + stride * u;
      if (g >= total) break;
      const int64_t row = g / cpr;
      const int64_t c0 = (g - row * cpr) * 8;
      uint32_t packed[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = c0 + 2 * e < n ? f32_to_bf16(v[u][2 * e]) : 0u;
        const uint32_t hi = c0 + 2 * e + 1 < n ? f32_to_bf16(v[u][2 * e + 1]) : 0u;
        packed[e] = lo | (hi << 16);
      }
      *reinterpret_cast<u32x4*>(Xs + row * ld + c0) = u32x4{packed[0], packed[1], packed[2], packed[3]};
    }
  }
}

__global__ __launch_bounds__(256) void store_f32_kernel(const float* __restrict__ X,
                                                        float* __restrict__ Xs, int64_t m,
                                                        int64_t n, int64_t ld) {
  const int64_t cpr = ld / 4;
  const int64_t total = m * cpr;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g < total;
       g += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t row = g / cpr;
    const int64_t c0 = (g - row * cpr) * 4;
    const float* src = X + row * n;
    float4 o;
    o.x = c0 < n ? src[c0] : 0.f;
    o.y = c0 + 1 < n ? src[c0 + 1] : 0.f;
    o.z = c0 + 2 < n ? src[c0 + 2] : 0.f;
    o.w = c0 + 3 < n ? src[c0 + 3] : 0.f;
    *reinterpret_cast<float4*>(Xs + row * ld + c0) = o;
  }
}

// Sample + gather: one workgroup of 256 lanes copies 256/GS rows (the row
// copy itself is in casgd_gather.h).
template <int GS>
__global__ __launch_bounds__(256) void gather_kernel(
    const u32x4* __restrict__ Xs, const float* __restrict__ y, int64_t m, int64_t cpr, int sb,
    uint64_t seed, const int32_t* __restrict__ idx_in, int32_t* __restrict__ idx_out,
    u32x4* __restrict__ Y, float* __restrict__ yB) {
  const int row = blockIdx.x * (256 / GS) + threadIdx.x / GS;
  gather::copy_row<GS>(Xs, y, m, cpr, sb, seed, idx_in, idx_out, Y, yB, row, threadIdx.x % GS);
}

template <int GS>
hipError_t gather_t(const void* Xs, const float* y, int64_t m, int64_t cpr, int sb, uint64_t seed,
                    const int32_t* idx_in, int32_t* idx_out, void* Y, float* yB, hipStream_t st,
                    const LaunchTimer& tm) {
  const int rows_per_block = 256 / GS;
  const int grid = (sb + rows_per_block - 1) / rows_per_block;
  return launch_kernel(gather_kernel<GS>, dim3(grid), dim3(256), 0, st, tm,
                       static_cast<const u32x4*>(Xs), y, m, cpr, sb, seed, idx_in, idx_out,
                       static_cast<u32x4*>(Y), yB);
}

}  // namespace

hipError_t launch_store(int storage, const float* X, void* Xs, int64_t m, int64_t n, int64_t ld,
                        hipStream_t st) {
  const int64_t chunks = m * (ld / (storage == kStoreBF16 ? 8 : 4));
  const int64_t want = (chunks + 256 * kSU - 1) / (256 * kSU);
  const int grid = static_cast<int>(want < (1 << 20) ? (want > 0 ? want : 1) : (1 << 20));
  if (storage == kStoreBF16) {
    if (n % 4 == 0 && (reinterpret_cast<uintptr_t>(X) & 15) == 0)
      store_bf16_kernel<true><<<grid, 256, 0, st>>>(X, static_cast<uint16_t*>(Xs), m, n, ld);
    else
      store_bf16_kernel<false><<<grid, 256, 0, st>>>(X, static_cast<uint16_t*>(Xs), m, n, ld);
  }
  else
    store_f32_kernel<<<grid, 256, 0, st>>>(X, static_cast<float*>(Xs), m, n, ld);
  return hipGetLastError();
}

hipError_t launch_gather(int storage, const void* Xs, const float* y, int64_t m, int64_t ld,
                         int sb, uint64_t seed, const int32_t* idx_in, int32_t* idx_out, void* Y,
                         float* yB, hipStream_t st, const LaunchTimer& tm) {
  const int64_t cpr = ld / (storage == kStoreBF16 ? 8 : 4);  // 16-byte chunks per row
  if (cpr >= 64) return gather_t<64>(Xs, y, m, cpr, sb, seed, idx_in, idx_out, Y, yB, st, tm);
  if (cpr >= 32) return gather_t<32>(Xs, y, m, cpr, sb, seed, idx_in, idx_out, Y, yB, st, tm);
  if (cpr >= 16) return gather_t<16>(Xs, y, m, cpr, sb, seed, idx_in, idx_out, Y, yB, st, tm);
  if (cpr >= 8) return gather_t<8>(Xs, y, m, cpr, sb, seed, idx_in, idx_out, Y, yB, st, tm);
  return gather_t<4>(Xs, y, m, cpr, sb, seed, idx_in, idx_out, Y, yB, st, tm);
}

}  // namespace casgd
