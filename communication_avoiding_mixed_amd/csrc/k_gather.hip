// Storage conversion (at create) and the per-step sample + gather kernel.
// The data matrix is kept in low precision, as the Abstract of "Mixed-
// Precision Communication-Avoiding SGD for Generalized Linear Models on GPUs"
// prescribes; rows are padded to ld (a multiple of 32 elements) so every row
// is a whole number of 16-byte chunks.
#include <cmath>

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

// Low-precision element formats of a stored row: E elements per 16-byte chunk.
template <int FMT>
struct Lp;
template <>
struct Lp<kStoreBF16> {
  static constexpr int E = 8;
  __device__ static uint32_t conv(float v, float) { return f32_to_bf16(v); }
};
template <>
struct Lp<kStoreF16> {
  static constexpr int E = 8;
  __device__ static uint32_t conv(float v, float) { return f32_to_f16(v); }
};
template <>
struct Lp<kStoreF8> {
  static constexpr int E = 16;
  // scaled by the matrix's power of two first (exact: no result leaves the
  // float32 normal range except below E4M3's rounding-to-zero threshold)
  __device__ static uint32_t conv(float v, float scale) { return f32_to_e4m3(v * scale); }
};

template <int FMT, bool VEC>
__global__ __launch_bounds__(256) void store_lp_kernel(const float* __restrict__ X,
                                                       uint8_t* __restrict__ Xs, int64_t m,
                                                       int64_t n, int64_t ld, float scale) {
  constexpr int E = Lp<FMT>::E;
  constexpr int BYTES = 16 / E;  // bytes per element
  const int64_t cpr = ld / E;    // chunks per row
  const int64_t total = m * cpr;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t g0 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g0 < total;
       g0 += stride * kSU) {
    float v[kSU][E];
#pragma unroll
    for (int u = 0; u < kSU; ++u) {
      const int64_t g = g0 + stride * u < total ? g0 + stride * u : g0;
      const int64_t row = g / cpr;
      const int64_t c0 = (g - row * cpr) * E;
      const float* src = X + row * n;
      if constexpr (VEC) {
        // a quarter chunk that starts at or past n reads the row's first
        // floats again; those elements are zeroed below
#pragma unroll
        for (int h = 0; h < E / 4; ++h) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(src + (c0 + 4 * h < n ? c0 + 4 * h : 0));
          v[u][4 * h] = a.x; v[u][4 * h + 1] = a.y; v[u][4 * h + 2] = a.z; v[u][4 * h + 3] = a.w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) v[u][e] = src[c0 + e < n ? c0 + e : n - 1];
      }
    }
#pragma unroll
    for (int u = 0; u < kSU; ++u) {
      const int64_t g = g0 + stride * u;
      if (g >= total) break;
      const int64_t row = g / cpr;
      const int64_t c0 = (g - row * cpr) * E;
      uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint32_t bits = c0 + e < n ? Lp<FMT>::conv(v[u][e], scale) : 0u;
        packed[(e * BYTES) / 4] |= bits << (8 * ((e * BYTES) % 4));
      }
      *reinterpret_cast<u32x4*>(Xs + (row * ld + c0) * BYTES) = u32x4{packed[0], packed[1], packed[2], packed[3]};
    }
  }
}

// Largest |x| of X as a float32 bit pattern (bit patterns of magnitudes order
// like the magnitudes; a NaN sorts above every finite value and infinity):
// per-workgroup maxima into partial[], then one workgroup reduces them.
__global__ __launch_bounds__(256) void maxabs_kernel(const float* __restrict__ X, int64_t count,
                                                     uint32_t* __restrict__ partial) {
  __shared__ uint32_t red[256];
  uint32_t mx = 0u;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < count;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const uint32_t a = __float_as_uint(X[i]) & 0x7FFFFFFFu;
    mx = a > mx ? a : mx;
  }
  red[threadIdx.x] = mx;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] = red[threadIdx.x + o] > red[threadIdx.x] ? red[threadIdx.x + o] : red[threadIdx.x];
    __syncthreads();
  }
  if (threadIdx.x == 0) partial[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(256) void maxabs_finish_kernel(const uint32_t* __restrict__ partial, int np,
                                                            uint32_t* __restrict__ out) {
  __shared__ uint32_t red[256];
  uint32_t mx = 0u;
  for (int i = threadIdx.x; i < np; i += 256) mx = partial[i] > mx ? partial[i] : mx;
  red[threadIdx.x] = mx;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] = red[threadIdx.x + o] > red[threadIdx.x] ? red[threadIdx.x + o] : red[threadIdx.x];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = red[0];
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

// Sample + gather of fp8 rows, widened to bf16 (gather::copy_row_f8).
template <int GS>
__global__ __launch_bounds__(256) void gather_f8_kernel(
    const u32x4* __restrict__ Xs, const float* __restrict__ y, int64_t m, int64_t cpr8, int sb,
    uint64_t seed, const int32_t* __restrict__ idx_in, int32_t* __restrict__ idx_out,
    u32x4* __restrict__ Y, float* __restrict__ yB, float unscale) {
  const int row = blockIdx.x * (256 / GS) + threadIdx.x / GS;
  gather::copy_row_f8<GS>(Xs, y, m, cpr8, sb, seed, idx_in, idx_out, Y, yB, unscale, row, threadIdx.x % GS);
}

template <int GS>
hipError_t gather_f8_t(const void* Xs, const float* y, int64_t m, int64_t cpr8, int sb, uint64_t seed,
                       const int32_t* idx_in, int32_t* idx_out, void* Y, float* yB, float unscale,
                       hipStream_t st, const LaunchTimer& tm) {
  const int rows_per_block = 256 / GS;
  const int grid = (sb + rows_per_block - 1) / rows_per_block;
  return launch_kernel(gather_f8_kernel<GS>, dim3(grid), dim3(256), 0, st, tm,
                       static_cast<const u32x4*>(Xs), y, m, cpr8, sb, seed, idx_in, idx_out,
                       static_cast<u32x4*>(Y), yB, unscale);
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
                        int fp8_exp, hipStream_t st) {
  const int E = storage == kStoreF32 ? 4 : storage == kStoreF8 ? 16 : 8;
  const int64_t chunks = m * (ld / E);
  const int64_t want = (chunks + 256 * kSU - 1) / (256 * kSU);
  const int grid = static_cast<int>(want < (1 << 20) ? (want > 0 ? want : 1) : (1 << 20));
  const bool vec = n % 4 == 0 && (reinterpret_cast<uintptr_t>(X) & 15) == 0;
  uint8_t* out = static_cast<uint8_t*>(Xs);
  const float scale = std::ldexp(1.0f, fp8_exp);
  switch (storage) {
    case kStoreBF16:
      if (vec) store_lp_kernel<kStoreBF16, true><<<grid, 256, 0, st>>>(X, out, m, n, ld, 1.f);
      else store_lp_kernel<kStoreBF16, false><<<grid, 256, 0, st>>>(X, out, m, n, ld, 1.f);
      break;
    case kStoreF16:
      if (vec) store_lp_kernel<kStoreF16, true><<<grid, 256, 0, st>>>(X, out, m, n, ld, 1.f);
      else store_lp_kernel<kStoreF16, false><<<grid, 256, 0, st>>>(X, out, m, n, ld, 1.f);
      break;
    case kStoreF8:
      if (vec) store_lp_kernel<kStoreF8, true><<<grid, 256, 0, st>>>(X, out, m, n, ld, scale);
      else store_lp_kernel<kStoreF8, false><<<grid, 256, 0, st>>>(X, out, m, n, ld, scale);
      break;
    default:
      store_f32_kernel<<<grid, 256, 0, st>>>(X, static_cast<float*>(Xs), m, n, ld);
  }
  return hipGetLastError();
}

hipError_t launch_maxabs(const float* X, int64_t count, uint32_t* partial, uint32_t* out_dev, hipStream_t st) {
  const int64_t want = (count + 256 * 16 - 1) / (256 * 16);
  const int grid = static_cast<int>(want < kMaxAbsBlocks ? (want > 0 ? want : 1) : kMaxAbsBlocks);
  maxabs_kernel<<<grid, 256, 0, st>>>(X, count, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  maxabs_finish_kernel<<<1, 256, 0, st>>>(partial, grid, out_dev);
  return hipGetLastError();
}

hipError_t launch_gather(int storage, const void* Xs, const float* y, int64_t m, int64_t ld,
                         int sb, uint64_t seed, const int32_t* idx_in, int32_t* idx_out, void* Y,
                         float* yB, int fp8_exp, hipStream_t st, const LaunchTimer& tm) {
  if (storage == kStoreF8) {
    const int64_t cpr8 = ld / 16;
    const float unscale = std::ldexp(1.0f, -fp8_exp);
    if (cpr8 >= 64) return gather_f8_t<64>(Xs, y, m, cpr8, sb, seed, idx_in, idx_out, Y, yB, unscale, st, tm);
    if (cpr8 >= 32) return gather_f8_t<32>(Xs, y, m, cpr8, sb, seed, idx_in, idx_out, Y, yB, unscale, st, tm);
    if (cpr8 >= 16) return gather_f8_t<16>(Xs, y, m, cpr8, sb, seed, idx_in, idx_out, Y, yB, unscale, st, tm);
    if (cpr8 >= 8) return gather_f8_t<8>(Xs, y, m, cpr8, sb, seed, idx_in, idx_out, Y, yB, unscale, st, tm);
    if (cpr8 >= 4) return gather_f8_t<4>(Xs, y, m, cpr8, sb, seed, idx_in, idx_out, Y, yB, unscale, st, tm);
    return gather_f8_t<2>(Xs, y, m, cpr8, sb, seed, idx_in, idx_out, Y, yB, unscale, st, tm);
  }
  const int64_t cpr = ld / (storage == kStoreF32 ? 4 : 8);  // 16-byte chunks per row
  if (cpr >= 64) return gather_t<64>(Xs, y, m, cpr, sb, seed, idx_in, idx_out, Y, yB, st, tm);
  if (cpr >= 32) return gather_t<32>(Xs, y, m, cpr, sb, seed, idx_in, idx_out, Y, yB, st, tm);
  if (cpr >= 16) return gather_t<16>(Xs, y, m, cpr, sb, seed, idx_in, idx_out, Y, yB, st, tm);
  if (cpr >= 8) return gather_t<8>(Xs, y, m, cpr, sb, seed, idx_in, idx_out, Y, yB, st, tm);
  return gather_t<4>(Xs, y, m, cpr, sb, seed, idx_in, idx_out, Y, yB, st, tm);
}

}  // namespace casgd
