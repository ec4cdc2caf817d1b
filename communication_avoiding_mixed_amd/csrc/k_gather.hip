// Storage conversion (at create) and the per-step sample + gather kernel.
// The data matrix is kept in low precision, as the Abstract of "Mixed-
// Precision Communication-Avoiding SGD for Generalized Linear Models on GPUs"
// prescribes; rows are padded to ld (a multiple of 32 elements) so every row
// is a whole number of 16-byte chunks.
#include "casgd_device.h"
#include "casgd_internal.h"

namespace casgd {
namespace {

// ---------------------------------------------------------------------------
// X (float32, m x n) -> Xs (m x ld).  One thread per 16-byte output chunk.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void store_bf16_kernel(const float* __restrict__ X,
                                                         uint16_t* __restrict__ Xs, int64_t m,
                                                         int64_t n, int64_t ld) {
  const int64_t cpr = ld / 8;  // chunks per row
  const int64_t total = m * cpr;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g < total;
       g += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t row = g / cpr;
    const int64_t c0 = (g - row * cpr) * 8;
    const float* src = X + row * n;
    uint32_t packed[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t c = c0 + 2 * e;
      const uint32_t lo = c < n ? f32_to_bf16(src[c]) : 0u;
      const uint32_t hi = c + 1 < n ? f32_to_bf16(src[c + 1]) : 0u;
      packed[e] = lo | (hi << 16);
    }
    *reinterpret_cast<uint4*>(Xs + row * ld + c0) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
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

// ---------------------------------------------------------------------------
// Sample + gather.  A group of GS lanes copies one row of Y with 16-byte
// loads and stores (GS chosen so the group spans the row's chunks); each lane
// issues all of its loads of a row before its stores, so a row costs one
// memory round trip.
// ---------------------------------------------------------------------------
template <int GS>
__global__ __launch_bounds__(256) void gather_kernel(
    const u32x4* __restrict__ Xs, const float* __restrict__ y, int64_t m, int64_t cpr, int sb,
    uint64_t seed, const int32_t* __restrict__ idx_in, int32_t* __restrict__ idx_out,
    u32x4* __restrict__ Y, float* __restrict__ yB) {
  constexpr int U = 4;
  const int lane = threadIdx.x % GS;
  const int row = blockIdx.x * (256 / GS) + threadIdx.x / GS;
  if (row >= sb) return;  // whole lane groups leave together
  int64_t src = idx_in ? static_cast<int64_t>(idx_in[row])
                       : static_cast<int64_t>(sample_row(seed, static_cast<uint64_t>(row),
                                                         static_cast<uint64_t>(m)));
  src = src < 0 ? 0 : (src >= m ? m - 1 : src);  // explicit indices are checked on the host
  if (lane == 0) {
    idx_out[row] = static_cast<int32_t>(src);
    yB[row] = y[src];
  }
  const u32x4* xr = Xs + src * cpr;
  u32x4* yr = Y + static_cast<int64_t>(row) * cpr;
  for (int64_t c0 = lane; c0 < cpr; c0 += GS * U) {
    u32x4 q[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + GS * u;
      q[u] = c < cpr ? xr[c] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + GS * u;
      if (c < cpr) yr[c] = q[u];
    }
  }
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
  const int64_t want = (chunks + 255) / 256;
  const int grid = static_cast<int>(want < 65536 ? (want > 0 ? want : 1) : 65536);
  if (storage == kStoreBF16)
    store_bf16_kernel<<<grid, 256, 0, st>>>(X, static_cast<uint16_t*>(Xs), m, n, ld);
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
