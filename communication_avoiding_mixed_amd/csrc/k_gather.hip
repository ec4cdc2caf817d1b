// Storage conversion (at create) and the per-step sample + gather + margins
// kernel.  The data matrix is kept in low precision, as the Abstract of
// "Mixed-Precision Communication-Avoiding SGD for Generalized Linear Models
// on GPUs" prescribes; rows are padded to ld (a multiple of 32 elements) so
// every row is a whole number of 16-byte chunks.
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

// Widen the elements of one 16-byte chunk to float.
template <typename T>
struct Chunk;

template <>
struct Chunk<uint16_t> {
  static constexpr int kElems = 8;
  __device__ static void widen(const uint4& q, float (&f)[8]) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = bf16_to_f32(w[e] & 0xFFFFu);
      f[2 * e + 1] = bf16_to_f32(w[e] >> 16);
    }
  }
};

template <>
struct Chunk<float> {
  static constexpr int kElems = 4;
  __device__ static void widen(const uint4& q, float (&f)[4]) {
    f[0] = __uint_as_float(q.x);
    f[1] = __uint_as_float(q.y);
    f[2] = __uint_as_float(q.z);
    f[3] = __uint_as_float(q.w);
  }
};

// ---------------------------------------------------------------------------
// Sample + gather + margins.  A group of GS lanes copies one row of Y with
// 16-byte loads/stores (GS chosen so the group spans the row's chunks) and
// accumulates the row's margin x . w in float32 (bf16 widened exactly).
// ---------------------------------------------------------------------------
template <typename T, int GS>
__global__ __launch_bounds__(256) void gather_kernel(
    const T* __restrict__ Xs, const float* __restrict__ y, int64_t m, int64_t n, int64_t ld,
    int sb, uint64_t seed, const int32_t* __restrict__ idx_in, int32_t* __restrict__ idx_out,
    T* __restrict__ Y, float* __restrict__ yB, const float* __restrict__ w,
    float* __restrict__ v) {
  constexpr int E = Chunk<T>::kElems;
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
  const int64_t cpr = ld / E;
  const uint4* xr = reinterpret_cast<const uint4*>(Xs + src * ld);
  uint4* yr = reinterpret_cast<uint4*>(Y + static_cast<int64_t>(row) * ld);
  float acc = 0.f;
  for (int64_t c = lane; c < cpr; c += GS) {
    const uint4 q = xr[c];
    yr[c] = q;
    if (w) {
      float f[E];
      Chunk<T>::widen(q, f);
      const int64_t col0 = c * E;
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (col0 + e < n) acc = fmaf(f[e], w[col0 + e], acc);
    }
  }
  if (w) {
    acc = group_sum<GS>(acc);
    if (lane == 0) v[row] = acc;
  }
}

template <typename T, int GS>
hipError_t gather_t(const void* Xs, const float* y, int64_t m, int64_t n, int64_t ld, int sb,
                    uint64_t seed, const int32_t* idx_in, int32_t* idx_out, void* Y, float* yB,
                    const float* w, float* v, hipStream_t st) {
  const int rows_per_block = 256 / GS;
  const int grid = (sb + rows_per_block - 1) / rows_per_block;
  gather_kernel<T, GS><<<grid, 256, 0, st>>>(static_cast<const T*>(Xs), y, m, n, ld, sb, seed,
                                             idx_in, idx_out, static_cast<T*>(Y), yB, w, v);
  return hipGetLastError();
}

template <typename T>
hipError_t gather_dispatch(const void* Xs, const float* y, int64_t m, int64_t n, int64_t ld,
                           int sb, uint64_t seed, const int32_t* idx_in, int32_t* idx_out,
                           void* Y, float* yB, const float* w, float* v, hipStream_t st) {
  const int64_t cpr = ld / Chunk<T>::kElems;
  if (cpr >= 64)
    return gather_t<T, 64>(Xs, y, m, n, ld, sb, seed, idx_in, idx_out, Y, yB, w, v, st);
  if (cpr >= 32)
    return gather_t<T, 32>(Xs, y, m, n, ld, sb, seed, idx_in, idx_out, Y, yB, w, v, st);
  if (cpr >= 16)
    return gather_t<T, 16>(Xs, y, m, n, ld, sb, seed, idx_in, idx_out, Y, yB, w, v, st);
  if (cpr >= 8)
    return gather_t<T, 8>(Xs, y, m, n, ld, sb, seed, idx_in, idx_out, Y, yB, w, v, st);
  return gather_t<T, 4>(Xs, y, m, n, ld, sb, seed, idx_in, idx_out, Y, yB, w, v, st);
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

hipError_t launch_gather(int storage, const void* Xs, const float* y, int64_t m, int64_t n,
                         int64_t ld, int sb, uint64_t seed, const int32_t* idx_in,
                         int32_t* idx_out, void* Y, float* yB, const float* w, float* v,
                         hipStream_t st) {
  if (storage == kStoreBF16)
    return gather_dispatch<uint16_t>(Xs, y, m, n, ld, sb, seed, idx_in, idx_out, Y, yB, w, v, st);
  return gather_dispatch<float>(Xs, y, m, n, ld, sb, seed, idx_in, idx_out, Y, yB, w, v, st);
}

}  // namespace casgd
