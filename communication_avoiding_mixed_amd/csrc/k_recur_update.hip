// Inner recurrence and weight update of one CA-SGD outer iteration, both in
// float32 (the Abstract of "Mixed-Precision Communication-Avoiding SGD for
// Generalized Linear Models on GPUs" runs the inner recurrence and the weight
// update in high precision).
//
//   z_j = v_j - c * sum_{t<j} G_{j,t} r_t,   r_j = l'(z_j, y_j),   c = eta / b
//   w   = w0 - c * Y^T r
#include "casgd_device.h"
#include "casgd_internal.h"

namespace casgd {
namespace {

// One workgroup walks the s minibatches in order.  Block-row j of G is a
// b x (j*b) row-major matrix, so each of its rows is one contiguous dot
// product with r[0 .. j*b), which lives in LDS.  A wave owns a row at a time.
template <int LOSS>
__global__ __launch_bounds__(1024) void recur_kernel(const float* __restrict__ G,
                                                     const float* __restrict__ v,
                                                     const float* __restrict__ yB,
                                                     float* __restrict__ z, float* __restrict__ r,
                                                     int s, int b, float c) {
  extern __shared__ float rs[];  // r of the minibatches finished so far
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int nwaves = blockDim.x >> 6;
  for (int j = 0; j < s; ++j) {
    const int jb = j * b;
    const float* Gj = G + static_cast<int64_t>(b) * b * (static_cast<int64_t>(j) * (j - 1) / 2);
    for (int i = wave; i < b; i += nwaves) {
      const float* row = Gj + static_cast<int64_t>(i) * jb;
      float acc = 0.f;
      if ((reinterpret_cast<uintptr_t>(row) & 15) == 0 && (jb & 3) == 0) {
        const float4* row4 = reinterpret_cast<const float4*>(row);
        const float4* r4 = reinterpret_cast<const float4*>(rs);
        for (int q = lane; q < (jb >> 2); q += 64) {
          const float4 g = row4[q];
          const float4 rr = r4[q];
          acc = fmaf(g.x, rr.x, acc);
          acc = fmaf(g.y, rr.y, acc);
          acc = fmaf(g.z, rr.z, acc);
          acc = fmaf(g.w, rr.w, acc);
        }
      } else {
        for (int q = lane; q < jb; q += 64) acc = fmaf(row[q], rs[q], acc);
      }
      acc = group_sum<64>(acc);
      if (lane == 0) {
        const float zz = v[jb + i] - c * acc;
        const float rv = loss_deriv<LOSS>(zz, yB[jb + i]);
        z[jb + i] = zz;
        r[jb + i] = rv;
        rs[jb + i] = rv;
      }
    }
    __syncthreads();
  }
}

template <typename T>
struct Chunk16;
template <>
struct Chunk16<uint16_t> {
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
struct Chunk16<float> {
  static constexpr int kElems = 4;
  __device__ static void widen(const uint4& q, float (&f)[4]) {
    f[0] = __uint_as_float(q.x);
    f[1] = __uint_as_float(q.y);
    f[2] = __uint_as_float(q.z);
    f[3] = __uint_as_float(q.w);
  }
};

// w <- w - c * Y^T r.  A workgroup owns 8 consecutive 16-byte column chunks
// (8 lanes per row) and all s*b rows, split over 32 row groups whose partial
// sums are then added in a fixed order: the result does not depend on timing.
template <typename T>
__global__ __launch_bounds__(256) void update_kernel(const T* __restrict__ Y, int64_t ld, int64_t n,
                                                     int sb, const float* __restrict__ r, float c,
                                                     float* __restrict__ w) {
  constexpr int E = Chunk16<T>::kElems;
  constexpr int COLS = 8 * E;
  __shared__ float red[32][COLS + 1];
  const int lane = threadIdx.x & 7;
  const int rg = threadIdx.x >> 3;
  const int64_t cpr = ld / E;
  const int64_t chunk = static_cast<int64_t>(blockIdx.x) * 8 + lane;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  if (chunk < cpr) {
    const uint4* Y4 = reinterpret_cast<const uint4*>(Y);
    for (int i = rg; i < sb; i += 32) {
      const uint4 q = Y4[static_cast<int64_t>(i) * cpr + chunk];
      const float ri = r[i];
      float f[E];
      Chunk16<T>::widen(q, f);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fmaf(f[e], ri, acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) red[rg][lane * E + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < COLS) {
    float sum = 0.f;
#pragma unroll 8
    for (int g = 0; g < 32; ++g) sum += red[g][threadIdx.x];
    const int64_t col = static_cast<int64_t>(blockIdx.x) * COLS + threadIdx.x;
    if (col < n) w[col] = w[col] - c * sum;
  }
}

}  // namespace

hipError_t launch_recur(int loss, const float* G, const float* v, const float* yB, float* z,
                        float* r, int s, int b, float c, hipStream_t st) {
  const size_t lds = static_cast<size_t>(s) * b * sizeof(float);
  switch (loss) {
    case kLogistic:
      recur_kernel<kLogistic><<<1, 1024, lds, st>>>(G, v, yB, z, r, s, b, c);
      break;
    case kSquared:
      recur_kernel<kSquared><<<1, 1024, lds, st>>>(G, v, yB, z, r, s, b, c);
      break;
    default:
      recur_kernel<kPoisson><<<1, 1024, lds, st>>>(G, v, yB, z, r, s, b, c);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_update(int storage, const void* Y, int64_t ld, int64_t n, int sb,
                         const float* r, float c, float* w, hipStream_t st) {
  if (storage == kStoreBF16) {
    const int64_t cpr = ld / 8;
    const int grid = static_cast<int>((cpr + 7) / 8);
    update_kernel<uint16_t><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(Y), ld, n, sb, r, c, w);
  } else {
    const int64_t cpr = ld / 4;
    const int grid = static_cast<int>((cpr + 7) / 8);
    update_kernel<float><<<grid, 256, 0, st>>>(static_cast<const float*>(Y), ld, n, sb, r, c, w);
  }
  return hipGetLastError();
}

}  // namespace casgd
