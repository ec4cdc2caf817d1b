// Mean loss over every stored row, f(w) = (1/m) sum_i l(x_i . w, y_i): the
// quantity by which the Abstract of "Mixed-Precision Communication-Avoiding
// SGD for Generalized Linear Models on GPUs" compares the method with float32
// SGD.  Margins are float32 dot products of the stored rows; loss terms and
// all sums are float64, reduced in a fixed order (no atomics).
#include <cmath>

#include "casgd_device.h"
#include "casgd_internal.h"

namespace casgd {
namespace {

template <typename T>
struct Widen;
template <>
struct Widen<uint16_t> {
  static constexpr int kElems = 8;
  __device__ static void run(const u32x4& q, float (&f)[8]) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = bf16_to_f32(w[e] & 0xFFFFu);
      f[2 * e + 1] = bf16_to_f32(w[e] >> 16);
    }
  }
};
template <>
struct Widen<_Float16> {
  static constexpr int kElems = 8;
  __device__ static void run(const u32x4& q, float (&f)[8]) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = f16_to_f32_hw(w[e] & 0xFFFFu);
      f[2 * e + 1] = f16_to_f32_hw(w[e] >> 16);
    }
  }
};
// fp8 rows: the stored E4M3 values, still scaled by the matrix's 2^k (each
// row's dot product is scaled back once, exactly)
template <>
struct Widen<uint8_t> {
  static constexpr int kElems = 16;
  __device__ static void run(const u32x4& q, float (&f)[16]) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int e = 0; e < 16; ++e) f[e] = e4m3_to_f32((w[e / 4] >> (8 * (e % 4))) & 0xFFu);
  }
};
template <>
struct Widen<float> {
  static constexpr int kElems = 4;
  __device__ static void run(const u32x4& q, float (&f)[4]) {
    f[0] = __uint_as_float(q.x);
    f[1] = __uint_as_float(q.y);
    f[2] = __uint_as_float(q.z);
    f[3] = __uint_as_float(q.w);
  }
};

// Grid-stride over pairs of rows; a group of GS lanes per row, R = 2 rows per
// group at a time.  w is staged in LDS (zero past n), so the dot products
// need no bounds checks and every row chunk of a pass is loaded before any is
// used (kU chunks per lane per row, clamped addresses, zeroed when used).
// Each block writes one float64 partial sum.
constexpr int kU = 4;
constexpr int64_t kLossWlMax = 8192;  // floats of w staged in LDS

template <typename T, int LOSS, int GS, bool WLDS>
__global__ __launch_bounds__(256) void loss_kernel(const T* __restrict__ Xs,
                                                   const float* __restrict__ y, int64_t m,
                                                   int64_t n, int64_t ld,
                                                   const float* __restrict__ w,
                                                   double* __restrict__ partial, float unscale) {
  constexpr int E = Widen<T>::kElems;
  constexpr int R = 2;
  __shared__ __attribute__((aligned(16))) float wl[WLDS ? kLossWlMax : 4];
  const int lane = threadIdx.x % GS;
  const int64_t groups = static_cast<int64_t>(gridDim.x) * (256 / GS);
  const int64_t cpr = ld / E;
  if constexpr (WLDS) {
    for (int64_t c = threadIdx.x; c < ld; c += 256) wl[c] = c < n ? w[c] : 0.f;
    __syncthreads();
  }
  auto wval = [&](int64_t col) -> float {
    if constexpr (WLDS) return wl[col];
    else return col < n ? w[col] : 0.f;
  };
  double acc = 0.0;
  for (int64_t row0 = (static_cast<int64_t>(blockIdx.x) * (256 / GS) + threadIdx.x / GS) * R; row0 < m;
       row0 += groups * R) {
    float d[R] = {};
    for (int64_t c0 = lane; c0 < cpr; c0 += GS * kU) {
      u32x4 q[R][kU];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t row = row0 + r < m ? row0 + r : row0;
        const u32x4* xr = reinterpret_cast<const u32x4*>(Xs + row * ld);
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int64_t c = c0 + GS * u;
          q[r][u] = xr[c < cpr ? c : 0];
        }
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t c = c0 + GS * u;
        if (c >= cpr) break;
        float wv[E];
#pragma unroll
        for (int e = 0; e < E; ++e) wv[e] = wval(c * E + e);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float f[E];
          Widen<T>::run(q[r][u], f);
#pragma unroll
          for (int e = 0; e < E; ++e) d[r] = fmaf(f[e], wv[e], d[r]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float tot = group_sum<GS>(d[r]) * unscale;
      if (lane == 0 && row0 + r < m)
        acc += loss_value<LOSS>(static_cast<double>(tot), static_cast<double>(y[row0 + r]));
    }
  }
  __shared__ double red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) partial[blockIdx.x] = red[0];
}

// Narrow rows (at most GS 16-byte chunks, GS = 4 or 8): a wave takes 64
// consecutive rows per pass.  Load r (r < GS) reads rows base + r*G ... base +
// r*G + G-1 (G = 64/GS lane groups, one row per group, lane c of a group
// chunk c), so each load instruction covers G whole consecutive rows; the
// group sums give every lane of group g the margins of its GS rows, and lane
// (g, c) keeps row c's, so the float64 loss terms of the 64 rows run on all 64
// lanes.  A row's float32 dot product is summed in the same order as in
// loss_kernel (chunk elements in order, then the group butterfly).
template <typename T, int LOSS, int GS>
__global__ __launch_bounds__(256) void loss_narrow_kernel(const T* __restrict__ Xs,
                                                          const float* __restrict__ y, int64_t m,
                                                          int64_t n, int64_t ld,
                                                          const float* __restrict__ w,
                                                          double* __restrict__ partial, float unscale) {
  constexpr int E = Widen<T>::kElems;
  constexpr int G = 64 / GS;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane % GS;  // chunk of this lane
  const int g = lane / GS;  // lane group
  const int64_t cpr = ld / E;
  float wv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int64_t col = static_cast<int64_t>(c) * E + e;
    wv[e] = (c < cpr && col < n) ? w[col] : 0.f;
  }
  const int cc = c < cpr ? c : 0;  // chunks past the row read chunk 0 against zero weights
  double acc = 0.0;
  for (int64_t base = (static_cast<int64_t>(blockIdx.x) * 4 + wave) * 64; base < m;
       base += static_cast<int64_t>(gridDim.x) * 256) {
    u32x4 q[GS];
#pragma unroll
    for (int r = 0; r < GS; ++r) {
      const int64_t row = base + r * G + g;
      const int64_t rc = row < m ? row : m - 1;
      q[r] = reinterpret_cast<const u32x4*>(Xs + rc * ld)[cc];
    }
    float mine = 0.f;
#pragma unroll
    for (int r = 0; r < GS; ++r) {
      float f[E];
      Widen<T>::run(q[r], f);
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) d = fmaf(f[e], wv[e], d);
      const float tot = group_sum<GS>(d) * unscale;
      if (c == r) mine = tot;
    }
    const int64_t myrow = base + c * G + g;
    if (myrow < m) acc += loss_value<LOSS>(static_cast<double>(mine), static_cast<double>(y[myrow]));
  }
  __shared__ double red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) partial[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(256) void loss_finish_kernel(const double* __restrict__ partial, int np,
                                                          double inv_m, double* __restrict__ out) {
  __shared__ double red[256];
  double acc = 0.0;
  for (int i = threadIdx.x; i < np; i += 256) acc += partial[i];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = red[0] * inv_m;
}

template <typename T, int LOSS, int GS>
void loss_g(const T* X, const float* y, int64_t m, int64_t n, int64_t ld, const float* w, double* partial,
            float unscale, hipStream_t st) {
  if (ld <= kLossWlMax)
    loss_kernel<T, LOSS, GS, true><<<kLossBlocks, 256, 0, st>>>(X, y, m, n, ld, w, partial, unscale);
  else
    loss_kernel<T, LOSS, GS, false><<<kLossBlocks, 256, 0, st>>>(X, y, m, n, ld, w, partial, unscale);
}

// A narrow-kernel block takes 256 rows per pass: no more blocks than passes need.
inline int narrow_blocks(int64_t m) {
  const int64_t need = (m + 255) / 256;
  return static_cast<int>(need < kLossBlocks ? need : kLossBlocks);
}

// Partial sums of the loss kernel for rows of cpr 16-byte chunks.
inline int partials_for(int64_t cpr, int64_t m) { return cpr > 8 ? kLossBlocks : narrow_blocks(m); }

// Launches the loss kernel for this row width; returns the partial sums it writes.
template <typename T, int LOSS>
int loss_gs(const void* Xs, const float* y, int64_t m, int64_t n, int64_t ld, const float* w,
             double* partial, float unscale, hipStream_t st) {
  const int64_t cpr = ld / Widen<T>::kElems;
  const T* X = static_cast<const T*>(Xs);
  if (cpr >= 64)
    loss_g<T, LOSS, 64>(X, y, m, n, ld, w, partial, unscale, st);
  else if (cpr >= 32)
    loss_g<T, LOSS, 32>(X, y, m, n, ld, w, partial, unscale, st);
  else if (cpr >= 16)
    loss_g<T, LOSS, 16>(X, y, m, n, ld, w, partial, unscale, st);
  else if (cpr > 8)
    loss_g<T, LOSS, 8>(X, y, m, n, ld, w, partial, unscale, st);
  else if (cpr > 4)  // the narrow kernels read chunks [0, GS) only
    loss_narrow_kernel<T, LOSS, 8><<<narrow_blocks(m), 256, 0, st>>>(X, y, m, n, ld, w, partial, unscale);
  else
    loss_narrow_kernel<T, LOSS, 4><<<narrow_blocks(m), 256, 0, st>>>(X, y, m, n, ld, w, partial, unscale);
  return partials_for(cpr, m);
}

template <typename T>
int loss_t(int loss, const void* Xs, const float* y, int64_t m, int64_t n, int64_t ld,
           const float* w, double* partial, float unscale, hipStream_t st) {
  if (loss == kLogistic) return loss_gs<T, kLogistic>(Xs, y, m, n, ld, w, partial, unscale, st);
  if (loss == kSquared) return loss_gs<T, kSquared>(Xs, y, m, n, ld, w, partial, unscale, st);
  return loss_gs<T, kPoisson>(Xs, y, m, n, ld, w, partial, unscale, st);
}

}  // namespace

int loss_partials(int storage, int64_t m, int64_t ld) {
  const int64_t cpr = ld / (16 / elem_bytes(storage));
  return partials_for(cpr, m);
}

hipError_t launch_loss(int storage, int loss, const void* Xs, const float* y, int64_t m, int64_t n,
                       int64_t ld, const float* w, double* partial, double* out_dev, int fp8_exp,
                       hipStream_t st) {
  int np;
  switch (storage) {
    case kStoreBF16: np = loss_t<uint16_t>(loss, Xs, y, m, n, ld, w, partial, 1.f, st); break;
    case kStoreF16: np = loss_t<_Float16>(loss, Xs, y, m, n, ld, w, partial, 1.f, st); break;
    case kStoreF8:
      np = loss_t<uint8_t>(loss, Xs, y, m, n, ld, w, partial, std::ldexp(1.0f, -fp8_exp), st);
      break;
    default: np = loss_t<float>(loss, Xs, y, m, n, ld, w, partial, 1.f, st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  loss_finish_kernel<<<1, 256, 0, st>>>(partial, np, 1.0 / static_cast<double>(m), out_dev);
  return hipGetLastError();
}

}  // namespace casgd
