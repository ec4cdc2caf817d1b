// Sample + gather of one row of Y, as a device function shared by the
// stand-alone gather kernel and the pipelined step kernel.  Row i of the
// outer step is stored row idx_i (sampled from the step seed, or given), the
// low-precision storage the Abstract of "Mixed-Precision Communication-
// Avoiding SGD for Generalized Linear Models on GPUs" prescribes, copied bit
// for bit.
#pragma once

#include "casgd_device.h"

namespace casgd {
namespace gather {

// A group of GS lanes copies row `row` of Y with 16-byte loads and stores (GS
// chosen so the group spans the row's cpr chunks); each lane issues all of its
// loads of a row before its stores, so a row costs one memory round trip.
// Rows at or past sb are skipped (whole lane groups together).
template <int GS>
__device__ __forceinline__ void copy_row(const u32x4* __restrict__ Xs, const float* __restrict__ y,
                                         int64_t m, int64_t cpr, int sb, uint64_t seed,
                                         const int32_t* __restrict__ idx_in,
                                         int32_t* __restrict__ idx_out, u32x4* __restrict__ Y,
                                         float* __restrict__ yB, int row, int lane) {
  constexpr int U = 4;
  if (row >= sb) return;
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

// The same for fp8 rows (16 E4M3 values per 16-byte chunk, cpr8 chunks),
// widened to bf16 as they are copied: the stored value e4m3 * 2^-k
// (unscale = 2^-k) has at most four significant bits and stays in bf16's
// range, so the bf16 row holds exactly the stored values.  Row `row` of Y
// has 2 * cpr8 chunks.
template <int GS>
__device__ __forceinline__ void copy_row_f8(const u32x4* __restrict__ Xs, const float* __restrict__ y,
                                            int64_t m, int64_t cpr8, int sb, uint64_t seed,
                                            const int32_t* __restrict__ idx_in,
                                            int32_t* __restrict__ idx_out, u32x4* __restrict__ Y,
                                            float* __restrict__ yB, float unscale, int row, int lane) {
  constexpr int U = 4;
  if (row >= sb) return;
  int64_t src = idx_in ? static_cast<int64_t>(idx_in[row])
                       : static_cast<int64_t>(sample_row(seed, static_cast<uint64_t>(row),
                                                         static_cast<uint64_t>(m)));
  src = src < 0 ? 0 : (src >= m ? m - 1 : src);
  if (lane == 0) {
    idx_out[row] = static_cast<int32_t>(src);
    yB[row] = y[src];
  }
  const u32x4* xr = Xs + src * cpr8;
  u32x4* yr = Y + static_cast<int64_t>(row) * cpr8 * 2;
  for (int64_t c0 = lane; c0 < cpr8; c0 += GS * U) {
    u32x4 q[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + GS * u;
      q[u] = c < cpr8 ? xr[c] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + GS * u;
      if (c >= cpr8) break;
      const uint32_t w[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
      uint32_t o[8];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t lo = f32_to_bf16(e4m3_to_f32((w[i] >> (16 * h)) & 0xFFu) * unscale);
          const uint32_t hi = f32_to_bf16(e4m3_to_f32((w[i] >> (16 * h + 8)) & 0xFFu) * unscale);
          o[2 * i + h] = lo | (hi << 16);
        }
      yr[2 * c] = u32x4{o[0], o[1], o[2], o[3]};
      yr[2 * c + 1] = u32x4{o[4], o[5], o[6], o[7]};
    }
  }
}

// Lanes per row for rows of cpr 16-byte chunks.
__host__ __device__ inline int group_size(int64_t cpr) {
  return cpr >= 64 ? 64 : cpr >= 32 ? 32 : cpr >= 16 ? 16 : cpr >= 8 ? 8 : 4;
}

}  // namespace gather
}  // namespace casgd
