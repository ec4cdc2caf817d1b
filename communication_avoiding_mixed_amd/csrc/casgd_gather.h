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

// Lanes per row for rows of cpr 16-byte chunks.
__host__ __device__ inline int group_size(int64_t cpr) {
  return cpr >= 64 ? 64 : cpr >= 32 ? 32 : cpr >= 16 ? 16 : cpr >= 8 ? 8 : 4;
}

}  // namespace gather
}  // namespace casgd
