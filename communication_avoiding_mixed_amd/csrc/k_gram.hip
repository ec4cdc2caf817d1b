// Strictly-lower block triangle of the Gram matrix G = Y Y^T.
//
// The Abstract of "Mixed-Precision Communication-Avoiding SGD for Generalized
// Linear Models on GPUs" forms the sb x sb Gram from low-precision inputs with
// high-precision accumulation on the GPU's matrix hardware; the inner
// recurrence only ever reads blocks G_{j,t} with t < j, so only those are
// computed.  bf16 storage uses the MFMA tile of casgd_gram.h; float32 storage
// runs the same tiles on the vector ALUs.
#include "casgd_device.h"
#include "casgd_gram.h"
#include "casgd_internal.h"

namespace casgd {
namespace {

using gram::kTile;

// One 64 x 64 output tile per workgroup; `order` maps workgroups to tiles
// (XCD-grouped) and holds -1 for the workgroups that pad the grid.
template <int BK, int D>
__global__ __launch_bounds__(256) void gram_bf16_kernel(const uint16_t* __restrict__ Y,
                                                        int64_t ld, int b, int tps,
                                                        float* __restrict__ G,
                                                        const int* __restrict__ order) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[gram::lds_elems<BK>()];
  const int tile = order[blockIdx.x];
  if (tile < 0) return;
  gram::bf16_tile<BK, D>(Y, ld, b, tps, G, tile, lds);
}

// float32 storage: the same tiles on the vector ALUs (each lane a 4 x 4
// register block), used when the data are kept in float32.
__global__ __launch_bounds__(256) void gram_f32_kernel(const float* __restrict__ Y, int64_t ld,
                                                       int b, int tps, float* __restrict__ G,
                                                       const int* __restrict__ order) {
  constexpr int BK = 16;
  __shared__ float As[BK][kTile + 4];
  __shared__ float Bs[BK][kTile + 4];
  const int nt2 = tps * tps;
  const int tile = order[blockIdx.x];
  if (tile < 0) return;
  const int p = tile / nt2;
  const int rem = tile - p * nt2;
  const int ti = rem / tps;
  const int tj = rem - ti * tps;
  int j, t;
  block_of(p, j, t);
  const float* Yp = Y;
  float* Gj = G + static_cast<int64_t>(b) * b * (static_cast<int64_t>(j) * (j - 1) / 2);
  const int64_t ldg = static_cast<int64_t>(j) * b;
  const int a0 = ti * kTile, b0 = tj * kTile;

  // loader: 64 rows x 16 k per stage = 256 float4
  const int lr = threadIdx.x >> 2;
  const int lk = (threadIdx.x & 3) * 4;
  const bool aok = a0 + lr < b, bok = b0 + lr < b;
  const float* ap = Yp + (static_cast<int64_t>(j) * b + a0 + (aok ? lr : 0)) * ld + lk;
  const float* bp = Yp + (static_cast<int64_t>(t) * b + b0 + (bok ? lr : 0)) * ld + lk;

  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int64_t k0 = 0; k0 < ld; k0 += BK) {
    const bool kin = k0 + lk < ld;
    const float4 av = (aok && kin) ? *reinterpret_cast<const float4*>(ap + k0) : make_float4(0, 0, 0, 0);
    const float4 bv = (bok && kin) ? *reinterpret_cast<const float4*>(bp + k0) : make_float4(0, 0, 0, 0);
    As[lk + 0][lr] = av.x;
    As[lk + 1][lr] = av.y;
    As[lk + 2][lr] = av.z;
    As[lk + 3][lr] = av.w;
    Bs[lk + 0][lr] = bv.x;
    Bs[lk + 1][lr] = bv.y;
    Bs[lk + 2][lr] = bv.z;
    Bs[lk + 3][lr] = bv.w;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      const float4 a4 = *reinterpret_cast<const float4*>(&As[k][ty * 4]);
      const float4 b4 = *reinterpret_cast<const float4*>(&Bs[k][tx * 4]);
      const float a[4] = {a4.x, a4.y, a4.z, a4.w};
      const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[u][q] = fmaf(a[u], bb[q], acc[u][q]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = a0 + ty * 4 + u;
    if (row >= b) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int col = b0 + tx * 4 + q;
      if (col < b) Gj[row * ldg + static_cast<int64_t>(t) * b + col] = acc[u][q];
    }
  }
}

}  // namespace

GramPlan gram_plan(int storage, int s, int b, int64_t ld) {
  (void)storage;
  (void)ld;
  GramPlan p;
  const int tps = (b + kTile - 1) / kTile;
  p.tiles = s * (s - 1) / 2 * tps * tps;
  p.slots = (p.tiles + kXcds - 1) / kXcds * kXcds;
  return p;
}

// Workgroups are dealt to the XCDs round-robin (workgroup w runs on XCD w mod
// 8, each XCD with its own L2).  Tiles are listed in super-blocks of S x S
// blocks (S chosen so a super-block holds about one XCD's share), the list is
// cut into 8 consecutive runs, and run x is placed on the workgroups of XCD x:
// the tiles that share rows of Y then share an L2.
std::vector<int> gram_order(int s, int b) {
  const int tps = (b + kTile - 1) / kTile;
  const int tiles = s * (s - 1) / 2 * tps * tps;
  const int per = (tiles + kXcds - 1) / kXcds;
  int S = 1;
  while (S < s && (S + 1) * (S + 1) * tps * tps <= per) ++S;
  std::vector<int> list;
  list.reserve(tiles);
  for (int J = 0; J * S < s; ++J)
    for (int T = 0; T <= J; ++T)
      for (int j = J * S; j < (J + 1) * S && j < s; ++j)
        for (int t = T * S; t < (T + 1) * S && t < j; ++t)
          for (int q = 0; q < tps * tps; ++q) list.push_back((j * (j - 1) / 2 + t) * tps * tps + q);
  std::vector<int> order(static_cast<size_t>(per) * kXcds, -1);
  for (int x = 0; x < kXcds; ++x)
    for (int k = 0; k < per; ++k) {
      const int idx = x * per + k;
      if (idx < tiles) order[static_cast<size_t>(k) * kXcds + x] = list[idx];
    }
  return order;
}

hipError_t launch_gram(int storage, const void* Y, int64_t ld, int s, int b, float* G,
                       const GramPlan& plan, const int* order, hipStream_t st, const LaunchTimer& tm) {
  (void)s;
  if (plan.tiles == 0) return hipSuccess;
  const int tps = (b + kTile - 1) / kTile;
  const dim3 grid(static_cast<unsigned>(plan.slots));
  if (storage == kStoreBF16) {
    const uint16_t* Yb = static_cast<const uint16_t*>(Y);
    switch (gram_variant(ld)) {
      case 0: return launch_kernel(gram_bf16_kernel<32, 1>, grid, dim3(256), 0, st, tm, Yb, ld, b, tps, G, order);
      case 1: return launch_kernel(gram_bf16_kernel<64, 8>, grid, dim3(256), 0, st, tm, Yb, ld, b, tps, G, order);
      case 2: return launch_kernel(gram_bf16_kernel<64, 4>, grid, dim3(256), 0, st, tm, Yb, ld, b, tps, G, order);
      default: return launch_kernel(gram_bf16_kernel<64, 2>, grid, dim3(256), 0, st, tm, Yb, ld, b, tps, G, order);
    }
  }
  return launch_kernel(gram_f32_kernel, grid, dim3(256), 0, st, tm, static_cast<const float*>(Y), ld, b,
                       tps, G, order);
}

}  // namespace casgd
