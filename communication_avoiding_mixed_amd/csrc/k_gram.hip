// Strictly-lower block triangle of the Gram matrix G = Y Y^T.
//
// The Abstract of "Mixed-Precision Communication-Avoiding SGD for Generalized
// Linear Models on GPUs" forms the sb x sb Gram from low-precision inputs with
// high-precision accumulation on the GPU's matrix hardware; the inner
// recurrence only ever reads blocks G_{j,t} with t < j, so only those are
// computed.  bf16 and fp16 rows use the MFMA tile of casgd_gram.h (bf16 or
// fp16 MFMA); float32 rows run the same tiles on the vector ALUs.  gr rounds
// every entry once to bf16 as it is stored (G communicated in low precision).
#include "casgd_device.h"
#include "casgd_gram.h"
#include "casgd_internal.h"

namespace casgd {
namespace {

using gram::kTile;

// One 64 x 64 output tile per workgroup; `order` maps workgroups to tiles
// (XCD-grouped) and holds -1 for the workgroups that pad the grid.
template <int BK, int D, bool F16>
__global__ __launch_bounds__(256) void gram_bf16_kernel(const uint16_t* __restrict__ Y,
                                                        int64_t ld, int b, int tps,
                                                        float* __restrict__ G,
                                                        const int* __restrict__ order, int gr) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[gram::lds_elems<BK>()];
  const int tile = order[blockIdx.x];
  if (tile < 0) return;
  gram::bf16_tile<BK, D, false, gram::SameRow, F16>(Y, ld, b, tps, G, tile, lds, gram::SameRow{}, gr != 0);
}

// float32 storage: the same tiles on the vector ALUs (casgd_gram.h).
__global__ __launch_bounds__(256) void gram_f32_kernel(const float* __restrict__ Y, int64_t ld,
                                                       int b, int tps, float* __restrict__ G,
                                                       const int* __restrict__ order, int gr) {
  __shared__ __attribute__((aligned(16))) float lds[gram::kF32LdsElems];
  const int tile = order[blockIdx.x];
  if (tile < 0) return;
  gram::f32_tile(Y, ld, b, tps, G, tile, lds, gram::SameRow{}, gr != 0);
}

template <bool F16>
hipError_t gram_lp(const uint16_t* Yb, int64_t ld, int b, int tps, float* G, const int* order, int gr,
                   dim3 grid, hipStream_t st, const LaunchTimer& tm) {
  switch (gram_variant(ld)) {
    case 0: return launch_kernel(gram_bf16_kernel<32, 1, F16>, grid, dim3(256), 0, st, tm, Yb, ld, b, tps, G, order, gr);
    case 1: return launch_kernel(gram_bf16_kernel<64, 8, F16>, grid, dim3(256), 0, st, tm, Yb, ld, b, tps, G, order, gr);
    case 2: return launch_kernel(gram_bf16_kernel<64, 4, F16>, grid, dim3(256), 0, st, tm, Yb, ld, b, tps, G, order, gr);
    default: return launch_kernel(gram_bf16_kernel<64, 2, F16>, grid, dim3(256), 0, st, tm, Yb, ld, b, tps, G, order, gr);
  }
}

}  // namespace

GramPlan gram_plan(int storage, int s, int b, int64_t ld, int nx) {
  (void)storage;
  (void)ld;
  GramPlan p;
  const int tps = (b + kTile - 1) / kTile;
  p.tiles = s * (s - 1) / 2 * tps * tps;
  p.slots = (p.tiles + nx - 1) / nx * nx;
  return p;
}

// Workgroups are dealt to the XCDs round-robin (workgroup w runs on XCD w mod
// 8, each XCD with its own L2; in the pipelined step launch the Gram's
// workgroups cycle over nx = 7 XCDs).  Tiles are listed in super-blocks of
// S x S blocks (S chosen so a super-block holds about one XCD's share), the
// list is cut into nx consecutive runs, and run x is placed on the workgroups
// g with g mod nx = x: the tiles that share rows of Y then share an L2.
std::vector<int> gram_order(int s, int b, int nx) {
  const int tps = (b + kTile - 1) / kTile;
  const int tiles = s * (s - 1) / 2 * tps * tps;
  const int per = (tiles + nx - 1) / nx;
  int S = 1;
  while (S < s && (S + 1) * (S + 1) * tps * tps <= per) ++S;
  std::vector<int> list;
  list.reserve(tiles);
  for (int J = 0; J * S < s; ++J)
    for (int T = 0; T <= J; ++T)
      for (int j = J * S; j < (J + 1) * S && j < s; ++j)
        for (int t = T * S; t < (T + 1) * S && t < j; ++t)
          for (int q = 0; q < tps * tps; ++q) list.push_back((j * (j - 1) / 2 + t) * tps * tps + q);
  std::vector<int> order(static_cast<size_t>(per) * nx, -1);
  for (int x = 0; x < nx; ++x)
    for (int k = 0; k < per; ++k) {
      const int idx = x * per + k;
      if (idx < tiles) order[static_cast<size_t>(k) * nx + x] = list[idx];
    }
  return order;
}

hipError_t launch_gram(int kind, const void* Y, int64_t ld, int s, int b, float* G,
                       const GramPlan& plan, const int* order, int gr, hipStream_t st, const LaunchTimer& tm) {
  (void)s;
  if (plan.tiles == 0) return hipSuccess;
  const int tps = (b + kTile - 1) / kTile;
  const dim3 grid(static_cast<unsigned>(plan.slots));
  if (kind == kStoreBF16) return gram_lp<false>(static_cast<const uint16_t*>(Y), ld, b, tps, G, order, gr, grid, st, tm);
  if (kind == kStoreF16) return gram_lp<true>(static_cast<const uint16_t*>(Y), ld, b, tps, G, order, gr, grid, st, tm);
  return launch_kernel(gram_f32_kernel, grid, dim3(256), 0, st, tm, static_cast<const float*>(Y), ld, b,
                       tps, G, order, gr);
}

}  // namespace casgd
