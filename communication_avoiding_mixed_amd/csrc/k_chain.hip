// The weight-dependent part of one CA-SGD outer iteration in a single launch:
// margins, inner recurrence and weight update (Abstract of "Mixed-Precision
// Communication-Avoiding SGD for Generalized Linear Models on GPUs": the inner
// recurrence and the weight update run in high precision, here float32).
//
//   v   = Y w0
//   z_j = v_j - c * sum_{t<j} G_{j,t} r_t,   r_j = l'(z_j, y_j),   c = eta / b
//   w   = w0 - c * Y^T r
//
// Q workgroups split the b rows of every minibatch: workgroup q owns rows
// i = q, q + Q, q + 2Q, ... of each minibatch, computes their margins, and at
// inner step j the dot products of its rows of block-row j of G with the r
// values of the earlier minibatches.  The new r values are exchanged through
// 64-bit words that carry the launch's epoch tag in their upper half, so a
// reader spins on the data itself (one one-way trip through the coherent
// memory per inner step, no barriers, no separate flags).  Each value is
// written to one mailbox per reading workgroup, so no memory location is
// polled by more than one workgroup.  Every spin is
// bounded: on expiry the kernel flags an error in `status` and returns.
// After the last inner step every workgroup holds all of r and updates its
// own slice of columns of w in a fixed summation order (no float atomics).
#include "casgd_chain.h"

namespace casgd {
namespace {

using chain::Elems;
using chain::kSpinLimit;
using chain::kThreads;
using chain::kWaves;
using chain::tagged;

// LDS layout (floats): rs[sb] | vown[s * nown_max] | yown[s * nown_max] |
// region, where region
// holds this workgroup's rows of G (when a.preload) during the recurrence and
// the update's reduction scratch afterwards.
struct ChainLayout {
  int64_t rs, vown, yown, region, region_len, total;
};

__host__ __device__ inline ChainLayout chain_layout(int s, int b, int Q, bool preload) {
  ChainLayout L;
  const int64_t sb = static_cast<int64_t>(s) * b;
  const int64_t nown_max = (b + Q - 1) / Q;
  L.rs = 0;
  L.vown = (sb + 3) & ~3LL;
  L.yown = L.vown + ((s * nown_max + 3) & ~3LL);
  L.region = L.yown + ((s * nown_max + 3) & ~3LL);
  const int64_t gl = preload ? nown_max * b * (static_cast<int64_t>(s) * (s - 1) / 2) : 0;
  L.region_len = gl > 2048 ? gl : 2048;
  L.total = L.region + L.region_len;
  return L;
}

template <typename T, int LOSS>
__global__ __launch_bounds__(kThreads) void chain_kernel(ChainArgs a) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  const int s = a.s, b = a.b, Q = a.Q;
  const int sb = s * b;
  const int q = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int nown = (b - q + Q - 1) / Q;  // rows q, q+Q, ... below b
  const ChainLayout L = chain_layout(s, b, Q, a.preload);
  float* rs = sm + L.rs;      // r of all rows done so far
  float* vown = sm + L.vown;  // margins of the own rows
  float* yown = sm + L.yown;  // labels / targets of the own rows
  float* gl = sm + L.region;  // own rows of G, then update scratch
  __shared__ int abort_flag;
  if (threadIdx.x == 0) abort_flag = 0;

  const T* Y = static_cast<const T*>(a.Y);
  const int64_t P = static_cast<int64_t>(b) * (static_cast<int64_t>(s) * (s - 1) / 2);

  // ---- this workgroup's rows of every block-row of G into LDS, 16 loads in
  // flight per lane.  Float4 f of own row t covers block-row j, columns
  // 4k..4k+3 with f - t*P/4 = (b/4) j(j-1)/2 + k; its LDS slot is f itself.
  if (a.preload) {
    const int64_t P4 = P / 4;
    const int64_t T4 = nown * P4;
    const int b4 = b / 4;
    const f32x4* G4 = reinterpret_cast<const f32x4*>(a.G);
    f32x4* gl4 = reinterpret_cast<f32x4*>(gl);
    for (int64_t f0 = threadIdx.x; f0 < T4; f0 += kThreads * 16) {
      f32x4 tmp[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int64_t f = f0 + static_cast<int64_t>(kThreads) * u;
        tmp[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (f < T4) {
          const int t = static_cast<int>(f / P4);
          const int64_t fr = f - t * P4;
          const int64_t chunk = fr / b4;  // = j(j-1)/2 + k/b4
          int j, kb;
          block_of(static_cast<int>(chunk), j, kb);
          const int64_t k4 = fr - static_cast<int64_t>(b4) * (static_cast<int64_t>(j) * (j - 1) / 2);
          const int64_t i = q + static_cast<int64_t>(Q) * t;
          tmp[u] = G4[(static_cast<int64_t>(b) * b * (static_cast<int64_t>(j) * (j - 1) / 2) +
                       i * j * b) / 4 + k4];
        }
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int64_t f = f0 + static_cast<int64_t>(kThreads) * u;
        if (f < T4) gl4[f] = tmp[u];
      }
    }
  }

  // ---- margins of the own rows (row p = (j, t) is minibatch j's row q + Q t)
  chain::margins<T>(
      Y, a.ld, a.n, a.w, s * nown,
      [&](int p) {
        const int j = p / nown;
        return static_cast<int64_t>(j) * b + q + static_cast<int64_t>(Q) * (p - j * nown);
      },
      [&](int p, int64_t row, float v) {
        vown[p] = v;
        yown[p] = a.yB[row];
        a.v[row] = v;
      },
      wave, lane);
  __syncthreads();  // vown and the G rows ready

  // ---- inner recurrence.  Waves 1..3 compute and publish the own rows;
  // wave 0 only polls for the step's r values, so its waits never queue
  // behind another wave's memory traffic.
  const bool vec = (b & 3) == 0;  // G rows are float4-aligned
  for (int j = 0; j < s; ++j) {
    const int jb = j * b;
    if (wave > 0) {
      const float* Gj = a.G + static_cast<int64_t>(b) * b * (static_cast<int64_t>(j) * (j - 1) / 2);
      for (int t = wave - 1; t < nown; t += kWaves - 1) {
        const int i = q + Q * t;
        float acc = 0.f;
        if (a.preload) {
          const f32x4* g4 = reinterpret_cast<const f32x4*>(gl + t * P + static_cast<int64_t>(b) * (static_cast<int64_t>(j) * (j - 1) / 2));
          const f32x4* r4 = reinterpret_cast<const f32x4*>(rs);
          for (int k4 = lane; k4 < (jb >> 2); k4 += 64) {
            const f32x4 g = g4[k4];
            const f32x4 rr = r4[k4];
            acc = fmaf(g.x, rr.x, acc);
            acc = fmaf(g.y, rr.y, acc);
            acc = fmaf(g.z, rr.z, acc);
            acc = fmaf(g.w, rr.w, acc);
          }
        } else if (vec) {
          const f32x4* g4 = reinterpret_cast<const f32x4*>(Gj + static_cast<int64_t>(i) * jb);
          const f32x4* r4 = reinterpret_cast<const f32x4*>(rs);
          const int n4 = jb >> 2;
          for (int k0 = lane; k0 < n4; k0 += 64 * 8) {
            f32x4 g[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              const int k4 = k0 + 64 * u;
              g[u] = k4 < n4 ? g4[k4] : f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              const int k4 = k0 + 64 * u;
              if (k4 < n4) {
                const f32x4 rr = r4[k4];
                acc = fmaf(g[u].x, rr.x, acc);
                acc = fmaf(g[u].y, rr.y, acc);
                acc = fmaf(g[u].z, rr.z, acc);
                acc = fmaf(g[u].w, rr.w, acc);
              }
            }
          }
        } else {
          const float* grow = Gj + static_cast<int64_t>(i) * jb;
          for (int k = lane; k < jb; k += 64) acc = fmaf(grow[k], rs[k], acc);
        }
        acc = group_sum<64>(acc);  // every lane holds the sum
        const int64_t row = jb + i;
        const float zz = vown[j * nown + t] - a.c * acc;
        const float rv = loss_deriv<LOSS>(zz, yown[j * nown + t]);
        const uint64_t word = tagged(a.epoch, rv);
        // one copy per reader: each workgroup polls only its own mailbox
        for (int dst = lane; dst < Q; dst += 64)
          __hip_atomic_store(&a.xbuf[static_cast<int64_t>(dst) * sb + row], word, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        if (lane == 0) {
          a.z[row] = zz;
          a.r[row] = rv;
        }
      }
    } else {
      // collect r_j of every row from this workgroup's mailbox
      const unsigned long long* mbox = a.xbuf + static_cast<int64_t>(q) * sb;
      for (int k = lane; k < b; k += 64) {
        uint64_t x = 0;
        long it = 0;
        while (true) {
          x = __hip_atomic_load(&mbox[jb + k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (static_cast<uint32_t>(x >> 32) == a.epoch) break;
          if (++it > kSpinLimit) {
            abort_flag = 1;
            atomicOr(a.status, 1);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        rs[jb + k] = __uint_as_float(static_cast<uint32_t>(x));
      }
    }
    __syncthreads();
    if (abort_flag) return;
  }

  // ---- update of this workgroup's columns of w; the G rows are no longer needed
  chain::update_columns<T>(Y, a.ld, a.n, sb, rs, a.c, a.w, q, Q, gl);
}

template <typename T, int LOSS>
hipError_t chain_t(const ChainArgs& a, size_t lds, hipStream_t st, const LaunchTimer& tm) {
  // dynamic LDS above the default 64 KB cap must be requested per kernel
  static size_t granted = 64 * 1024;
  if (lds > granted) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chain_kernel<T, LOSS>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
    granted = lds;
  }
  return launch_kernel(chain_kernel<T, LOSS>, dim3(a.Q), dim3(kThreads), lds, st, tm, a);
}

}  // namespace

// Whole-CU LDS per workgroup keeps other kernels' workgroups off the CUs that
// run the recurrence, whose inner steps are latency-bound.
constexpr size_t kLdsBudget = 160 * 1024 - 256;
constexpr size_t kLdsReserve = 136 * 1024;

bool chain_preload(int s, int b, int Q) {
  if ((b & 3) != 0) return false;
  return static_cast<size_t>(chain_layout(s, b, Q, true).total) * sizeof(float) <= kLdsBudget;
}

size_t chain_lds_bytes(int s, int b, int Q) {
  const size_t need = static_cast<size_t>(chain_layout(s, b, Q, chain_preload(s, b, Q)).total) * sizeof(float);
  return need > kLdsReserve ? need : kLdsReserve;
}

int chain_workgroups(int s, int b) {
  (void)s;
  return b < kChainMaxWorkgroups ? b : kChainMaxWorkgroups;
}

hipError_t launch_chain(int storage, int loss, const ChainArgs& a_in, hipStream_t st,
                        const LaunchTimer& tm) {
  ChainArgs a = a_in;
  a.preload = chain_preload(a.s, a.b, a.Q) ? 1 : 0;
  const size_t lds = chain_lds_bytes(a.s, a.b, a.Q);
  if (storage == kStoreBF16) {
    if (loss == kLogistic) return chain_t<uint16_t, kLogistic>(a, lds, st, tm);
    if (loss == kSquared) return chain_t<uint16_t, kSquared>(a, lds, st, tm);
    return chain_t<uint16_t, kPoisson>(a, lds, st, tm);
  }
  if (loss == kLogistic) return chain_t<float, kLogistic>(a, lds, st, tm);
  if (loss == kSquared) return chain_t<float, kSquared>(a, lds, st, tm);
  return chain_t<float, kPoisson>(a, lds, st, tm);
}

}  // namespace casgd
