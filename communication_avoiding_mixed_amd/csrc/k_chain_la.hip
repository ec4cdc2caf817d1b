// Lookahead form of the weight-dependent kernel (margins, inner recurrence,
// update; Abstract of "Mixed-Precision Communication-Avoiding SGD for
// Generalized Linear Models on GPUs": inner recurrence and weight update in
// high precision, here float32):
//
//   z_j = v_j - c * sum_{t<j} G_{j,t} r_t,   r_j = l'(z_j, y_j),   c = eta / b
//
// splits every z_j into a far part (t < j - d), known d steps ahead, and a
// near part (the d latest blocks).  One critical workgroup (C) computes all b
// rows of every step from the near blocks alone and publishes r_j; M helper
// workgroups own b/M rows each and fold every new r_t into the far sums of
// the later steps, sending
//
//   F'_k = v_k - c * sum_{t < k-d} G_{k,t} r_t
//
// to C as soon as its last term (t = k-d-1) is in.  C then needs no hand-off
// from another workgroup inside a step, and each r_t -> F'_{t+d+1} round trip
// has d steps to complete.  The remaining workgroups (receivers) only collect
// r for the column-sliced update.  Values travel as epoch-tagged 64-bit words;
// every wait is bounded.  All sums run in fixed orders (bit-reproducible).
//
// Exchange buffer (words): C's inbox [s*b] | helper inboxes [M][s*b] | a
// broadcast copy of r [s*b].
#include "casgd_chain.h"

namespace casgd {
namespace {

using chain::Elems;
using chain::kThreads;
using chain::put;
using chain::take;
using chain::tagged;

constexpr int kMaxB = 64;     // rows per minibatch handled by C's lanes
constexpr int kMaxD = 3;      // near blocks per step
constexpr int kBandRegs = 16; // float4 per lane: a third of a band row (d*b/4 <= 48)

struct LaLayout {
  int64_t rs, yb, fbuf, part, band, red, total;  // C
  int64_t hgl, hv, hacc;                          // helpers (after rs)
};

__host__ __device__ inline LaLayout la_layout(int s, int b, int d, int H) {
  LaLayout L;
  const int64_t sb = static_cast<int64_t>(s) * b;
  auto up4 = [](int64_t x) { return (x + 3) & ~3LL; };
  L.rs = 0;
  // critical workgroup
  L.yb = up4(sb);
  L.fbuf = L.yb + up4(sb);
  L.part = L.fbuf + 2 * kMaxB;
  L.band = L.part + 3 * kMaxB;
  L.red = L.band;
  const int64_t c_total = L.red + 8 * kThreads;
  // helpers: own rows of G, then margins and far sums
  const int64_t P = static_cast<int64_t>(b) * (static_cast<int64_t>(s) * (s - 1) / 2);
  L.hgl = up4(sb);
  L.hv = L.hgl + up4(H * P > 8 * kThreads ? H * P : 8 * kThreads);
  L.hacc = L.hv + up4(static_cast<int64_t>(s) * H);
  const int64_t h_total = L.hacc + up4(static_cast<int64_t>(s) * H);
  L.total = c_total > h_total ? c_total : h_total;
  return L;
}

template <typename T, int LOSS>
__global__ __launch_bounds__(kThreads) void chain_la_kernel(ChainArgs a, int d, int M) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  const int s = a.s, b = a.b, Q = a.Q;
  const int sb = s * b;
  const int H = b / M;  // rows per helper
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const LaLayout L = la_layout(s, b, d, H);
  float* rs = sm + L.rs;
  __shared__ int abort_flag;
  if (threadIdx.x == 0) abort_flag = 0;
  __syncthreads();

  const T* Y = static_cast<const T*>(a.Y);
  unsigned long long* inbox_c = a.xbuf;
  unsigned long long* inbox_h = a.xbuf + sb;
  unsigned long long* bcast = a.xbuf + static_cast<int64_t>(M + 1) * sb;
  const int role = blockIdx.x;  // 0: critical, 1..M: helpers, above: receivers
  float* red = nullptr;

  if (role == 0) {
    // ------------------------------------------------------------ critical
    float* yb = sm + L.yb;
    float* fbuf = sm + L.fbuf;
    float* part = sm + L.part;
    red = sm + L.red;
    for (int k = threadIdx.x; k < sb; k += kThreads) yb[k] = a.yB[k];

    // Band of step jj: the d_j = min(jj, d) latest blocks of block-row jj,
    // d_j*b/4 float4 per row.  Wave w' = wave - 1 (waves 1..3) holds, for row
    // `lane`, the float4 k = w' + 3u (u < kBandRegs) of the row in registers;
    // it is loaded two steps before its use, and wave 0 (the poller) issues
    // no loads of its own so its waits never queue behind these.
    const int w3 = wave - 1;
    f32x4 setA[kBandRegs], setB[kBandRegs];
    auto load_band = [&](f32x4 (&set)[kBandRegs], int jj) {
      const int dj = jj < d ? jj : d;
      const int n4r = dj * b / 4;  // float4 per row
      const bool row_ok = wave > 0 && lane < b && jj >= 1 && jj < s;
      const float* rowp = row_ok ? a.G + static_cast<int64_t>(b) * b * (static_cast<int64_t>(jj) * (jj - 1) / 2) +
                                       static_cast<int64_t>(lane) * jj * b + static_cast<int64_t>(jj - dj) * b
                                 : a.G;
#pragma unroll
      for (int u = 0; u < kBandRegs; ++u) {
        const int k = w3 + 3 * u;
        const bool ok = row_ok && k < n4r;
        // lanes with nothing to load read G's first float4, so no address leaves G
        const f32x4 v = *reinterpret_cast<const f32x4*>(ok ? rowp + 4 * k : a.G);
        set[u] = ok ? v : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    };
    load_band(setA, 0);  // step 0 has no band
    load_band(setB, 1);

    // one inner step; `cur` holds band j (loaded two steps ago) and is then
    // refilled with band j + 2
    auto step = [&](int j, f32x4 (&cur)[kBandRegs]) {
      const int jb = j * b;
      if (wave == 0) {
        for (int k = lane; k < b; k += 64)
          fbuf[(j & 1) * kMaxB + k] = take(&inbox_c[jb + k], a.epoch, a.status, &abort_flag, 0, a.spin);
      }
      __syncthreads();
      if (abort_flag) return;
      if (wave > 0) {
        // near part: wave w' sums its third of the band of row `lane`
        const int dj = j < d ? j : d;
        const int n4r = dj * b / 4;
        const f32x4* r4 = reinterpret_cast<const f32x4*>(rs + (j - dj) * b);
        float acc = 0.f;
#pragma unroll
        for (int u = 0; u < kBandRegs; ++u) {
          const int k = w3 + 3 * u;
          if (j >= 1 && k < n4r) {
            const f32x4 g = cur[u];
            const f32x4 rr = r4[k];
            acc = fmaf(g.x, rr.x, acc);
            acc = fmaf(g.y, rr.y, acc);
            acc = fmaf(g.z, rr.z, acc);
            acc = fmaf(g.w, rr.w, acc);
          }
        }
        if (lane < b) part[w3 * kMaxB + lane] = acc;
        load_band(cur, j + 2);
      }
      __syncthreads();
      if (wave == 1 && lane < b) {
        const float near = (part[lane] + part[kMaxB + lane]) + part[2 * kMaxB + lane];
        const float zz = fbuf[(j & 1) * kMaxB + lane] - a.c * near;
        const float rv = loss_deriv<LOSS>(zz, yb[jb + lane]);
        rs[jb + lane] = rv;
        const uint64_t word = tagged(a.epoch, rv);
        for (int h = 0; h < M; ++h) put(&inbox_h[static_cast<int64_t>(h) * sb + jb + lane], word);
        put(&bcast[jb + lane], word);
        a.z[jb + lane] = zz;
        a.r[jb + lane] = rv;
      }
    };
    for (int j0 = 0; j0 < s; j0 += 2) {
      step(j0, setA);
      if (abort_flag) return;
      if (j0 + 1 < s) step(j0 + 1, setB);
      if (abort_flag) return;
    }
    __syncthreads();  // rs complete; the band slots become the update scratch
  } else if (role <= M) {
    // ------------------------------------------------------------- helper
    const int h = role - 1;
    float* gl = sm + L.hgl;
    float* vown = sm + L.hv;
    float* acc = sm + L.hacc;
    red = gl;
    const int64_t P = static_cast<int64_t>(b) * (static_cast<int64_t>(s) * (s - 1) / 2);
    // Own rows of every block-row of G go to LDS: float4 f of own row u covers
    // block-row j, columns 4k.. with f - u*P/4 = (b/4) j(j-1)/2 + k.  The
    // first batch of these loads is issued before the margins so that both
    // are in flight together.
    const int64_t P4 = P / 4;
    const int64_t T4 = H * P4;
    const int b4 = b / 4;
    const f32x4* G4 = reinterpret_cast<const f32x4*>(a.G);
    f32x4* gl4 = reinterpret_cast<f32x4*>(gl);
    f32x4 tmp[16];
    auto load_batch = [&](int64_t f0) {
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int64_t f = f0 + static_cast<int64_t>(kThreads) * u;
        int64_t src = 0;
        if (f < T4) {
          const int uu = static_cast<int>(f / P4);
          const int64_t fr = f - uu * P4;
          int j, kb;
          block_of(static_cast<int>(fr / b4), j, kb);
          const int64_t k4 = fr - static_cast<int64_t>(b4) * (static_cast<int64_t>(j) * (j - 1) / 2);
          const int64_t i = h + static_cast<int64_t>(M) * uu;
          src = (static_cast<int64_t>(b) * b * (static_cast<int64_t>(j) * (j - 1) / 2) + i * j * b) / 4 + k4;
        }
        const f32x4 v = G4[src];
        tmp[u] = f < T4 ? v : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    };
    auto store_batch = [&](int64_t f0) {
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int64_t f = f0 + static_cast<int64_t>(kThreads) * u;
        if (f < T4) gl4[f] = tmp[u];
      }
    };
    load_batch(threadIdx.x);
    // margins of the own rows i = h + M u (row p = (j, u))
    chain::margins<T>(
        Y, a.ld, a.n, a.w, s * H,
        [&](int p) {
          const int j = p / H;
          return static_cast<int64_t>(j) * b + h + static_cast<int64_t>(M) * (p - j * H);
        },
        [&](int p, int64_t row, float v) {
          v = chain::stored_margin(v, a.vround);
          vown[p] = v;
          a.v[row] = v;
        },
        wave, lane);
    for (int k = threadIdx.x; k < s * H; k += kThreads) acc[k] = 0.f;
    __syncthreads();
    // steps with no far part: F' = v, sent at once (after every margin is read)
    for (int p = threadIdx.x; p < s * H; p += kThreads) {
      const int j = p / H;
      if (j <= d) put(&inbox_c[j * b + h + M * (p - j * H)], tagged(a.epoch, vown[p]));
    }
    store_batch(threadIdx.x);
    for (int64_t f0 = threadIdx.x + kThreads * 16; f0 < T4; f0 += kThreads * 16) {
      load_batch(f0);
      store_batch(f0);
    }
    __syncthreads();
    // G_{k,t} row i_u (b floats) in LDS
    auto grow = [&](int u, int k, int t) {
      return gl + u * P + static_cast<int64_t>(b) * (static_cast<int64_t>(k) * (k - 1) / 2) +
             static_cast<int64_t>(t) * b;
    };
    const int lpr = 64 / H;  // lanes per own row in the urgent dot
    for (int t = 0; t < s; ++t) {
      const int tb = t * b;
      if (wave == 0) {
        for (int k = lane; k < b; k += 64)
          rs[tb + k] = take(&inbox_h[static_cast<int64_t>(h) * sb + tb + k], a.epoch, a.status, &abort_flag, 0, a.spin);
      }
      __syncthreads();
      if (abort_flag) return;
      const int ku = t + d + 1;  // the step whose far part r_t completes
      if (wave == 1 && ku < s) {
        const int u = lane / lpr;
        const int l = lane - u * lpr;
        float dot = 0.f;
        if (u < H) {
          const float* g = grow(u, ku, t);
          for (int k = l; k < b; k += lpr) dot = fmaf(g[k], rs[tb + k], dot);
        }
        // sum over the lpr lanes of the row (lpr is 16, 32 or 64)
        for (int o = lpr / 2; o > 0; o >>= 1) dot += __shfl_xor(dot, o, lpr);
        if (u < H && l == 0) {
          const float far = acc[ku * H + u] + dot;
          acc[ku * H + u] = far;
          put(&inbox_c[ku * b + h + M * u], tagged(a.epoch, vown[ku * H + u] - a.c * far));
        }
      } else if (wave >= 2) {
        // the later steps' far sums: one (step, row) pair per lane
        const int npairs = (s - (ku + 1)) * H;
        for (int pr = threadIdx.x - 128; pr < npairs; pr += 128) {
          const int k = ku + 1 + pr / H;
          const int u = pr - (k - ku - 1) * H;
          const float* g = grow(u, k, t);
          float dot = 0.f;
          for (int c4 = 0; c4 < b; c4 += 4) {
            const f32x4 gg = *reinterpret_cast<const f32x4*>(g + c4);
            const f32x4 rr = *reinterpret_cast<const f32x4*>(rs + tb + c4);
            dot = fmaf(gg.x, rr.x, dot);
            dot = fmaf(gg.y, rr.y, dot);
            dot = fmaf(gg.z, rr.z, dot);
            dot = fmaf(gg.w, rr.w, dot);
          }
          acc[k * H + u] += dot;
        }
      }
    }
    __syncthreads();
  } else {
    // ----------------------------------------------------------- receiver
    red = sm + L.yb;  // unused by receivers otherwise
    for (int k = threadIdx.x; k < sb; k += kThreads) {
      rs[k] = take(&bcast[k], a.epoch, a.status, &abort_flag, 1, a.spin);
      if (abort_flag) break;
    }
    __syncthreads();
    if (abort_flag) return;
  }

  // ---- update of this workgroup's columns of w (every workgroup holds all r)
  chain::update_columns<T>(Y, a.ld, a.n, sb, rs, a.c, a.w, blockIdx.x, Q, red);
}

template <typename T, int LOSS>
hipError_t la_t(const ChainArgs& a, int d, int M, size_t lds, hipStream_t st, const LaunchTimer& tm) {
  static size_t granted = 64 * 1024;
  if (lds > granted) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chain_la_kernel<T, LOSS>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    granted = lds;
  }
  return launch_kernel(chain_la_kernel<T, LOSS>, dim3(a.Q), dim3(kThreads), lds, st, tm, a, d, M);
}

constexpr size_t kLaLdsBudget = 160 * 1024 - 256;
constexpr size_t kLaLdsReserve = 136 * 1024;

}  // namespace

LaPlan la_plan(int s, int b) {
  LaPlan p;
  if (s < 2 || b < 16 || b > kMaxB || b % 16 != 0) return p;
  const int d = s - 1 < kMaxD ? s - 1 : kMaxD;
  // two rows per helper first (their preload and margins start fast), then one, then four
  for (int H : {2, 1, 4}) {
    if (b % H) continue;
    const int M = b / H;
    if (M + 1 > kChainMaxWorkgroups) continue;
    const size_t need = static_cast<size_t>(la_layout(s, b, d, H).total) * sizeof(float);
    if (need <= kLaLdsBudget) {
      p.ok = true;
      p.d = d;
      p.M = M;
      p.lds = need > kLaLdsReserve ? need : kLaLdsReserve;
      return p;
    }
  }
  return p;
}

hipError_t launch_chain_la(int storage, int loss, const ChainArgs& a, const LaPlan& p,
                           hipStream_t st, const LaunchTimer& tm) {
  if (storage == kStoreBF16) {
    if (loss == kLogistic) return la_t<uint16_t, kLogistic>(a, p.d, p.M, p.lds, st, tm);
    if (loss == kSquared) return la_t<uint16_t, kSquared>(a, p.d, p.M, p.lds, st, tm);
    return la_t<uint16_t, kPoisson>(a, p.d, p.M, p.lds, st, tm);
  }
  if (storage == kStoreF16) {
    if (loss == kLogistic) return la_t<_Float16, kLogistic>(a, p.d, p.M, p.lds, st, tm);
    if (loss == kSquared) return la_t<_Float16, kSquared>(a, p.d, p.M, p.lds, st, tm);
    return la_t<_Float16, kPoisson>(a, p.d, p.M, p.lds, st, tm);
  }
  if (loss == kLogistic) return la_t<float, kLogistic>(a, p.d, p.M, p.lds, st, tm);
  if (loss == kSquared) return la_t<float, kSquared>(a, p.d, p.M, p.lds, st, tm);
  return la_t<float, kPoisson>(a, p.d, p.M, p.lds, st, tm);
}

}  // namespace casgd
