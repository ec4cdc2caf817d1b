// casgd_train's whole loop of outer iterations in ONE persistent launch.
//
// Every outer step k (Abstract of "Mixed-Precision Communication-Avoiding SGD
// for Generalized Linear Models on GPUs": Gram from low-precision rows with
// float32 accumulation, then the inner recurrence and the weight update in
// float32) is carried out by three kinds of resident workgroups that loop
// over the steps and hand results to each other inside the launch:
//
//   chain   Q workgroups (on one XCD when the layout puts them there): load
//           their rows of G_k into LDS, take the margins v_k, run the inner
//           recurrence (casgd_step.h, the code of the one-step launch) and
//           write their column slice of w_k;
//   margin  workgroups that compute v_k = Y_k w_{k-1} as soon as w_{k-1} is
//           complete and send each margin to the chain as a tagged word;
//   Gram    workgroups that compute the tiles of G_k into a ring of three
//           buffers, up to three steps ahead of the chain.
//
// Nothing gathers Y: every role reads the rows it needs from the stored data
// through the step's sampled indices (read-only data, cached normally), in
// the same summation orders as the one-step launch, so results are
// bit-identical to casgd_outer_step.  What crosses XCDs inside the launch (G,
// the tagged margins and weights, progress words) is written with
// device-scope stores, which write through to memory, and read with
// device-scope loads, which do not take a stale line of their own XCD's L2.
// Progress is published as monotone step tags in per-workgroup words:
//   gprog[g]  Gram workgroup g has written its tiles of step k (tag of k)
//   gfree[q]  chain workgroup q has copied its rows of G_k to LDS
//   wdone[q]  chain workgroup q has written its slice of w_k
// Every wait is bounded; an expired wait sets the status word, which every
// other wait of the launch checks, so a failure ends the launch quickly.
#pragma once

#include "casgd_step.h"

namespace casgd {
namespace persist {

using chain::Elems;
using chain::kThreads;
using chain::tagged;
using step::tri;

constexpr int kRing = 3;  // G buffers: the Gram may run this many steps ahead

struct TrainArgs {
  const void* Xs;        // stored rows, m x ld
  const float* y;        // labels / targets, m
  int64_t m, n, ld;
  int s, b, Q, stride, loss, vround;
  int gbf16;             // the Gram role rounds each entry of G once to bf16
  float c;
  int n_outer;
  uint64_t base_seed, first;  // step k samples with splitmix64(base_seed, first + k)
  float* w;              // weights, in place
  float *v, *z, *r;      // exported margins, z and r of the latest step
  float* G[kRing];       // ring of G buffers (block-row layout)
  unsigned long long* xbuf;   // r of every row, s*b tagged words
  unsigned long long* vbox;   // margins, s*b words
  unsigned long long* wbox;   // new weights, n words
  unsigned long long* place;  // XCD of each chain workgroup
  unsigned long long* prog;   // progress words: gfree[64] | wdone[64] | gprog[...]
  uint32_t tag0;              // tag of step 0; step k uses tag0 + k
  int* status;
  long spin;
  // roles: non-chain workgroups numbered o as in PipeArgs
  int ochain;
  int mar_wgs, mar_rows;      // o in [0, mar_wgs)
  int gram0, gram_wgs;        // o in [gram0, gram0 + gram_wgs)
  int tiles, tps, slots;      // Gram tiles per step; order has `slots` entries per step
  const int* order;           // slot -> tile (-1: none), XCD-grouped
  int dbl;                    // two G buffers in the chain's LDS: G_{k+1} prefetched during step k
  int cus;                    // CUs of the device (host side)
};

__device__ __forceinline__ unsigned long long* gfree(const TrainArgs& A) { return A.prog; }
__device__ __forceinline__ unsigned long long* wdone(const TrainArgs& A) { return A.prog + 64; }
__device__ __forceinline__ unsigned long long* gprog(const TrainArgs& A) { return A.prog + 128; }

__device__ __forceinline__ void publish(unsigned long long* p, uint32_t tag) {
  chain::put(p, static_cast<unsigned long long>(tag));
}

// One wave waits until every word p[0..count) has reached tag `want` (tags
// grow by one per step; words from older launches hold smaller tags).  A
// sleep between polls keeps waiting roles from flooding the memory system.
// False on expiry or when another workgroup has reported a failure.
__device__ __forceinline__ bool wait_all(const unsigned long long* p, int count, uint32_t want, int* status,
                                         long limit, int sleep) {
  const int lane = threadIdx.x & 63;
  long it = 0;
  while (true) {
    bool ok = true;
    for (int k = lane; k < count; k += 64) {
      const uint32_t x = static_cast<uint32_t>(__hip_atomic_load(&p[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      ok = ok && static_cast<int32_t>(x - want) >= 0;
    }
    if (__all(ok)) return true;
    ++it;
    if (it > limit || chain::failed_elsewhere(it, status)) {
      if (lane == 0) atomicOr(status, 1);
      return false;
    }
    if (sleep) __builtin_amdgcn_s_sleep(1);
  }
}

// Row index in the stored data of row `row` of step `seed`'s sample.
__device__ __forceinline__ int64_t sample(uint64_t seed, int row, int64_t m) {
  return sample_row(seed, static_cast<uint64_t>(row), static_cast<uint64_t>(m));
}

// Offset (floats) of the chain's two index lists in LDS: past the layout's
// end, the second G buffer (dbl) and the update's own scratch (dbl with a
// partial-sum region under 2048 floats).
__host__ __device__ inline int64_t idx_offset(const step::Layout& L, int NO, bool dbl, int64_t acc_len) {
  int64_t end = L.total;
  if (dbl) {
    int64_t e2 = L.gl + 2 * NO * L.P + (acc_len < 2048 ? 2048 : 0);
    if (e2 > end) end = e2;
  }
  return (end + 3) & ~3LL;
}

template <typename T, int NO, int CP>
__device__ __forceinline__ void chain_role(const TrainArgs& A, int q) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  const int s = A.s, b = A.b, Q = A.Q;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  const int nown = (b - q + Q - 1) / Q;
  const step::Layout L = step::layout(s, b, NO, CP);
  constexpr int LW = 64 * CP;
  __shared__ int abort_flag;
  __shared__ int r_ready;
  __shared__ int acc_ready[3];
  __shared__ int xloc;
  __shared__ int have_next;  // G_{k+1} is in the other buffer
  __shared__ int pf_state;   // this step's early copy of G_{k+1}: 0 undecided, 1 under way, 2 not taken
  step::RecLds S{sm + L.rs, sm + L.vown, sm + L.yown, sm + L.acc, sm + L.gl, static_cast<int>(L.P),
                 &abort_flag, &r_ready, acc_ready};
  if (threadIdx.x == 0) {
    abort_flag = 0;
    xloc = 0;
    have_next = 0;
    if (A.place) chain::put(&A.place[q], tagged(A.tag0, __uint_as_float(chain::xcd_id())));
  }
  uint64_t place_w = 0;
  if (A.place && wave == 0)
    place_w = __hip_atomic_load(&A.place[lane < Q ? lane : 0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (A.place && wave == 0) {
    ChainArgs pa;  // only the fields the placement check reads
    pa.Q = Q;
    pa.place = A.place;
    pa.epoch = A.tag0;
    pa.status = A.status;
    pa.spin = A.spin;
    const bool all = step::all_on_this_xcd(pa, place_w, &abort_flag);
    if (lane == 0) xloc = all ? 1 : 0;
  }
  const u32x4* X4 = static_cast<const u32x4*>(A.Xs);
  const int64_t cpr = A.ld / Elems<T>::E;
  const int sb = s * b;
  float* gbuf[2] = {S.gl, S.gl + (A.dbl ? NO * S.P : 0)};
  // sampled row indices of the current and the next step, past the chain's
  // layout, the G buffers and the update's scratch (train_lds counts them)
  int* ibuf[2];
  float* ybuf[2];  // labels of the own rows of the current and the next step
  {
    int* base = reinterpret_cast<int*>(sm + idx_offset(L, NO, A.dbl != 0, s * NO * LW));
    ibuf[0] = base;
    ibuf[1] = base + ((sb + 3) & ~3);
    ybuf[0] = S.yown;
    ybuf[1] = reinterpret_cast<float*>(ibuf[1] + ((sb + 3) & ~3));
  }
  for (int p = threadIdx.x; p < sb; p += kThreads)
    ibuf[0][p] = static_cast<int>(sample(splitmix64(A.base_seed, A.first), p, A.m));
  for (int k = 0; k < A.n_outer; ++k) {
    const uint32_t tag = A.tag0 + k;
    float* gl = gbuf[k & 1];
    const int* idx = ibuf[k & 1];
    const bool loaded = have_next != 0;  // (read before the barrier below)
    // G_k complete: every Gram workgroup has passed step k (already checked
    // by the prefetch when it ran)
    if (s > 1 && !loaded && wave == 0 && !wait_all(gprog(A), A.gram_wgs, tag, A.status, A.spin, 0))
      abort_flag = 1;
    __syncthreads();  // (also: this step's indices are in LDS)
    if (abort_flag) break;
    if (s > 1 && !loaded) step::load_g_rows<16>(A.G[k % kRing], gl, s, b, Q, q, nown, S.P);
    for (int i = threadIdx.x; i < s * NO * LW; i += kThreads) S.acc[i] = 0.f;
    if (k == 0)
      for (int p = threadIdx.x; p < s * NO; p += kThreads) {
        const int j = p / NO, t = p - (p / NO) * NO;
        ybuf[0][p] = t < nown ? A.y[idx[j * b + q + Q * t]] : 0.f;
      }
    if (threadIdx.x == 0) {
      r_ready = 0;
      acc_ready[0] = acc_ready[1] = acc_ready[2] = 0;
      have_next = 0;
      pf_state = 0;
    }
    __builtin_amdgcn_s_waitcnt(0);  // G_k (loaded now or prefetched) has landed
    __syncthreads();
    // this workgroup is done with G_k's buffer; published by wave 1, so the
    // critical wave's first poll does not also wait for this store
    if (threadIdx.x == 64) publish(&gfree(A)[q], tag);
    step::Rec R;
    R.s = s;
    R.b = b;
    R.Q = Q;
    R.q = q;
    R.nown = nown;
    R.loss = A.loss;
    R.c = A.c;
    R.tag = tag;
    R.vbox = A.vbox;
    R.xbuf = A.xbuf;
    R.xl = xloc != 0;
    R.z = A.z;
    R.r = A.r;
    R.w = A.w;
    R.wbox = A.wbox;
    R.n = A.n;
    R.ld = A.ld;
    R.status = A.status;
    R.spin = A.spin;
    step::RecLds Sk = S;
    Sk.gl = gl;
    Sk.yown = ybuf[k & 1];
    // the update after the recurrence (if any) must not touch the other G
    // buffer, which may already hold G_{k+1}: scratch in acc when it is large
    // enough, else past both buffers
    if (A.dbl && s * NO * LW < 2048) Sk.red = S.gl + 2 * NO * S.P;
    // G_{k+1} goes into the other buffer early in the step if the Gram has
    // finished it by then (one look), else after wave 1's folds.  A wave's
    // LDS accesses wait for all of its direct-to-LDS copies in flight (about
    // 8 us for these rows, which one XCD streams from memory), so the early
    // copy goes to the wave with the most slack: the update wave when the
    // update runs overlapped (its per-block sums catch up long before the
    // step ends), else wave 1 (before its first fold).  Wave 2, after its
    // folds, draws the next step's row indices and labels.  All of it has
    // landed when the next step starts (its barrier and s_waitcnt).
    const bool upd = step::update_overlapped(b, Q, A.ld, Elems<T>::E);
    auto prefetch = [&](int wv, int phase) {
      if (k + 1 >= A.n_outer) return;
      const bool pre = A.dbl && s >= 2;
      if (phase == 0) {
        if (!pre || wv != (upd ? 3 : 1)) return;
        // one look only: the recurrence must not wait for the Gram
        bool ok = true;
        for (int g = lane; g < A.gram_wgs; g += 64)
          ok = ok && static_cast<int32_t>(static_cast<uint32_t>(__hip_atomic_load(
                         &gprog(A)[g], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) - (tag + 1)) >= 0;
        const bool go = __all(ok);
        // the decision goes out before the copy (a later LDS store would wait for it)
        if (lane == 0) __hip_atomic_store(&pf_state, go ? 1 : 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (!go) return;
        step::load_g_rows<16>(A.G[(k + 1) % kRing], gbuf[(k + 1) & 1], s, b, Q, q, nown, S.P, wv, 1);
        if (lane == 0) have_next = 1;
        return;
      }
      if (wv == 1) {
        // the copy the early look did not take
        if (!pre || !step::lds_wait(&pf_state, 1, &abort_flag, A.status, A.spin) ||
            __hip_atomic_load(&pf_state, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 1)
          return;
        if (!wait_all(gprog(A), A.gram_wgs, tag + 1, A.status, A.spin, 0)) {
          abort_flag = 1;
          return;
        }
        step::load_g_rows<16>(A.G[(k + 1) % kRing], gbuf[(k + 1) & 1], s, b, Q, q, nown, S.P, 1, 1);
        if (lane == 0) have_next = 1;
        return;
      }
      // wave 2
      const uint64_t seed1 = splitmix64(A.base_seed, A.first + static_cast<uint64_t>(k + 1));
      int* nidx = ibuf[(k + 1) & 1];
      for (int p = lane; p < sb; p += 64) nidx[p] = static_cast<int>(sample(seed1, p, A.m));
      // and the labels of the own rows (rows of the next step: own row t of
      // minibatch j is row j*b + q + Q*t)
      float* ny = ybuf[(k + 1) & 1];
      for (int p = lane; p < s * NO; p += 64) {
        const int j = p / NO, t = p - (p / NO) * NO;
        ny[p] = t < nown ? A.y[static_cast<int>(sample(seed1, j * b + q + Q * t, A.m))] : 0.f;
      }
    };
    step::recurrence<T, NO, CP>(R, Sk, [&](int row) { return X4 + static_cast<int64_t>(idx[row]) * cpr; },
                                prefetch);
    // every wave has issued its stores of w_k and its tagged copy; a margin
    // workgroup that comes early re-polls the tagged words
    if (abort_flag) break;
    if (threadIdx.x == 0) publish(&wdone(A)[q], tag);
  }
}

// Margins of rows [mw * mar_rows, ...) of every step.  The step's rows are
// copied to LDS (direct-to-LDS loads) while w_{k-1} is still being formed;
// then every tagged word of w_{k-1} is polled at once (from w itself for the
// first step) and each row's dot product is summed exactly as the one-step
// launch's margin workgroups sum it: lane l takes 16-byte chunks l, l + 64,
// ... in order, element by element, then one wave reduction.
template <typename T>
__device__ __forceinline__ void margin_role(const TrainArgs& A, int mw) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  constexpr int E = Elems<T>::E;
  const int sb = A.s * A.b;
  const int r0 = mw * A.mar_rows;
  const int nrows = sb - r0 < A.mar_rows ? sb - r0 : A.mar_rows;
  if (nrows <= 0) return;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  const int ld = static_cast<int>(A.ld);
  const int cpr = ld / E;
  __shared__ int fail;
  float* wl = sm;                                                  // w_{k-1}, ld floats
  u32x4* rows = reinterpret_cast<u32x4*>(sm + ((ld + 3) & ~3));    // nrows x cpr chunks
  const u32x4* X4 = static_cast<const u32x4*>(A.Xs);
  const f32x4* w4 = reinterpret_cast<const f32x4*>(wl);
  int dummy_abort = 0;
  if (threadIdx.x == 0) fail = 0;
  for (int k = 0; k < A.n_outer; ++k) {
    const uint32_t tag = A.tag0 + k;
    const uint64_t seed = splitmix64(A.base_seed, A.first + static_cast<uint64_t>(k));
    // this step's rows to LDS: row r's chunks are consecutive, so one wave
    // instruction copies up to 64 chunks of one row
    const int per_row = (cpr + 63) / 64;
    for (int g = wave; g < nrows * per_row; g += chain::kWaves) {
      const int r = g / per_row;
      const int c0 = (g - r * per_row) * 64;
      const int c = c0 + lane;
      if (c < cpr) {
        const u32x4* src = X4 + sample(seed, r0 + r, A.m) * cpr + c;
        __builtin_amdgcn_global_load_lds(src, (step::lds_void*)(rows + r * cpr + c0), 16, 0, 0);
      }
    }
    // (no sleep: one load per poll, and the margins are on the critical path)
    if (k > 0 && wave == 0 && !wait_all(wdone(A), A.Q, tag - 1, A.status, A.spin, 0)) fail = 1;
    __syncthreads();
    if (fail) return;
    // w_{k-1}: all of a thread's tagged words polled together
    {
      constexpr int U = 8;
      float x[U];
      uint32_t need = 0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        x[u] = 0.f;
        const int col = threadIdx.x + kThreads * u;
        if (col < A.n && k > 0) need |= 1u << u;
        if (col < A.n && k == 0) x[u] = A.w[col];
      }
      long it = 0;
      while (need) {
        uint64_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int col = threadIdx.x + kThreads * u;
          v[u] = __hip_atomic_load(&A.wbox[col < A.n ? col : 0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (((need >> u) & 1u) && static_cast<uint32_t>(v[u] >> 32) == tag - 1) {
            x[u] = __uint_as_float(static_cast<uint32_t>(v[u]));
            need &= ~(1u << u);
          }
        if (need && (++it > A.spin || chain::failed_elsewhere(it, A.status))) {
          atomicOr(A.status, 1);
          dummy_abort = 1;
          break;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int col = threadIdx.x + kThreads * u;
        if (col < ld) wl[col] = x[u];
      }
      // columns past 8 per thread (ld > 2048) one at a time
      for (int col = threadIdx.x + kThreads * U; col < ld; col += kThreads)
        wl[col] = col >= A.n ? 0.f
                  : k == 0  ? A.w[col]
                            : chain::take(&A.wbox[col], tag - 1, A.status, &dummy_abort, 0, A.spin);
    }
    __builtin_amdgcn_s_waitcnt(0);  // the rows have landed
    __syncthreads();
    if (dummy_abort) fail = 1;
    // a wave's rows (r = wave, wave + 4, ...) four at a time: each weight
    // chunk read once for all of them; every row still sums its own chunks
    // in order
    constexpr int RB = 4;
    for (int r0w = wave; r0w < nrows; r0w += chain::kWaves * RB) {
      float acc[RB];
#pragma unroll
      for (int u = 0; u < RB; ++u) acc[u] = 0.f;
      for (int c = lane; c < cpr; c += 64) {
        float wv[E];
#pragma unroll
        for (int h = 0; h < E / 4; ++h) {
          const f32x4 ww = w4[c * (E / 4) + h];
          wv[4 * h + 0] = ww.x;
          wv[4 * h + 1] = ww.y;
          wv[4 * h + 2] = ww.z;
          wv[4 * h + 3] = ww.w;
        }
#pragma unroll
        for (int u = 0; u < RB; ++u) {
          const int r = r0w + chain::kWaves * u;
          if (r < nrows) {
            float f[E];
            Elems<T>::widen(rows[r * cpr + c], f);
#pragma unroll
            for (int e = 0; e < E; ++e) acc[u] = fmaf(f[e], wv[e], acc[u]);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        const int r = r0w + chain::kWaves * u;
        if (r >= nrows) break;
        float v = group_sum<64>(acc[u]);
        if (lane == 0) {
          v = chain::stored_margin(v, A.vround);
          chain::put(&A.vbox[r0 + r], tagged(tag, v));
          A.v[r0 + r] = v;
        }
      }
    }
    __syncthreads();  // rows and wl are refilled for the next step
    if (fail) return;
  }
}

// Gram workgroup gw: slot p of step k's tile order goes to workgroup
// (k * slots + p) mod gram_wgs, so a slot keeps its XCD whatever the step.
// Before writing buffer k mod kRing the workgroup waits until every chain
// workgroup has copied G_{k - kRing} out of it; after its tiles of step k it
// publishes its progress (also for steps in which it has no tile).
template <typename T, int BK, int D>
__device__ __forceinline__ void gram_role(const TrainArgs& A, int gw) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  __shared__ int fail;
  if (threadIdx.x == 0) fail = 0;
  for (int k = 0; k < A.n_outer; ++k) {
    const uint32_t tag = A.tag0 + k;
    const uint64_t seed = splitmix64(A.base_seed, A.first + static_cast<uint64_t>(k));
    const int64_t base = static_cast<int64_t>(k) * A.slots;
    int p = static_cast<int>((gw - base % A.gram_wgs + A.gram_wgs) % A.gram_wgs);
    if (p < A.slots && k >= kRing && wave == 0 &&
        !wait_all(gfree(A), A.Q, tag - kRing, A.status, A.spin, 1))
      fail = 1;
    __syncthreads();
    if (fail) return;
    auto row_of = [&](int r) { return sample(seed, r, A.m); };
    for (; p < A.slots; p += A.gram_wgs) {
      const int tile = A.order[p];
      if (tile < 0) continue;
      if constexpr (std::is_same<T, float>::value)
        gram::f32_tile<true>(static_cast<const float*>(A.Xs), A.ld, A.b, A.tps, A.G[k % kRing], tile, sm, row_of,
                             A.gbf16 != 0);
      else
        gram::bf16_tile<BK, D, true>(static_cast<const uint16_t*>(A.Xs), A.ld, A.b, A.tps, A.G[k % kRing], tile,
                                     reinterpret_cast<uint16_t*>(sm), row_of, A.gbf16 != 0);
      __syncthreads();  // the tile's LDS is reused by the next one
    }
    __builtin_amdgcn_s_waitcnt(0);  // this workgroup's G stores written through
    __syncthreads();
    if (threadIdx.x == 0) publish(&gprog(A)[gw], tag);
  }
}

template <typename T, int NO, int CP, int BK, int D>
__global__ __launch_bounds__(kThreads) void train_kernel(TrainArgs A) {
  const int wg = blockIdx.x;
  int w;
  if (A.stride == 1) {
    if (wg < A.Q) {
      chain_role<T, NO, CP>(A, wg);
      return;
    }
    w = wg - A.ochain;
    if (w < 0) return;
  } else {
    const int slot = wg / A.stride, x = wg % A.stride;
    if (x == 0) {
      if (slot < A.Q) chain_role<T, NO, CP>(A, slot);
      return;
    }
    w = slot * (A.stride - 1) + x - 1;
  }
  if (w < A.mar_wgs) {
    margin_role<T>(A, w);
    return;
  }
  if (w >= A.gram0 && w < A.gram0 + A.gram_wgs) gram_role<T, BK, D>(A, w - A.gram0);
}

template <typename T, int NO, int CP, int BK, int D>
hipError_t launch_t(const TrainArgs& A, int grid, size_t lds, hipStream_t st, const LaunchTimer& tm) {
  static size_t granted = 64 * 1024;
  const void* fn = reinterpret_cast<const void*>(&train_kernel<T, NO, CP, BK, D>);
  if (lds > granted) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    granted = lds;
  }
  // every workgroup of the launch waits on others: all must be resident
  int occ = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, kThreads, lds);
  if (e != hipSuccess) return e;
  if (static_cast<int64_t>(occ) * A.cus < grid) return hipErrorLaunchOutOfResources;
  return launch_kernel(train_kernel<T, NO, CP, BK, D>, dim3(grid), dim3(kThreads), lds, st, tm, A);
}

template <int NO, int CP>
hipError_t launch_variant(int storage, const TrainArgs& A, int grid, size_t lds, hipStream_t st,
                          const LaunchTimer& tm) {
  if (storage == kStoreF32) return launch_t<float, NO, CP, 0, 0>(A, grid, lds, st, tm);
  if (storage != kStoreBF16) return hipErrorInvalidValue;  // reads stored rows: bf16 and float32 storage only
  switch (gram_variant(A.ld)) {
    case 0: return launch_t<uint16_t, NO, CP, 32, 1>(A, grid, lds, st, tm);
    case 1: return launch_t<uint16_t, NO, CP, 64, 8>(A, grid, lds, st, tm);
    case 2: return launch_t<uint16_t, NO, CP, 64, 4>(A, grid, lds, st, tm);
    default: return launch_t<uint16_t, NO, CP, 64, 2>(A, grid, lds, st, tm);
  }
}

}  // namespace persist
}  // namespace casgd
