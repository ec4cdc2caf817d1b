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
// memory per inner step, no barriers, no separate flags).  The fast path
// writes each value once into one array that every reader polls (measured
// 2% faster at b = 128, s = 32 than a copy per reader); the general path
// writes one mailbox per reading workgroup.  Every spin is bounded: on
// expiry the kernel flags an error in `status` and returns.
// After the last inner step every workgroup holds all of r and updates its
// own slice of columns of w in a fixed summation order (no float atomics).
#include <type_traits>

#include "casgd_chain.h"
#include "casgd_gather.h"
#include "casgd_gram.h"

namespace casgd {
namespace {

using chain::Elems;
using chain::kThreads;
using chain::kWaves;
using chain::tagged;

// LDS layout (floats): rs[sb] | vown[s * nown_max] | yown[s * nown_max] |
// acc[s * nown_max * 64 * cpl] (b <= kFastMaxB) | region, where region holds
// this workgroup's rows of G (when a.preload) during the recurrence and the
// update's reduction scratch afterwards.
// Whole-CU LDS per workgroup keeps other kernels' workgroups off the CUs that
// run the recurrence, whose inner steps are latency-bound.
constexpr size_t kLdsBudget = 160 * 1024 - 256;
constexpr size_t kLdsReserve = 136 * 1024;
// Explicit address spaces keep the two sources of a G element from being
// merged into one generic (flat) load.
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(1))) float global_f32;
constexpr int kFastMaxB = 256;  // per-lane accumulators: up to 4 columns per lane
constexpr int kMaxCpl = kFastMaxB / 64;
constexpr int kMaxOwn = 4;      // own rows per minibatch on the fast path

// Columns per lane of the fast-path variant chain_body runs for nown_max own
// rows and cpl = ceil(b / 64) columns per lane (also the accumulators' pitch
// in units of 64 floats).
__host__ __device__ inline int fast_cols(int64_t nown_max, int64_t cpl) {
  return (nown_max == 1 && cpl == 1) ? 1 : (nown_max <= 2 && cpl <= 2) ? 2 : kMaxCpl;
}

using chain::kWlMax;
using chain::margins_wlds;

struct ChainLayout {
  int64_t rs, vown, yown, acc, acc_len, region, region_len, wl, wl_len, total;
};

__host__ __device__ inline ChainLayout chain_layout(int s, int b, int Q, int64_t ld, bool preload) {
  ChainLayout L;
  const int64_t sb = static_cast<int64_t>(s) * b;
  const int64_t nown_max = (b + Q - 1) / Q;
  const int64_t cpl = fast_cols(nown_max, (b + 63) / 64);
  L.rs = 0;
  L.vown = (sb + 3) & ~3LL;
  L.yown = L.vown + ((s * nown_max + 3) & ~3LL);
  L.acc = L.yown + ((s * nown_max + 3) & ~3LL);
  // the fast path needs its accumulators next to the update scratch
  const int64_t acc_len = s * nown_max * 64 * cpl;
  const bool fits = (L.acc + acc_len + 2048) * 4 <= static_cast<int64_t>(kLdsBudget);
  L.acc_len = (b <= kFastMaxB && nown_max <= kMaxOwn && fits) ? acc_len : 0;
  L.region = L.acc + L.acc_len;
  const int64_t gl = preload ? nown_max * b * (static_cast<int64_t>(s) * (s - 1) / 2) : 0;
  L.region_len = gl > 2048 ? gl : 2048;
  L.wl = L.region + L.region_len;
  L.wl_len = ld <= kWlMax ? ld : 0;
  L.total = L.wl + L.wl_len;
  return L;
}

// Spin (bounded) until the LDS word *flag reaches `want` or the workgroup
// aborts; false on abort or expiry.
__device__ __forceinline__ bool lds_wait(const int* flag, int want, int* abort_flag, int* status, long limit) {
  long it = 0;
  while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < want) {
    if (__hip_atomic_load(abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) return false;
    if (++it > limit) {
      *abort_flag = 1;
      atomicOr(status, 1);
      return false;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  return true;
}

// Publish `v` to the LDS word *flag after this wave's earlier LDS writes
// (an LDS-only release: global stores in flight are not waited for).
__device__ __forceinline__ void lds_publish(int* flag, int v) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __hip_atomic_store(flag, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// This workgroup's rows of every block-row of G, copied to LDS: own row t of
// block-row j is a contiguous run of j*b/4 float4 in G and in LDS (at
// t*P/4 + (b/4) j(j-1)/2).  Slots enumerate (t, j, c4) on power-of-two
// strides so a slot decodes with shifts; slots past a run's end are skipped.
struct GPreload {
  const f32x4* G4;
  f32x4* gl4;
  int64_t T4, P4;  // slots (0: nothing to copy), float4 per own row
  int lgW, lgJ, s, b, b4, q, Q;

  __device__ __forceinline__ bool slot(int64_t g, int64_t& src, int64_t& dst) const {
    const int c4 = static_cast<int>(g & ((1 << lgW) - 1));
    const int j = 1 + static_cast<int>((g >> lgW) & ((1 << lgJ) - 1));
    const int t = static_cast<int>(g >> (lgW + lgJ));
    if (g >= T4 || j >= s || c4 >= j * b4) return false;
    const int64_t tri = static_cast<int64_t>(j) * (j - 1) / 2;
    const int64_t i = q + static_cast<int64_t>(Q) * t;
    src = (static_cast<int64_t>(b) * b * tri + i * j * b) / 4 + c4;
    dst = t * P4 + b4 * tri + c4;
    return true;
  }
  // N slots g0, g0 + stride, ...: unconditional loads (skipped slots read
  // G's first float4), then the stores of the slots that exist
  template <int N>
  __device__ __forceinline__ void issue(f32x4 (&tmp)[N], int64_t g0, int stride) const {
#pragma unroll
    for (int u = 0; u < N; ++u) {
      int64_t src = 0, dst = 0;
      slot(g0 + static_cast<int64_t>(stride) * u, src, dst);
      tmp[u] = G4[src];
    }
  }
  template <int N>
  __device__ __forceinline__ void store(const f32x4 (&tmp)[N], int64_t g0, int stride) const {
#pragma unroll
    for (int u = 0; u < N; ++u) {
      int64_t src = 0, dst = 0;
      if (slot(g0 + static_cast<int64_t>(stride) * u, src, dst)) gl4[dst] = tmp[u];
    }
  }
};

// Everything a fast-path recurrence needs from chain_body.
struct FastCtx {
  const ChainArgs* a;
  int q, nown, nown_max, lane, wave;
  float *rs, *vown, *yown, *acc, *gl;
  int64_t P;
  int *abort_flag, *r_ready, *acc_ready;
  const unsigned long long* mbox;
  bool xl;  // every chain workgroup on this one's XCD: r goes out with plain stores
};

constexpr int kUpdRows = 4;  // rows per lane per block the update wave prefetches

// Inner recurrence, fast path, for at most NO own rows per minibatch and CP
// columns per lane (b <= 64 CP).  Wave 0 alone is on the critical path: it
// collects r of block j-1 from its mailbox (lane l holds columns l, l+64,
// ...), finishes z of its rows of block j with the one block G_{j,j-1} on
// top of the per-lane partial sums, reduces once, and publishes r.  The fold
// waves fold each block t of r into the per-lane partial sums of the rows of
// blocks k >= t+2 while wave 0 waits for the next block, so
//   z_j = v_j - c * sum_lanes(acc_j + G_{j,j-1} r_{j-1}).
// Waves 1..3 fold (block k to wave 1 + k mod 3).  When the workgroup's column
// slice of w allows (at most 64 chunks, at most kUpdRows rows per lane per
// block), wave 3 also accumulates the update Y^T r of its columns block by
// block as r arrives (the rows of the next block prefetched), reduces over
// its lanes and writes w, and the function returns true; otherwise the
// caller runs the update afterwards.
// PRE: where the rows of G are, 1 in LDS (a.preload), 0 in global memory,
// fixed at compile time so the critical wave's loop carries no branch on
// it; 2 reads a.preload at run time.  Measured on MI355X, the compile-time
// forms are 3-10% faster per step for 2 and 4 rows per workgroup and the
// run-time form 8% faster for one row and one column per lane, so each
// variant is launched in its faster form.
template <typename T, int LOSS, int NO, int CP, int PRE>
__device__ __forceinline__ bool recurrence_fast(const FastCtx& x) {
  const ChainArgs& a = *x.a;
  const int s = a.s, b = a.b, Q = a.Q, sb = s * b;
  const int q = x.q, nown = x.nown, nown_max = x.nown_max, lane = x.lane;
  float* rs = x.rs;
  const float* vown = x.vown;  // (wave 0 fills it first when a.vbox is set)
  const float* yown = x.yown;
  float* acc = x.acc;
  int& abort_flag = *x.abort_flag;
  int& r_ready = *x.r_ready;
  int* acc_ready = x.acc_ready;
  const unsigned long long* mbox = x.mbox;
  auto gval = [&](int k, int t, int col) -> float {
    const int64_t tri = static_cast<int64_t>(k) * (k - 1) / 2;
    if (PRE == 1 || (PRE == 2 && a.preload)) return ((const lds_f32*)x.gl)[t * x.P + static_cast<int64_t>(b) * tri + col];
    const int64_t i = q + static_cast<int64_t>(Q) * t;
    return ((const global_f32*)a.G)[static_cast<int64_t>(b) * b * tri + i * k * b + col];
  };
  const int wave = x.wave;
  const int wv = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform
  constexpr int LWc = 64 * CP;  // acc row pitch
  // the update plan (same in every wave)
  constexpr int E = Elems<T>::E;
  const int64_t cpr = a.ld / E;
  const int64_t per = (cpr + Q - 1) / Q;
  int cw = 1;
  while (cw < per && cw < 64) cw <<= 1;
  const int rgw = 64 / cw;
  const int rpl = (b + rgw - 1) / rgw;
  const bool upd = per <= 64 && rpl <= kUpdRows;
  const int nf = kWaves - 1;  // fold waves
  if (wv == 0) {
    if (a.vbox) {
      // margins of the own rows, from the launch's margin workgroups (they
      // finish together, so all are taken at once; only this wave uses them)
      float* vw = x.vown;
      for (int p = lane; p < s * nown; p += 64) {
        const int j = p / nown, t = p - (p / nown) * nown;
        vw[j * nown_max + t] = chain::take(&a.vbox[static_cast<int64_t>(j) * b + q + Q * t], a.epoch, a.status, &abort_flag, 0, a.spin);
      }
    }
    float rp[CP];
#pragma unroll
    for (int u = 0; u < CP; ++u) rp[u] = 0.f;
    for (int j = 0; j < s; ++j) {
      const int jb = j * b;
      // everything of step j that does not depend on r of block j-1 is
      // read before the wait: G_{j,j-1} of the own rows, their margins and
      // labels, and their partial sums if the helper has finished them
      float gv[NO][CP], av[NO][CP], vj[NO], yj[NO];
      const int* ready = &acc_ready[j % nf];
      const bool acc_now = j < 2 || __hip_atomic_load(ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= j - 1;
      if (acc_now) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
#pragma unroll
      for (int t = 0; t < NO; ++t) {
        vj[t] = t < nown ? vown[j * nown_max + t] : 0.f;
        yj[t] = t < nown ? yown[j * nown_max + t] : 0.f;
#pragma unroll
        for (int u = 0; u < CP; ++u) {
          const int l = lane + 64 * u;
          const bool on = j > 0 && t < nown && l < b;
          gv[t][u] = on ? gval(j, t, (j - 1) * b + l) : 0.f;
          av[t][u] = (on && acc_now) ? acc[(j * nown_max + t) * LWc + l] : 0.f;
        }
      }
      if (j > 0) {
        chain::take_n<CP>(&mbox[jb - b], lane, b, a.epoch, rp, a.status, &abort_flag, a.spin);
#pragma unroll
        for (int u = 0; u < CP; ++u) {
          const int l = lane + 64 * u;
          if (l < b) rs[jb - b + l] = rp[u];
        }
        lds_publish(&r_ready, j);
        if (!acc_now) {
          if (!lds_wait(ready, j - 1, &abort_flag, a.status, a.spin)) break;
#pragma unroll
          for (int t = 0; t < NO; ++t)
#pragma unroll
            for (int u = 0; u < CP; ++u) {
              const int l = lane + 64 * u;
              if (t < nown && l < b) av[t][u] = acc[(j * nown_max + t) * LWc + l];
            }
        }
      }
#pragma unroll
      for (int t = 0; t < NO; ++t) {
        if (t >= nown) break;
        const int i = q + Q * t;
        float part = 0.f;
#pragma unroll
        for (int u = 0; u < CP; ++u)
          part += fmaf(gv[t][u], rp[u], av[t][u]);
        const float tot = wave_sum(part);
        const int64_t row = jb + i;
        const float zz = vj[t] - a.c * tot;
        const float rv = loss_deriv<LOSS>(zz, yj[t]);
        const uint64_t word = tagged(a.epoch, rv);
        if (lane == 0) chain::put_x(&a.xbuf[row], word, x.xl);
        if (lane == 0) {
          a.z[row] = zz;
          a.r[row] = rv;
        }
      }
      // a wait that expired ends the loop (its zero values went out with the
      // step, but the status word reports the failure)
      if (abort_flag) break;
    }
    // the last block's r, for the update
    if (!abort_flag) {
      const int jb = (s - 1) * b;
      float rl[CP];
      chain::take_n<CP>(&mbox[jb], lane, b, a.epoch, rl, a.status, &abort_flag, a.spin);
#pragma unroll
      for (int u = 0; u < CP; ++u)
        if (lane + 64 * u < b) rs[jb + lane + 64 * u] = rl[u];
      if (!abort_flag) lds_publish(&r_ready, s);
    }
  } else {
    // fold wave h = wv - 1 owns the rows of the blocks k = h (mod 3); after
    // r of block tb is in, it folds G_{k,tb} r_tb into their partial sums
    // for every k >= tb + 2, two blocks at a time with all loads issued first
    const int h = wv - 1;
    // G in global memory (rows too large for LDS): up to NBW blocks' loads
    // are all issued (clamped, unconditional) before any is used, so a fold
    // step waits about one memory latency per batch, not one per pair.  Past
    // the last block the clamped loads are wasted, so the batch is kept
    // short: on MI355X at b = 128, s = 32 batches of 3 / 4 / 6 / 8 / 12 / 16
    // blocks gave 101 / 97.6 / 97.3 / 97.6 / 103.7 / 116 us per outer step.
    // The loads do not depend on r, so the first batch of fold(tb), and the
    // second when the fold has one, are issued before the wait for r of block
    // tb (g0, g1) and their latency overlaps it.
    constexpr int NBW = NO * CP <= 4 ? 6 : 3;
    const bool glob = PRE == 0 || (PRE == 2 && !a.preload);
    float g0[NBW][NO][CP], g1[NBW][NO][CP];
    bool two = false;  // g1 holds the second batch of the coming fold
    auto first_k = [&](int tb) {
      int k0 = tb + 2;
      return k0 + (h - k0 % nf + nf) % nf;  // first k >= tb+2 with k = h (mod nf)
    };
    auto load_batch = [&](int tb, int k, float (&gb)[NBW][NO][CP]) {
#pragma unroll
      for (int e = 0; e < NBW; ++e) {
        const int kk = k + e * nf;
        const int kc = kk < s ? kk : s - 1;
#pragma unroll
        for (int t = 0; t < NO; ++t)
#pragma unroll
          for (int u = 0; u < CP; ++u) {
            const int l = lane + 64 * u;
            gb[e][t][u] = gval(kc, t < nown ? t : 0, tb * b + (l < b ? l : 0));
          }
      }
    };
    auto use_batch = [&](int k, const float (&gb)[NBW][NO][CP], const float (&rr)[CP]) {
#pragma unroll
      for (int e = 0; e < NBW; ++e) {
        const int kk = k + e * nf;
#pragma unroll
        for (int t = 0; t < NO; ++t)
#pragma unroll
          for (int u = 0; u < CP; ++u) {
            const int l = lane + 64 * u;
            if (kk < s && t < nown && l < b) {
              float* ap = &acc[(kk * nown_max + t) * LWc + l];
              *ap = fmaf(gb[e][t][u], rr[u], *ap);
            }
          }
      }
    };
    // before the wait for r of block tb: the first one or two batches of
    // fold(tb)
    auto pre_load = [&](int tb) {
      if (glob && tb + 2 < s) {
        const int k0 = first_k(tb);
        load_batch(tb, k0, g0);
        two = k0 + NBW * nf < s;
        if (two) load_batch(tb, k0 + NBW * nf, g1);
      }
    };
    // after r of block tb is in: fold G_{k,tb} r_tb into the partial sums of
    // this wave's blocks k >= tb + 2 (pre_load(tb) ran first)
    auto fold = [&](int tb) {
      float rr[CP];
#pragma unroll
      for (int u = 0; u < CP; ++u) {
        const int l = lane + 64 * u;
        rr[u] = (l < b) ? rs[tb * b + l] : 0.f;
      }
      const int k0 = first_k(tb);
      if (glob) {
        int k = k0;
        if (k < s) {
          use_batch(k, g0, rr);
          k += NBW * nf;
        }
        if (two) {
          use_batch(k, g1, rr);
          k += NBW * nf;
        }
        for (; k < s; k += NBW * nf) {
          float gb[NBW][NO][CP];
          load_batch(tb, k, gb);
          use_batch(k, gb, rr);
        }
        lds_publish(&acc_ready[h], tb + 1);
        return;
      }
      for (int k = k0; k < s; k += 2 * nf) {
        float gb[2][NO][CP], ab[2][NO][CP];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int kk = k + e * nf;
#pragma unroll
          for (int t = 0; t < NO; ++t)
#pragma unroll
            for (int u = 0; u < CP; ++u) {
              const int l = lane + 64 * u;
              const bool on = kk < s && t < nown && l < b;
              gb[e][t][u] = on ? gval(kk, t, tb * b + l) : 0.f;
              ab[e][t][u] = on ? acc[(kk * nown_max + t) * LWc + l] : 0.f;
            }
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int kk = k + e * nf;
#pragma unroll
          for (int t = 0; t < NO; ++t)
#pragma unroll
            for (int u = 0; u < CP; ++u) {
              const int l = lane + 64 * u;
              if (kk < s && t < nown && l < b)
                acc[(kk * nown_max + t) * LWc + l] = fmaf(gb[e][t][u], rr[u], ab[e][t][u]);
            }
        }
      }
      lds_publish(&acc_ready[h], tb + 1);
    };
    if (!(upd && wv == kWaves - 1)) {
      for (int tb = 0; tb + 2 < s; ++tb) {
        pre_load(tb);
        if (!lds_wait(&r_ready, tb + 1, &abort_flag, a.status, a.spin)) break;
        fold(tb);
      }
    } else {
      // the last wave also accumulates the update of this workgroup's chunks
      // [ch0, ch1) of w: lane = (rgl, cl) sums rows rgl, rgl + rgw, ... of
      // every block for chunk ch0 + cl, right after folding the block
      const int64_t ch0 = static_cast<int64_t>(q) * per;
      const int64_t ch1 = ch0 + per < cpr ? ch0 + per : cpr;
      const int cl = lane % cw, rgl = lane / cw;
      const int64_t ch = ch0 + cl;
      const bool col_ok = ch < ch1;
      const u32x4* Y4 = reinterpret_cast<const u32x4*>(a.Y);
      float accw[E];
#pragma unroll
      for (int e = 0; e < E; ++e) accw[e] = 0.f;
      // rows of block tb (clamped to the last block) for this lane, unconditional loads
      auto load_blk = [&](int tb, u32x4 (&dst)[kUpdRows]) {
        const int tbc = tb < s ? tb : s - 1;
#pragma unroll
        for (int i = 0; i < kUpdRows; ++i) {
          const int rl = rgl + rgw * i;
          const bool ok = i < rpl && rl < b && col_ok;
          dst[i] = Y4[(ok ? static_cast<int64_t>(tbc) * b + rl : 0) * cpr + (ok ? ch : 0)];
        }
      };
      auto step = [&](int tb, const u32x4 (&src)[kUpdRows]) -> bool {
        pre_load(tb);
        if (!lds_wait(&r_ready, tb + 1, &abort_flag, a.status, a.spin)) return false;
        if (tb + 2 < s) fold(tb);
#pragma unroll
        for (int i = 0; i < kUpdRows; ++i) {
          const int rl = rgl + rgw * i;
          if (i < rpl && rl < b && col_ok) {
            const float rr = rs[tb * b + rl];
            float f[E];
            Elems<T>::widen(src[i], f);
#pragma unroll
            for (int e = 0; e < E; ++e) accw[e] = fmaf(f[e], rr, accw[e]);
          }
        }
        return true;
      };
      u32x4 ya[kUpdRows], yb[kUpdRows];
      load_blk(0, ya);
      bool ok = true;
      for (int tb = 0; tb < s; tb += 2) {
        load_blk(tb + 1, yb);
        ok = step(tb, ya);
        if (!ok || tb + 1 >= s) break;
        load_blk(tb + 2, ya);
        ok = step(tb + 1, yb);
        if (!ok) break;
      }
      if (ok) {
        for (int off = cw; off < 64; off <<= 1)
#pragma unroll
          for (int e = 0; e < E; ++e) accw[e] += __shfl_xor(accw[e], off, 64);
        if (rgl == 0 && col_ok) {
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const int64_t col = ch * E + e;
            if (col < a.n) a.w[col] = a.w[col] - a.c * accw[e];
          }
        }
      }
    }
  }
  return upd;
}

// The work of workgroup q (0 <= q < a.Q); called by all 256 lanes.
template <typename T, int LOSS>
__device__ __forceinline__ void chain_body(const ChainArgs& a, int q) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  const int s = a.s, b = a.b, Q = a.Q;
  const int sb = s * b;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int nown = (b - q + Q - 1) / Q;  // rows q, q+Q, ... below b
  const int nown_max = (b + Q - 1) / Q;
  const ChainLayout L = chain_layout(s, b, Q, a.ld, a.preload);
  const bool fast = L.acc_len > 0;
  const int cpl = (b + 63) / 64;
  float* rs = sm + L.rs;      // r of all rows done so far
  float* vown = sm + L.vown;  // margins of the own rows
  float* yown = sm + L.yown;  // labels / targets of the own rows
  float* acc = sm + L.acc;    // per-lane partial sums of the own rows (fast path)
  float* gl = sm + L.region;  // own rows of G, then update scratch
  __shared__ int abort_flag;
  __shared__ int r_ready;                  // blocks whose r is in rs (wave 0)
  __shared__ int acc_ready[kWaves - 1];    // blocks folded into acc (waves 1..3)
  __shared__ int xloc;                     // all chain workgroups on this XCD
  if (threadIdx.x == 0) {
    abort_flag = 0;
    r_ready = 0;
    xloc = 0;
    for (int k = 0; k < kWaves - 1; ++k) acc_ready[k] = 0;
    // where this workgroup runs, for the others' choice of store
    if (a.place) chain::put(&a.place[q], tagged(a.epoch, __uint_as_float(chain::xcd_id())));
  }
  // every chain workgroup's XCD, read early by wave 0 and checked below
  uint64_t place_w = 0;
  if (a.place && wave == 0)
    place_w = __hip_atomic_load(&a.place[lane < Q ? lane : 0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int64_t k = threadIdx.x; k < L.acc_len; k += kThreads) acc[k] = 0.f;

  const T* Y = static_cast<const T*>(a.Y);
  const int64_t P = static_cast<int64_t>(b) * (static_cast<int64_t>(s) * (s - 1) / 2);

  // ---- this workgroup's rows of G to LDS (when a.preload), the first batch
  // in flight beside the margins' loads.
  GPreload gp;
  gp.G4 = reinterpret_cast<const f32x4*>(a.G);
  gp.gl4 = reinterpret_cast<f32x4*>(gl);
  gp.P4 = P / 4;
  gp.s = s;
  gp.b = b;
  gp.b4 = b / 4;
  gp.q = q;
  gp.Q = Q;
  gp.lgW = 0;
  gp.lgJ = 0;
  while ((1 << gp.lgW) < (s - 1) * gp.b4) ++gp.lgW;
  while ((1 << gp.lgJ) < s - 1) ++gp.lgJ;
  gp.T4 = (a.preload && s > 1) ? static_cast<int64_t>(nown) << (gp.lgW + gp.lgJ) : 0;
  const int64_t T4 = gp.T4;
  constexpr int kGB = 8;  // float4 per lane per preload batch
  {
    // own row p = (j, t) is minibatch j's row q + Q t; its label is loaded
    // now and stored after the margins, so the load overlaps them
    const int nrows = s * nown;
    auto row_of = [&](int p) {
      const int j = p / nown;
      return static_cast<int64_t>(j) * b + q + static_cast<int64_t>(Q) * (p - j * nown);
    };
    auto slot_of = [&](int p) {
      const int j = p / nown;
      return j * nown_max + (p - j * nown);
    };
    // (an unconditional load: a load under a branch is waited for at the join)
    const int yp = static_cast<int>(threadIdx.x) < nrows ? static_cast<int>(threadIdx.x) : nrows - 1;
    const float ylab = a.yB[row_of(yp)];
    f32x4 tmp[kGB];
    auto out = [&](int p, int64_t row, float v) {
      v = chain::stored_margin(v, a.vround);
      vown[slot_of(p)] = v;
      a.v[row] = v;
    };
    auto more = [&] {
      if (T4 > 0) gp.issue<kGB>(tmp, threadIdx.x, kThreads);
    };
    if (a.vbox)
      more();  // margins are computed by other workgroups of the launch
    else if (L.wl_len > 0)
      margins_wlds<T>(Y, a.ld, a.n, a.w, nrows, row_of, out, sm + L.wl, more);
    else
      chain::margins<T>(Y, a.ld, a.n, a.w, nrows, row_of, out, wave, lane, more);
    if (static_cast<int>(threadIdx.x) < nrows) yown[slot_of(threadIdx.x)] = ylab;
    for (int p = threadIdx.x + kThreads; p < nrows; p += kThreads) yown[slot_of(p)] = a.yB[row_of(p)];
    if (T4 > 0) gp.store<kGB>(tmp, threadIdx.x, kThreads);
    for (int64_t g0 = threadIdx.x + kThreads * kGB; g0 < T4; g0 += kThreads * kGB) {
      gp.issue<kGB>(tmp, g0, kThreads);
      gp.store<kGB>(tmp, g0, kThreads);
    }
  }
  if (a.place && wave == 0) {
    // plain stores for r only if all Q chain workgroups share this XCD (a
    // wait that expires counts as a mismatch and is reported)
    const uint32_t mine = chain::xcd_id();
    bool same = true;
    if (lane < Q) {
      uint32_t x = static_cast<uint32_t>(place_w);
      if (static_cast<uint32_t>(place_w >> 32) != a.epoch)
        x = __float_as_uint(chain::take(&a.place[lane], a.epoch, a.status, &abort_flag, 0, a.spin));
      same = x == mine && !abort_flag;
    }
    const bool all = __all(same);
    if (lane == 0) xloc = all ? 1 : 0;
  }
  __syncthreads();  // vown, acc, flags, the G rows and xloc ready
  const bool xl = xloc != 0;


  const unsigned long long* mbox = a.xbuf + static_cast<int64_t>(q) * sb;

  if (fast) {
    // the fast path polls the one shared array
    FastCtx x{&a, q, nown, nown_max, lane, wave, rs, vown, yown, acc, gl, P, &abort_flag, &r_ready, acc_ready, a.xbuf, xl};
    const int fc = fast_cols(nown_max, cpl);
    bool updated;
    if (fc == 1) updated = recurrence_fast<T, LOSS, 1, 1, 2>(x);
    else if (fc == 2) updated = a.preload ? recurrence_fast<T, LOSS, 2, 2, 1>(x) : recurrence_fast<T, LOSS, 2, 2, 0>(x);
    else updated = a.preload ? recurrence_fast<T, LOSS, kMaxOwn, kMaxCpl, 1>(x)
                             : recurrence_fast<T, LOSS, kMaxOwn, kMaxCpl, 0>(x);
    __syncthreads();
    if (abort_flag || updated) return;
  } else {
    // ---- inner recurrence, any b.  Waves 1..3 compute and publish the own rows;
    // wave 0 only polls for the step's r values, so its waits never queue
    // behind another wave's memory traffic.
    const bool vec = (b & 3) == 0;  // G rows are float4-aligned
    for (int j = 0; j < s; ++j) {
      const int jb = j * b;
      if (wave > 0) {
        const float* Gj = a.G + static_cast<int64_t>(b) * b * (static_cast<int64_t>(j) * (j - 1) / 2);
        for (int t = wave - 1; t < nown; t += kWaves - 1) {
          const int i = q + Q * t;
          float dot = 0.f;
          if (a.preload) {
            const f32x4* g4 = reinterpret_cast<const f32x4*>(gl + t * P + static_cast<int64_t>(b) * (static_cast<int64_t>(j) * (j - 1) / 2));
            const f32x4* r4 = reinterpret_cast<const f32x4*>(rs);
            for (int k4 = lane; k4 < (jb >> 2); k4 += 64) {
              const f32x4 g = g4[k4];
              const f32x4 rr = r4[k4];
              dot = fmaf(g.x, rr.x, dot);
              dot = fmaf(g.y, rr.y, dot);
              dot = fmaf(g.z, rr.z, dot);
              dot = fmaf(g.w, rr.w, dot);
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
                  dot = fmaf(g[u].x, rr.x, dot);
                  dot = fmaf(g[u].y, rr.y, dot);
                  dot = fmaf(g[u].z, rr.z, dot);
                  dot = fmaf(g[u].w, rr.w, dot);
                }
              }
            }
          } else {
            const float* grow = Gj + static_cast<int64_t>(i) * jb;
            for (int k = lane; k < jb; k += 64) dot = fmaf(grow[k], rs[k], dot);
          }
          dot = group_sum<64>(dot);  // every lane holds the sum
          const int64_t row = jb + i;
          const float zz = vown[j * nown_max + t] - a.c * dot;
          const float rv = loss_deriv<LOSS>(zz, yown[j * nown_max + t]);
          const uint64_t word = tagged(a.epoch, rv);
          // one copy per reader: each workgroup polls only its own mailbox
          for (int dst = lane; dst < Q; dst += 64)
            chain::put_x(&a.xbuf[static_cast<int64_t>(dst) * sb + row], word, xl);
          if (lane == 0) {
            a.z[row] = zz;
            a.r[row] = rv;
          }
        }
      } else {
        // collect r_j of every row from this workgroup's mailbox
        for (int k = lane; k < b; k += 64) {
          uint64_t x = 0;
          long it = 0;
          while (true) {
            x = __hip_atomic_load(&mbox[jb + k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (static_cast<uint32_t>(x >> 32) == a.epoch) break;
            if (++it > a.spin) {
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
  }

  // ---- update of this workgroup's columns of w; the G rows are no longer needed
  chain::update_columns<T>(Y, a.ld, a.n, sb, rs, a.c, a.w, q, Q, gl);
}

template <typename T, int LOSS>
__global__ __launch_bounds__(kThreads) void chain_kernel(ChainArgs a) {
  const int w = blockIdx.x;
  if (w % a.stride != 0) return;  // launch slots between chain workgroups
  chain_body<T, LOSS>(a, w / a.stride);
}

// One launch of the pipelined training loop: the recurrence of outer step k
// (workgroups [0, Q)), the Gram of step k+1 and the gather of step k+2, each
// on buffers no other role of the launch touches, so the three need no
// synchronisation with each other; stream order between consecutive launches
// supplies every dependence.
template <int GS>
__device__ __forceinline__ void pipe_gather(const PipeArgs& p, int g) {
  constexpr int RPW = kThreads / GS;  // rows per workgroup pass
  for (int row0 = g * RPW; row0 < p.sb; row0 += p.gath_wgs * RPW)
    gather::copy_row<GS>(static_cast<const u32x4*>(p.Xs), p.y, p.m, p.cpr, p.sb, p.seed, nullptr,
                         p.idx_out, static_cast<u32x4*>(p.Yo), p.yBo,
                         row0 + static_cast<int>(threadIdx.x) / GS, threadIdx.x % GS);
}

// T = uint16_t: bf16 storage, Gram on MFMA with (BK, D) stages; T = float:
// float32 storage, Gram on the vector ALUs (BK, D unused).
// Margins of rows [m * mar_rows, (m+1) * mar_rows) of step k for the chain
// workgroups: each value goes out as a tagged word to vbox[row] (and to v).
template <typename T>
__device__ __forceinline__ void pipe_margins(const PipeArgs& p, int m, float* sm) {
  const ChainArgs& a = p.a;
  const int sb = a.s * a.b;
  const int r0 = m * p.mar_rows;
  const int nrows = sb - r0 < p.mar_rows ? sb - r0 : p.mar_rows;
  if (nrows <= 0) return;
  auto row_of = [&](int i) { return static_cast<int64_t>(r0 + i); };
  auto out = [&](int, int64_t row, float v) {
    v = chain::stored_margin(v, a.vround);
    chain::put(&p.vbox_out[row], tagged(a.epoch, v));
    a.v[row] = v;
  };
  const T* Y = static_cast<const T*>(a.Y);
  if (a.ld <= kWlMax)
    margins_wlds<T>(Y, a.ld, a.n, a.w, nrows, row_of, out, sm, [] {});
  else
    chain::margins<T>(Y, a.ld, a.n, a.w, nrows, row_of, out, threadIdx.x >> 6, threadIdx.x & 63);
}

template <typename T, int LOSS, int BK, int D>
__global__ __launch_bounds__(kThreads) void pipe_kernel(PipeArgs p) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  const int wg = blockIdx.x;
  int w;  // number among the non-chain workgroups
  if (p.a.stride == 1) {
    if (wg < p.a.Q) {
      chain_body<T, LOSS>(p.a, wg);
      return;
    }
    w = wg - p.ochain;
    if (w < 0) return;
  } else {
    const int slot = wg / p.a.stride, x = wg % p.a.stride;
    if (x == 0) {
      if (slot < p.a.Q) chain_body<T, LOSS>(p.a, slot);
      return;
    }
    w = slot * (p.a.stride - 1) + x - 1;
  }
  if (w >= p.mar0 && w < p.mar0 + p.mar_wgs) {
    pipe_margins<T>(p, w - p.mar0, sm);
    return;
  }
  if (w >= p.gram0 && w < p.gram0 + p.gram_slots) {
    const int tile = p.order[w - p.gram0];
    if (tile >= 0) {
      if constexpr (std::is_same<T, float>::value)
        gram::f32_tile(static_cast<const float*>(p.gY), p.a.ld, p.a.b, p.tps, p.gG, tile, sm, gram::SameRow{},
                       p.gbf16 != 0);
      else
        gram::bf16_tile<BK, D, false, gram::SameRow, std::is_same<T, _Float16>::value>(
            static_cast<const uint16_t*>(p.gY), p.a.ld, p.a.b, p.tps, p.gG, tile, reinterpret_cast<uint16_t*>(sm),
            gram::SameRow{}, p.gbf16 != 0);
    }
    return;
  }
  if (w >= p.gath0 && w < p.gath0 + p.gath_wgs) {
    const int g = w - p.gath0;
    switch (p.gs) {
      case 64: pipe_gather<64>(p, g); break;
      case 32: pipe_gather<32>(p, g); break;
      case 16: pipe_gather<16>(p, g); break;
      case 8: pipe_gather<8>(p, g); break;
      default: pipe_gather<4>(p, g); break;
    }
  }
}

// The chain workgroups wait for each other inside the launch, so all Q of
// them must be resident at once: Q per XCD group of CUs (one XCD when they
// are placed there, all CUs otherwise) times the kernel's occupancy.
template <typename K>
hipError_t check_resident(K kernel, size_t lds, const ChainArgs& a) {
  int occ = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(kernel),
                                                              kThreads, lds);
  if (e != hipSuccess) return e;
  const int cus = a.stride > 1 ? a.cus / a.stride : a.cus;
  return static_cast<int64_t>(occ) * cus >= a.Q ? hipSuccess : hipErrorLaunchOutOfResources;
}

template <typename T, int LOSS, int BK, int D>
hipError_t pipe_t(const PipeArgs& p, int grid, size_t lds, hipStream_t st, const LaunchTimer& tm) {
  static size_t granted = 64 * 1024;
  if (lds > granted) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&pipe_kernel<T, LOSS, BK, D>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
    granted = lds;
  }
  hipError_t e = check_resident(&pipe_kernel<T, LOSS, BK, D>, lds, p.a);
  if (e != hipSuccess) return e;
  return launch_kernel(pipe_kernel<T, LOSS, BK, D>, dim3(grid), dim3(kThreads), lds, st, tm, p);
}

template <int LOSS>
hipError_t pipe_l(int storage, const PipeArgs& p, int grid, size_t lds, hipStream_t st, const LaunchTimer& tm) {
  if (storage != kStoreBF16) return pipe_t<float, LOSS, 0, 0>(p, grid, lds, st, tm);
  switch (gram_variant(p.a.ld)) {
    case 0: return pipe_t<uint16_t, LOSS, 32, 1>(p, grid, lds, st, tm);
    case 1: return pipe_t<uint16_t, LOSS, 64, 8>(p, grid, lds, st, tm);
    case 2: return pipe_t<uint16_t, LOSS, 64, 4>(p, grid, lds, st, tm);
    default: return pipe_t<uint16_t, LOSS, 64, 2>(p, grid, lds, st, tm);
  }
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
  hipError_t e = check_resident(&chain_kernel<T, LOSS>, lds, a);
  if (e != hipSuccess) return e;
  const int grid = a.stride * (a.Q - 1) + 1;
  return launch_kernel(chain_kernel<T, LOSS>, dim3(grid), dim3(kThreads), lds, st, tm, a);
}

}  // namespace

bool chain_preload(int s, int b, int Q, int64_t ld) {
  if ((b & 3) != 0) return false;
  return static_cast<size_t>(chain_layout(s, b, Q, ld, true).total) * sizeof(float) <= kLdsBudget;
}

bool chain_fast(int s, int b, int Q, int64_t ld) {
  return chain_layout(s, b, Q, ld, chain_preload(s, b, Q, ld)).acc_len > 0;
}

size_t chain_lds_bytes(int s, int b, int Q, int64_t ld) {
  const size_t need = static_cast<size_t>(chain_layout(s, b, Q, ld, chain_preload(s, b, Q, ld)).total) * sizeof(float);
  return need > kLdsReserve ? need : kLdsReserve;
}

// Exact LDS of the chain workgroups, for launches whose other workgroups never
// share an XCD with them.
size_t chain_lds_need(int s, int b, int Q, int64_t ld) {
  return static_cast<size_t>(chain_layout(s, b, Q, ld, chain_preload(s, b, Q, ld)).total) * sizeof(float);
}

// layout 0 picks the first that holds of: the lean recurrence on one XCD
// (one workgroup per CU; an exchange round through one XCD's L2 costs a third
// of one through memory, 0.4 against 1.2 us measured at 32 and 64
// workgroups); the lean recurrence spread over the XCDs (one workgroup per
// row up to 64); the general recurrence spread.  1 forces the spread form, 2
// the one-XCD form with one workgroup per CU, 3 the one-XCD form with up to
// two workgroups per CU.
ChainPlan chain_plan(int s, int b, int64_t ld, int xcds, int cus_per_xcd, int layout) {
  ChainPlan spread;
  spread.Q = b < kChainMaxWorkgroups ? b : kChainMaxWorkgroups;
  spread.stride = 1;
  if (xcds <= 1) {
    // one XCD in all: the same form, and the exchange is XCD-local anyway
    spread.Q = b < cus_per_xcd ? b : cus_per_xcd;
    spread.lean = step_fits(s, b, spread.Q, ld);
    return spread;
  }
  spread.lean = step_fits(s, b, spread.Q, ld);
  ChainPlan one;
  one.Q = b < cus_per_xcd ? b : cus_per_xcd;
  one.stride = xcds;
  one.lean = step_fits(s, b, one.Q, ld);
  ChainPlan two = one;
  const int q2 = 2 * cus_per_xcd < kChainMaxWorkgroups ? 2 * cus_per_xcd : kChainMaxWorkgroups;
  two.Q = b < q2 ? b : q2;
  two.lean = step_fits(s, b, two.Q, ld);
  if (layout == 1) return spread;
  if (layout == 2) return one;
  if (layout == 3) return two;
  if (one.lean) return one;
  return spread;
}

hipError_t launch_chain(int storage, int loss, const ChainArgs& a_in, hipStream_t st,
                        const LaunchTimer& tm) {
  ChainArgs a = a_in;
  a.preload = chain_preload(a.s, a.b, a.Q, a.ld) ? 1 : 0;
  // spread over the XCDs: whole-CU LDS keeps other kernels off their CUs;
  // packed on one XCD (possibly two per CU): their own LDS only
  const size_t lds = a.stride == 1 ? chain_lds_bytes(a.s, a.b, a.Q, a.ld) : chain_lds_need(a.s, a.b, a.Q, a.ld);
  if (storage == kStoreBF16) {
    if (loss == kLogistic) return chain_t<uint16_t, kLogistic>(a, lds, st, tm);
    if (loss == kSquared) return chain_t<uint16_t, kSquared>(a, lds, st, tm);
    return chain_t<uint16_t, kPoisson>(a, lds, st, tm);
  }
  if (storage == kStoreF16) {
    if (loss == kLogistic) return chain_t<_Float16, kLogistic>(a, lds, st, tm);
    if (loss == kSquared) return chain_t<_Float16, kSquared>(a, lds, st, tm);
    return chain_t<_Float16, kPoisson>(a, lds, st, tm);
  }
  if (loss == kLogistic) return chain_t<float, kLogistic>(a, lds, st, tm);
  if (loss == kSquared) return chain_t<float, kSquared>(a, lds, st, tm);
  return chain_t<float, kPoisson>(a, lds, st, tm);
}

hipError_t launch_pipe(int storage, int loss, const PipeArgs& p_in, hipStream_t st, const LaunchTimer& tm) {
  if (storage != kStoreBF16 && storage != kStoreF32) return hipErrorInvalidValue;  // bf16 and float32 rows only
  PipeArgs p = p_in;
  p.a.preload = chain_preload(p.a.s, p.a.b, p.a.Q, p.a.ld) ? 1 : 0;
  // Spread chain workgroups share XCDs with the other roles: whole-CU LDS
  // keeps those off their CUs.  On their own XCD they need only their own.
  size_t lds = p.a.stride == 1 ? chain_lds_bytes(p.a.s, p.a.b, p.a.Q, p.a.ld)
                               : chain_lds_need(p.a.s, p.a.b, p.a.Q, p.a.ld);
  const size_t glds = storage != kStoreBF16 ? sizeof(float) * gram::kF32LdsElems
                      : sizeof(uint16_t) * (gram_variant(p.a.ld) == 0 ? gram::lds_elems<32>() : gram::lds_elems<64>());
  if (glds > lds) lds = glds;
  // non-chain workgroups needed, in o numbering
  int others = 0;
  if (p.mar_wgs > 0) others = p.mar0 + p.mar_wgs;
  if (p.gram_slots > 0) others = p.gram0 + p.gram_slots;
  if (p.gath_wgs > 0) others = p.gath0 + p.gath_wgs;
  int grid;
  if (p.a.stride == 1) {
    grid = others > 0 ? p.ochain + others : p.a.Q;
  } else {
    const int per = p.a.stride - 1;
    const int slots_o = (others + per - 1) / per;
    const int slots = slots_o > p.a.Q ? slots_o : p.a.Q;
    grid = slots * p.a.stride;
  }
  if (loss == kLogistic) return pipe_l<kLogistic>(storage, p, grid, lds, st, tm);
  if (loss == kSquared) return pipe_l<kSquared>(storage, p, grid, lds, st, tm);
  return pipe_l<kPoisson>(storage, p, grid, lds, st, tm);
}

}  // namespace casgd
