// The pipelined outer-step launch with the lean form of the inner recurrence.
//
// Abstract of "Mixed-Precision Communication-Avoiding SGD for Generalized
// Linear Models on GPUs": the Gram matrix comes from low-precision rows with
// high-precision accumulation, the inner recurrence and the weight update
// run in high precision (float32 here):
//
//   v   = Y w0
//   z_j = v_j - c * sum_{t<j} G_{j,t} r_t,   r_j = l'(z_j, y_j),   c = eta / b
//   w   = w0 - c * Y^T r
//
// One launch carries up to four roles on disjoint workgroups and buffers:
// the recurrence and update of outer step k ("chain", Q workgroups), the
// margins v of step k (handed to the chain as tagged words), the Gram of
// step k+1 and the sample + gather of step k+2.  Stream order between
// launches supplies every dependence between steps.
//
// Chain workgroup q owns rows i = q, q + Q, ... (at most NO of them) of every
// minibatch; each lane holds CP columns (b <= 64 CP).  Its rows of every
// block-row of G sit in LDS, copied there at the start with direct-to-LDS
// loads.  Wave 0 is the only wave on the critical path of an inner step: it
// reads everything of step j that does not depend on the newest r (its rows
// of G_{j,j-1}, margins, labels, partial sums) from LDS, polls r of block
// j-1, finishes z_j = v_j - c * sum_lanes(acc_j + G_{j,j-1} r_{j-1}) with one
// wave reduction per row, applies l' and publishes r_j: every value needed
// by a branch is loaded unconditionally (clamped addresses, then selects),
// so its loop holds no branch on per-lane data and no global load besides
// the polls.  Waves 1..3 fold each block t of r into the per-lane partial
// sums acc_k of blocks k >= t+2 (block k to wave 1 + k mod 3); wave 3 also
// accumulates the update of the workgroup's column slice as r arrives.
// r travels as 64-bit words tagged with the launch epoch, written once into
// one array that every chain workgroup polls; with every chain workgroup on
// one XCD (ChainArgs::place) through that XCD's L2.  Every wait is bounded.  All sums run in fixed
// orders, so results are bit-reproducible.
#pragma once

#include <type_traits>

#include "casgd_chain.h"
#include "casgd_gather.h"
#include "casgd_gram.h"

namespace casgd {
namespace step {

using chain::Elems;
using chain::kThreads;
using chain::tagged;

// bytes of LDS one workgroup may ask for (the static flags need a few)
constexpr int64_t kLdsBudget = 160 * 1024 - 512;
constexpr int kUR = 8;  // rows per lane per block the update wave holds

// Loss derivative with the loss chosen at run time (a wave-uniform branch).
__device__ __forceinline__ float dloss(int loss, float z, float y) {
  if (loss == kLogistic) return loss_deriv<kLogistic>(z, y);
  if (loss == kSquared) return loss_deriv<kSquared>(z, y);
  return loss_deriv<kPoisson>(z, y);
}

// LDS layout of a chain workgroup (floats): rs[sb] r so far | vown[s*NO] |
// yown[s*NO] | acc[s][NO][64 CP] per-lane partial sums | gl[NO][P] own rows
// of G (P = b * s(s-1)/2; own row t of block-row j at t*P + b*j(j-1)/2).
// After the recurrence acc serves as the update's reduction scratch, so at
// least 2048 floats follow its start.
struct Layout {
  int64_t rs, vown, yown, acc, gl, P, LW, total;
};

__host__ __device__ inline Layout layout(int s, int b, int NO, int CP) {
  Layout L;
  const int64_t sb = static_cast<int64_t>(s) * b;
  L.P = static_cast<int64_t>(b) * (static_cast<int64_t>(s) * (s - 1) / 2);
  L.LW = 64 * CP;
  L.rs = 0;
  L.vown = (sb + 3) & ~3LL;
  L.yown = L.vown + ((static_cast<int64_t>(s) * NO + 3) & ~3LL);
  L.acc = L.yown + ((static_cast<int64_t>(s) * NO + 3) & ~3LL);
  L.gl = L.acc + static_cast<int64_t>(s) * NO * L.LW;
  L.total = L.gl + NO * L.P;
  if (L.total < L.acc + 2048) L.total = L.acc + 2048;
  return L;
}

typedef __attribute__((address_space(3))) void lds_void;

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

// Publish `v` to the LDS word *flag after this wave's earlier LDS writes.
__device__ __forceinline__ void lds_publish(int* flag, int v) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __hip_atomic_store(flag, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// The same without waiting for the writes to complete: the LDS performs one
// wave's accesses in the order they are issued, so a wave that sees the flag
// (and then fences, lds_wait) sees the earlier writes; only the compiler must
// keep the order, which the signal fence asks of it.
__device__ __forceinline__ void lds_publish_inorder(int* flag, int v) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __hip_atomic_store(flag, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ int tri(int j) { return j * (j - 1) / 2; }

// What one run of the inner recurrence of a chain workgroup needs besides
// its LDS (filled by the caller: yown, acc zeroed, the own rows of G in gl,
// flags reset).
struct Rec {
  int s, b, Q, q, nown, loss;
  float c;
  uint32_t tag;                        // tag of this step's exchanged words
  const unsigned long long* vbox;      // margins of the step, tagged, by row
  unsigned long long* xbuf;            // r of every row, s*b tagged words (one array for all readers)
  bool xl;                             // r goes out with plain stores (one XCD)
  float *z, *r, *w;                    // exported z, r; weights (in place)
  unsigned long long* wbox;            // tagged copy of the new weights, or nullptr
  int64_t n, ld;
  int* status;
  long spin;
};

// Whether the update runs overlapped with the recurrence, on the last wave
// (at most 64 chunks of w per workgroup and kUR rows per lane per block);
// otherwise the whole workgroup runs it afterwards.  E: elements per chunk.
__host__ __device__ inline bool update_overlapped(int b, int Q, int64_t ld, int E) {
  const int64_t cpr = ld / E;
  const int64_t per = (cpr + Q - 1) / Q;
  int cw = 1;
  while (cw < per && cw < 64) cw <<= 1;
  const int rgw = 64 / cw;
  const int rpl = (b + rgw - 1) / rgw;
  return per <= 64 && rpl <= kUR;
}

struct RecLds {
  float *rs, *vown, *yown, *acc, *gl;
  int P;
  int *abort_flag, *r_ready, *acc_ready;
  float* red = nullptr;  // 2048 floats for the update after the recurrence (nullptr: acc)
};

// w0[col] with a device-scope load: this workgroup wrote it last, possibly
// in an earlier step of the same launch, and L1 may hold an older copy.
__device__ __forceinline__ float read_w0(const Rec& R, int64_t col) {
  return __hip_atomic_load(&R.w[col], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The new weight w[col] = w0 - c * sum of the column; it also goes out as a
// tagged word when wbox is set.
__device__ __forceinline__ void write_w(const Rec& R, int64_t col, float w0, float sum) {
  const float w1 = w0 - R.c * sum;
  R.w[col] = w1;
  if (R.wbox) chain::put(&R.wbox[col], tagged(R.tag, w1));
}

// The update after the recurrence by the whole workgroup, for column slices
// too wide for the overlapped form: the same fixed-order sums as
// chain::update_columns, rows read through rowp.  red: kWaves * 64 * E floats.
template <typename T, typename RowPtr>
__device__ __forceinline__ void update_after(const Rec& R, const float* rs, float* red, RowPtr rowp) {
  constexpr int E = Elems<T>::E;
  const int sb = R.s * R.b;
  const int64_t cpr = R.ld / E;
  const int64_t per = (cpr + R.Q - 1) / R.Q;
  const int64_t ch0 = static_cast<int64_t>(R.q) * per;
  const int64_t ch1 = ch0 + per < cpr ? ch0 + per : cpr;
  int cw = 1;
  while (cw < per && cw < 64) cw <<= 1;
  const int rgn = kThreads / cw;
  const int cl = threadIdx.x % cw;
  const int rg = threadIdx.x / cw;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  for (int64_t cb = ch0; cb < ch1; cb += cw) {
    const int64_t ch = cb + cl;
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    if (ch < ch1) {
      int row = rg;
      for (; row + 15 * rgn < sb; row += 16 * rgn) {
        u32x4 qv[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) qv[u] = rowp(row + u * rgn)[ch];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          float f[E];
          Elems<T>::widen(qv[u], f);
          const float rr = rs[row + u * rgn];
#pragma unroll
          for (int e = 0; e < E; ++e) acc[e] = fmaf(f[e], rr, acc[e]);
        }
      }
      for (; row < sb; row += rgn) {
        float f[E];
        Elems<T>::widen(rowp(row)[ch], f);
        const float rr = rs[row];
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = fmaf(f[e], rr, acc[e]);
      }
    }
    for (int off = cw; off < 64; off <<= 1)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += __shfl_xor(acc[e], off, 64);
    __syncthreads();  // red is reused across column blocks
    if (lane < cw)
#pragma unroll
      for (int e = 0; e < E; ++e) red[wave * (64 * E) + lane * E + e] = acc[e];
    __syncthreads();
    for (int o = threadIdx.x; o < cw * E; o += kThreads) {
      float sum = red[o];
      for (int g = 1; g < chain::kWaves; ++g) sum += red[g * (64 * E) + o];
      const int64_t chunk = cb + o / E;
      const int64_t col = chunk * E + o % E;
      if (chunk < ch1 && col < R.n) write_w(R, col, read_w0(R, col), sum);
    }
  }
}

// The inner recurrence and the update of one chain workgroup; called by all
// 256 lanes.  rowp(row) points at the 16-byte chunks of row `row` (0 <=
// row < s*b) of the step's Y.  Ends with the new weights of the workgroup's
// columns written (and every wave past its last LDS access).
// after_folds(wave, phase) lets a caller run other work on the waves with
// slack: phase 0 on waves 1 and 2 before their first fold and on the update
// wave (when the update is overlapped) before its first block, phase 1 on
// waves 1 and 2 after their last fold.
struct NoHook {
  __device__ void operator()(int, int) const {}
};

template <typename T, int NO, int CP, typename RowPtr, typename Hook = NoHook>
__device__ __forceinline__ void recurrence(const Rec& R, const RecLds& S, RowPtr rowp, Hook after_folds = {}) {
  const int s = R.s, b = R.b, Q = R.Q, q = R.q, nown = R.nown, sb = s * b;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  const int P = S.P;
  constexpr int LW = 64 * CP;
  float* rs = S.rs;
  float* vown = S.vown;
  const float* yown = S.yown;
  float* acc = S.acc;
  const float* gl = S.gl;
  int& abort_flag = *S.abort_flag;
  int& r_ready = *S.r_ready;
  int* acc_ready = S.acc_ready;
  // every workgroup publishes each of its own rows' r once; every reader
  // polls the same words (one mailbox for the whole launch)
  const unsigned long long* mbox = R.xbuf;
  // update plan (the same in every wave): chunks [ch0, ch1) of w
  constexpr int E = Elems<T>::E;
  const int cpr = static_cast<int>(R.ld / E);
  const int per = (cpr + Q - 1) / Q;
  int cw = 1;
  while (cw < per && cw < 64) cw <<= 1;
  const int rgw = 64 / cw;
  const int rpl = (b + rgw - 1) / rgw;
  const bool upd = update_overlapped(b, Q, R.ld, E);
  // fold waves 1..nf; with the update overlapped, wave 3 only updates (its
  // row loads then never hold back a fold)
  const int nf = upd ? 2 : 3;

  if (wave == 0) {
    // ------------------------------------------------ the critical wave
    // first claim on the CU's shared issue resources (LDS, memory, scalar)
    __builtin_amdgcn_s_setprio(3);
    // margins of the own rows, from the launch's margin workgroups
    for (int p = lane; p < s * NO; p += 64) {
      const int j = p / NO, t = p - (p / NO) * NO;
      float v = 0.f;
      if (t < nown) v = chain::take(&R.vbox[j * b + q + Q * t], R.tag, R.status, &abort_flag, 0, R.spin);
      vown[p] = v;
    }
    float rp[CP];
#pragma unroll
    for (int u = 0; u < CP; ++u) rp[u] = 0.f;
    for (int j = 0; j < s; ++j) {
      if (__hip_atomic_load(&abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) break;
      const int jb = j * b;
      // everything of step j that does not wait for r of block j-1
      float vj[NO], yj[NO], gv[NO][CP], av[NO][CP];
      const int* ready = &acc_ready[j % nf];
      const bool acc_now = j < 2 || __hip_atomic_load(ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= j - 1;
      if (acc_now) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      const int goff = b * tri(j) + (j - 1) * b;  // G_{j,j-1} inside an own row
#pragma unroll
      for (int t = 0; t < NO; ++t) {
        vj[t] = vown[j * NO + t];
        yj[t] = yown[j * NO + t];
#pragma unroll
        for (int u = 0; u < CP; ++u) {
          const int col = lane + 64 * u;
          const int colc = col < b ? col : b - 1;
          // rows t >= nown hold no G: read row 0 and drop the value
          const float g = j > 0 ? gl[(t < nown ? t : 0) * P + goff + colc] : 0.f;
          gv[t][u] = t < nown ? g : 0.f;
          av[t][u] = acc[(j * NO + t) * LW + col];
        }
      }
      if (j > 0) {
        chain::take_n<CP>(&mbox[jb - b], lane, b, R.tag, rp, R.status, &abort_flag, R.spin);
#pragma unroll
        for (int u = 0; u < CP; ++u) {
          const int col = lane + 64 * u;
          if (col < b) rs[jb - b + col] = rp[u];
        }
        lds_publish_inorder(&r_ready, j);
        if (!acc_now) {
          if (!lds_wait(ready, j - 1, &abort_flag, R.status, R.spin)) break;
#pragma unroll
          for (int t = 0; t < NO; ++t)
#pragma unroll
            for (int u = 0; u < CP; ++u) av[t][u] = acc[(j * NO + t) * LW + lane + 64 * u];
        }
      }
      // from here to the stores is the step's critical path
      float part[NO], zz[NO], rv[NO];
#pragma unroll
      for (int t = 0; t < NO; ++t) {
        part[t] = 0.f;
#pragma unroll
        for (int u = 0; u < CP; ++u) part[t] += fmaf(gv[t][u], rp[u], av[t][u]);
      }
#pragma unroll
      for (int t = 0; t < NO; ++t) part[t] = wave_sum(part[t]);
#pragma unroll
      for (int t = 0; t < NO; ++t) {
        zz[t] = vj[t] - R.c * part[t];
        rv[t] = dloss(R.loss, zz[t], yj[t]);
      }
      // each own row's r once, lane t for own row t: NO stores per workgroup
      // (a copy per reader, NO * Q stores, measured 2-7% slower)
      {
        float x = rv[0];
#pragma unroll
        for (int t = 1; t < NO; ++t) x = lane == t ? rv[t] : x;
        if (lane < nown) chain::put_x(&R.xbuf[jb + q + Q * lane], tagged(R.tag, x), R.xl);
      }
      // the exported z and r
      if (lane == 0) {
#pragma unroll
        for (int t = 0; t < NO; ++t)
          if (t < nown) {
            R.z[jb + q + Q * t] = zz[t];
            R.r[jb + q + Q * t] = rv[t];
          }
      }
    }
    // the last block's r, for the update
    if (!abort_flag) {
      const int jb = (s - 1) * b;
      float rl[CP];
      chain::take_n<CP>(&mbox[jb], lane, b, R.tag, rl, R.status, &abort_flag, R.spin);
#pragma unroll
      for (int u = 0; u < CP; ++u)
        if (lane + 64 * u < b) rs[jb + lane + 64 * u] = rl[u];
      if (!abort_flag) lds_publish(&r_ready, s);
    }
    __builtin_amdgcn_s_setprio(0);
  } else {
    // ------------------------------------------------ fold waves 1..nf
    // wave h + 1 owns the partial sums of blocks k = h (mod nf); once r of
    // block tb is in, it adds G_{k,tb} r_tb for every such k >= tb + 2
    const int h = wave - 1;
    auto fold = [&](int tb) {
      float rr[CP];
      int colc[CP];
#pragma unroll
      for (int u = 0; u < CP; ++u) {
        const int col = lane + 64 * u;
        rr[u] = col < b ? rs[tb * b + col] : 0.f;  // columns past b add 0
        colc[u] = col < b ? col : b - 1;
      }
      int k0 = tb + 2;
      k0 += (h - k0 % nf + nf) % nf;
      for (int k = k0; k < s; k += nf) {
        const int goff = b * tri(k) + tb * b;
#pragma unroll
        for (int t = 0; t < NO; ++t) {
          if (t >= nown) break;
#pragma unroll
          for (int u = 0; u < CP; ++u) {
            float* ap = &acc[(k * NO + t) * LW + lane + 64 * u];
            *ap = fmaf(gl[t * P + goff + colc[u]], rr[u], *ap);
          }
        }
      }
      lds_publish_inorder(&acc_ready[h], tb + 1);
    };
    if (!(upd && wave == chain::kWaves - 1)) {
      // waves 1 and 2 may start work of the next step now (phase 0, before
      // their first fold) and when their folds are done (phase 1)
      if (wave == 1 || wave == 2) after_folds(wave, 0);
      for (int tb = 0; tb + 2 < s; ++tb) {
        if (!lds_wait(&r_ready, tb + 1, &abort_flag, R.status, R.spin)) break;
        fold(tb);
      }
      if (wave == 1 || wave == 2) after_folds(wave, 1);
    } else {
      // the last wave accumulates the update of this workgroup's chunks
      // [ch0, ch1) of w: lane (rgl, cl) sums rows rgl, rgl + rgw, ... of every
      // block for chunk ch0 + cl as soon as the block's r is in.  It may
      // start work of the next step first (phase 0): its sums have slack.
      after_folds(wave, 0);
      const int ch0 = q * per;
      const int ch1 = ch0 + per < cpr ? ch0 + per : cpr;
      const int cl = lane % cw, rgl = lane / cw;
      const int ch = ch0 + cl;
      const bool col_ok = ch < ch1;
      float accw[E], w0[E];
#pragma unroll
      for (int e = 0; e < E; ++e) accw[e] = 0.f;
      // the old weights of the lane's columns, all loads issued at once now
      // (device-scope atomics stay in program order, so loading each one at
      // the end would cost one round trip per column)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int64_t col = static_cast<int64_t>(ch) * E + e;
        w0[e] = (rgl == 0 && col_ok && col < R.n) ? read_w0(R, col) : 0.f;
      }
      // rows of block tb (clamped to the last block) for this lane, unconditional loads
      auto load_blk = [&](int tb, u32x4 (&dst)[kUR]) {
        const int tbc = tb < s ? tb : s - 1;
#pragma unroll
        for (int i = 0; i < kUR; ++i) {
          const int rl = rgl + rgw * i;
          const bool ok = i < rpl && rl < b && col_ok;
          dst[i] = rowp(ok ? tbc * b + rl : 0)[ok ? ch : 0];
        }
      };
      auto blk = [&](int tb, const u32x4 (&src)[kUR]) -> bool {
        if (!lds_wait(&r_ready, tb + 1, &abort_flag, R.status, R.spin)) return false;
#pragma unroll
        for (int i = 0; i < kUR; ++i) {
          const int rl = rgl + rgw * i;
          const bool ok = i < rpl && rl < b && col_ok;
          const float rr = ok ? rs[tb * b + rl] : 0.f;
          float f[E];
          Elems<T>::widen(src[i], f);
#pragma unroll
          for (int e = 0; e < E; ++e) accw[e] = fmaf(f[e], rr, accw[e]);
        }
        return true;
      };
      // loads stop at the last block: a load issued for nothing would still
      // be waited for before the final reduction
      u32x4 ya[kUR], yb[kUR];
      load_blk(0, ya);
      bool ok = true;
      for (int tb = 0; tb < s; tb += 2) {
        if (tb + 1 < s) load_blk(tb + 1, yb);
        ok = blk(tb, ya);
        if (!ok || tb + 1 >= s) break;
        if (tb + 2 < s) load_blk(tb + 2, ya);
        ok = blk(tb + 1, yb);
        if (!ok) break;
      }
      if (ok) {
        for (int off = cw; off < 64; off <<= 1)
#pragma unroll
          for (int e = 0; e < E; ++e) accw[e] += __shfl_xor(accw[e], off, 64);
        if (rgl == 0 && col_ok) {
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const int64_t col = static_cast<int64_t>(ch) * E + e;
            if (col < R.n) write_w(R, col, w0[e], accw[e]);
          }
        }
      }
    }
  }
  __syncthreads();
  // the update after the recurrence, by the whole workgroup (acc is free now)
  if (!upd && !abort_flag) {
    update_after<T>(R, rs, S.red ? S.red : acc, rowp);
    __syncthreads();
  }
}

// Own rows of G to LDS (gl[t * P ...]) for own rows t < nown: own row t of
// block-row j is a run of j*b/4 float4, contiguous in G and in LDS (at t*P +
// b*j(j-1)/2).  Each run is copied with direct-to-LDS loads of up to 64
// float4 (one per lane); all run addresses are wave-uniform (scalar), so a
// lane adds only its own offset.  The instructions are dealt round-robin to
// the `nwaves` waves starting at wave `wave0`; all are in flight together.
// AUX: the loads' cache policy (device scope for G written by other XCDs in
// the same launch).  The caller waits (s_waitcnt) and synchronises.
template <int AUX>
__device__ __forceinline__ void load_g_rows(const float* G, float* gl, int s, int b, int Q, int q, int nown, int P,
                                            int wave0 = 0, int nwaves = chain::kWaves) {
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6) - wave0;
  const int lane = threadIdx.x & 63;
  const int b4 = b / 4;
  const f32x4* G4 = reinterpret_cast<const f32x4*>(G);
  f32x4* gl4 = reinterpret_cast<f32x4*>(gl);
  int g = 0;
  for (int t = 0; t < nown; ++t) {
    const int i = q + Q * t;
    for (int j = 1; j < s; ++j) {
      const int len = j * b4;
      const int src0 = (b * b * tri(j) + i * j * b) / 4;
      const int dst0 = t * (P / 4) + b4 * tri(j);
      for (int c0 = 0; c0 < len; c0 += 64, ++g) {
        if (g % nwaves != wave) continue;
        if (c0 + lane < len)
          __builtin_amdgcn_global_load_lds(G4 + src0 + c0 + lane, (lds_void*)(gl4 + dst0 + c0), 16, 0, AUX);
      }
    }
  }
}

// Placement check of the chain workgroups (wave 0): true if all Q of them
// run on this XCD.  place_w: this lane's early read of place[lane].
__device__ __forceinline__ bool all_on_this_xcd(const ChainArgs& a, uint64_t place_w, int* abort_flag) {
  const int lane = threadIdx.x & 63;
  const uint32_t mine = chain::xcd_id();
  bool same = true;
  if (lane < a.Q) {
    uint32_t x = static_cast<uint32_t>(place_w);
    if (static_cast<uint32_t>(place_w >> 32) != a.epoch)
      x = __float_as_uint(chain::take(&a.place[lane], a.epoch, a.status, abort_flag, 0, a.spin));
    same = x == mine && !*abort_flag;
  }
  return __all(same);
}

// Chain workgroup q of the one-step launch; called by all 256 lanes.
template <typename T, int NO, int CP>
__device__ __forceinline__ void chain(const ChainArgs& a, int q, int loss) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  const int s = a.s, b = a.b, Q = a.Q;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  const int nown = (b - q + Q - 1) / Q;  // own rows q, q + Q, ... below b
  const Layout L = layout(s, b, NO, CP);
  constexpr int LW = 64 * CP;
  __shared__ int abort_flag;
  __shared__ int r_ready;        // blocks whose r is in rs (wave 0)
  __shared__ int acc_ready[3];   // blocks folded into acc (waves 1..3)
  __shared__ int xloc;           // all chain workgroups on this XCD
  RecLds S{sm + L.rs, sm + L.vown, sm + L.yown, sm + L.acc, sm + L.gl, static_cast<int>(L.P),
           &abort_flag, &r_ready, acc_ready};
  if (threadIdx.x == 0) {
    abort_flag = 0;
    r_ready = 0;
    xloc = 0;
    acc_ready[0] = acc_ready[1] = acc_ready[2] = 0;
    if (a.place) chain::put(&a.place[q], tagged(a.epoch, __uint_as_float(chain::xcd_id())));
  }
  uint64_t place_w = 0;
  if (a.place && wave == 0)
    place_w = __hip_atomic_load(&a.place[lane < Q ? lane : 0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  load_g_rows<0>(a.G, S.gl, s, b, Q, q, nown, S.P);
  for (int k = threadIdx.x; k < s * NO * LW; k += kThreads) S.acc[k] = 0.f;
  for (int p = threadIdx.x; p < s * NO; p += kThreads) {
    const int j = p / NO, t = p - (p / NO) * NO;
    S.yown[p] = t < nown ? a.yB[j * b + q + Q * t] : 0.f;
  }
  if (a.place && wave == 0) {
    const bool all = all_on_this_xcd(a, place_w, &abort_flag);
    if (lane == 0) xloc = all ? 1 : 0;
  }
  __builtin_amdgcn_s_waitcnt(0);  // the direct-to-LDS copies have landed
  __syncthreads();
  Rec R;
  R.s = s;
  R.b = b;
  R.Q = Q;
  R.q = q;
  R.nown = nown;
  R.loss = loss;
  R.c = a.c;
  R.tag = a.epoch;
  R.vbox = a.vbox;
  R.xbuf = a.xbuf;
  R.xl = xloc != 0;
  R.z = a.z;
  R.r = a.r;
  R.w = a.w;
  R.wbox = nullptr;
  R.n = a.n;
  R.ld = a.ld;
  R.status = a.status;
  R.spin = a.spin;
  const u32x4* Y4 = reinterpret_cast<const u32x4*>(a.Y);
  const int64_t cpr = a.ld / Elems<T>::E;
  recurrence<T, NO, CP>(R, S, [&](int row) { return Y4 + row * cpr; });
}

// Margins of rows [m * mar_rows, (m+1) * mar_rows) of step k for the chain
// workgroups: each value goes out as a tagged word to vbox[row] (and to v).
template <typename T>
__device__ __forceinline__ void margins(const PipeArgs& p, int m) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
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
  if (a.ld <= chain::kWlMax)
    chain::margins_wlds<T>(Y, a.ld, a.n, a.w, nrows, row_of, out, sm, [] {});
  else
    chain::margins<T>(Y, a.ld, a.n, a.w, nrows, row_of, out, threadIdx.x >> 6, threadIdx.x & 63);
}

template <int GS>
__device__ __forceinline__ void gather_rows(const PipeArgs& p, int g) {
  constexpr int RPW = kThreads / GS;  // rows per workgroup pass
  for (int row0 = g * RPW; row0 < p.sb; row0 += p.gath_wgs * RPW) {
    const int row = row0 + static_cast<int>(threadIdx.x) / GS;
    if (p.gf8)
      gather::copy_row_f8<GS>(static_cast<const u32x4*>(p.Xs), p.y, p.m, p.cpr, p.sb, p.seed, nullptr, p.idx_out,
                              static_cast<u32x4*>(p.Yo), p.yBo, p.unscale, row, threadIdx.x % GS);
    else
      gather::copy_row<GS>(static_cast<const u32x4*>(p.Xs), p.y, p.m, p.cpr, p.sb, p.seed, nullptr, p.idx_out,
                           static_cast<u32x4*>(p.Yo), p.yBo, row, threadIdx.x % GS);
  }
}

// T = uint16_t: bf16 rows, Gram on bf16 MFMA with (BK, D) stages; T =
// _Float16: fp16 rows, Gram on fp16 MFMA; T = float: float32 rows, Gram on
// the vector ALUs (BK, D unused).
template <typename T, int NO, int CP, int BK, int D>
__global__ __launch_bounds__(kThreads) void step_kernel(PipeArgs p, int loss) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  const int wg = blockIdx.x;
  int w;  // number among the non-chain workgroups
  if (p.a.stride == 1) {
    if (wg < p.a.Q) {
      chain<T, NO, CP>(p.a, wg, loss);
      return;
    }
    w = wg - p.ochain;
    if (w < 0) return;
  } else {
    const int slot = wg / p.a.stride, x = wg % p.a.stride;
    if (x == 0) {
      if (slot < p.a.Q) chain<T, NO, CP>(p.a, slot, loss);
      return;
    }
    w = slot * (p.a.stride - 1) + x - 1;
  }
  if (w >= p.mar0 && w < p.mar0 + p.mar_wgs) {
    margins<T>(p, w - p.mar0);
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
      case 64: gather_rows<64>(p, g); break;
      case 32: gather_rows<32>(p, g); break;
      case 16: gather_rows<16>(p, g); break;
      case 8: gather_rows<8>(p, g); break;
      default: gather_rows<4>(p, g); break;
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

template <typename T, int NO, int CP, int BK, int D>
hipError_t launch_t(const PipeArgs& p, int loss, int grid, size_t lds, hipStream_t st, const LaunchTimer& tm) {
  static size_t granted = 64 * 1024;
  if (lds > granted) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&step_kernel<T, NO, CP, BK, D>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    granted = lds;
  }
  hipError_t e = check_resident(&step_kernel<T, NO, CP, BK, D>, lds, p.a);
  if (e != hipSuccess) return e;
  return launch_kernel(step_kernel<T, NO, CP, BK, D>, dim3(grid), dim3(kThreads), lds, st, tm, p, loss);
}

// All kernels of one (NO, CP) variant; `lds` and `grid` come from the caller.
template <int NO, int CP>
hipError_t launch_variant(int storage, int loss, const PipeArgs& p, int grid, size_t lds, hipStream_t st,
                          const LaunchTimer& tm) {
  if (storage == kStoreF32) return launch_t<float, NO, CP, 0, 0>(p, loss, grid, lds, st, tm);
  if (storage == kStoreF16) {
    switch (gram_variant(p.a.ld)) {
      case 0: return launch_t<_Float16, NO, CP, 32, 1>(p, loss, grid, lds, st, tm);
      case 1: return launch_t<_Float16, NO, CP, 64, 8>(p, loss, grid, lds, st, tm);
      case 2: return launch_t<_Float16, NO, CP, 64, 4>(p, loss, grid, lds, st, tm);
      default: return launch_t<_Float16, NO, CP, 64, 2>(p, loss, grid, lds, st, tm);
    }
  }
  switch (gram_variant(p.a.ld)) {
    case 0: return launch_t<uint16_t, NO, CP, 32, 1>(p, loss, grid, lds, st, tm);
    case 1: return launch_t<uint16_t, NO, CP, 64, 8>(p, loss, grid, lds, st, tm);
    case 2: return launch_t<uint16_t, NO, CP, 64, 4>(p, loss, grid, lds, st, tm);
    default: return launch_t<uint16_t, NO, CP, 64, 2>(p, loss, grid, lds, st, tm);
  }
}

}  // namespace step
}  // namespace casgd
