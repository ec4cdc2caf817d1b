// Device building blocks shared by the two weight-dependent kernels (the
// all-to-all recurrence in k_chain.hip and the lookahead recurrence in
// k_chain_la.hip): widening of 16-byte chunks, tagged exchange words,
// batched margins of a set of rows, and the column-sliced weight update.
#pragma once

#include <type_traits>

#include "casgd_device.h"
#include "casgd_internal.h"

namespace casgd {
namespace chain {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr long kSpinLimit = 1L << 22;  // default poll bound: seconds, far above any real wait

template <typename T>
struct Elems;
template <>
struct Elems<uint16_t> {
  static constexpr int E = 8;
  __device__ static void widen(const u32x4& q, float (&f)[8]) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = bf16_to_f32(w[e] & 0xFFFFu);
      f[2 * e + 1] = bf16_to_f32(w[e] >> 16);
    }
  }
};
template <>
struct Elems<_Float16> {
  static constexpr int E = 8;
  __device__ static void widen(const u32x4& q, float (&f)[8]) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = f16_to_f32_hw(w[e] & 0xFFFFu);
      f[2 * e + 1] = f16_to_f32_hw(w[e] >> 16);
    }
  }
};
template <>
struct Elems<float> {
  static constexpr int E = 4;
  __device__ static void widen(const u32x4& q, float (&f)[4]) {
    f[0] = __uint_as_float(q.x);
    f[1] = __uint_as_float(q.y);
    f[2] = __uint_as_float(q.z);
    f[3] = __uint_as_float(q.w);
  }
};

// A float r value travels with the launch's epoch in the upper half of a
// 64-bit word, so a reader spins on the data itself.
__device__ __forceinline__ uint64_t tagged(uint32_t epoch, float x) {
  return (static_cast<uint64_t>(epoch) << 32) | __float_as_uint(x);
}

// A device-scope store writes through to memory, where a device-scope load
// on any XCD finds it.
__device__ __forceinline__ void put(unsigned long long* p, uint64_t word) {
  __hip_atomic_store(p, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A wavefront-scope atomic store is a plain store (no cache-policy bits): it
// passes the CU's write-through L1 and stays in the L2 of its XCD, where the
// device-scope loads of workgroups on the same XCD find it (such loads skip
// the L1 and read a line this XCD has modified from its L2).  Only for
// readers on the writer's XCD; measured on MI355X, an all-to-all round among
// 32 workgroups of one XCD takes 0.4 us this way against 1.8 us with stores
// written through.
__device__ __forceinline__ void put_xcd(unsigned long long* p, uint64_t word) {
  __hip_atomic_store(p, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
}

__device__ __forceinline__ void put_x(unsigned long long* p, uint64_t word, bool same_xcd) {
  if (same_xcd)
    put_xcd(p, word);
  else
    put(p, word);
}

// The XCD (accelerator complex die) this wave runs on: bits 3:0 of the
// XCC_ID hardware register (gfx942 / gfx950).
__device__ __forceinline__ uint32_t xcd_id() {
  return __builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11)) & 0xFu;
}

// Spin until *p carries `epoch`; returns its float.  Bounded by `limit`
// polls: on expiry sets *abort (LDS) and bit 0 of *status and returns 0.
// True when another workgroup has reported an expired wait (read every 1024
// polls, so one failure ends every wait of the launch soon after).
__device__ __forceinline__ bool failed_elsewhere(long it, const int* status) {
  return (it & 1023) == 0 && __hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}

__device__ __forceinline__ float take(const unsigned long long* p, uint32_t epoch, int* status,
                                      int* abort_flag, int sleep, long limit) {
  long it = 0;
  while (true) {
    const uint64_t x = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (static_cast<uint32_t>(x >> 32) == epoch) return __uint_as_float(static_cast<uint32_t>(x));
    if (++it > limit || failed_elsewhere(it, status)) {
      *abort_flag = 1;
      atomicOr(status, 1);
      return 0.f;
    }
    if (sleep) __builtin_amdgcn_s_sleep(2);
  }
}

// Spin until every word p[lane + 64 u] with lane + 64 u < cnt (u < N)
// carries `epoch`; out[u] gets its float (0 for words past cnt).  The N words
// of a lane are polled together, so a lane that holds several columns waits
// one round trip per poll, not one per column.  Bounded like take(): on
// expiry sets *abort and bit 0 of *status, and the missing words read 0.
template <int N>
__device__ __forceinline__ void take_n(const unsigned long long* p, int lane, int cnt, uint32_t epoch,
                                       float (&out)[N], int* status, int* abort_flag, long limit) {
  uint32_t need = 0;
#pragma unroll
  for (int u = 0; u < N; ++u) {
    out[u] = 0.f;
    if (lane + 64 * u < cnt) need |= 1u << u;
  }
  long it = 0;
  while (need) {
    uint64_t x[N];
    // every load unconditional (words past cnt read word 0), then all checked
#pragma unroll
    for (int u = 0; u < N; ++u) {
      const int k = lane + 64 * u;
      x[u] = __hip_atomic_load(&p[k < cnt ? k : 0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int u = 0; u < N; ++u)
      if (((need >> u) & 1u) && static_cast<uint32_t>(x[u] >> 32) == epoch) {
        out[u] = __uint_as_float(static_cast<uint32_t>(x[u]));
        need &= ~(1u << u);
      }
    if (need && (++it > limit || failed_elsewhere(it, status))) {
      *abort_flag = 1;
      atomicOr(status, 1);
      break;
    }
  }
}

// A margin as the recurrence stores it: float32, or (vround) rounded to the
// nearest bf16, ties to even, and held in a float.
__device__ __forceinline__ float stored_margin(float v, int vround) {
  return vround ? bf16_to_f32(f32_to_bf16(v)) : v;
}

// Margins x . w of `nrows` rows of Y, row number row_of(p) for p < nrows.
// Each wave takes kRB rows at a time so their loads are in flight together;
// the weights of the same columns are loaded in the same batch.  `issued()`
// runs once, right after the first batch's loads are issued and before any
// of them is waited for, so a caller can put its own loads in flight beside
// them.  lane 0 of the wave calls out(p, row, value).
template <typename T, typename RowOf, typename Out, typename Issued>
__device__ __forceinline__ void margins(const T* Y, int64_t ld, int64_t n, const float* w, int nrows,
                                        RowOf row_of, Out out, int wave, int lane, Issued issued) {
  constexpr int E = Elems<T>::E;
  constexpr int kRB = 4;
  const int64_t cpr = ld / E;
  const bool w_vec = (reinterpret_cast<uintptr_t>(w) & 15) == 0;
  bool first = true;
  // every wave makes the same number of passes, so `issued` runs in all of them
  const int passes = (nrows + kWaves * kRB - 1) / (kWaves * kRB);
  for (int pass = 0; pass < (passes > 0 ? passes : 1); ++pass) {
    const int p0 = (pass * kWaves + wave) * kRB;
    float acc[kRB];
#pragma unroll
    for (int r = 0; r < kRB; ++r) acc[r] = 0.f;
    for (int64_t c0 = lane; c0 < cpr || first; c0 += 64 * 4) {
      // every load is unconditional (clamped addresses); out-of-range data
      // are zeroed only when used, so no load waits before all are issued
      u32x4 qv[kRB][4];
      float wv[4][E];
#pragma unroll
      for (int r = 0; r < kRB; ++r) {
        const int p = p0 + r;
        const u32x4* yr = reinterpret_cast<const u32x4*>(Y + row_of(p < nrows ? p : 0) * ld);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t c = c0 + 64 * u;
          qv[r][u] = yr[c < cpr ? c : 0];
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        // whole 16-byte pieces of w where they exist, else clamped elements
        const int64_t col0 = (c0 + 64 * u) * E;
        if (w_vec && col0 + E <= n) {
          const f32x4* w4 = reinterpret_cast<const f32x4*>(w + col0);
#pragma unroll
          for (int h = 0; h < E / 4; ++h) {
            const f32x4 ww = w4[h];
            wv[u][4 * h + 0] = ww.x;
            wv[u][4 * h + 1] = ww.y;
            wv[u][4 * h + 2] = ww.z;
            wv[u][4 * h + 3] = ww.w;
          }
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) wv[u][e] = w[col0 + e < n ? col0 + e : n - 1];
        }
      }
      if (first) {
        issued();
        first = false;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t c = c0 + 64 * u;
#pragma unroll
        for (int r = 0; r < kRB; ++r) {
          float f[E];
          Elems<T>::widen(qv[r][u], f);
          const bool on = p0 + r < nrows && c < cpr;
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const float ww = (on && c * E + e < n) ? wv[u][e] : 0.f;
            acc[r] = fmaf(f[e], ww, acc[r]);
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kRB; ++r) {
      const float tot = group_sum<64>(acc[r]);
      const int p = p0 + r;
      if (lane == 0 && p < nrows) out(p, row_of(p), tot);
    }
  }
}

template <typename T, typename RowOf, typename Out>
__device__ __forceinline__ void margins(const T* Y, int64_t ld, int64_t n, const float* w, int nrows,
                                        RowOf row_of, Out out, int wave, int lane) {
  margins<T>(Y, ld, n, w, nrows, row_of, out, wave, lane, [] {});
}

constexpr int64_t kWlMax = 2048;  // w staged in LDS for ld up to this

// Margins x . w of nrows rows of Y with w staged in LDS (ld <= kWlMax).  Every global
// load of the first batch is issued before any is waited for: w (clamped
// element loads, for the staging copy), the rows of Y, then whatever
// `issued()` adds; w goes to LDS (zero past n) behind a workgroup barrier and
// the dot products read it from there.  kRB rows per wave per batch; lane 0
// calls out(p, row, value).  Called by the whole workgroup.
template <typename T, typename RowOf, typename Out, typename Issued>
__device__ __forceinline__ void margins_wlds(const T* Y, int64_t ld, int64_t n, const float* w, int nrows,
                                             RowOf row_of, Out out, float* wl, Issued issued) {
  constexpr int E = Elems<T>::E;
  constexpr int kRB = 4;
  constexpr int kWv = static_cast<int>(kWlMax / kThreads);  // w elements per thread
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t cpr = ld / E;
  float wtmp[kWv];
#pragma unroll
  for (int e = 0; e < kWv; ++e) {
    const int64_t col = threadIdx.x + static_cast<int64_t>(kThreads) * e;
    wtmp[e] = w[col < n ? col : n - 1];
  }
  // One batch: kRB rows of this wave, 4 chunks per lane from c0.  The first
  // batch is separate code (FIRST), so no wait placed for the later batches
  // can hold back the loads `issued()` adds to the first.
  auto batch = [&](auto first_tag, int pass, int64_t c0, float (&acc)[kRB]) {
    constexpr bool FIRST = decltype(first_tag)::value;
    const int p0 = (pass * kWaves + wave) * kRB;
    u32x4 qv[kRB][4];
#pragma unroll
    for (int r = 0; r < kRB; ++r) {
      const int p = p0 + r;
      const u32x4* yr = reinterpret_cast<const u32x4*>(Y + row_of(p < nrows ? p : 0) * ld);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t c = c0 + 64 * u;
        qv[r][u] = yr[c < cpr ? c : 0];
      }
    }
    if constexpr (FIRST) {
      issued();
      // the copies of w are touched only now, so no load above is waited
      // for before every one of them is in flight
#pragma unroll
      for (int e = 0; e < kWv; ++e) asm volatile("" : "+v"(wtmp[e]) : : "memory");
#pragma unroll
      for (int e = 0; e < kWv; ++e) {
        const int64_t col = threadIdx.x + static_cast<int64_t>(kThreads) * e;
        if (col < ld) wl[col] = col < n ? wtmp[e] : 0.f;
      }
      __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t c = c0 + 64 * u;
      const f32x4* w4 = reinterpret_cast<const f32x4*>(wl + (c < cpr ? c : 0) * E);
      float wv[E];
#pragma unroll
      for (int h = 0; h < E / 4; ++h) {
        const f32x4 ww = w4[h];
        wv[4 * h + 0] = ww.x;
        wv[4 * h + 1] = ww.y;
        wv[4 * h + 2] = ww.z;
        wv[4 * h + 3] = ww.w;
      }
#pragma unroll
      for (int r = 0; r < kRB; ++r) {
        float f[E];
        Elems<T>::widen(qv[r][u], f);
        const bool on = p0 + r < nrows && c < cpr;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[r] = fmaf(f[e], on ? wv[e] : 0.f, acc[r]);
      }
    }
  };
  auto finish = [&](int pass, const float (&acc)[kRB]) {
    const int p0 = (pass * kWaves + wave) * kRB;
#pragma unroll
    for (int r = 0; r < kRB; ++r) {
      const float tot = group_sum<64>(acc[r]);
      const int p = p0 + r;
      if (lane == 0 && p < nrows) out(p, row_of(p), tot);
    }
  };
  const int passes = (nrows + kWaves * kRB - 1) / (kWaves * kRB);
  for (int pass = 0; pass < passes; ++pass) {
    float acc[kRB];
#pragma unroll
    for (int r = 0; r < kRB; ++r) acc[r] = 0.f;
    int64_t c0 = lane;
    if (pass == 0) {
      batch(std::integral_constant<bool, true>{}, 0, c0, acc);
      c0 += 64 * 4;
    }
    for (; c0 < cpr; c0 += 64 * 4) batch(std::integral_constant<bool, false>{}, pass, c0, acc);
    finish(pass, acc);
  }
}


// w[col] -= c * sum_rows Y[row][col] r[row] for the 16-byte column chunks
// [q*per, (q+1)*per) of this workgroup (per = ceil(chunks / Q)).  Thread
// (rg, cl) sums rows rg, rg + rgn, ... of chunk cl in a fixed order; the row
// groups of a wave are then added by an xor butterfly (every lane ends with
// the same, order-independent value: each level adds two equal-rank partial
// sums, a commutative step), and the four wave sums through `red`
// (kWaves * 64 * E floats of LDS) in a fixed order.  No float atomics: the
// result is bit-reproducible.  Must be called by the whole workgroup; rs
// holds r for all sb rows.
template <typename T>
__device__ __forceinline__ void update_columns(const T* Y, int64_t ld, int64_t n, int sb, const float* rs,
                                               float c, float* w, int q, int Q, float* red) {
  constexpr int E = Elems<T>::E;
  const int64_t cpr = ld / E;
  const int64_t per = (cpr + Q - 1) / Q;
  const int64_t ch0 = static_cast<int64_t>(q) * per;
  const int64_t ch1 = ch0 + per < cpr ? ch0 + per : cpr;
  int cw = 1;
  while (cw < per && cw < 64) cw <<= 1;
  const int rgn = kThreads / cw;
  const int cl = threadIdx.x % cw;
  const int rg = threadIdx.x / cw;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const u32x4* Y4 = reinterpret_cast<const u32x4*>(Y);
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
        for (int u = 0; u < 16; ++u) qv[u] = Y4[static_cast<int64_t>(row + u * rgn) * cpr + ch];
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
        Elems<T>::widen(Y4[static_cast<int64_t>(row) * cpr + ch], f);
        const float rr = rs[row];
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = fmaf(f[e], rr, acc[e]);
      }
    }
    // row groups of this wave: lanes cl, cl + cw, ... hold the same chunk
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
      for (int g = 1; g < kWaves; ++g) sum += red[g * (64 * E) + o];
      const int64_t chunk = cb + o / E;
      const int64_t col = chunk * E + o % E;
      if (chunk < ch1 && col < n) w[col] = w[col] - c * sum;
    }
  }
}

}  // namespace chain
}  // namespace casgd
