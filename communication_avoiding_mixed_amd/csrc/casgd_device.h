// Device-side helpers shared by the CA-SGD kernels: the counter-based row
// sampler, bfloat16 storage conversion and the three GLM losses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace casgd {

// Native clang vectors for 16-byte loads and stores.  Arrays of these stay in
// registers; arrays of HIP's struct vector types (uint4, float4) can end up in
// scratch or LDS memory instead.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kLogistic = 0;
constexpr int kSquared = 1;
constexpr int kPoisson = 2;

// SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): output i of the stream
// seeded with `seed` mixes seed + (i + 1) * golden-gamma.  Counter-based, so
// every row index of an outer step is computed independently.
__host__ __device__ __forceinline__ uint64_t splitmix64(uint64_t seed, uint64_t i) {
  uint64_t z = seed + (i + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Row i of an outer step: floor(x_i * m / 2^64), the multiply-high range
// reduction (Lemire 2019).  Uniform with replacement over [0, m).
__device__ __forceinline__ int32_t sample_row(uint64_t seed, uint64_t i, uint64_t m) {
  return static_cast<int32_t>(__umul64hi(splitmix64(seed, i), m));
}

// float32 -> bfloat16 bits, round to nearest with ties to even; NaN -> quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even of a float32 magnitude (bit pattern a, below the
// target format's smallest normal) to a count of the target's subnormal
// quanta 2^qexp: a = mant * 2^(e - 150) with the implicit bit, so the count is
// mant * 2^(e - 150 - qexp), a right shift by sh = 150 + qexp - e (at least
// 14 here).  Host and device share these conversions.
__host__ __device__ __forceinline__ uint32_t subnormal_quanta(uint32_t a, int qexp) {
  const int e = static_cast<int>(a >> 23);
  const int sh = 150 + qexp - e;
  if (e == 0 || sh > 24) return 0u;  // below half a quantum (or a float32 subnormal)
  const uint32_t mant = (a & 0x7FFFFFu) | 0x800000u;
  const uint32_t q = mant >> sh;
  const uint32_t rem = mant & ((1u << sh) - 1u);
  const uint32_t half = 1u << (sh - 1);
  return q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u);
}

// float32 -> IEEE binary16 bits: round to nearest even, subnormals kept,
// overflow (|x| >= 65520 after rounding, infinities) to infinity, NaN -> quiet
// NaN with the sign kept.
__host__ __device__ __forceinline__ uint16_t f32_to_f16(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  const uint32_t sign = (u >> 16) & 0x8000u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return static_cast<uint16_t>(sign | 0x7E00u);
  if (a >= 0x477FF000u) return static_cast<uint16_t>(sign | 0x7C00u);  // 65520: rounds past 65504
  if (a >= 0x38800000u) {                                              // 2^-14: a binary16 normal
    uint32_t r = a - (112u << 23);                                     // rebias 127 -> 15
    r += 0xFFFu + ((r >> 13) & 1u);                                    // 13 dropped fraction bits
    return static_cast<uint16_t>(sign | (r >> 13));
  }
  return static_cast<uint16_t>(sign | subnormal_quanta(a, -24));  // 1024 quanta is 2^-14, bits 0x400
}

// Exact float32 value of binary16 bits.
__host__ __device__ __forceinline__ float f16_to_f32(uint32_t h) {
  const uint32_t sign = (h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1Fu, f = h & 0x3FFu;
  uint32_t bits;
  if (e == 0)
    bits = sign | __builtin_bit_cast(uint32_t, static_cast<float>(f) * 0x1p-24f);
  else if (e == 31)
    bits = sign | 0x7F800000u | (f << 13);
  else
    bits = sign | ((e + 112u) << 23) | (f << 13);
  return __builtin_bit_cast(float, bits);
}

// The same decode with the hardware conversion (v_cvt_f32_f16), which the
// kernels use: every binary16 value, subnormals included, is a normal
// float32, and the default float mode keeps f16 denormals, so it is exact.
// A GPU test pins it on subnormal inputs; it needs a fraction of the
// integer decode's instructions, which measured 3x slower steps.
__device__ __forceinline__ float f16_to_f32_hw(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

// float32 -> OCP E4M3 bits: round to nearest even, subnormals (quanta of
// 2^-9) kept, magnitudes from 448 up (and infinities) saturated to 448, NaN
// -> 0x7F with the sign kept.  Magnitudes in (448, 464] round to 448 and
// larger ones would round past it, so every a >= 448 gives 448.
__host__ __device__ __forceinline__ uint8_t f32_to_e4m3(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return static_cast<uint8_t>(sign | 0x7Fu);
  if (a >= 0x43E00000u) return static_cast<uint8_t>(sign | 0x7Eu);
  if (a >= 0x3C800000u) {             // 2^-6: an E4M3 normal
    uint32_t r = a - (120u << 23);     // rebias 127 -> 7
    r += 0x7FFFFu + ((r >> 20) & 1u);  // 20 dropped fraction bits
    return static_cast<uint8_t>(sign | (r >> 20));
  }
  return static_cast<uint8_t>(sign | subnormal_quanta(a, -9));  // 8 quanta is 2^-6, bits 0x08
}

// Exact float32 value of E4M3 bits (0x7F / 0xFF are NaN).
__host__ __device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t sign = (b & 0x80u) << 24;
  const uint32_t e = (b >> 3) & 0xFu, f = b & 7u;
  uint32_t bits;
  if (e == 0)
    bits = sign | __builtin_bit_cast(uint32_t, static_cast<float>(f) * 0x1p-9f);
  else if (e == 15 && f == 7)
    bits = sign | 0x7FC00000u;
  else
    bits = sign | ((e + 120u) << 23) | (f << 20);
  return __builtin_bit_cast(float, bits);
}

// Derivative of the per-row loss with respect to the margin z, in float32.
//   logistic: -y * sigmoid(-y z) (exp of a non-positive argument only)
//   squared:  z - y
//   poisson:  exp(z) - y
// It sits on the recurrence's critical path once per inner step, so it uses
// the hardware exponential (v_exp_f32 of x log2 e) and reciprocal
// (v_rcp_f32, 1 ulp): a few float32 ulps, far below the recurrence's
// float32 rounding of z.
__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }

template <int LOSS>
__device__ __forceinline__ float loss_deriv(float z, float y) {
  if constexpr (LOSS == kLogistic) {
    const float u = -y * z;
    const float e = exp_hw(-fabsf(u));
    const float inv = __builtin_amdgcn_rcpf(1.f + e);
    const float sig = u >= 0.f ? inv : e * inv;
    return -y * sig;
  } else if constexpr (LOSS == kSquared) {
    return z - y;
  } else {
    return exp_hw(z) - y;
  }
}

// Per-row loss in float64 from a float32 margin.
//   logistic: softplus(-y z); squared: (z - y)^2 / 2; poisson: exp(z) - y z
template <int LOSS>
__device__ __forceinline__ double loss_value(double z, double y) {
  if constexpr (LOSS == kLogistic) {
    const double u = -y * z;
    return fmax(u, 0.0) + log1p(exp(-fabs(u)));
  } else if constexpr (LOSS == kSquared) {
    const double d = z - y;
    return 0.5 * d * d;
  } else {
    return exp(z) - y * z;
  }
}

// Cross-lane move inside rows of 16 lanes (DPP).  CTRL: 0xB1 / 0x4E swap
// neighbours 1 / 2 apart in each quad, 0x124 / 0x128 rotate a row by 4 / 8.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes of a wavefront, the same value in every lane.  Rows
// of 16 are summed with DPP moves, then the four row sums are read out and
// added in a fixed order, so the result does not depend on timing.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_move<0xB1>(v);
  v += dpp_move<0x4E>(v);
  v += dpp_move<0x124>(v);
  v += dpp_move<0x128>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return ((r0 + r1) + r2) + r3;
}

// Reduction over the `width` lanes of an aligned lane group (width a power of
// two up to the 64-lane wavefront).
template <int WIDTH>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (WIDTH == 64) {
    return wave_sum(x);
  } else {
#pragma unroll
    for (int o = WIDTH / 2; o > 0; o >>= 1) x += __shfl_xor(x, o, WIDTH);
    return x;
  }
}

template <int WIDTH>
__device__ __forceinline__ double group_sum_d(double x) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) x += __shfl_xor(x, o, WIDTH);
  return x;
}

// Strictly-lower block (j, t), t < j, from its linear number p = j(j-1)/2 + t.
__device__ __forceinline__ void block_of(int p, int& j, int& t) {
  int jj = static_cast<int>((1.0f + sqrtf(1.0f + 8.0f * static_cast<float>(p))) * 0.5f);
  while (jj * (jj - 1) / 2 > p) --jj;
  while ((jj + 1) * jj / 2 <= p) ++jj;
  j = jj;
  t = p - jj * (jj - 1) / 2;
}

}  // namespace casgd
