// One 64 x 64 output tile of the strictly-lower block triangle of G = Y Y^T,
// on bf16 MFMA (v_mfma_f32_32x32x16_bf16, float32 accumulators) for bf16
// rows, on fp16 MFMA (v_mfma_f32_32x32x16_f16, the same operand layout) for
// fp16 rows, or on the vector ALUs for float32 rows, as device functions so
// both the stand-alone Gram kernel and the pipelined step kernel run the same
// code.  The Abstract of "Mixed-Precision Communication-Avoiding
// SGD for Generalized Linear Models on GPUs" forms the Gram from low-precision
// inputs with high-precision accumulation on the matrix hardware.
//
// Output layout (block-row): block-row j (1 <= j < s) is the b x (j*b)
// row-major matrix [G_{j,0} ... G_{j,j-1}] starting at element b*b*j(j-1)/2.
#pragma once

#include "casgd_device.h"

namespace casgd {
namespace gram {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kTile = 64;  // output tile edge; 4 waves of 32 x 32

// LDS the tile function needs: two buffers of A and of B, kTile rows of
// BK + 8 bf16 each (the pad breaks bank aliasing).
template <int BK>
constexpr int lds_elems() {
  return 2 * 2 * kTile * (BK + 8);
}

// Tile `tile` enumerates (block (j,t), tile row, tile col); a workgroup of
// 256 lanes computes it.  Output rows and columns past the block edge (b not
// a multiple of 64) are not stored.  K is walked in BK-wide stages: each
// stage's global loads are issued D stages before it is used (a ring of D
// register sets per lane), then the stage is copied into one of two LDS
// buffers and consumed by the MFMAs.  Loads carry no branches and their data
// is not touched until the LDS copy, so the compiler waits for exactly the
// stage it needs and D stages stay in flight.  The stage count is padded to a
// multiple of D with zero stages.  `lds` holds lds_elems<BK>() elements.
// Row r of the step's Y is row row_of(r) of `Y` (the gathered rows
// themselves, or the stored data read through the sampled indices).  WT
// writes G through to memory (device-scope stores), for readers on other
// XCDs inside the same launch.
struct SameRow {
  __device__ int64_t operator()(int r) const { return r; }
};

// gr: G communicated in low precision, each float32 entry rounded once to
// the nearest bf16 (ties to even) as it is stored.
template <bool WT>
__device__ __forceinline__ void store_g(float* p, float v, bool gr) {
  if (gr) v = bf16_to_f32(f32_to_bf16(v));
  if constexpr (WT)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}

// F16: the 16-bit rows are fp16 (else bf16).
template <int BK, int D, bool WT = false, typename RowOf = SameRow, bool F16 = false>
__device__ __forceinline__ void bf16_tile(const uint16_t* __restrict__ Y, int64_t ld, int b, int tps,
                                          float* __restrict__ G, int tile, uint16_t* lds, RowOf row_of = {},
                                          bool gr = false) {
  constexpr int CPR = BK / 8;          // 16-byte chunks per tile row per stage
  constexpr int RPP = 256 / CPR;       // tile rows loaded per pass
  constexpr int PASSES = kTile / RPP;  // passes per operand per stage
  constexpr int LW = BK + 8;           // LDS row pitch (elements)
  constexpr int BUF = kTile * LW;
  uint16_t* As = lds;            // [2][BUF]
  uint16_t* Bs = lds + 2 * BUF;  // [2][BUF]

  const int nt2 = tps * tps;
  const int p = tile / nt2;
  const int rem = tile - p * nt2;
  const int ti = rem / tps;
  const int tj = rem - ti * tps;
  int j, t;
  block_of(p, j, t);

  float* Gj = G + static_cast<int64_t>(b) * b * (static_cast<int64_t>(j) * (j - 1) / 2);
  const int64_t ldg = static_cast<int64_t>(j) * b;
  const int a0 = ti * kTile;  // first row of the A tile inside block-row j
  const int b0 = tj * kTile;  // first row of the B tile inside block-row t

  // Rows past the block edge read rows of the same block instead; they only
  // feed output rows / columns that are never stored.
  const int lrow = threadIdx.x / CPR;
  const int lchunk = threadIdx.x - lrow * CPR;
  const uint16_t* aptr[PASSES];
  const uint16_t* bptr[PASSES];
#pragma unroll
  for (int q = 0; q < PASSES; ++q) {
    const int r = lrow + q * RPP;
    const int ar = a0 + r < b ? r : 0;
    const int br = b0 + r < b ? r : 0;
    aptr[q] = Y + row_of(j * b + a0 + ar) * ld + lchunk * 8;
    bptr[q] = Y + row_of(t * b + b0 + br) * ld + lchunk * 8;
  }

  // Chunks past the end of the row (a half-width last stage, or the zero
  // stages that pad the count to a multiple of D) read column 0 and are
  // zeroed when copied to LDS, D stages later, so no load waits early.
  u32x4 ra[D][PASSES], rb[D][PASSES];
  bool kin[D];
  const int64_t nstage = (ld + BK - 1) / BK;
  const int64_t nst_pad = (nstage + D - 1) / D * D;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  auto load_stage = [&](int slot, int64_t st) {
    const int64_t k0 = st * BK;
    kin[slot] = k0 + lchunk * 8 < ld;
    const int64_t off = kin[slot] ? k0 : 0;
#pragma unroll
    for (int q = 0; q < PASSES; ++q) {
      ra[slot][q] = *reinterpret_cast<const u32x4*>(aptr[q] + off);
      rb[slot][q] = *reinterpret_cast<const u32x4*>(bptr[q] + off);
    }
  };

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int arow = wm * 32 + (lane & 31);
  const int brow = wn * 32 + (lane & 31);
  const int kofs = (lane >> 5) * 8;

  // one accumulator per 16-wide K slice of a stage: the MFMAs of a stage are
  // independent and issue back to back instead of waiting on each other
  constexpr int NACC = BK / 16;
  f32x16_t acc[NACC];
#pragma unroll
  for (int kk = 0; kk < NACC; ++kk)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[kk][e] = 0.f;

#pragma unroll
  for (int d = 0; d < D; ++d) load_stage(d, d);

  for (int64_t st0 = 0; st0 < nst_pad; st0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int buf = static_cast<int>((st0 + d) & 1);
#pragma unroll
      for (int q = 0; q < PASSES; ++q) {
        const int r = lrow + q * RPP;
        *reinterpret_cast<u32x4*>(&As[buf * BUF + r * LW + lchunk * 8]) = kin[d] ? ra[d][q] : zero;
        *reinterpret_cast<u32x4*>(&Bs[buf * BUF + r * LW + lchunk * 8]) = kin[d] ? rb[d][q] : zero;
      }
      __syncthreads();
      load_stage(d, st0 + d + D);
#pragma unroll
      for (int kk = 0; kk < NACC; ++kk) {
        if constexpr (F16) {
          const f16x8_t av = *reinterpret_cast<const f16x8_t*>(&As[buf * BUF + arow * LW + kk * 16 + kofs]);
          const f16x8_t bv = *reinterpret_cast<const f16x8_t*>(&Bs[buf * BUF + brow * LW + kk * 16 + kofs]);
          acc[kk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, acc[kk], 0, 0, 0);
        } else {
          const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(&As[buf * BUF + arow * LW + kk * 16 + kofs]);
          const bf16x8_t bv = *reinterpret_cast<const bf16x8_t*>(&Bs[buf * BUF + brow * LW + kk * 16 + kofs]);
          acc[kk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[kk], 0, 0, 0);
        }
      }
    }
  }
#pragma unroll
  for (int kk = 1; kk < NACC; ++kk)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[0][e] += acc[kk][e];

  // Accumulator element e of lane l holds row 8*(e/4) + 4*(l/32) + e%4,
  // column l%32 of the wave's 32 x 32 sub-tile.
  const int col = b0 + wn * 32 + (lane & 31);
  if (col < b) {
    float* gcol = Gj + static_cast<int64_t>(t) * b + col;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = a0 + wm * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      if (row < b) store_g<WT>(&gcol[row * ldg], acc[0][e], gr);
    }
  }
}

// float32 storage: the same tiles on the vector ALUs, each lane a 4 x 4
// register block, K in 16-wide stages through LDS.  `lds` holds
// kF32LdsElems floats.
constexpr int kF32BK = 16;
constexpr int kF32LdsElems = 2 * kF32BK * (kTile + 4);

template <bool WT = false, typename RowOf = SameRow>
__device__ __forceinline__ void f32_tile(const float* __restrict__ Y, int64_t ld, int b, int tps,
                                         float* __restrict__ G, int tile, float* lds, RowOf row_of = {},
                                         bool gr = false) {
  constexpr int BK = kF32BK;
  constexpr int LW = kTile + 4;
  float* As = lds;            // [BK][LW]
  float* Bs = lds + BK * LW;  // [BK][LW]
  const int nt2 = tps * tps;
  const int p = tile / nt2;
  const int rem = tile - p * nt2;
  const int ti = rem / tps;
  const int tj = rem - ti * tps;
  int j, t;
  block_of(p, j, t);
  float* Gj = G + static_cast<int64_t>(b) * b * (static_cast<int64_t>(j) * (j - 1) / 2);
  const int64_t ldg = static_cast<int64_t>(j) * b;
  const int a0 = ti * kTile, b0 = tj * kTile;

  // loader: 64 rows x 16 k per stage = 256 float4
  const int lr = threadIdx.x >> 2;
  const int lk = (threadIdx.x & 3) * 4;
  const bool aok = a0 + lr < b, bok = b0 + lr < b;
  const float* ap = Y + row_of(j * b + a0 + (aok ? lr : 0)) * ld + lk;
  const float* bp = Y + row_of(t * b + b0 + (bok ? lr : 0)) * ld + lk;

  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int64_t k0 = 0; k0 < ld; k0 += BK) {
    const bool kin = k0 + lk < ld;
    const float4 av = (aok && kin) ? *reinterpret_cast<const float4*>(ap + k0) : make_float4(0, 0, 0, 0);
    const float4 bv = (bok && kin) ? *reinterpret_cast<const float4*>(bp + k0) : make_float4(0, 0, 0, 0);
    As[(lk + 0) * LW + lr] = av.x;
    As[(lk + 1) * LW + lr] = av.y;
    As[(lk + 2) * LW + lr] = av.z;
    As[(lk + 3) * LW + lr] = av.w;
    Bs[(lk + 0) * LW + lr] = bv.x;
    Bs[(lk + 1) * LW + lr] = bv.y;
    Bs[(lk + 2) * LW + lr] = bv.z;
    Bs[(lk + 3) * LW + lr] = bv.w;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      const float4 a4 = *reinterpret_cast<const float4*>(&As[k * LW + ty * 4]);
      const float4 b4 = *reinterpret_cast<const float4*>(&Bs[k * LW + tx * 4]);
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
      if (col < b) store_g<WT>(&Gj[row * ldg + static_cast<int64_t>(t) * b + col], acc[u][q], gr);
    }
  }
}

}  // namespace gram
}  // namespace casgd
