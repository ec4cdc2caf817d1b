// Launchers of the CA-SGD kernels (host side).  Each queues its kernels on
// `stream` and returns the launch status; shapes are validated by the C ABI
// layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace casgd {

constexpr int kStoreBF16 = 0;
constexpr int kStoreF32 = 1;

// X (float32 m x n) -> stored rows (m x ld, zero-padded), bf16 or f32.
hipError_t launch_store(int storage, const float* X, void* Xs, int64_t m, int64_t n,
                        int64_t ld, hipStream_t stream);

// Sample (or take idx_in), gather rows into Y and labels into yB.
hipError_t launch_gather(int storage, const void* Xs, const float* y, int64_t m, int64_t ld,
                         int sb, uint64_t seed, const int32_t* idx_in, int32_t* idx_out,
                         void* Y, float* yB, hipStream_t stream);

// Strictly-lower block triangle of Y Y^T in block-row layout, one 64 x 64
// output tile per workgroup.
struct GramPlan {
  int tiles = 0;  // 64 x 64 output tiles
};
GramPlan gram_plan(int storage, int s, int b, int64_t ld);
hipError_t launch_gram(int storage, const void* Y, int64_t ld, int s, int b, float* G,
                       const GramPlan& plan, hipStream_t stream);

// Margins, inner recurrence and update in one launch of Q workgroups.
struct ChainArgs {
  const void* Y;
  int64_t ld;
  int64_t n;
  int s, b, Q;
  float c;
  const float* G;
  const float* yB;
  float* v;
  float* z;
  float* r;
  float* w;
  unsigned long long* xbuf;  // Q mailboxes of s*b tagged words each
  uint32_t epoch;            // distinct per launch on this exchange buffer
  int* status;               // bit 0 set if an exchange wait expired
  int preload;               // set by launch_chain: own rows of G staged in LDS
};
size_t chain_lds_bytes(int s, int b, int Q);
int chain_workgroups(int s, int b);
constexpr int kChainMaxWorkgroups = 64;
hipError_t launch_chain(int storage, int loss, const ChainArgs& a, hipStream_t stream);

// Mean loss over all m stored rows into out_dev (one double); partial must
// hold kLossBlocks doubles.
constexpr int kLossBlocks = 2048;
hipError_t launch_loss(int storage, int loss, const void* Xs, const float* y, int64_t m,
                       int64_t n, int64_t ld, const float* w, double* partial, double* out_dev,
                       hipStream_t stream);

}  // namespace casgd
