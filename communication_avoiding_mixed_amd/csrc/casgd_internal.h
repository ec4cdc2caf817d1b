// Launchers of the CA-SGD kernels (host side).  Each queues one or two kernels
// on `stream` and returns the launch status; shapes are validated by the C ABI
// layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace casgd {

constexpr int kStoreBF16 = 0;
constexpr int kStoreF32 = 1;

// X (float32 m x n) -> stored rows (m x ld, zero-padded), bf16 or f32.
hipError_t launch_store(int storage, const float* X, void* Xs, int64_t m, int64_t n,
                        int64_t ld, hipStream_t stream);

// Sample (or take idx_in), gather rows into Y, labels into yB; when w is
// non-null also margins v = Y w.
hipError_t launch_gather(int storage, const void* Xs, const float* y, int64_t m, int64_t n,
                         int64_t ld, int sb, uint64_t seed, const int32_t* idx_in,
                         int32_t* idx_out, void* Y, float* yB, const float* w, float* v,
                         hipStream_t stream);

// Strictly-lower block triangle of Y Y^T in block-row layout, for `nprob`
// independent problems spaced y_stride / g_stride elements apart.
hipError_t launch_gram(int storage, const void* Y, int64_t ld, int s, int b, float* G, int nprob,
                       int64_t y_stride, int64_t g_stride, hipStream_t stream);

// Inner recurrence over the s minibatches: z, r from G, v, yB.
hipError_t launch_recur(int loss, const float* G, const float* v, const float* yB, float* z,
                        float* r, int s, int b, float c, hipStream_t stream);

// w <- w - c * Y^T r over the first n columns.
hipError_t launch_update(int storage, const void* Y, int64_t ld, int64_t n, int sb,
                         const float* r, float c, float* w, hipStream_t stream);

// Mean loss over all m stored rows into out_dev (one double); partial must
// hold kLossBlocks doubles.
constexpr int kLossBlocks = 2048;
hipError_t launch_loss(int storage, int loss, const void* Xs, const float* y, int64_t m,
                       int64_t n, int64_t ld, const float* w, double* partial, double* out_dev,
                       hipStream_t stream);

}  // namespace casgd
