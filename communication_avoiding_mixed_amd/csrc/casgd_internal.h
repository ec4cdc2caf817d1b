// Launchers of the CA-SGD kernels (host side).  Each queues its kernels on
// `stream` and returns the launch status; shapes are validated by the C ABI
// layer before any of these is called.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

namespace casgd {

// Optional pair of HIP events stamped by the kernel dispatch itself (start and
// end of the kernel), so a timed launch measures the kernel and not the queue.
struct LaunchTimer {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

template <typename... Params, typename... Args>
hipError_t launch_kernel(void (*kernel)(Params...), dim3 grid, dim3 block, size_t lds,
                         hipStream_t stream, const LaunchTimer& tm, Args... args) {
  if (tm.start)
    hipExtLaunchKernelGGL(kernel, grid, block, static_cast<uint32_t>(lds), stream, tm.start, tm.stop,
                          0u, static_cast<Params>(args)...);
  else
    kernel<<<grid, block, lds, stream>>>(static_cast<Params>(args)...);
  return hipGetLastError();
}

constexpr int kStoreBF16 = 0;
constexpr int kStoreF32 = 1;
constexpr int kStoreF16 = 2;
constexpr int kStoreF8 = 3;  // OCP E4M3 of X * 2^k, k one exponent per matrix

// Element type of the gathered rows Y, which the Gram, the margins, the
// recurrence and the update read: the storage type, except that fp8 rows
// are widened (exactly) to bf16 by the gather.
inline int row_kind(int storage) { return storage == kStoreF8 ? kStoreBF16 : storage; }
inline int elem_bytes(int kind) { return kind == kStoreF32 ? 4 : kind == kStoreF8 ? 1 : 2; }

// X (float32 m x n) -> stored rows (m x ld, zero-padded) of the storage type;
// fp8 stores e4m3(x * 2^fp8_exp).
hipError_t launch_store(int storage, const float* X, void* Xs, int64_t m, int64_t n,
                        int64_t ld, int fp8_exp, hipStream_t stream);
// Largest |x| over count floats as a float32 bit pattern into *out_dev (a
// NaN above every number); partial holds kMaxAbsBlocks words.
constexpr int kMaxAbsBlocks = 1024;
hipError_t launch_maxabs(const float* X, int64_t count, uint32_t* partial, uint32_t* out_dev,
                         hipStream_t stream);

// Sample (or take idx_in), gather rows into Y (of row_kind(storage)) and
// labels into yB; fp8 rows are divided by 2^fp8_exp as they are widened.
hipError_t launch_gather(int storage, const void* Xs, const float* y, int64_t m, int64_t ld,
                         int sb, uint64_t seed, const int32_t* idx_in, int32_t* idx_out,
                         void* Y, float* yB, int fp8_exp, hipStream_t stream, const LaunchTimer& tm = {});

// Strictly-lower block triangle of Y Y^T in block-row layout, one 64 x 64
// output tile per workgroup.
// `order` (device, plan.slots ints) maps workgroups to tiles so that tiles
// sharing rows of Y run on the same XCD; build it with gram_order for the
// number of XCDs the tiles are spread over (workgroup g of the Gram runs on
// XCD g mod nx of those).
constexpr int kXcds = 8;
struct GramPlan {
  int tiles = 0;  // 64 x 64 output tiles
  int slots = 0;  // workgroups launched: tiles rounded up to a multiple of nx
};
GramPlan gram_plan(int storage, int s, int b, int64_t ld, int nx = kXcds);
// bf16 tile variant for rows of ld elements: 0 -> 32-wide K stages, one in
// flight (ld <= 32); 1, 2, 3 -> 64-wide stages, 8, 4 or 2 in flight.
inline int gram_variant(int64_t ld) {
  if (ld <= 32) return 0;
  const int64_t nstage = (ld + 63) / 64;
  return nstage >= 8 ? 1 : nstage >= 4 ? 2 : 3;
}
std::vector<int> gram_order(int s, int b, int nx = kXcds);
// kind: row_kind of the storage; gr: round each entry of G once to bf16.
hipError_t launch_gram(int kind, const void* Y, int64_t ld, int s, int b, float* G,
                       const GramPlan& plan, const int* order, int gr, hipStream_t stream,
                       const LaunchTimer& tm = {});

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
  long spin;                 // polls before a wait between workgroups expires
  int vround;                // margins stored as bf16 (rounded when formed) instead of float32
  // Margins as tagged words (epoch, float) at vbox[row], written by other
  // workgroups of the same launch; nullptr: the chain computes them itself.
  const unsigned long long* vbox = nullptr;
  // Chain workgroup q runs as workgroup q * stride of the launch.  With
  // stride = the XCD count, dispatch places all of them on XCD 0, where the
  // r values can travel through that XCD's L2 (see place).
  int stride = 1;
  // Q tagged words: the XCD of each chain workgroup, written at its start.
  // When every chain workgroup finds all Q on its own XCD it publishes r with
  // plain stores (they land in the shared L2, where the other workgroups'
  // device-scope loads find them); otherwise, or with place == nullptr, with
  // device-scope stores that write through to memory.
  unsigned long long* place = nullptr;
  // CUs of the device (host side only): a launch whose Q chain workgroups
  // cannot all be resident at once fails with hipErrorLaunchOutOfResources
  // instead of waiting on workgroups that never start.
  int cus = 0;
};
// Whether chain workgroups of shape (s, b, Q, ld) run the fast recurrence
// (the only one that can take its margins from vbox).
bool chain_fast(int s, int b, int Q, int64_t ld);
size_t chain_lds_bytes(int s, int b, int Q, int64_t ld);
constexpr int kChainMaxWorkgroups = 64;
// How the recurrence's workgroups are laid out for a shape: Q workgroups at
// launch indices q * stride.  one_xcd asks for all of them on one XCD (Q at
// most cus_per_xcd); they must then all fit the fast recurrence path.
struct ChainPlan {
  int Q = 1;
  int stride = 1;
  bool lean = false;  // the shape runs the lean recurrence (launch_step)
};
ChainPlan chain_plan(int s, int b, int64_t ld, int xcds, int cus_per_xcd, int layout);
hipError_t launch_chain(int storage, int loss, const ChainArgs& a, hipStream_t stream,
                        const LaunchTimer& tm = {});

// One launch of the pipelined training loop: the chain of outer step k on
// the a.Q chain workgroups (see ChainArgs::stride), and on the other
// workgroups the margins of step k (mar_wgs > 0; handed to the chain through
// a.vbox), the Gram of step k+1 (gram_slots > 0; gram0 a multiple of the
// number of XCDs the other roles run on, 8 or 7, so the tile order's XCD
// grouping holds) and the sample + gather of step k+2 (gath_wgs > 0).  The
// three roles use disjoint buffers; Y/G/yB of the chain, Y/G of the Gram and
// idx/Y/yB of the gather belong to three different steps.
struct PipeArgs {
  ChainArgs a;
  // Non-chain roles are numbered o = 0, 1, ... over the workgroups that are
  // not chain workgroups: with a.stride == 1 the chain is [0, Q) and o = w -
  // ochain (ochain = Q rounded up to a multiple of 8); with a.stride == 8 the
  // chain owns the multiples of 8 below 8Q, the other multiples of 8 exit at
  // once, and o = 7 * (w / 8) + (w % 8) - 1 (XCDs 1..7).  The ranges below
  // are in o.
  int ochain = 0;
  int mar0 = 0, mar_wgs = 0, mar_rows = 0;  // margins: mar_rows rows per workgroup, into a.vbox
  unsigned long long* vbox_out = nullptr;   // = a.vbox, writable
  int gram0 = 0, gram_slots = 0, tps = 0;
  const void* gY = nullptr;  // Y of step k+1 (stored type)
  float* gG = nullptr;           // G of step k+1
  const int* order = nullptr;
  int gbf16 = 0;  // the Gram role rounds each entry of G once to bf16
  int gath0 = 0, gath_wgs = 0, gs = 0;  // gs: lanes per row (gather::group_size)
  int gf8 = 0;          // stored rows are fp8: widened to bf16 (times unscale) as they are gathered
  float unscale = 1.f;  // 2^-k of fp8 storage
  const void* Xs = nullptr;
  const float* y = nullptr;
  int64_t m = 0, cpr = 0;  // cpr: 16-byte chunks of a stored row
  int sb = 0;
  uint64_t seed = 0;  // seed of step k+2
  int32_t* idx_out = nullptr;
  void* Yo = nullptr;
  float* yBo = nullptr;
};
hipError_t launch_pipe(int storage, int loss, const PipeArgs& p, hipStream_t stream,
                       const LaunchTimer& tm = {});

// The same launch with the lean recurrence (casgd_step.h) for shapes where
// step_fits holds (b a multiple of 4, at most 4 own rows per minibatch and 4
// columns per lane, the workgroup's rows of G in LDS).  Needs the margins
// role (mar_wgs > 0, a.vbox); a.preload is ignored.
bool step_fits(int s, int b, int Q, int64_t ld);
hipError_t launch_step(int storage, int loss, const PipeArgs& p, hipStream_t stream,
                       const LaunchTimer& tm = {});

// casgd_train's whole loop as one persistent launch of `grid` workgroups
// (casgd_train.h); for shapes where step_fits holds.
namespace persist {
struct TrainArgs;
}
hipError_t launch_train(int storage, const persist::TrainArgs& A, int grid, hipStream_t stream,
                        const LaunchTimer& tm = {});
// Dynamic LDS bytes of that launch (0: it does not fit in one workgroup).
size_t train_lds(int storage, int s, int b, int Q, int64_t ld, int mar_rows, bool dbl);

// Lookahead form of the same kernel (one critical workgroup for the d latest
// blocks of every step, M helpers for the rest, receivers for the update);
// ok is false for shapes it does not take (then launch_chain is used).
struct LaPlan {
  bool ok = false;
  int d = 0;       // near blocks per step
  int M = 0;       // helper workgroups (b / M rows each)
  size_t lds = 0;  // dynamic LDS bytes per workgroup
};
LaPlan la_plan(int s, int b);
hipError_t launch_chain_la(int storage, int loss, const ChainArgs& a, const LaPlan& plan,
                           hipStream_t stream, const LaunchTimer& tm = {});

// Mean loss over all m stored rows into out_dev (one double); partial must
// hold kLossBlocks doubles.
constexpr int kLossBlocks = 2048;
hipError_t launch_loss(int storage, int loss, const void* Xs, const float* y, int64_t m,
                       int64_t n, int64_t ld, const float* w, double* partial, double* out_dev,
                       int fp8_exp, hipStream_t stream);
// The partial sums launch_loss writes for this shape (at most kLossBlocks).
int loss_partials(int storage, int64_t m, int64_t ld);

// Calibration kernels (k_peak.hip): a copy of bytes (a multiple of 16) from
// src to dst, and workgroups x 256 lanes of iters x 4 dependent bf16 MFMAs
// (32x32x16) per wave, each lane's accumulator sum written to out.
hipError_t launch_peak_copy(const void* src, void* dst, int64_t bytes, int cus, hipStream_t stream);
hipError_t launch_peak_mfma(float* out, int workgroups, int iters, hipStream_t stream);
// workgroups read bytes (a multiple of 16) of src, each a contiguous slice,
// with direct-to-LDS loads; out[workgroups * 8] receives ring words.
hipError_t launch_peak_read(const void* src, int64_t bytes, float* out, int workgroups, hipStream_t stream);

}  // namespace casgd
