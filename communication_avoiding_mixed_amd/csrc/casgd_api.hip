// C ABI of the CA-SGD library: argument checks, handle-owned device memory,
// streams, optional per-kernel event timing, and the launches that make one
// outer iteration (Abstract of "Mixed-Precision Communication-Avoiding SGD for
// Generalized Linear Models on GPUs").
//
// An outer iteration is split at its only weight dependence.  Sampling,
// gathering and the Gram matrix depend on the seed alone; they run on the
// handle's internal "prep" stream into one of two buffer sets.  Margins, the
// inner recurrence and the update need the weights; they run as one kernel on
// the caller's stream once the step's prep is done.  Consecutive steps
// alternate buffer sets, so the next step's gather and Gram overlap the
// current step's recurrence.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "casgd.h"
#include "casgd_device.h"
#include "casgd_gather.h"
#include "casgd_chain.h"
#include "casgd_internal.h"
#include "casgd_train.h"

// Static scratch of casgd_loss_noalloc: the loss reduction's per-workgroup
// partial sums.  Each GPU the library runs on holds its own copy until the
// process ends; every call on that GPU shares it.  Host code never uses this
// name as an address: the device address comes from hipGetSymbolAddress.
constexpr int kNoAllocPartials = casgd::kLossBlocks;
// casgd_create finds fp8's max |x| in the loss buffers
static_assert(sizeof(double) * casgd::kLossBlocks >= sizeof(uint32_t) * casgd::kMaxAbsBlocks, "max-abs partials");
static __device__ __align__(256) double scratch[kNoAllocPartials];

namespace {

thread_local std::string g_last_error;

// device address of `scratch` per device id, resolved once per device
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_addr;

// With dev current: the address of its copy of `scratch`.
hipError_t scratch_address(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (dev < 0) return hipErrorInvalidDevice;
  if (static_cast<int>(g_scratch_addr.size()) <= dev) g_scratch_addr.resize(dev + 1, nullptr);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return hipSuccess;
}

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(CASGD_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

constexpr int kMaxSB = 16384;
constexpr int kPipeGatherWgs = 64;  // gather workgroups of a pipelined step launch
constexpr int kMarginRows = 8;      // rows per margin workgroup of a pipelined step launch
// progress words of the persistent launch: gfree[64] | wdone[64] | gprog[up to kMaxGramWgs]
constexpr int kMaxGramWgs = 1024;
constexpr int kProgWords = 128 + kMaxGramWgs;

struct EventPair {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

struct StepBuffers {
  int32_t* idx = nullptr;
  void* Y = nullptr;
  float* yB = nullptr;
  float* G = nullptr;
};

}  // namespace

struct casgd_ctx {
  int64_t m = 0, n = 0, ld = 0;
  int loss = 0, storage = 0;
  size_t esize = 0;  // bytes of a stored element
  size_t ysize = 0;  // bytes of an element of the gathered rows Y (row_kind)
  int fp8_exp = 0;   // fp8 storage: X is stored as e4m3(x * 2^fp8_exp)
  int gram_bf16 = 0; // CASGD_OPT_GRAM_BF16
  void* Xs = nullptr;
  float* y = nullptr;
  hipStream_t stream = nullptr;  // caller's stream: weight-dependent work
  hipStream_t prep = nullptr;    // internal: sampling, gather, Gram
  hipEvent_t ev_prep[2] = {nullptr, nullptr};
  hipEvent_t ev_chain[2] = {nullptr, nullptr};
  hipEvent_t ev_switch = nullptr;  // orders a new caller stream after the old one
  int xcds = 1, cus = 1;           // XCDs and CUs of the device

  // workspace, sized for cap_sb rows and cap_g Gram elements
  int cap_sb = 0;
  int64_t cap_g = 0;
  StepBuffers buf[3];  // outer steps use sets 0 and 1; casgd_train's pipeline all three
  float* v = nullptr;
  float* z = nullptr;
  float* r = nullptr;
  int32_t* idx_user = nullptr;
  unsigned long long* xbuf = nullptr;
  // Gram workgroup -> tile tables for (order_s, order_b): [0] for tiles over
  // all XCDs (stand-alone Gram), [1] over the XCDs left to the other roles of
  // a pipelined step launch whose recurrence sits on one XCD
  int* order[2] = {nullptr, nullptr};
  int order_cap[2] = {0, 0}, order_s[2] = {0, 0}, order_b[2] = {0, 0}, order_nx[2] = {0, 0};
  unsigned long long* place = nullptr;  // XCD of each chain workgroup (tagged words)
  int* status = nullptr;
  double* loss_partial = nullptr;
  double* loss_out = nullptr;
  double* scratch = nullptr;  // this device's copy of the static scratch (casgd_loss_noalloc)
  uint32_t epoch = 0;
  int recurrence = 0;  // CASGD_OPT_RECURRENCE
  long spin = 0;       // CASGD_OPT_SPIN_LIMIT (0: the default bound)
  int margin_bf16 = 0; // CASGD_OPT_MARGIN_BF16
  int layout = 0;      // CASGD_OPT_CHAIN_LAYOUT
  int train_form = 0;  // CASGD_OPT_TRAIN_FORM
  unsigned long long* prog = nullptr;  // progress words of the persistent launch
  unsigned long long* wbox = nullptr;  // tagged weights of the persistent launch (n words)

  int next_buf = 0;
  int last_buf = 0;
  int last_s = 0, last_b = 0;

  int timing = 0;  // 0 off, else stamp every timing-th launch of each kernel
  int64_t issued[CASGD_K_COUNT] = {};
  std::vector<EventPair> pending[CASGD_K_COUNT];
  std::vector<EventPair> pool;
  double total_ms[CASGD_K_COUNT] = {};
  int64_t launches[CASGD_K_COUNT] = {};
};

namespace {

template <typename P>
void release(P*& p) {
  if (p) (void)hipFree(p);
  p = nullptr;
}

void free_workspace(casgd_ctx* h) {
  for (auto& bset : h->buf) {
    release(bset.idx);
    release(bset.Y);
    release(bset.yB);
    release(bset.G);
  }
  release(h->v);
  release(h->z);
  release(h->r);
  release(h->idx_user);
  release(h->xbuf);
  for (int i = 0; i < 2; ++i) {
    release(h->order[i]);
    h->order_cap[i] = h->order_s[i] = h->order_b[i] = h->order_nx[i] = 0;
  }
  h->cap_sb = 0;
  h->cap_g = 0;
}

hipError_t sync_all(casgd_ctx* h) {
  hipError_t e = hipStreamSynchronize(h->prep);
  hipError_t e2 = hipStreamSynchronize(h->stream);
  return e != hipSuccess ? e : e2;
}

template <typename P>
bool grab(P*& p, size_t bytes) {
  void* q = nullptr;
  if (hipMalloc(&q, bytes > 0 ? bytes : 16) != hipSuccess) return false;
  p = static_cast<P*>(q);
  return true;
}

int ensure_workspace(casgd_ctx* h, int s, int b) {
  const int sb = s * b;
  const int64_t gsz = static_cast<int64_t>(b) * b * s * (s - 1) / 2;
  if (sb <= h->cap_sb && gsz <= h->cap_g) return CASGD_OK;
  hipError_t e = sync_all(h);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  const int new_sb = sb > h->cap_sb ? sb : h->cap_sb;
  const int64_t new_g = gsz > h->cap_g ? gsz : h->cap_g;
  free_workspace(h);
  bool ok = true;
  for (auto& bset : h->buf) {
    ok = ok && grab(bset.idx, sizeof(int32_t) * new_sb) && grab(bset.Y, h->ysize * h->ld * new_sb) &&
         grab(bset.yB, sizeof(float) * new_sb) && grab(bset.G, sizeof(float) * new_g);
  }
  ok = ok && grab(h->v, sizeof(float) * new_sb) && grab(h->z, sizeof(float) * new_sb) &&
       grab(h->r, sizeof(float) * new_sb) && grab(h->idx_user, sizeof(int32_t) * new_sb) &&
       grab(h->xbuf, sizeof(unsigned long long) * (casgd::kChainMaxWorkgroups + 1) * new_sb);
  if (ok) {
    ok = hipMemset(h->xbuf, 0, sizeof(unsigned long long) * (casgd::kChainMaxWorkgroups + 1) * new_sb) ==
             hipSuccess &&
         hipDeviceSynchronize() == hipSuccess;
  }
  if (!ok) {
    (void)hipGetLastError();
    free_workspace(h);
    return fail(CASGD_ENOMEM, "device allocation of the outer-step workspace failed");
  }
  h->cap_sb = new_sb;
  h->cap_g = new_g;
  return CASGD_OK;
}

// The Gram's XCD-grouped tile order for shape (s, b) over nx XCDs in table
// `which`, rebuilt when the shape changes.
int ensure_order(casgd_ctx* h, int which, int s, int b, int nx) {
  if (h->order[which] && h->order_s[which] == s && h->order_b[which] == b && h->order_nx[which] == nx)
    return CASGD_OK;
  const std::vector<int> order = casgd::gram_order(s, b, nx);
  hipError_t e = sync_all(h);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  if (static_cast<int>(order.size()) > h->order_cap[which]) {
    release(h->order[which]);
    h->order_cap[which] = 0;
    if (!grab(h->order[which], sizeof(int) * (order.size() > 0 ? order.size() : 1)))
      return fail(CASGD_ENOMEM, "device allocation of the Gram tile order failed");
    h->order_cap[which] = static_cast<int>(order.size());
  }
  if (!order.empty()) {
    e = hipMemcpy(h->order[which], order.data(), sizeof(int) * order.size(), hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "uploading the Gram tile order");
  }
  h->order_s[which] = s;
  h->order_b[which] = b;
  h->order_nx[which] = nx;
  return CASGD_OK;
}

// Layout of the recurrence's workgroups for (s, b) on this handle.
casgd::ChainPlan plan_chain(const casgd_ctx* h, int s, int b) {
  return casgd::chain_plan(s, b, h->ld, h->xcds, h->cus / h->xcds, h->layout);
}

int launch_fail(hipError_t e, const char* what) {
  if (e == hipErrorLaunchOutOfResources)
    return fail(CASGD_EHIP, std::string(what) +
                                ": the recurrence's workgroups cannot all be resident at once on this device");
  return hip_fail(e, what);
}

EventPair take_pair(casgd_ctx* h) {
  if (!h->pool.empty()) {
    EventPair p = h->pool.back();
    h->pool.pop_back();
    return p;
  }
  EventPair p;
  (void)hipEventCreate(&p.start);
  (void)hipEventCreate(&p.stop);
  return p;
}

// Call fn(timer): with timing on, the timer's events are stamped by the
// kernel's own dispatch (start and end of that kernel).
template <typename Fn>
hipError_t timed(casgd_ctx* h, int kernel, Fn&& fn) {
  if (!h->timing || h->issued[kernel]++ % h->timing != 0) return fn(casgd::LaunchTimer{});
  EventPair p = take_pair(h);
  hipError_t e = fn(casgd::LaunchTimer{p.start, p.stop});
  h->pending[kernel].push_back(p);
  return e;
}

int check_step_args(casgd_ctx* h, int s, int b, const float* w) {
  if (!h) return fail(CASGD_EINVAL, "NULL handle");
  if (s < 1 || b < 1) return fail(CASGD_EINVAL, "s and b must be >= 1");
  if (static_cast<int64_t>(s) * b > kMaxSB) return fail(CASGD_EINVAL, "s*b exceeds 16384");
  if (!w) return fail(CASGD_EINVAL, "NULL weight pointer");
  return CASGD_OK;
}

// Check the kernels' error word (exchange waits that expired); streams are synced.
int check_status(casgd_ctx* h) {
  int st = 0;
  hipError_t e = hipMemcpy(&st, h->status, sizeof(int), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "reading the status word");
  if (st != 0) {
    (void)hipMemset(h->status, 0, sizeof(int));
    return fail(CASGD_EHIP, "an inner-step exchange between workgroups timed out");
  }
  return CASGD_OK;
}

// The launches of one outer iteration.  idx_in == nullptr: sample with `seed`.
int run_outer(casgd_ctx* h, int s, int b, float eta, uint64_t seed, const int32_t* idx_in,
              float* w) {
  int rc = ensure_workspace(h, s, b);
  if (rc != CASGD_OK) return rc;
  rc = ensure_order(h, 0, s, b, casgd::kXcds);
  if (rc != CASGD_OK) return rc;
  const int sb = s * b;
  const float c = eta / static_cast<float>(b);
  const int k = h->next_buf;
  StepBuffers& B = h->buf[k];
  hipError_t e;

  // weight-independent part, on the prep stream
  e = hipStreamWaitEvent(h->prep, h->ev_chain[k], 0);
  if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  e = timed(h, CASGD_K_GATHER, [&](const casgd::LaunchTimer& tm) {
    return casgd::launch_gather(h->storage, h->Xs, h->y, h->m, h->ld, sb, seed, idx_in, B.idx,
                                B.Y, B.yB, h->fp8_exp, h->prep, tm);
  });
  if (e != hipSuccess) return hip_fail(e, "gather launch");
  const casgd::GramPlan plan = casgd::gram_plan(h->storage, s, b, h->ld);
  e = timed(h, CASGD_K_GRAM, [&](const casgd::LaunchTimer& tm) {
    return casgd::launch_gram(casgd::row_kind(h->storage), B.Y, h->ld, s, b, B.G, plan, h->order[0],
                              h->gram_bf16, h->prep, tm);
  });
  if (e != hipSuccess) return hip_fail(e, "gram launch");
  e = hipEventRecord(h->ev_prep[k], h->prep);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");

  // weight-dependent part, on the caller's stream
  e = hipStreamWaitEvent(h->stream, h->ev_prep[k], 0);
  if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  casgd::ChainArgs a;
  a.Y = B.Y;
  a.ld = h->ld;
  a.n = h->n;
  a.s = s;
  a.b = b;
  const casgd::ChainPlan cp = plan_chain(h, s, b);
  a.Q = cp.Q;
  a.stride = cp.stride;
  a.place = (cp.stride > 1 || h->xcds == 1) ? h->place : nullptr;
  a.cus = h->cus;
  a.c = c;
  a.G = B.G;
  a.yB = B.yB;
  a.v = h->v;
  a.z = h->z;
  a.r = h->r;
  a.w = w;
  a.xbuf = h->xbuf;
  a.epoch = ++h->epoch == 0 ? ++h->epoch : h->epoch;
  a.status = h->status;
  a.spin = h->spin > 0 ? h->spin : casgd::chain::kSpinLimit;
  a.vround = h->margin_bf16;
  // The all-to-all kernel is the faster one on every measured shape, so it is
  // the default; the lookahead form runs only when asked for.
  const casgd::LaPlan la = h->recurrence == 2 ? casgd::la_plan(s, b) : casgd::LaPlan{};
  if (la.ok) {
    a.Q = casgd::kChainMaxWorkgroups;
    a.stride = 1;
    a.place = nullptr;
  }
  if (!la.ok && cp.lean) {
    // the lean recurrence with its margins computed by workgroups of the same
    // launch (the launch casgd_train uses, without the Gram and gather roles)
    casgd::PipeArgs p;
    p.a = a;
    p.a.preload = 0;
    p.vbox_out = h->xbuf + static_cast<int64_t>(casgd::kChainMaxWorkgroups) * sb;
    p.a.vbox = p.vbox_out;
    p.ochain = (a.Q + casgd::kXcds - 1) / casgd::kXcds * casgd::kXcds;
    p.mar0 = 0;
    p.mar_rows = kMarginRows;
    p.mar_wgs = (sb + kMarginRows - 1) / kMarginRows;
    e = timed(h, CASGD_K_CHAIN, [&](const casgd::LaunchTimer& tm) {
      return casgd::launch_step(casgd::row_kind(h->storage), h->loss, p, h->stream, tm);
    });
  } else {
    e = timed(h, CASGD_K_CHAIN, [&](const casgd::LaunchTimer& tm) {
      return la.ok ? casgd::launch_chain_la(casgd::row_kind(h->storage), h->loss, a, la, h->stream, tm)
                   : casgd::launch_chain(casgd::row_kind(h->storage), h->loss, a, h->stream, tm);
    });
  }
  if (e != hipSuccess) return launch_fail(e, "recurrence launch");
  e = hipEventRecord(h->ev_chain[k], h->stream);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");

  h->last_buf = k;
  h->next_buf = k ^ 1;
  h->last_s = s;
  h->last_b = b;
  return CASGD_OK;
}

// Rows per margin workgroup of the persistent launch for (s, b): about half
// of the workgroups besides the recurrence's compute margins (few rows each,
// so a step's margins come out soon after its weights), at least
// kMarginRows rows each, fewer when their rows (staged in LDS) would not
// fit; 0 if no choice fits, or the margins would need more than half of
// those workgroups.
int persist_margin_rows(const casgd_ctx* h, const casgd::ChainPlan& cp, int s, int b) {
  const int cus_per_xcd = h->cus / h->xcds;
  const int others = cp.stride > 1 ? (cp.stride - 1) * cus_per_xcd : h->cus - cp.Q;
  const int sb = s * b;
  if (others < 16) return 0;
  int rows = (sb + others / 2 - 1) / (others / 2);
  if (rows < kMarginRows) rows = kMarginRows;
  while (rows > 1 && casgd::train_lds(h->storage, s, b, cp.Q, h->ld, rows, false) == 0) --rows;
  if (casgd::train_lds(h->storage, s, b, cp.Q, h->ld, rows, false) == 0) return 0;
  return (sb + rows - 1) / rows <= others / 2 ? rows : 0;
}

// casgd_train as one persistent launch (casgd_train.h): the recurrence's
// workgroups, margin workgroups and Gram workgroups stay resident for all n
// steps; G of step i lives in buffer set i mod 3.  A gather of the last
// step's rows follows, for the exports.
int run_train_persist(casgd_ctx* h, const casgd::ChainPlan& cp, int s, int b, float eta, uint64_t base_seed,
                      uint64_t first, int n, float* w) {
  int rc = ensure_workspace(h, s, b);
  if (rc != CASGD_OK) return rc;
  const int nx = cp.stride > 1 ? cp.stride - 1 : casgd::kXcds;
  rc = ensure_order(h, 1, s, b, nx);
  if (rc != CASGD_OK) return rc;
  const int sb = s * b;
  const casgd::GramPlan gp = casgd::gram_plan(h->storage, s, b, h->ld, nx);
  auto round_up = [](int x, int k) { return (x + k - 1) / k * k; };
  // workgroups besides the recurrence's: everything the device holds at once
  const int cus_per_xcd = h->cus / h->xcds;
  const int grid = cp.stride > 1 ? cp.stride * cus_per_xcd : h->cus;
  const int others = cp.stride > 1 ? (cp.stride - 1) * cus_per_xcd : h->cus - cp.Q;
  const int mar_rows = persist_margin_rows(h, cp, s, b);
  if (mar_rows <= 0) return fail(CASGD_EHIP, "persistent train launch: no layout of the margin workgroups fits");
  const int mar_wgs = (sb + mar_rows - 1) / mar_rows;
  // a second G buffer when it fits: G_{k+1} then arrives during step k
  const bool dbl = casgd::train_lds(h->storage, s, b, cp.Q, h->ld, mar_rows, true) != 0;
  // the Gram's workgroups start at a multiple of nx (counted in launch
  // indices when the recurrence is spread) and come in multiples of nx
  int gram0 = round_up(mar_wgs, nx);
  if (cp.stride == 1) gram0 = round_up(cp.Q + mar_wgs, nx) - cp.Q;
  int gram_wgs = (others - gram0) / nx * nx;
  if (gram_wgs > kMaxGramWgs) gram_wgs = kMaxGramWgs / nx * nx;
  if (s == 1) gram_wgs = 0;
  if (gram_wgs <= 0 && s > 1) return fail(CASGD_EHIP, "persistent train launch: no workgroups left for the Gram");
  casgd::persist::TrainArgs A{};
  A.Xs = h->Xs;
  A.y = h->y;
  A.m = h->m;
  A.n = h->n;
  A.ld = h->ld;
  A.s = s;
  A.b = b;
  A.Q = cp.Q;
  A.stride = cp.stride;
  A.loss = h->loss;
  A.vround = h->margin_bf16;
  A.gbf16 = h->gram_bf16;
  A.c = eta / static_cast<float>(b);
  A.n_outer = n;
  A.base_seed = base_seed;
  A.first = first;
  A.w = w;
  A.v = h->v;
  A.z = h->z;
  A.r = h->r;
  for (int i = 0; i < casgd::persist::kRing; ++i) A.G[i] = h->buf[i].G;
  A.xbuf = h->xbuf;
  A.vbox = h->xbuf + static_cast<int64_t>(casgd::kChainMaxWorkgroups) * sb;
  A.wbox = h->wbox;
  A.place = (cp.stride > 1 || h->xcds == 1) ? h->place : nullptr;
  A.prog = h->prog;
  // tags of steps 0 .. n-1 (never 0: the buffers start zeroed)
  if (h->epoch + static_cast<uint32_t>(n) + 1 < h->epoch) h->epoch = 0;
  A.tag0 = h->epoch + 1;
  h->epoch += static_cast<uint32_t>(n);
  A.status = h->status;
  A.spin = h->spin > 0 ? h->spin : casgd::chain::kSpinLimit;
  A.ochain = cp.Q;
  A.mar_wgs = mar_wgs;
  A.mar_rows = mar_rows;
  A.gram0 = gram0;
  A.gram_wgs = gram_wgs;
  A.tiles = gp.tiles;
  A.tps = (b + 63) / 64;
  A.slots = gp.slots;
  A.order = h->order[1];
  A.dbl = dbl ? 1 : 0;
  A.cus = h->cus;
  // work queued earlier on the prep stream uses the buffer sets
  hipError_t e = hipEventRecord(h->ev_prep[0], h->prep);
  if (e == hipSuccess) e = hipStreamWaitEvent(h->stream, h->ev_prep[0], 0);
  if (e != hipSuccess) return hip_fail(e, "ordering the prep stream before the training launch");
  e = timed(h, CASGD_K_TRAIN, [&](const casgd::LaunchTimer& tm) {
    return casgd::launch_train(h->storage, A, grid, h->stream, tm);
  });
  if (e != hipSuccess) return launch_fail(e, "persistent training launch");
  StepBuffers& B = h->buf[(n - 1) % 3];
  e = casgd::launch_gather(h->storage, h->Xs, h->y, h->m, h->ld, sb,
                           casgd::splitmix64(base_seed, first + static_cast<uint64_t>(n - 1)), nullptr, B.idx, B.Y,
                           B.yB, h->fp8_exp, h->stream);
  if (e != hipSuccess) return hip_fail(e, "gather of the last step");
  e = hipEventRecord(h->ev_chain[0], h->stream);
  if (e == hipSuccess) e = hipEventRecord(h->ev_chain[1], h->stream);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  h->last_buf = (n - 1) % 3;
  h->last_s = s;
  h->last_b = b;
  return CASGD_OK;
}

// casgd_train's pipelined loop (all-to-all recurrence): step i
// uses buffer set i mod 3.  Prologue: gather and Gram of step 0, gather of
// step 1.  Launch i: chain of step i, Gram of step i+1, gather of step i+2.
// The gather of step i+2 overwrites the set of step i-1, whose chain ended
// with the previous launch; everything runs on the caller's stream.
int run_train_pipe(casgd_ctx* h, int s, int b, float eta, uint64_t base_seed, uint64_t first,
                   int n, float* w) {
  int rc = ensure_workspace(h, s, b);
  if (rc != CASGD_OK) return rc;
  rc = ensure_order(h, 0, s, b, casgd::kXcds);
  if (rc != CASGD_OK) return rc;
  // recurrence on one XCD: the other roles cycle over the remaining ones
  const casgd::ChainPlan cp = plan_chain(h, s, b);
  const int nx = cp.stride > 1 ? cp.stride - 1 : casgd::kXcds;
  const int ot = cp.stride > 1 ? 1 : 0;  // tile-order table of the step launch
  rc = ensure_order(h, ot, s, b, nx);
  if (rc != CASGD_OK) return rc;
  const int sb = s * b;
  const float c = eta / static_cast<float>(b);
  auto seed_of = [&](int i) { return casgd::splitmix64(base_seed, first + static_cast<uint64_t>(i)); };
  hipError_t e;

  // work queued earlier on the prep stream reads or writes sets 0 and 1
  e = hipEventRecord(h->ev_prep[0], h->prep);
  if (e == hipSuccess) e = hipStreamWaitEvent(h->stream, h->ev_prep[0], 0);
  if (e != hipSuccess) return hip_fail(e, "ordering the prep stream before the pipeline");

  auto gather = [&](int i) {
    StepBuffers& A = h->buf[i % 3];
    return timed(h, CASGD_K_GATHER, [&](const casgd::LaunchTimer& tm) {
      return casgd::launch_gather(h->storage, h->Xs, h->y, h->m, h->ld, sb, seed_of(i), nullptr, A.idx,
                                  A.Y, A.yB, h->fp8_exp, h->stream, tm);
    });
  };
  const casgd::GramPlan plan = casgd::gram_plan(h->storage, s, b, h->ld);
  const casgd::GramPlan pplan = casgd::gram_plan(h->storage, s, b, h->ld, nx);
  e = gather(0);
  if (e == hipSuccess)
    e = timed(h, CASGD_K_GRAM, [&](const casgd::LaunchTimer& tm) {
      return casgd::launch_gram(casgd::row_kind(h->storage), h->buf[0].Y, h->ld, s, b, h->buf[0].G, plan,
                                h->order[0], h->gram_bf16, h->stream, tm);
    });
  if (e == hipSuccess && n > 1) e = gather(1);
  if (e != hipSuccess) return hip_fail(e, "pipeline prologue");

  const int Q = cp.Q;
  const bool fast = casgd::chain_fast(s, b, Q, h->ld);
  const int64_t cpr = h->ld / (16 / static_cast<int64_t>(h->esize));  // 16-byte chunks of a stored row
  const int gs = casgd::gather::group_size(cpr);
  const int rows_per_wg = 256 / gs;
  const int gather_wgs_all = (sb + rows_per_wg - 1) / rows_per_wg;
  auto round_up = [](int x, int k) { return (x + k - 1) / k * k; };
  for (int i = 0; i < n; ++i) {
    StepBuffers& C = h->buf[i % 3];
    casgd::PipeArgs p;
    casgd::ChainArgs& a = p.a;
    a.Y = C.Y;
    a.ld = h->ld;
    a.n = h->n;
    a.s = s;
    a.b = b;
    a.Q = Q;
    a.stride = cp.stride;
    a.place = (cp.stride > 1 || h->xcds == 1) ? h->place : nullptr;
    a.cus = h->cus;
    a.c = c;
    a.G = C.G;
    a.yB = C.yB;
    a.v = h->v;
    a.z = h->z;
    a.r = h->r;
    a.w = w;
    a.xbuf = h->xbuf;
    a.epoch = ++h->epoch == 0 ? ++h->epoch : h->epoch;
    a.status = h->status;
    a.spin = h->spin > 0 ? h->spin : casgd::chain::kSpinLimit;
    a.vround = h->margin_bf16;
    a.preload = 0;
    // The other roles are numbered from 0 over the non-chain workgroups
    // (PipeArgs); the Gram's range starts at a multiple of nx so its tile
    // order's XCD grouping holds.  Margins by their own workgroups
    // (kMarginRows rows each) when the chain takes them from the exchange
    // buffer's last s*b words.
    p.ochain = round_up(Q, casgd::kXcds);
    int next = 0;
    if (fast || cp.lean) {
      p.vbox_out = h->xbuf + static_cast<int64_t>(casgd::kChainMaxWorkgroups) * sb;
      a.vbox = p.vbox_out;
      p.mar0 = 0;
      p.mar_rows = kMarginRows;
      p.mar_wgs = (sb + kMarginRows - 1) / kMarginRows;
      next = round_up(p.mar_wgs, nx);
    }
    p.gram0 = next;
    if (i + 1 < n && pplan.tiles > 0) {
      const StepBuffers& N = h->buf[(i + 1) % 3];
      p.gram_slots = pplan.slots;
      p.tps = (b + 63) / 64;
      p.gY = N.Y;
      p.gG = N.G;
      p.order = h->order[ot];
    }
    p.gath0 = p.gram0 + p.gram_slots;
    if (i + 2 < n) {
      StepBuffers& A = h->buf[(i + 2) % 3];
      p.gath_wgs = gather_wgs_all < kPipeGatherWgs ? gather_wgs_all : kPipeGatherWgs;
      p.gs = gs;
      p.Xs = h->Xs;
      p.y = h->y;
      p.m = h->m;
      p.cpr = cpr;
      p.sb = sb;
      p.seed = seed_of(i + 2);
      p.idx_out = A.idx;
      p.Yo = A.Y;
      p.yBo = A.yB;
      p.gf8 = h->storage == CASGD_FP8 ? 1 : 0;
      p.unscale = std::ldexp(1.0f, -h->fp8_exp);
    }
    p.gbf16 = h->gram_bf16;
    e = timed(h, CASGD_K_PIPE, [&](const casgd::LaunchTimer& tm) {
      return cp.lean ? casgd::launch_step(casgd::row_kind(h->storage), h->loss, p, h->stream, tm)
                     : casgd::launch_pipe(h->storage, h->loss, p, h->stream, tm);
    });
    if (e != hipSuccess) return launch_fail(e, "pipelined step launch");
  }
  // later outer steps' prep work reuses sets 0 and 1 only after this loop
  e = hipEventRecord(h->ev_chain[0], h->stream);
  if (e == hipSuccess) e = hipEventRecord(h->ev_chain[1], h->stream);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  h->last_buf = (n - 1) % 3;
  h->last_s = s;
  h->last_b = b;
  return CASGD_OK;
}

}  // namespace

extern "C" {

const char* casgd_last_error(void) { return g_last_error.c_str(); }

int casgd_peak_copy(const void* src, void* dst, int64_t bytes, void* hip_stream) {
  if (!src || !dst) return fail(CASGD_EINVAL, "NULL pointer");
  if (bytes < 0 || bytes % 16 != 0) return fail(CASGD_EINVAL, "bytes must be a non-negative multiple of 16");
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0)
    return fail(CASGD_EINVAL, "src and dst must be 16-byte aligned");
  const char* a = static_cast<const char*>(src);
  const char* d = static_cast<const char*>(dst);
  if (a < d + bytes && d < a + bytes) return fail(CASGD_EINVAL, "src and dst overlap");
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "querying the compute unit count");
  e = casgd::launch_peak_copy(src, dst, bytes, cus, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? CASGD_OK : hip_fail(e, "copy calibration launch");
}

int casgd_peak_read(const void* src, int64_t bytes, float* out, int workgroups, void* hip_stream) {
  if (!src || !out) return fail(CASGD_EINVAL, "NULL pointer");
  if (bytes < 16 || bytes % 16 != 0) return fail(CASGD_EINVAL, "bytes must be a positive multiple of 16");
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0) return fail(CASGD_EINVAL, "src must be 16-byte aligned");
  if (workgroups < 1 || workgroups > (1 << 20)) return fail(CASGD_EINVAL, "workgroups must be in [1, 2^20]");
  hipError_t e = casgd::launch_peak_read(src, bytes, out, workgroups, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? CASGD_OK : hip_fail(e, "read calibration launch");
}

int casgd_peak_mfma(float* out, int workgroups, int iters, void* hip_stream) {
  if (!out) return fail(CASGD_EINVAL, "NULL pointer");
  if (workgroups < 1 || workgroups > (1 << 20) || iters < 1)
    return fail(CASGD_EINVAL, "workgroups must be in [1, 2^20] and iters >= 1");
  hipError_t e = casgd::launch_peak_mfma(out, workgroups, iters, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? CASGD_OK : hip_fail(e, "MFMA calibration launch");
}

uint64_t casgd_step_seed(uint64_t base_seed, uint64_t k) { return casgd::splitmix64(base_seed, k); }

int64_t casgd_gram_bytes(int s, int b, int packed) {
  if (s < 1 || b < 1) return -1;
  const int64_t sb = static_cast<int64_t>(s) * b;
  if (packed) return 4 * static_cast<int64_t>(b) * b * s * (s - 1) / 2;
  return 4 * sb * sb;
}

casgd_handle casgd_create(const float* X, const float* y, int64_t m, int64_t n, int loss,
                          int storage) {
  if (!X || !y) {
    fail(CASGD_EINVAL, "NULL data pointer");
    return nullptr;
  }
  if (m < 1 || m > 2147483647LL || n < 1 || n > (1LL << 24)) {
    fail(CASGD_EINVAL, "need 1 <= m <= 2^31-1 and 1 <= n <= 2^24");
    return nullptr;
  }
  if (loss < CASGD_LOGISTIC || loss > CASGD_POISSON) {
    fail(CASGD_EINVAL, "unknown loss");
    return nullptr;
  }
  if (storage != CASGD_BF16 && storage != CASGD_FP32 && storage != CASGD_FP16 && storage != CASGD_FP8) {
    fail(CASGD_EINVAL, "unknown storage type");
    return nullptr;
  }
  casgd_ctx* h = new casgd_ctx;
  h->m = m;
  h->n = n;
  h->ld = (n + 31) / 32 * 32;
  h->loss = loss;
  h->storage = storage;
  h->esize = casgd::elem_bytes(storage);
  h->ysize = casgd::elem_bytes(casgd::row_kind(storage));
  bool ok = hipStreamCreateWithFlags(&h->prep, hipStreamNonBlocking) == hipSuccess &&
            hipEventCreateWithFlags(&h->ev_switch, hipEventDisableTiming) == hipSuccess;
  for (int i = 0; i < 2 && ok; ++i)
    ok = hipEventCreateWithFlags(&h->ev_prep[i], hipEventDisableTiming) == hipSuccess &&
         hipEventCreateWithFlags(&h->ev_chain[i], hipEventDisableTiming) == hipSuccess;
  // where the recurrence's workgroups can be placed
  int dev = 0, xcds = 1, cus = 1;
  ok = ok && hipGetDevice(&dev) == hipSuccess &&
       hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess;
  if (ok && hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess) {
    (void)hipGetLastError();
    xcds = 1;
  }
  h->xcds = xcds >= 1 && cus % xcds == 0 ? xcds : 1;
  h->cus = cus >= 1 ? cus : 1;
  void* scratch_ptr = nullptr;
  ok = ok && scratch_address(dev, &scratch_ptr) == hipSuccess;
  h->scratch = static_cast<double*>(scratch_ptr);
  if (!ok) {
    (void)hipGetLastError();
    fail(CASGD_EHIP, "creating the handle's stream and events failed");
    casgd_destroy(h);
    return nullptr;
  }
  if (!grab(h->Xs, h->esize * h->ld * m) || !grab(h->y, sizeof(float) * m) ||
      !grab(h->loss_partial, sizeof(double) * casgd::kLossBlocks) ||
      !grab(h->loss_out, sizeof(double)) || !grab(h->status, sizeof(int)) ||
      !grab(h->place, sizeof(unsigned long long) * casgd::kChainMaxWorkgroups) ||
      !grab(h->prog, sizeof(unsigned long long) * kProgWords) || !grab(h->wbox, sizeof(unsigned long long) * n)) {
    (void)hipGetLastError();
    fail(CASGD_ENOMEM, "device allocation of the stored data failed");
    casgd_destroy(h);
    return nullptr;
  }
  hipError_t e = hipMemsetAsync(h->status, 0, sizeof(int), h->stream);
  if (e == hipSuccess)
    e = hipMemsetAsync(h->place, 0, sizeof(unsigned long long) * casgd::kChainMaxWorkgroups, h->stream);
  if (e == hipSuccess) e = hipMemsetAsync(h->prog, 0, sizeof(unsigned long long) * kProgWords, h->stream);
  if (e == hipSuccess) e = hipMemsetAsync(h->wbox, 0, sizeof(unsigned long long) * n, h->stream);
  if (e == hipSuccess && storage == CASGD_FP8) {
    // the scale exponent: the largest k with max|x| * 2^k <= 448 = 0.875 * 2^9
    uint32_t bits = 0;
    e = casgd::launch_maxabs(X, m * n, reinterpret_cast<uint32_t*>(h->loss_partial),
                             reinterpret_cast<uint32_t*>(h->loss_out), h->stream);
    if (e == hipSuccess)
      e = hipMemcpyAsync(&bits, h->loss_out, sizeof(bits), hipMemcpyDeviceToHost, h->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(h->stream);
    float mx = 0.f;
    std::memcpy(&mx, &bits, sizeof(mx));
    if (std::isfinite(mx) && mx > 0.f) {
      int E = 0;
      const double f = std::frexp(static_cast<double>(mx), &E);
      h->fp8_exp = f <= 0.875 ? 9 - E : 8 - E;
    }
  }
  if (e == hipSuccess) e = casgd::launch_store(storage, X, h->Xs, m, n, h->ld, h->fp8_exp, h->stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(h->y, y, sizeof(float) * m, hipMemcpyDeviceToDevice, h->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(h->stream);
  if (e != hipSuccess) {
    hip_fail(e, "storing the data");
    casgd_destroy(h);
    return nullptr;
  }
  return h;
}

void casgd_destroy(casgd_handle h) {
  if (!h) return;
  if (h->prep) (void)hipStreamSynchronize(h->prep);
  (void)hipStreamSynchronize(h->stream);
  free_workspace(h);
  release(h->Xs);
  release(h->y);
  release(h->loss_partial);
  release(h->loss_out);
  release(h->status);
  release(h->place);
  release(h->prog);
  release(h->wbox);
  for (auto& v : h->pending)
    for (auto& p : v) h->pool.push_back(p);
  for (auto& p : h->pool) {
    (void)hipEventDestroy(p.start);
    (void)hipEventDestroy(p.stop);
  }
  for (int i = 0; i < 2; ++i) {
    if (h->ev_prep[i]) (void)hipEventDestroy(h->ev_prep[i]);
    if (h->ev_chain[i]) (void)hipEventDestroy(h->ev_chain[i]);
  }
  if (h->ev_switch) (void)hipEventDestroy(h->ev_switch);
  if (h->prep) (void)hipStreamDestroy(h->prep);
  delete h;
}

int casgd_set_stream(casgd_handle h, void* stream) {
  if (!h) return fail(CASGD_EINVAL, "NULL handle");
  hipStream_t next = static_cast<hipStream_t>(stream);
  if (next == h->stream) return CASGD_OK;
  // The handle's buffers are shared by all its work: the new stream starts
  // only after everything already queued on the old one.
  hipError_t e = hipEventRecord(h->ev_switch, h->stream);
  if (e == hipSuccess) e = hipStreamWaitEvent(next, h->ev_switch, 0);
  if (e != hipSuccess) return hip_fail(e, "ordering the new stream after the old one");
  h->stream = next;
  return CASGD_OK;
}

int64_t casgd_ld(casgd_handle h) { return h ? h->ld : -1; }

int casgd_fp8_exponent(casgd_handle h) { return h ? h->fp8_exp : 0; }

int casgd_set_option(casgd_handle h, int option, int value) {
  if (!h) return fail(CASGD_EINVAL, "NULL handle");
  if (option == CASGD_OPT_RECURRENCE && value >= 0 && value <= 2) {
    h->recurrence = value;
    return CASGD_OK;
  }
  if (option == CASGD_OPT_SPIN_LIMIT && value >= 0) {
    h->spin = value;
    return CASGD_OK;
  }
  if (option == CASGD_OPT_MARGIN_BF16 && (value == 0 || value == 1)) {
    h->margin_bf16 = value;
    return CASGD_OK;
  }
  if (option == CASGD_OPT_CHAIN_LAYOUT && value >= 0 && value <= 3) {
    h->layout = value;
    return CASGD_OK;
  }
  if (option == CASGD_OPT_GRAM_BF16 && (value == 0 || value == 1)) {
    h->gram_bf16 = value;
    return CASGD_OK;
  }
  if (option == CASGD_OPT_TRAIN_FORM && (value == 0 || value == 1)) {
    h->train_form = value;
    return CASGD_OK;
  }
  return fail(CASGD_EINVAL, "unknown option or value");
}

int casgd_outer_step(casgd_handle h, int s, int b, float eta, uint64_t seed, float* w) {
  int rc = check_step_args(h, s, b, w);
  if (rc != CASGD_OK) return rc;
  return run_outer(h, s, b, eta, seed, nullptr, w);
}

int casgd_outer_step_indices(casgd_handle h, int s, int b, float eta, const int32_t* idx,
                             float* w) {
  int rc = check_step_args(h, s, b, w);
  if (rc != CASGD_OK) return rc;
  if (!idx) return fail(CASGD_EINVAL, "NULL index pointer");
  const int sb = s * b;
  std::vector<int32_t> host(sb);
  hipError_t e = hipMemcpyAsync(host.data(), idx, sizeof(int32_t) * sb, hipMemcpyDeviceToHost,
                                h->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(h->stream);
  if (e != hipSuccess) return hip_fail(e, "copying indices");
  for (int i = 0; i < sb; ++i)
    if (host[i] < 0 || host[i] >= h->m) return fail(CASGD_EINVAL, "row index out of range");
  rc = ensure_workspace(h, s, b);
  if (rc != CASGD_OK) return rc;
  // the previous step's gather may still read idx_user
  e = hipStreamSynchronize(h->prep);
  if (e == hipSuccess)
    e = hipMemcpy(h->idx_user, host.data(), sizeof(int32_t) * sb, hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e, "copying indices");
  return run_outer(h, s, b, eta, 0, h->idx_user, w);
}

int casgd_train(casgd_handle h, int s, int b, float eta, uint64_t base_seed, uint64_t first_step,
                int n_outer, float* w) {
  int rc = check_step_args(h, s, b, w);
  if (rc != CASGD_OK) return rc;
  if (n_outer < 0) return fail(CASGD_EINVAL, "n_outer must be >= 0");
  // The persistent launch and the general pipelined kernel read bf16 or
  // float32 stored rows themselves; the pipelined launch of the lean
  // recurrence also gathers fp16 rows and widens fp8 rows.  Other cases run
  // step by step.
  const bool fused = h->storage == CASGD_BF16 || h->storage == CASGD_FP32;
  if (n_outer > 0 && h->recurrence != 2) {
    const casgd::ChainPlan cp = plan_chain(h, s, b);
    if (fused && cp.lean && h->train_form == 0 && persist_margin_rows(h, cp, s, b) > 0)
      return run_train_persist(h, cp, s, b, eta, base_seed, first_step, n_outer, w);
    if (fused || cp.lean) return run_train_pipe(h, s, b, eta, base_seed, first_step, n_outer, w);
  }
  for (int k = 0; k < n_outer; ++k) {
    rc = run_outer(h, s, b, eta, casgd::splitmix64(base_seed, first_step + k), nullptr, w);
    if (rc != CASGD_OK) return rc;
  }
  return CASGD_OK;
}

int casgd_loss(casgd_handle h, const float* w, double* out) {
  if (!h) return fail(CASGD_EINVAL, "NULL handle");
  if (!w || !out) return fail(CASGD_EINVAL, "NULL pointer");
  hipError_t e = casgd::launch_loss(h->storage, h->loss, h->Xs, h->y, h->m, h->n, h->ld, w,
                                    h->loss_partial, h->loss_out, h->fp8_exp, h->stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(out, h->loss_out, sizeof(double), hipMemcpyDeviceToHost, h->stream);
  if (e == hipSuccess) e = sync_all(h);
  if (e != hipSuccess) return hip_fail(e, "loss");
  return check_status(h);
}

int casgd_loss_noalloc(casgd_handle h, const float* w, double* out_dev) {
  if (!h) return fail(CASGD_EINVAL, "NULL handle");
  if (!w || !out_dev) return fail(CASGD_EINVAL, "NULL pointer");
  if (!h->scratch) return fail(CASGD_EHIP, "the static scratch has no device address");
  const int np = casgd::loss_partials(h->storage, h->m, h->ld);
  if (np > kNoAllocPartials)
    return fail(CASGD_EINVAL, "the loss needs " + std::to_string(np) + " partial sums; the static scratch holds " +
                                  std::to_string(kNoAllocPartials));
  const hipError_t e = casgd::launch_loss(h->storage, h->loss, h->Xs, h->y, h->m, h->n, h->ld, w, h->scratch,
                                          out_dev, h->fp8_exp, h->stream);
  if (e != hipSuccess) return hip_fail(e, "loss launch");
  return CASGD_OK;
}

int casgd_debug_export(casgd_handle h, int what, void* dst, size_t bytes) {
  if (!h) return fail(CASGD_EINVAL, "NULL handle");
  if (!dst) return fail(CASGD_EINVAL, "NULL destination");
  if (h->last_s == 0) return fail(CASGD_EINVAL, "no outer step has run yet");
  const int s = h->last_s, b = h->last_b;
  const size_t sb = static_cast<size_t>(s) * b;
  const StepBuffers& B = h->buf[h->last_buf];
  const void* src = nullptr;
  size_t need = 0;
  switch (what) {
    case CASGD_EXPORT_IDX: src = B.idx; need = sb * sizeof(int32_t); break;
    case CASGD_EXPORT_Y: src = B.Y; need = sb * h->ld * h->ysize; break;
    case CASGD_EXPORT_YB: src = B.yB; need = sb * sizeof(float); break;
    case CASGD_EXPORT_G:
      src = B.G;
      need = sizeof(float) * static_cast<size_t>(b) * b * s * (s - 1) / 2;
      break;
    case CASGD_EXPORT_V: src = h->v; need = sb * sizeof(float); break;
    case CASGD_EXPORT_Z: src = h->z; need = sb * sizeof(float); break;
    case CASGD_EXPORT_R: src = h->r; need = sb * sizeof(float); break;
    default: return fail(CASGD_EINVAL, "unknown export");
  }
  if (bytes != need) return fail(CASGD_EINVAL, "export size mismatch: need " + std::to_string(need));
  hipError_t e = sync_all(h);
  if (e == hipSuccess && need > 0) e = hipMemcpy(dst, src, need, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "export");
  return check_status(h);
}

int casgd_export_rows(casgd_handle h, int64_t row0, int64_t nrows, void* dst, size_t bytes) {
  if (!h) return fail(CASGD_EINVAL, "NULL handle");
  if (!dst) return fail(CASGD_EINVAL, "NULL destination");
  if (row0 < 0 || nrows < 0 || row0 + nrows > h->m) return fail(CASGD_EINVAL, "rows out of range");
  const size_t need = static_cast<size_t>(nrows) * h->ld * h->esize;
  if (bytes != need) return fail(CASGD_EINVAL, "export size mismatch");
  if (need == 0) return CASGD_OK;
  const char* src = static_cast<const char*>(h->Xs) + static_cast<size_t>(row0) * h->ld * h->esize;
  hipError_t e = hipMemcpyAsync(dst, src, need, hipMemcpyDeviceToHost, h->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(h->stream);
  if (e != hipSuccess) return hip_fail(e, "export rows");
  return CASGD_OK;
}

int casgd_set_timing(casgd_handle h, int on) {
  if (!h) return fail(CASGD_EINVAL, "NULL handle");
  if (on < 0) return fail(CASGD_EINVAL, "timing period must be >= 0");
  h->timing = on;
  for (auto& c : h->issued) c = 0;
  return CASGD_OK;
}

int casgd_get_timing(casgd_handle h, int kernel, double* total_ms, int64_t* launches, int reset) {
  if (!h) return fail(CASGD_EINVAL, "NULL handle");
  if (kernel < 0 || kernel >= CASGD_K_COUNT) return fail(CASGD_EINVAL, "unknown kernel id");
  if (!total_ms || !launches) return fail(CASGD_EINVAL, "NULL output");
  hipError_t e = sync_all(h);
  if (e != hipSuccess) return hip_fail(e, "timing sync");
  for (int k = 0; k < CASGD_K_COUNT; ++k) {
    for (auto& p : h->pending[k]) {
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, p.start, p.stop) == hipSuccess) {
        h->total_ms[k] += ms;
        h->launches[k] += 1;
      }
      h->pool.push_back(p);
    }
    h->pending[k].clear();
  }
  *total_ms = h->total_ms[kernel];
  *launches = h->launches[kernel];
  if (reset) {
    h->total_ms[kernel] = 0.0;
    h->launches[kernel] = 0;
  }
  return check_status(h);
}

}  // extern "C"
