// C ABI of the CA-SGD library: argument checks, handle-owned device memory,
// stream handling, optional per-kernel event timing, and the sequence of
// launches that makes one outer iteration (Abstract of "Mixed-Precision
// Communication-Avoiding SGD for Generalized Linear Models on GPUs"):
// sample + gather + margins, strictly-lower Gram, inner recurrence, update.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <utility>
#include <vector>

#include "casgd.h"
#include "casgd_device.h"
#include "casgd_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(CASGD_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

constexpr int kMaxSB = 16384;

struct EventPair {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

}  // namespace

struct casgd_ctx {
  int64_t m = 0, n = 0, ld = 0;
  int loss = 0, storage = 0;
  size_t esize = 0;
  void* Xs = nullptr;
  float* y = nullptr;
  hipStream_t stream = nullptr;

  // workspace, sized for cap_sb rows and cap_g Gram elements
  int cap_sb = 0;
  int64_t cap_g = 0;
  int32_t* idx = nullptr;
  void* Y = nullptr;
  float* yB = nullptr;
  float* G = nullptr;
  float* v = nullptr;
  float* z = nullptr;
  float* r = nullptr;
  double* loss_partial = nullptr;
  double* loss_out = nullptr;

  // shape of the most recent outer step (for exports)
  int last_s = 0, last_b = 0;

  // timing
  bool timing = false;
  std::vector<EventPair> pending[CASGD_K_COUNT];
  std::vector<EventPair> pool;
  double total_ms[CASGD_K_COUNT] = {};
  int64_t launches[CASGD_K_COUNT] = {};
};

namespace {

void free_workspace(casgd_ctx* h) {
  (void)hipFree(h->idx);
  (void)hipFree(h->Y);
  (void)hipFree(h->yB);
  (void)hipFree(h->G);
  (void)hipFree(h->v);
  (void)hipFree(h->z);
  (void)hipFree(h->r);
  h->idx = nullptr;
  h->Y = nullptr;
  h->yB = h->G = h->v = h->z = h->r = nullptr;
  h->cap_sb = 0;
  h->cap_g = 0;
}

int ensure_workspace(casgd_ctx* h, int s, int b) {
  const int sb = s * b;
  const int64_t gsz = static_cast<int64_t>(b) * b * s * (s - 1) / 2;
  if (sb <= h->cap_sb && gsz <= h->cap_g) return CASGD_OK;
  hipError_t e = hipStreamSynchronize(h->stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  const int new_sb = sb > h->cap_sb ? sb : h->cap_sb;
  const int64_t new_g = gsz > h->cap_g ? gsz : h->cap_g;
  free_workspace(h);
  bool ok = hipMalloc(&h->idx, sizeof(int32_t) * new_sb) == hipSuccess &&
            hipMalloc(&h->Y, h->esize * h->ld * new_sb) == hipSuccess &&
            hipMalloc(&h->yB, sizeof(float) * new_sb) == hipSuccess &&
            hipMalloc(&h->G, sizeof(float) * (new_g > 0 ? new_g : 1)) == hipSuccess &&
            hipMalloc(&h->v, sizeof(float) * new_sb) == hipSuccess &&
            hipMalloc(&h->z, sizeof(float) * new_sb) == hipSuccess &&
            hipMalloc(&h->r, sizeof(float) * new_sb) == hipSuccess;
  if (!ok) {
    (void)hipGetLastError();
    free_workspace(h);
    return fail(CASGD_ENOMEM, "device allocation of the outer-step workspace failed");
  }
  h->cap_sb = new_sb;
  h->cap_g = new_g;
  return CASGD_OK;
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

// Launch `fn` on the handle's stream, bracketed by events when timing is on.
template <typename Fn>
hipError_t timed(casgd_ctx* h, int kernel, Fn&& fn) {
  if (!h->timing) return fn();
  EventPair p = take_pair(h);
  (void)hipEventRecord(p.start, h->stream);
  hipError_t e = fn();
  (void)hipEventRecord(p.stop, h->stream);
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

// The launches of one outer iteration.  idx_in == nullptr: sample with `seed`.
int run_outer(casgd_ctx* h, int s, int b, float eta, uint64_t seed, const int32_t* idx_in,
              float* w) {
  int rc = ensure_workspace(h, s, b);
  if (rc != CASGD_OK) return rc;
  const int sb = s * b;
  const float c = eta / static_cast<float>(b);
  hipError_t e;
  e = timed(h, CASGD_K_GATHER, [&] {
    return casgd::launch_gather(h->storage, h->Xs, h->y, h->m, h->n, h->ld, sb, seed, idx_in,
                                h->idx, h->Y, h->yB, w, h->v, h->stream);
  });
  if (e != hipSuccess) return hip_fail(e, "gather launch");
  e = timed(h, CASGD_K_GRAM, [&] {
    return casgd::launch_gram(h->storage, h->Y, h->ld, s, b, h->G, 1, 0, 0, h->stream);
  });
  if (e != hipSuccess) return hip_fail(e, "gram launch");
  e = timed(h, CASGD_K_RECUR, [&] {
    return casgd::launch_recur(h->loss, h->G, h->v, h->yB, h->z, h->r, s, b, c, h->stream);
  });
  if (e != hipSuccess) return hip_fail(e, "recurrence launch");
  e = timed(h, CASGD_K_UPDATE, [&] {
    return casgd::launch_update(h->storage, h->Y, h->ld, h->n, sb, h->r, c, w, h->stream);
  });
  if (e != hipSuccess) return hip_fail(e, "update launch");
  h->last_s = s;
  h->last_b = b;
  return CASGD_OK;
}

}  // namespace

extern "C" {

const char* casgd_last_error(void) { return g_last_error.c_str(); }

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
  if (storage != CASGD_BF16 && storage != CASGD_FP32) {
    fail(CASGD_EINVAL, "unknown storage type");
    return nullptr;
  }
  casgd_ctx* h = new casgd_ctx;
  h->m = m;
  h->n = n;
  h->ld = (n + 31) / 32 * 32;
  h->loss = loss;
  h->storage = storage;
  h->esize = storage == CASGD_BF16 ? 2 : 4;
  if (hipMalloc(&h->Xs, h->esize * h->ld * m) != hipSuccess ||
      hipMalloc(&h->y, sizeof(float) * m) != hipSuccess ||
      hipMalloc(&h->loss_partial, sizeof(double) * casgd::kLossBlocks) != hipSuccess ||
      hipMalloc(&h->loss_out, sizeof(double)) != hipSuccess) {
    (void)hipGetLastError();
    fail(CASGD_ENOMEM, "device allocation of the stored data failed");
    casgd_destroy(h);
    return nullptr;
  }
  hipError_t e = casgd::launch_store(storage, X, h->Xs, m, n, h->ld, h->stream);
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
  (void)hipStreamSynchronize(h->stream);
  free_workspace(h);
  (void)hipFree(h->Xs);
  (void)hipFree(h->y);
  (void)hipFree(h->loss_partial);
  (void)hipFree(h->loss_out);
  for (auto& v : h->pending)
    for (auto& p : v) h->pool.push_back(p);
  for (auto& p : h->pool) {
    (void)hipEventDestroy(p.start);
    (void)hipEventDestroy(p.stop);
  }
  delete h;
}

int casgd_set_stream(casgd_handle h, void* stream) {
  if (!h) return fail(CASGD_EINVAL, "NULL handle");
  h->stream = static_cast<hipStream_t>(stream);
  return CASGD_OK;
}

int64_t casgd_ld(casgd_handle h) { return h ? h->ld : -1; }

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
  return run_outer(h, s, b, eta, 0, idx, w);
}

int casgd_train(casgd_handle h, int s, int b, float eta, uint64_t base_seed, uint64_t first_step,
                int n_outer, float* w) {
  int rc = check_step_args(h, s, b, w);
  if (rc != CASGD_OK) return rc;
  if (n_outer < 0) return fail(CASGD_EINVAL, "n_outer must be >= 0");
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
                                    h->loss_partial, h->loss_out, h->stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(out, h->loss_out, sizeof(double), hipMemcpyDeviceToHost, h->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(h->stream);
  if (e != hipSuccess) return hip_fail(e, "loss");
  return CASGD_OK;
}

int casgd_debug_export(casgd_handle h, int what, void* dst, size_t bytes) {
  if (!h) return fail(CASGD_EINVAL, "NULL handle");
  if (!dst) return fail(CASGD_EINVAL, "NULL destination");
  if (h->last_s == 0) return fail(CASGD_EINVAL, "no outer step has run yet");
  const int s = h->last_s, b = h->last_b;
  const size_t sb = static_cast<size_t>(s) * b;
  const void* src = nullptr;
  size_t need = 0;
  switch (what) {
    case CASGD_EXPORT_IDX: src = h->idx; need = sb * sizeof(int32_t); break;
    case CASGD_EXPORT_Y: src = h->Y; need = sb * h->ld * h->esize; break;
    case CASGD_EXPORT_YB: src = h->yB; need = sb * sizeof(float); break;
    case CASGD_EXPORT_G:
      src = h->G;
      need = sizeof(float) * static_cast<size_t>(b) * b * s * (s - 1) / 2;
      break;
    case CASGD_EXPORT_V: src = h->v; need = sb * sizeof(float); break;
    case CASGD_EXPORT_Z: src = h->z; need = sb * sizeof(float); break;
    case CASGD_EXPORT_R: src = h->r; need = sb * sizeof(float); break;
    default: return fail(CASGD_EINVAL, "unknown export");
  }
  if (bytes != need) return fail(CASGD_EINVAL, "export size mismatch: need " + std::to_string(need));
  if (need == 0) return CASGD_OK;
  hipError_t e = hipMemcpyAsync(dst, src, need, hipMemcpyDeviceToHost, h->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(h->stream);
  if (e != hipSuccess) return hip_fail(e, "export");
  return CASGD_OK;
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
  h->timing = on != 0;
  return CASGD_OK;
}

int casgd_get_timing(casgd_handle h, int kernel, double* total_ms, int64_t* launches, int reset) {
  if (!h) return fail(CASGD_EINVAL, "NULL handle");
  if (kernel < 0 || kernel >= CASGD_K_COUNT) return fail(CASGD_EINVAL, "unknown kernel id");
  if (!total_ms || !launches) return fail(CASGD_EINVAL, "NULL output");
  hipError_t e = hipStreamSynchronize(h->stream);
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
  return CASGD_OK;
}

}  // extern "C"
