/*
 * casgd.h - C ABI of the MI355X (gfx950) mixed-precision communication-avoiding
 * SGD library for generalized linear models.
 *
 * Method: "Mixed-Precision Communication-Avoiding SGD for Generalized Linear
 * Models on GPUs" (paperdance.org/p/2606.18463), Abstract.  One outer
 * iteration replaces s minibatch SGD steps, each with its own AllReduce, by
 * one sb x sb Gram matrix: the data matrix is stored in low precision
 * (bfloat16), the Gram is formed from those low-precision rows with float32
 * accumulation, and the inner recurrence and the weight update run in float32.
 * Written out (the plain SGD step unrolled over s minibatches of b rows):
 *
 *   Y   = the s*b sampled rows of X, minibatch j = rows [j*b, (j+1)*b)
 *   G_{j,t} = Y_j Y_t^T            for 0 <= t < j < s  (strictly-lower blocks)
 *   v   = Y w0
 *   z_j = v_j - (eta/b) sum_{t<j} G_{j,t} r_t,   r_j = l'(z_j, y_j)
 *   w   = w0 - (eta/b) Y^T r
 *
 * Losses l(z, y): logistic log(1 + exp(-y z)) with y = +-1; squared
 * (z - y)^2 / 2; Poisson exp(z) - y z.
 *
 * Conventions for every entry point:
 *   - Pointers named "device" are HIP device pointers on the current device;
 *     "host" pointers are ordinary CPU memory.  No pointer is retained past
 *     the call unless stated.
 *   - Work is queued on the handle's stream (casgd_set_stream; default: the
 *     null stream) and returns without waiting unless stated.
 *   - Arguments are validated on the host before anything is queued; an
 *     invalid call returns CASGD_EINVAL and changes nothing (w untouched).
 *   - Errors: CASGD_EINVAL (bad argument), CASGD_ENOMEM (device allocation
 *     failed), CASGD_EHIP (a HIP runtime call failed).  casgd_last_error()
 *     returns a description of the last failure on the calling thread.
 *   - NaN and Inf in the data or weights are not checked; they propagate.
 *   - A handle is not thread-safe; distinct handles are independent.
 */
#ifndef CASGD_H
#define CASGD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct casgd_ctx* casgd_handle;

enum casgd_loss_kind { CASGD_LOGISTIC = 0, CASGD_SQUARED = 1, CASGD_POISSON = 2 };
enum casgd_storage { CASGD_BF16 = 0, CASGD_FP32 = 1, CASGD_FP16 = 2, CASGD_FP8 = 3 };
enum casgd_status { CASGD_OK = 0, CASGD_EINVAL = -1, CASGD_ENOMEM = -2, CASGD_EHIP = -3 };

/* What casgd_debug_export copies out (state of the most recent outer step). */
enum casgd_export_what {
  CASGD_EXPORT_IDX = 0, /* int32[s*b]   sampled row indices                        */
  CASGD_EXPORT_Y = 1,   /* [s*b][ld] gathered rows: bf16 bits (bf16 and fp8
                           storage), fp16 bits or float32                     */
  CASGD_EXPORT_YB = 2,  /* float[s*b]   gathered labels / targets                  */
  CASGD_EXPORT_G = 3,   /* float[b*b*s*(s-1)/2]  strictly-lower block triangle,     */
                        /*   block-row layout: block-row j (1 <= j < s) is a       */
                        /*   b x (j*b) row-major matrix [G_{j,0} ... G_{j,j-1}]    */
                        /*   starting at element b*b*j*(j-1)/2                     */
  CASGD_EXPORT_V = 4,   /* float[s*b]   margins v = Y w0                          */
  CASGD_EXPORT_Z = 5,   /* float[s*b]   recurrence values z                       */
  CASGD_EXPORT_R = 6    /* float[s*b]   loss derivatives r = l'(z, y)              */
};

/* Timers kept when timing is on (casgd_set_timing). */
enum casgd_kernel_id {
  CASGD_K_GATHER = 0, /* sample + gather of the s*b rows                        */
  CASGD_K_GRAM = 1,   /* strictly-lower Gram on bf16 MFMA                       */
  CASGD_K_CHAIN = 2,  /* margins + inner recurrence + weight update (one launch) */
  CASGD_K_PIPE = 3,   /* casgd_train's step launch: chain of step k, Gram of     */
                      /* step k+1 and gather of step k+2 together               */
  CASGD_K_TRAIN = 4,  /* casgd_train's single persistent launch of all steps    */
  CASGD_K_COUNT = 5
};

/*
 * Create a handle that owns the stored data.  The data matrix is the one the
 * Abstract says is kept in low precision.
 *   X      device, float32 [m][n] row-major contiguous; read during the call only
 *   y      device, float32 [m]: labels +-1 (logistic), targets (squared),
 *          counts (Poisson); read during the call only
 *   m      rows, 1 <= m <= 2^31 - 1
 *   n      features, n >= 1
 *   loss   enum casgd_loss_kind
 *   storage enum casgd_storage, the low-precision format X is stored in (a
 *          precision choice of the Abstract's analysis):
 *          CASGD_BF16 bfloat16, round to nearest, ties to even;
 *          CASGD_FP32 float32 as given;
 *          CASGD_FP16 IEEE binary16, round to nearest even, subnormals kept,
 *            overflow to infinity; the Gram runs on fp16 MFMA;
 *          CASGD_FP8 OCP E4M3 of x * 2^k, round to nearest even, saturating
 *            at 448, with one exponent k per matrix: the largest integer with
 *            max|x| * 2^k <= 448 (casgd_fp8_exponent); the stored value
 *            e4m3 * 2^-k is exactly a bf16 value, so the gathered rows are
 *            bf16 and the Gram runs on bf16 MFMA.
 * The stored rows are padded with zeros to ld = n rounded up to 32 elements.
 * Synchronises the stream once so that failures surface here.
 * Returns NULL on failure (see casgd_last_error).
 */
casgd_handle casgd_create(const float* X, const float* y, int64_t m, int64_t n,
                          int loss, int storage);

/* Free everything the handle owns.  NULL is allowed.  Synchronises its streams. */
void casgd_destroy(casgd_handle h);

/* Queue later work on hip_stream (a hipStream_t; NULL selects the null
 * stream).  When the stream changes, the new stream is first made to wait
 * (an event, no host synchronisation) for everything already queued on the
 * old one, since all work of a handle shares its buffers: switching streams
 * never lets two of the handle's calls overlap. */
int casgd_set_stream(casgd_handle h, void* hip_stream);

/*
 * One CA-SGD outer iteration (s inner SGD steps), Abstract.
 *   s, b   minibatches per outer step and rows per minibatch; 1 <= s,
 *          1 <= b, s*b <= 16384
 *   eta    learning rate (the step is eta/b times the minibatch sum)
 *   seed   sampling seed of this outer step: row index i (i < s*b) is
 *          floor(x_i * m / 2^64), x_i = output i of SplitMix64 seeded with seed
 *   w      device, float32 [n]; read as w0, overwritten with the new weights
 *          in stream order; must not alias handle memory
 * Asynchronous.  Workspace grows on the first call with a larger s*b.
 * Sampling, gathering and the Gram run on a stream the handle owns, ordered
 * before the weight-dependent kernel on the handle's stream; the next call's
 * sampling, gathering and Gram may overlap this call's recurrence.
 */
int casgd_outer_step(casgd_handle h, int s, int b, float eta, uint64_t seed, float* w);

/*
 * As casgd_outer_step but with explicit row indices instead of sampling
 * (for tests of degenerate minibatches).
 *   idx    device, int32 [s*b], each in [0, m); copied to the host and
 *          checked first, so this call synchronises the stream.
 */
int casgd_outer_step_indices(casgd_handle h, int s, int b, float eta,
                             const int32_t* idx, float* w);

/*
 * n_outer consecutive outer iterations; outer step k (k = first_step ...
 * first_step + n_outer - 1) samples with seed casgd_step_seed(base_seed, k).
 * Bit-identical to calling casgd_outer_step with those seeds.  Asynchronous.
 * With the default recurrence the loop runs on the handle's stream alone:
 *   - for shapes the lean recurrence takes (see CASGD_OPT_TRAIN_FORM), ONE
 *     persistent launch for all n_outer steps (timer CASGD_K_TRAIN): its
 *     workgroups stay resident and hand results to each other, the Gram of
 *     later steps running ahead of the recurrence; a small gather of the
 *     last step follows so that casgd_debug_export sees that step's rows;
 *   - otherwise, after a prologue (gather and Gram of the first step, gather
 *     of the second), ONE launch per step that runs the margins, recurrence
 *     and update of step k next to the Gram of step k+1 and the gather of
 *     step k+2 (timer CASGD_K_PIPE).
 * With the lookahead recurrence, and for fp16 and fp8 storage (whose rows
 * go through the gather kernel), each step is queued as by casgd_outer_step.
 * The persistent launch needs every one of its workgroups resident at once
 * (one per CU); if the device cannot hold them the call fails with
 * CASGD_EHIP before anything is queued.
 */
int casgd_train(casgd_handle h, int s, int b, float eta, uint64_t base_seed,
                uint64_t first_step, int n_outer, float* w);

/* Seed of outer step k: output k of SplitMix64 seeded with base_seed. */
uint64_t casgd_step_seed(uint64_t base_seed, uint64_t k);

/*
 * Mean loss over every stored row, f(w) = (1/m) sum_i l(x_i . w, y_i): float32
 * dot products, float64 loss terms and sums (the Abstract compares methods by
 * this loss).  w: device float32 [n].  out: host double.  Synchronises.
 * Also reports CASGD_EHIP if an earlier outer step's exchange between
 * workgroups timed out (a wait is bounded instead of hanging).
 */
int casgd_loss(casgd_handle h, const float* w, double* out);

/* casgd_loss for callers that cannot allocate or wait: code under HIP graph
 * capture, allocation-free serving and training loops, harnesses that forbid
 * hipMalloc.  The same mean loss f(w) as casgd_loss (the same kernels and
 * summation order, so the same bits), written to *out_dev (one device double)
 * on the handle's stream; returns without waiting.  Allocates nothing: the
 * per-workgroup partial sums go to a static device array of the library
 * holding 2048 doubles (16 KiB) per GPU, kept by each GPU the library runs on
 * until the process ends.  A shape whose reduction would need more partial
 * sums than that is refused with EINVAL (the loss uses at most 2048, so no
 * handle's shape is refused today).  Every call on one GPU shares that array:
 * calls that overlap on one GPU (other streams, other handles, other threads)
 * race and may return wrong values.  Every partial sum a call reads is written
 * by that call first, so nothing is cleared.  EINVAL for a NULL handle or
 * pointer. */
int casgd_loss_noalloc(casgd_handle h, const float* w, double* out_dev);

/*
 * Copy part of the most recent outer step's state to host memory (tests and
 * benchmarks).  what: enum casgd_export_what; bytes must equal the exact size
 * of that array.  Synchronises the stream.
 */
int casgd_debug_export(casgd_handle h, int what, void* dst_host, size_t bytes);

/* Copy stored rows [row0, row0 + nrows) (bf16 bits or float32, ld wide) to
 * host memory; bytes must equal nrows * ld * element size.  Synchronises. */
int casgd_export_rows(casgd_handle h, int64_t row0, int64_t nrows, void* dst_host,
                      size_t bytes);

/* Padded row length (elements) of the stored data. */
int64_t casgd_ld(casgd_handle h);

/* The exponent k of fp8 storage (X stored as E4M3 of x * 2^k); 0 for the
 * other storage types and for a NULL handle. */
int casgd_fp8_exponent(casgd_handle h);

/*
 * Bytes of the float32 Gram that the one AllReduce per outer step would carry
 * between processes (Abstract): packed != 0 gives the strictly-lower block
 * triangle (4 * b*b * s*(s-1)/2), packed == 0 the full sb x sb matrix.
 * On one process the AllReduce itself is omitted.  Returns -1 on bad input.
 * With CASGD_OPT_GRAM_BF16 the Gram would travel as bf16: half these bytes.
 */
int64_t casgd_gram_bytes(int s, int b, int packed);

/* Options (casgd_set_option). */
enum casgd_option {
  /* How the inner recurrence is spread over workgroups:
   *   0 (default) the fastest form for the shape, currently always 1;
   *   1 every workgroup owns rows of every minibatch and all exchange r each
   *     inner step;
   *   2 lookahead: one workgroup computes every step from the latest blocks
   *     of G while helper workgroups add the older blocks ahead of time
   *     (taken for 16 <= b <= 64, b a multiple of 16, s >= 2; otherwise 1).
   * All forms give bit-identical results for a given shape and form; the
   * forms differ from each other only in float32 rounding order. */
  CASGD_OPT_RECURRENCE = 0,
  /* Bound, in polls, of every wait between workgroups of the recurrence
   * (0, the default: 2^22 polls, seconds, far beyond any real wait).  For
   * tests of the failure path: a small bound makes the waits expire, every
   * kernel still ends, the step's results are invalid, and the next
   * casgd_loss / casgd_debug_export / casgd_get_timing reports CASGD_EHIP
   * (once; the error word is then cleared). */
  CASGD_OPT_SPIN_LIMIT = 1,
  /* Precision of the stored margin vector v = Y w0 (Abstract of
   * "Mixed-Precision Communication-Avoiding SGD for Generalized Linear Models
   * on GPUs": the recipe keeps the margin vector in low precision).
   *   0 (default) float32;
   *   1 each margin is accumulated in float32 and rounded once to bfloat16
   *     (nearest, ties to even) when formed; the recurrence starts from the
   *     rounded value and CASGD_EXPORT_V returns it, widened to float.
   * Applies to every recurrence form and to casgd_train. */
  CASGD_OPT_MARGIN_BF16 = 2,
  /* Placement of the all-to-all recurrence's workgroups (they exchange r
   * at every inner step):
   *   0 (default) on one XCD, whose shared L2 carries the exchange, whenever
   *     the shape allows it (at most 4 rows per minibatch per workgroup with
   *     one workgroup per CU of that XCD), else spread over all XCDs;
   *   1 spread over all XCDs, one workgroup per row up to 64;
   *   2 on one XCD whatever the shape.
   * A launch whose recurrence workgroups cannot all be resident at once
   * fails with CASGD_EHIP.  Results depend on the layout only through the
   * float32 summation order of the weight update. */
  CASGD_OPT_CHAIN_LAYOUT = 3,
  /* How casgd_train runs its steps:
   *   0 (default) one persistent launch for all steps whenever the shape
   *     runs the lean recurrence (b a multiple of 4, at most 4 rows per
   *     minibatch per recurrence workgroup and 4 columns per lane, the
   *     workgroup's rows of G in LDS), else one launch per step;
   *   1 one launch per step.
   * Both give bit-identical results. */
  CASGD_OPT_TRAIN_FORM = 4,
  /* Precision in which G reaches the recurrence (a precision choice of the
   * Abstract's analysis: the Gram communicated in low or high precision):
   *   0 (default) float32 as accumulated (the recipe's high precision);
   *   1 each entry rounded once to the nearest bfloat16, ties to even, as it
   *     is stored (what a bf16 AllReduce would deliver at P = 1). */
  CASGD_OPT_GRAM_BF16 = 5
};

/* Set an option of the handle; later outer steps use it.  EINVAL for an
 * unknown option or value. */
int casgd_set_option(casgd_handle h, int option, int value);

/* Time hot-path kernel launches with HIP events that the kernel's own
 * dispatch stamps at its start and end.  on = 0: off; on = 1: every launch;
 * on = k > 1: every k-th launch of each kernel (the first one included), so
 * the stamping perturbs a long run less.  EINVAL for on < 0. */
int casgd_set_timing(casgd_handle h, int on);

/* Total milliseconds and count of the timed launches of one kernel (enum
 * casgd_kernel_id) since timing was switched on; synchronises.  reset != 0
 * clears them after. */
int casgd_get_timing(casgd_handle h, int kernel, double* total_ms, int64_t* launches,
                     int reset);

/* Calibration kernels for roofline reporting (not part of the method).
 *
 * casgd_peak_copy: copy `bytes` (a multiple of 16) from device src to device
 * dst, both 16-byte aligned and not overlapping, with a plain grid-stride
 * kernel on hip_stream (NULL: the null stream).  It reads and writes `bytes`
 * each: the achievable HBM rate, and a kernel of known traffic that scales
 * the HBM byte counters.  EINVAL for bad sizes, alignment or overlap.
 *
 * casgd_peak_mfma: launch `workgroups` workgroups of 256 lanes; each wave
 * runs iters x 4 bf16 MFMAs (32x32x16, float32 accumulators) on four
 * independent accumulator chains and each lane stores its accumulator sum to
 * device out[workgroups * 256].  It does workgroups * 4 waves * 4 chains *
 * iters * 32768 flops: the achievable dense bf16 matrix-core rate under
 * sustained load.  EINVAL for workgroups outside [1, 2^20] or iters < 1. */
int casgd_peak_copy(const void* src, void* dst, int64_t bytes, void* hip_stream);
/* casgd_peak_read: `workgroups` workgroups of 256 lanes read `bytes` (a
 * positive multiple of 16) of device src, 16-byte aligned, each a contiguous
 * slice, with direct-to-LDS loads (the achievable HBM read rate); workgroup
 * w writes 8 words of its LDS ring to device out[8 w .. 8 w + 7] (all of
 * them read from src when each slice spans at least 8 x 64 x 16 bytes).
 * EINVAL for bad sizes, alignment or workgroup count. */
int casgd_peak_read(const void* src, int64_t bytes, float* out, int workgroups, void* hip_stream);
int casgd_peak_mfma(float* out, int workgroups, int iters, void* hip_stream);

/* Text of the last error on the calling thread ("" if none). */
const char* casgd_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CASGD_H */
