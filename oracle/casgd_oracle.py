"""FP64 CPU oracle for mixed-precision communication-avoiding SGD (CA-SGD) on
generalized linear models.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test-suite, the package smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library
and imports nothing from the package; the two meet only through the seeded
input generators, which hold none of the method's arithmetic.

Source of the method: "Mixed-Precision Communication-Avoiding SGD for
Generalized Linear Models on GPUs" (paperdance.org/p/2606.18463), Abstract.
The abstract names the pieces (an outer iteration of s minibatch steps whose
s AllReduces become one AllReduce of an sb x sb Gram matrix; data stored in
low precision; the Gram built from low-precision inputs with high-precision
accumulation; inner recurrence and weight update in high precision) but prints
no formula.  The algebra below is the plain minibatch-SGD step unrolled over s
minibatches, which is what replacing s AllReduces by one Gram requires:

    SGD on minibatch j:   w_j = w_{j-1} - (eta/b) * Y_j^T r_j,
                          r_j = l'(Y_j w_{j-1}, y_j)
    unrolled:             Y_j w_{j-1} = Y_j w_0 - (eta/b) * sum_{t<j} (Y_j Y_t^T) r_t
    so with v = Y w_0 and G_{j,t} = Y_j Y_t^T:
                          z_j = v_j - (eta/b) * sum_{t<j} G_{j,t} r_t,  r_j = l'(z_j, y_j)
                          w_s = w_0 - (eta/b) * Y^T [r_1; ...; r_s]

Readings taken where the page is silent (each is listed in the design notes):
  * sampling: i.i.d. uniform with replacement; index i of an outer step with
    seed S is floor(x_i * m / 2^64) where x_i is output i of the SplitMix64
    stream seeded with S (Steele, Lea & Flood, OOPSLA 2014; multiply-high range
    reduction as in Lemire, ACM TOMS 2019).  The seed of outer step k is output
    k of the SplitMix64 stream seeded with the run's base seed.
  * the step is eta/b times the minibatch SUM of per-row derivatives.
  * "linear" regression uses the squared loss l = (z - y)^2 / 2.
  * no regularisation.
  * low precision = bfloat16 with round-to-nearest, ties to even.  The other
    storage formats the precision analysis allows are IEEE binary16 (fp16:
    round to nearest even, overflow to infinity) and OCP 8-bit E4M3 (fp8:
    round to nearest even, saturating at +-448, no infinities).  fp8 scales
    X by one power of two 2^k first, k the largest integer with
    max|X| * 2^k <= 448, and the stored value is e4m3(x * 2^k) * 2^-k; the
    page gives no scaling, but without one the entries of unit-norm rows of
    a few thousand columns sit in E4M3's subnormal range, where its roundoff
    is not the format's unit roundoff 2^-4.
  * "communicating G in low precision" (a precision choice of the analysis)
    forms each Gram entry at float32 precision and rounds it once to bf16.
  * the margin vector is float32 by default; its bfloat16 form (the recipe's
    low-precision margins) rounds each float32 margin once.
  * eta enters as the float32 value the GPU receives, widened to float64.

Parity status of each function:
  splitmix64, sample_indices ...... pinned (published known-answer values,
                                     big-integer range reduction, chi-square)
  bf16_bits / stored_values ....... pinned (torch CPU conversion, built ties)
  f16_bits / e4m3_bits ............ pinned (built ties, subnormals and limits
                                     in tests/golden; NumPy's float16 and
                                     torch's float8_e4m3fn conversions; the
                                     formats' unit roundoffs)
  fp8_exponent .................... pinned (hand-derived exponents at and
                                     around the 448 boundary)
  stored_gram (bf16 G) ............ pinned (built ties; a step whose G entries
                                     are bf16 values equals the fp32-G step)
  loss_terms / loss_derivative .... pinned (finite differences, closed forms)
  gram_blocks ..................... pinned (brute-force triple loop)
  outer_step ...................... pinned (equals s plain SGD steps; s = 1;
                                     squared loss = linear solve; exact
                                     rational arithmetic; orthogonal rows)
  stored_margins / bf16 margins ... pinned (hand-placed ties and near-ties
                                     with known rounded values; an exact
                                     s = 2 step in rational arithmetic)
  margin_choices .................. pinned (hand-placed boundaries and a
                                     cancelling row; every float32 summation
                                     order of random rows lands in the range)
  full_loss / full_gradient ....... pinned (closed forms at w = 0; finite
                                     differences)
  train (many outer steps) ........ parity unpinned beyond the per-step pins
"""

from __future__ import annotations

import numpy as np

MASK64 = (1 << 64) - 1
# SplitMix64 constants, as published with the generator (Steele, Lea & Flood 2014).
SPLITMIX_GAMMA = 0x9E3779B97F4A7C15
SPLITMIX_M1 = 0xBF58476D1CE4E5B9
SPLITMIX_M2 = 0x94D049BB133111EB

LOSSES = ("logistic", "squared", "poisson")


# --------------------------------------------------------------------------
# sampling
# --------------------------------------------------------------------------
def splitmix64(seed: int, i: int) -> int:
    """Output number i (0-based) of the SplitMix64 stream seeded with `seed`.

    The generator's state advances by the golden-ratio increment before each
    output, so output i mixes seed + (i + 1) * gamma.  Pure Python integers.
    """
    z = (int(seed) + (int(i) + 1) * SPLITMIX_GAMMA) & MASK64
    z = ((z ^ (z >> 30)) * SPLITMIX_M1) & MASK64
    z = ((z ^ (z >> 27)) * SPLITMIX_M2) & MASK64
    return z ^ (z >> 31)


def step_seed(base_seed: int, k: int) -> int:
    """Seed of outer step k: output k of the stream seeded with the base seed."""
    return splitmix64(base_seed, k)


def sample_indices(seed: int, m: int, count: int) -> np.ndarray:
    """Row indices of one outer step: floor(x_i * m / 2^64), i < count.

    Sampling with replacement (a reading: the page does not say how
    minibatches are drawn).  Minibatch j is entries [j*b, (j+1)*b).
    """
    out = np.empty(count, dtype=np.int64)
    for i in range(count):
        out[i] = (splitmix64(seed, i) * int(m)) >> 64
    return out


# --------------------------------------------------------------------------
# low-precision storage
# --------------------------------------------------------------------------
def bf16_bits(x) -> np.ndarray:
    """bfloat16 bit patterns of float32 values, round-to-nearest ties-to-even.

    Integer formulation: add 0x7FFF plus the lowest kept bit, then drop the
    16 low bits.  NaNs keep their sign and become quiet NaNs.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    is_nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> 16) & 1
    rounded = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    quiet = ((u >> 16) | 0x0040) & 0xFFFF
    return np.where(is_nan, quiet, rounded).astype(np.uint16)


def bf16_to_f64(bits) -> np.ndarray:
    """Exact float64 value of bfloat16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def _round_to_grid(a, emin: int, mbits: int) -> np.ndarray:
    """Round non-negative float64 values to the nearest value of a binary
    floating-point grid with `mbits` fraction bits whose smallest normal
    binade is [2^emin, 2^(emin+1)) (evenly spaced subnormals below it), ties
    to even, with no upper limit.

    In the binade [2^e, 2^(e+1)) the grid spacing is 2^(e - mbits); below
    2^emin it is 2^(emin - mbits).  a / spacing is exact for float32-derived
    a, so np.rint (round half to even) takes the whole decision.
    """
    a = np.asarray(a, dtype=np.float64)
    _, E = np.frexp(a)                    # a = f * 2^E with f in [0.5, 1)
    e = np.maximum(E - 1, emin)           # binade exponent, at least emin
    q = np.ldexp(1.0, e - mbits)
    return np.rint(a / q) * q


F16_MAX = 65504.0
E4M3_MAX = 448.0


def f16_round(x) -> np.ndarray:
    """IEEE binary16 value of float32/float64 values: round to nearest, ties
    to even, with subnormals; beyond the largest finite value 65504 after
    rounding: +-inf; NaN stays NaN."""
    x = np.asarray(x, dtype=np.float64)
    r = _round_to_grid(np.abs(x), -14, 10)
    r = np.where(r > F16_MAX, np.inf, r)
    return np.where(np.isnan(x), np.nan, np.copysign(r, x))


def e4m3_round(x) -> np.ndarray:
    """OCP E4M3 value: round to nearest, ties to even, with subnormals
    (spacing 2^-9 below 2^-6); magnitudes that round above 448 (and
    infinities) saturate to +-448; NaN stays NaN."""
    x = np.asarray(x, dtype=np.float64)
    r = np.minimum(_round_to_grid(np.abs(x), -6, 3), E4M3_MAX)
    return np.where(np.isnan(x), np.nan, np.copysign(r, x))


def _encode(v, emin: int, mbits: int, ebias: int) -> np.ndarray:
    """Bit pattern (without sign) of finite grid values v >= 0."""
    v = np.asarray(v, dtype=np.float64)
    _, E = np.frexp(v)
    normal = v >= np.ldexp(1.0, emin)
    sub = np.rint(v / np.ldexp(1.0, emin - mbits))
    expo = np.where(normal, E - 1 + ebias, 0)
    frac = np.where(normal, np.rint((v / np.ldexp(1.0, np.where(normal, E - 1, 0)) - 1.0) * (1 << mbits)), 0)
    return np.where(normal, expo * (1 << mbits) + frac, sub).astype(np.int64)


def f16_bits(x) -> np.ndarray:
    """binary16 bit patterns of f16_round(x) (NaN -> 0x7E00 with x's sign)."""
    x = np.asarray(x, dtype=np.float64)
    r = f16_round(x)
    mag = np.abs(np.where(np.isfinite(r), r, 0.0))
    body = np.where(np.isinf(r), 0x7C00, np.where(np.isnan(r), 0x7E00, _encode(mag, -14, 10, 15)))
    return (body | (np.signbit(x).astype(np.int64) << 15)).astype(np.uint16)


def f16_to_f64(bits) -> np.ndarray:
    """Exact float64 value of binary16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(b >> 15, -1.0, 1.0)
    expo, frac = (b >> 10) & 0x1F, b & 0x3FF
    val = np.where(expo == 0, np.ldexp(frac.astype(np.float64), -24),
                   np.ldexp((1024 + frac).astype(np.float64), expo - 25))
    val = np.where(expo == 31, np.where(frac == 0, np.inf, np.nan), val)
    return sign * val


def e4m3_bits(x) -> np.ndarray:
    """OCP E4M3 bit patterns of e4m3_round(x) (NaN -> 0x7F with x's sign)."""
    x = np.asarray(x, dtype=np.float64)
    r = e4m3_round(x)
    mag = np.abs(np.where(np.isnan(r), 0.0, r))
    body = np.where(np.isnan(r), 0x7F, _encode(mag, -6, 3, 7))
    return (body | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def e4m3_to_f64(bits) -> np.ndarray:
    """Exact float64 value of OCP E4M3 bit patterns (0x7F / 0xFF are NaN)."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    expo, frac = (b >> 3) & 0xF, b & 0x7
    val = np.where(expo == 0, np.ldexp(frac.astype(np.float64), -9),
                   np.ldexp((8 + frac).astype(np.float64), expo - 10))
    val = np.where((expo == 15) & (frac == 7), np.nan, val)
    return sign * val


def fp8_exponent(max_abs: float) -> int:
    """Largest integer k with max_abs * 2^k <= 448 (0 for max_abs 0 or not
    finite).  With max_abs = f * 2^E, f in [0.5, 1), and 448 = 0.875 * 2^9:
    k = 9 - E if f <= 0.875, else 8 - E."""
    max_abs = float(max_abs)
    if not np.isfinite(max_abs) or max_abs <= 0.0:
        return 0
    f, E = np.frexp(max_abs)
    return int(9 - E) if f <= 0.875 else int(8 - E)


def fp8_exponent_of(X_f32) -> int:
    """The fp8 scale exponent of a whole float32 data matrix."""
    X = np.asarray(X_f32, dtype=np.float32)
    return fp8_exponent(float(np.max(np.abs(X))) if X.size else 0.0)


def stored_values(x_f32, storage: str, fp8_exp: int | None = None) -> np.ndarray:
    """The values the method stores for float32 data, as float64.  fp8 needs
    the data matrix's scale exponent (fp8_exponent_of the whole X)."""
    if storage == "bf16":
        return bf16_to_f64(bf16_bits(x_f32))
    if storage == "fp32":
        return np.asarray(x_f32, dtype=np.float32).astype(np.float64)
    if storage == "fp16":
        return f16_round(np.asarray(x_f32, dtype=np.float32))
    if storage == "fp8":
        if fp8_exp is None:
            raise ValueError("fp8 storage needs the data matrix's scale exponent")
        x = np.asarray(x_f32, dtype=np.float32).astype(np.float64)
        return np.ldexp(e4m3_round(np.ldexp(x, fp8_exp)), -fp8_exp)
    raise ValueError(f"unknown storage {storage!r}")


STORAGES = ("bf16", "fp32", "fp16", "fp8")


# --------------------------------------------------------------------------
# per-row losses of the three generalized linear models
# --------------------------------------------------------------------------
def _softplus(u):
    return np.maximum(u, 0.0) + np.log1p(np.exp(-np.abs(u)))


def _sigmoid(u):
    out = np.empty_like(u)
    pos = u >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-u[pos]))
    e = np.exp(u[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def loss_terms(z, y, loss: str) -> np.ndarray:
    """Per-row loss l(z, y).

    logistic (y = +-1):  log(1 + exp(-y z))
    squared:             (z - y)^2 / 2
    poisson (counts y):  exp(z) - y z
    """
    z = np.asarray(z, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    if loss == "logistic":
        return _softplus(-y * z)
    if loss == "squared":
        return 0.5 * (z - y) ** 2
    if loss == "poisson":
        return np.exp(z) - y * z
    raise ValueError(f"unknown loss {loss!r}")


def loss_derivative(z, y, loss: str) -> np.ndarray:
    """d l(z, y) / dz.

    logistic:  -y * sigmoid(-y z)
    squared:   z - y
    poisson:   exp(z) - y
    """
    z = np.atleast_1d(np.asarray(z, dtype=np.float64))
    y = np.atleast_1d(np.asarray(y, dtype=np.float64))
    if loss == "logistic":
        return -y * _sigmoid(-y * z)
    if loss == "squared":
        return z - y
    if loss == "poisson":
        return np.exp(z) - y
    raise ValueError(f"unknown loss {loss!r}")


# --------------------------------------------------------------------------
# one outer iteration
# --------------------------------------------------------------------------
def step_size(eta, b: int) -> float:
    """eta / b with eta taken as the float32 value handed to the GPU."""
    return float(np.float64(np.float32(eta))) / float(b)


def gather(X_f32, y_f32, idx, storage: str, fp8_exp: int | None = None):
    """Y = stored rows X[idx] and y_B = y[idx], both float64.

    Rounding is elementwise, so rounding the gathered rows equals gathering
    rounded rows; this keeps the oracle's memory at the sample's size.  For
    fp8 the scale exponent is the whole matrix's (computed from X_f32 when
    not given).
    """
    idx = np.asarray(idx, dtype=np.int64)
    if storage == "fp8" and fp8_exp is None:
        fp8_exp = fp8_exponent_of(X_f32)
    Y = stored_values(np.asarray(X_f32)[idx], storage, fp8_exp)
    yB = np.asarray(y_f32, dtype=np.float32)[idx].astype(np.float64)
    return Y, yB


def gram_blocks(Y, s: int, b: int) -> dict:
    """G_{j,t} = Y_j Y_t^T for 0 <= t < j < s (0-based minibatch numbers).

    Only the strictly-lower block triangle: the recurrence never reads the
    diagonal blocks or the upper triangle.  With bfloat16 inputs every product
    is exact in float64, so the blocks are the exact Gram up to float64 sums.
    """
    G = {}
    for j in range(s):
        Yj = Y[j * b:(j + 1) * b]
        for t in range(j):
            G[(j, t)] = Yj @ Y[t * b:(t + 1) * b].T
    return G


def recurrence(G: dict, v, yB, s: int, b: int, eta, loss: str):
    """Inner recurrence: z_j = v_j - (eta/b) sum_{t<j} G_{j,t} r_t, r_j = l'(z_j, y_j)."""
    c = step_size(eta, b)
    z = np.empty(s * b)
    r = np.empty(s * b)
    for j in range(s):
        acc = np.zeros(b)
        for t in range(j):
            acc += G[(j, t)] @ r[t * b:(t + 1) * b]
        z[j * b:(j + 1) * b] = v[j * b:(j + 1) * b] - c * acc
        r[j * b:(j + 1) * b] = loss_derivative(z[j * b:(j + 1) * b], yB[j * b:(j + 1) * b], loss)
    return z, r


def stored_margins(v, margin: str) -> np.ndarray:
    """The margin vector as the recurrence receives it.

    The Abstract's recipe keeps the margin vector in low precision.  "fp32":
    v is used as formed (the high-precision reading).  "bf16": v is formed at
    float32 precision and each value is then rounded to the nearest
    bfloat16, ties to even; the float32 step makes the rounding decision in
    the precision the GPU takes it in, so for a v that float32 holds exactly
    both sides round the same value.
    """
    v = np.asarray(v, dtype=np.float64)
    if margin == "fp32":
        return v
    if margin == "bf16":
        return bf16_to_f64(bf16_bits(v.astype(np.float32)))
    raise ValueError(f"unknown margin precision {margin!r}")


def margin_choices(Y, w0):
    """The range of admissible bf16 margins when v is formed in float32.

    A float32 dot product of n terms, summed in any order with rounding to
    nearest, is within e = gamma_n * sum_k |y_k w_k| of the exact value
    (gamma_n = n u / (1 - n u), u = 2^-24; Higham, Accuracy and Stability of
    Numerical Algorithms, 2nd ed., section 3.1), and rounding is monotone, so
    every admissible stored margin is a bf16 value in [round(v - e),
    round(v + e)].  Returns (nearest, lo, hi): the rounding of the exact v and
    the two ends of that range.
    """
    Y = np.asarray(Y, dtype=np.float64)
    w0 = np.asarray(w0, dtype=np.float64)
    v = Y @ w0
    nu = Y.shape[1] * 2.0 ** -24
    # widened by the float32 step that precedes each rounding below
    e = nu / (1.0 - nu) * (np.abs(Y) @ np.abs(w0)) + 2.0 ** -23 * np.abs(v)
    return stored_margins(v, "bf16"), stored_margins(v - e, "bf16"), stored_margins(v + e, "bf16")


def stored_gram(G: dict, gram: str) -> dict:
    """The Gram blocks as the recurrence receives them.  "fp32": as formed
    (the high-precision reading).  "bf16": each entry formed at float32
    precision, then rounded once to the nearest bfloat16, ties to even (the
    low-precision communication choice), by the same reading as the bf16
    margins."""
    if gram == "fp32":
        return G
    if gram == "bf16":
        return {k: bf16_to_f64(bf16_bits(np.asarray(g, np.float64).astype(np.float32))) for k, g in G.items()}
    raise ValueError(f"unknown Gram precision {gram!r}")


def gram_choices(Y, s: int, b: int):
    """The range of admissible bf16 Gram entries when each is formed in
    float32 and rounded once: like margin_choices, a float32 dot product of
    n terms in any order is within gamma_n * sum_k |y_jk y_tk| of the exact
    value, widened by the float32 step before the rounding.  The unit
    roundoff is taken as 2^-23, which also covers sums truncated toward zero:
    matrix units do not specify their accumulation order or rounding.
    Returns (nearest, lo, hi) as dicts of blocks."""
    Y = np.asarray(Y, dtype=np.float64)
    nu = Y.shape[1] * 2.0 ** -23
    G = gram_blocks(Y, s, b)
    A = np.abs(Y)
    near, lo, hi = {}, {}, {}
    for (j, t), g in G.items():
        e = nu / (1.0 - nu) * (A[j * b:(j + 1) * b] @ A[t * b:(t + 1) * b].T) + 2.0 ** -23 * np.abs(g)
        near[(j, t)] = stored_margins(g, "bf16")
        lo[(j, t)] = stored_margins(g - e, "bf16")
        hi[(j, t)] = stored_margins(g + e, "bf16")
    return near, lo, hi


def outer_step_rows(Y, yB, w0, s: int, b: int, eta, loss: str, margin: str = "fp32",
                    gram: str = "fp32", G=None) -> dict:
    """One CA-SGD outer iteration on already-gathered rows Y (s*b x n).

    `margin` is the stored precision of v = Y w0 (see stored_margins),
    `gram` that of G (see stored_gram); G, when given, replaces the Gram
    blocks the step would form (a test hands in admissible bf16 blocks)."""
    w0 = np.asarray(w0, dtype=np.float64)
    c = step_size(eta, b)
    G = stored_gram(gram_blocks(Y, s, b), gram) if G is None else G
    v = stored_margins(Y @ w0, margin)
    z, r = recurrence(G, v, yB, s, b, eta, loss)
    w = w0 - c * (Y.T @ r)
    return {"G": G, "v": v, "z": z, "r": r, "w": w}


def outer_step(X_f32, y_f32, w0, s: int, b: int, eta, seed: int, loss: str,
               storage: str = "bf16", idx=None, margin: str = "fp32", gram: str = "fp32",
               fp8_exp: int | None = None) -> dict:
    """One outer step from the full data: sample (or take idx), gather, step."""
    m = np.asarray(X_f32).shape[0]
    if idx is None:
        idx = sample_indices(seed, m, s * b)
    Y, yB = gather(X_f32, y_f32, idx, storage, fp8_exp)
    out = outer_step_rows(Y, yB, w0, s, b, eta, loss, margin, gram)
    out["idx"] = np.asarray(idx, dtype=np.int64)
    out["Y"] = Y
    out["yB"] = yB
    return out


# --------------------------------------------------------------------------
# plain minibatch SGD (what CA-SGD reorganises)
# --------------------------------------------------------------------------
def sgd_steps(Y, yB, w0, s: int, b: int, eta, loss: str) -> np.ndarray:
    """s plain minibatch SGD steps on the minibatches of Y, in order."""
    c = step_size(eta, b)
    w = np.array(w0, dtype=np.float64)
    for j in range(s):
        Yj = Y[j * b:(j + 1) * b]
        w = w - c * (Yj.T @ loss_derivative(Yj @ w, yB[j * b:(j + 1) * b], loss))
    return w


# --------------------------------------------------------------------------
# loss over the whole data set, and multi-step runs
# --------------------------------------------------------------------------
def full_loss(X_f32, y_f32, w, loss: str, storage: str = "bf16", fp8_exp: int | None = None) -> float:
    """f(w) = (1/m) sum_i l(x_i . w, y_i) over every row, in float64."""
    X_f32 = np.asarray(X_f32)
    m = X_f32.shape[0]
    if storage == "fp8" and fp8_exp is None:
        fp8_exp = fp8_exponent_of(X_f32)
    chunk = max(1, (1 << 21) // max(1, X_f32.shape[1]))
    w = np.asarray(w, dtype=np.float64)
    total = 0.0
    for a in range(0, m, chunk):
        Xc = stored_values(X_f32[a:a + chunk], storage, fp8_exp)
        total += float(np.sum(loss_terms(Xc @ w, np.asarray(y_f32[a:a + chunk], np.float64), loss)))
    return total / m


def full_gradient(X_f32, y_f32, w, loss: str, storage: str = "bf16") -> np.ndarray:
    """grad f(w) = (1/m) X^T l'(X w, y) over every row."""
    X = stored_values(X_f32, storage, fp8_exponent_of(X_f32) if storage == "fp8" else None)
    y = np.asarray(y_f32, dtype=np.float64)
    return X.T @ loss_derivative(X @ np.asarray(w, np.float64), y, loss) / X.shape[0]


def train(X_f32, y_f32, w0, s: int, b: int, eta, loss: str, base_seed: int,
          n_outer: int, storage: str = "bf16", first_step: int = 0,
          method: str = "ca", margin: str = "fp32", gram: str = "fp32",
          fp8_exp: int | None = None) -> np.ndarray:
    """n_outer outer steps from w0; step k samples with step_seed(base_seed, k).

    method "ca" runs the CA-SGD outer iteration (margins stored at `margin`
    precision, G at `gram` precision), "sgd" runs s plain SGD steps on the
    same minibatches.
    """
    m = np.asarray(X_f32).shape[0]
    w = np.array(w0, dtype=np.float64)
    if storage == "fp8" and fp8_exp is None:
        fp8_exp = fp8_exponent_of(X_f32)
    for k in range(first_step, first_step + n_outer):
        idx = sample_indices(step_seed(base_seed, k), m, s * b)
        Y, yB = gather(X_f32, y_f32, idx, storage, fp8_exp)
        if method == "ca":
            w = outer_step_rows(Y, yB, w, s, b, eta, loss, margin, gram)["w"]
        elif method == "sgd":
            w = sgd_steps(Y, yB, w, s, b, eta, loss)
        else:
            raise ValueError(method)
    return w


def gram_bytes(s: int, b: int, packed: bool) -> int:
    """Bytes of the float32 Gram an AllReduce would carry: full sb x sb, or the
    strictly-lower block triangle only (s(s-1)/2 blocks of b x b)."""
    if packed:
        return 4 * b * b * s * (s - 1) // 2
    return 4 * (s * b) ** 2
