"""Pins of the CPU oracle to facts it does not compute itself.

Each test checks the oracle against something independent of its own code:
published known-answer values, a library routine, a closed form, brute force,
exact rational arithmetic, or the identity that defines the method (CA-SGD is
s plain minibatch SGD steps reorganised around the Gram matrix; Abstract of
"Mixed-Precision Communication-Avoiding SGD for Generalized Linear Models on
GPUs").  The last test plants plausible mistakes in a copy of the oracle's
recurrence and checks that the pins catch every one.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import casgd_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LOSSES = ("logistic", "squared", "poisson")


def _read_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def _targets(rng, k, loss):
    if loss == "logistic":
        return np.where(rng.random(k) < 0.5, -1.0, 1.0)
    if loss == "squared":
        return rng.standard_normal(k)
    return rng.poisson(1.5, k).astype(np.float64)


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


# ---------------------------------------------------------------- sampler
def test_splitmix64_known_answers():
    rows = _read_rows("splitmix64_kat.txt")
    assert len(rows) >= 6
    for seed, i, out in rows:
        assert O.splitmix64(int(seed), int(i)) == int(out)


def test_step_seed_is_stream_output():
    # outer step k's seed is output k of the base stream (known answers above)
    assert O.step_seed(0, 0) == 16294208416658607535
    assert O.step_seed(0, 2) == 487617019471545679


def test_sample_power_of_two_takes_top_bits():
    # for m = 2^k the multiply-high range reduction keeps the top k bits
    for k in (1, 7, 20, 31):
        idx = O.sample_indices(12345, 1 << k, 64)
        top = [O.splitmix64(12345, i) >> (64 - k) for i in range(64)]
        assert idx.tolist() == top


def test_sample_matches_exact_division():
    m = 400_000
    idx = O.sample_indices(99, m, 256)
    for i in range(256):
        x = O.splitmix64(99, i)
        assert idx[i] == math.floor(Fraction(x * m, 1 << 64))
    assert idx.min() >= 0 and idx.max() < m


def test_sample_uniform_chi_square():
    from scipy.stats import chisquare
    m = 1000
    idx = O.sample_indices(7, m, 200_000)
    counts = np.bincount(idx, minlength=m)
    assert chisquare(counts).pvalue > 1e-4


# ---------------------------------------------------------------- bf16
def test_bf16_hand_built_cases():
    for f32, bf, *_ in _read_rows("bf16_rne_cases.txt"):
        x = np.array([int(f32, 16)], dtype=np.uint32).view(np.float32)
        assert int(O.bf16_bits(x)[0]) == int(bf, 16), f32


def test_bf16_matches_torch_cpu_conversion():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),
        rng.integers(0, 1 << 32, 20000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    x = x[~np.isnan(x)]  # torch canonicalises NaN payloads; NaNs are covered above
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_bits(x), ref)


def test_bf16_values_exact_and_close():
    x = np.linspace(-3, 3, 1001).astype(np.float32)
    v = O.stored_values(x, "bf16")
    assert np.all(np.abs(v - x) <= np.abs(x) * 2.0 ** -8 + 1e-45)
    assert np.array_equal(O.stored_values(x, "fp32"), x.astype(np.float64))


# ---------------------------------------------------------------- losses
@pytest.mark.parametrize("loss", LOSSES)
def test_derivative_matches_finite_differences(loss):
    rng = np.random.default_rng(11)
    z = rng.uniform(-3, 3, 64)
    y = _targets(rng, 64, loss)
    h = 1e-6
    fd = (O.loss_terms(z + h, y, loss) - O.loss_terms(z - h, y, loss)) / (2 * h)
    d = O.loss_derivative(z, y, loss)
    assert np.max(np.abs(fd - d) / (1 + np.abs(d))) < 1e-7


def test_closed_forms_at_zero():
    rng = np.random.default_rng(5)
    X = rng.standard_normal((50, 4)).astype(np.float32)
    w = np.zeros(4)
    ylog = np.where(rng.random(50) < 0.5, -1.0, 1.0).astype(np.float32)
    ysq = rng.standard_normal(50).astype(np.float32)
    ypo = rng.poisson(2.0, 50).astype(np.float32)
    assert abs(O.full_loss(X, ylog, w, "logistic") - math.log(2.0)) < 1e-15
    assert abs(O.full_loss(X, ysq, w, "squared") - 0.5 * np.mean(ysq.astype(np.float64) ** 2)) < 1e-15
    assert abs(O.full_loss(X, ypo, w, "poisson") - 1.0) < 1e-15
    z0 = np.zeros(50)
    assert np.array_equal(O.loss_derivative(z0, ylog, "logistic"), -ylog / 2.0)
    assert np.array_equal(O.loss_derivative(z0, ysq, "squared"), -ysq.astype(np.float64))
    assert np.array_equal(O.loss_derivative(z0, ypo, "poisson"), 1.0 - ypo)


def test_logistic_is_stable_at_large_margins():
    z = np.array([-800.0, -40.0, 40.0, 800.0])
    y = np.ones(4)
    lt = O.loss_terms(z, y, "logistic")
    assert np.all(np.isfinite(lt))
    assert abs(lt[0] - 800.0) < 1e-12 and lt[3] < 1e-300
    d = O.loss_derivative(z, y, "logistic")
    assert np.all(np.isfinite(d)) and abs(d[0] + 1.0) < 1e-15 and abs(d[3]) < 1e-300


# ---------------------------------------------------------------- Gram
def test_gram_blocks_brute_force():
    rng = np.random.default_rng(2)
    s, b, n = 4, 3, 5
    Y = rng.standard_normal((s * b, n))
    G = O.gram_blocks(Y, s, b)
    assert sorted(G) == [(j, t) for j in range(s) for t in range(j)]
    for (j, t), blk in G.items():
        for i in range(b):
            for k in range(b):
                ref = sum(Y[j * b + i, c] * Y[t * b + k, c] for c in range(n))
                assert abs(blk[i, k] - ref) < 1e-12


# ---------------------------------------------------------------- outer step
@pytest.mark.parametrize("loss", LOSSES)
@pytest.mark.parametrize("s,b", [(1, 4), (2, 3), (4, 8), (7, 1), (5, 16)])
def test_ca_step_equals_s_sgd_steps(loss, s, b):
    rng = np.random.default_rng(100 * s + b)
    n = 9
    Y = O.stored_values(rng.standard_normal((s * b, n)).astype(np.float32) * 0.4, "bf16")
    yB = _targets(rng, s * b, loss)
    w0 = rng.standard_normal(n) * 0.5
    ca = O.outer_step_rows(Y, yB, w0, s, b, 0.7, loss)["w"]
    sgd = O.sgd_steps(Y, yB, w0, s, b, 0.7, loss)
    assert _rel(ca, sgd) <= 1e-10


@pytest.mark.parametrize("loss", LOSSES)
def test_s1_reduces_to_one_sgd_step(loss):
    rng = np.random.default_rng(17)
    b, n = 6, 5
    Y = rng.standard_normal((b, n))
    yB = _targets(rng, b, loss)
    w0 = rng.standard_normal(n)
    out = O.outer_step_rows(Y, yB, w0, 1, b, 0.3, loss)
    assert out["G"] == {}
    assert np.array_equal(out["z"], Y @ w0)
    c = float(np.float32(0.3)) / b
    g = O.loss_derivative(Y @ w0, yB, loss)
    manual = w0 - c * np.array([sum(Y[i, k] * g[i] for i in range(b)) for k in range(n)])
    assert _rel(out["w"], manual) <= 1e-13


def test_squared_recurrence_is_a_block_triangular_solve():
    rng = np.random.default_rng(23)
    s, b, n = 6, 4, 7
    Y = rng.standard_normal((s * b, n))
    yB = rng.standard_normal(s * b)
    w0 = rng.standard_normal(n)
    eta = 0.25
    out = O.outer_step_rows(Y, yB, w0, s, b, eta, "squared")
    c = float(np.float32(eta)) / b
    full = Y @ Y.T
    L = np.zeros_like(full)
    for j in range(s):
        L[j * b:(j + 1) * b, :j * b] = full[j * b:(j + 1) * b, :j * b]
    v = Y @ w0
    z = np.linalg.solve(np.eye(s * b) + c * L, v + c * L @ yB)
    assert _rel(out["z"], z) <= 1e-12


def test_squared_step_matches_exact_rationals():
    # dyadic inputs are exact in float64; plain SGD in Fractions is the exact answer
    rng = np.random.default_rng(29)
    s, b, n = 3, 2, 3
    Yi = rng.integers(-8, 9, (s * b, n))
    yi = rng.integers(-8, 9, s * b)
    wi = rng.integers(-8, 9, n)
    Y = Yi / 8.0
    yB = yi / 4.0
    w0 = wi / 16.0
    eta = 0.375  # exact in float32
    c = Fraction(3, 8) / b
    w = [Fraction(int(v), 16) for v in wi]
    for j in range(s):
        rows = range(j * b, (j + 1) * b)
        g = [sum(Fraction(int(Yi[i, k]), 8) * w[k] for k in range(n)) - Fraction(int(yi[i]), 4) for i in rows]
        w = [w[k] - c * sum(Fraction(int(Yi[i, k]), 8) * g[ii] for ii, i in enumerate(rows)) for k in range(n)]
    exact = np.array([float(x) for x in w])
    got = O.outer_step_rows(Y, yB, w0, s, b, eta, "squared")["w"]
    assert _rel(got, exact) <= 1e-14


@pytest.mark.parametrize("loss", LOSSES)
def test_orthogonal_rows_decouple(loss):
    n = 12
    X = np.eye(n, dtype=np.float32)
    rng = np.random.default_rng(31)
    y = _targets(rng, n, loss).astype(np.float32)
    idx = rng.permutation(n)[:8]
    w0 = (rng.standard_normal(n) * 0.5).astype(np.float32).astype(np.float64)
    out = O.outer_step(X, y, w0, 4, 2, 0.5, 0, loss, storage="fp32", idx=idx)
    for blk in out["G"].values():
        assert not np.any(blk)
    c = float(np.float32(0.5)) / 2
    expect = w0.copy()
    for i in idx:
        expect[i] -= c * O.loss_derivative(w0[i], y[i], loss)[0]
    assert _rel(out["w"], expect) <= 1e-15


@pytest.mark.parametrize("loss", LOSSES)
def test_full_gradient_matches_finite_differences(loss):
    rng = np.random.default_rng(37)
    m, n = 8, 3
    X = (rng.standard_normal((m, n)) * 0.5).astype(np.float32)
    y = _targets(rng, m, loss).astype(np.float32)
    w = rng.standard_normal(n) * 0.3
    g = O.full_gradient(X, y, w, loss)
    h = 1e-6
    for k in range(n):
        e = np.zeros(n)
        e[k] = h
        fd = (O.full_loss(X, y, w + e, loss) - O.full_loss(X, y, w - e, loss)) / (2 * h)
        assert abs(fd - g[k]) <= 1e-7 * (1 + abs(g[k]))


@pytest.mark.parametrize("loss", LOSSES)
def test_training_run_ca_equals_sgd(loss):
    rng = np.random.default_rng(41)
    m, n = 300, 6
    X = (rng.standard_normal((m, n)) * 0.4).astype(np.float32)
    y = _targets(rng, m, loss).astype(np.float32)
    w0 = np.zeros(n)
    a = O.train(X, y, w0, 4, 8, 0.2, loss, base_seed=5, n_outer=10, method="ca")
    b = O.train(X, y, w0, 4, 8, 0.2, loss, base_seed=5, n_outer=10, method="sgd")
    assert _rel(a, b) <= 1e-10
    # resuming after 4 steps reproduces the indices exactly
    w4 = O.train(X, y, w0, 4, 8, 0.2, loss, base_seed=5, n_outer=4)
    w10 = O.train(X, y, w4, 4, 8, 0.2, loss, base_seed=5, n_outer=6, first_step=4)
    assert np.array_equal(w10, a)


def test_gram_bytes():
    assert O.gram_bytes(16, 64, packed=False) == 4 * 1024 * 1024
    assert O.gram_bytes(16, 64, packed=True) == 120 * 64 * 64 * 4
    assert O.gram_bytes(1, 64, packed=True) == 0


# ---------------------------------------------------------------- pin sensitivity
def _broken_recurrences():
    def drop_last(G, v, yB, s, b, eta, loss):
        c = O.step_size(eta, b)
        z = np.empty(s * b)
        r = np.empty(s * b)
        for j in range(s):
            acc = np.zeros(b)
            for t in range(j - 1):  # the t = j-1 term dropped
                acc += G[(j, t)] @ r[t * b:(t + 1) * b]
            z[j * b:(j + 1) * b] = v[j * b:(j + 1) * b] - c * acc
            r[j * b:(j + 1) * b] = O.loss_derivative(z[j * b:(j + 1) * b], yB[j * b:(j + 1) * b], loss)
        return z, r

    def wrong_sign(G, v, yB, s, b, eta, loss):
        c = O.step_size(eta, b)
        z = np.empty(s * b)
        r = np.empty(s * b)
        for j in range(s):
            acc = np.zeros(b)
            for t in range(j):
                acc += G[(j, t)] @ r[t * b:(t + 1) * b]
            z[j * b:(j + 1) * b] = v[j * b:(j + 1) * b] + c * acc
            r[j * b:(j + 1) * b] = O.loss_derivative(z[j * b:(j + 1) * b], yB[j * b:(j + 1) * b], loss)
        return z, r

    def transposed_block(G, v, yB, s, b, eta, loss):
        c = O.step_size(eta, b)
        z = np.empty(s * b)
        r = np.empty(s * b)
        for j in range(s):
            acc = np.zeros(b)
            for t in range(j):
                acc += G[(j, t)].T @ r[t * b:(t + 1) * b]
            z[j * b:(j + 1) * b] = v[j * b:(j + 1) * b] - c * acc
            r[j * b:(j + 1) * b] = O.loss_derivative(z[j * b:(j + 1) * b], yB[j * b:(j + 1) * b], loss)
        return z, r

    def wrong_index(G, v, yB, s, b, eta, loss):
        c = O.step_size(eta, b)
        z = np.empty(s * b)
        r = np.empty(s * b)
        for j in range(s):
            acc = np.zeros(b)
            for t in range(j):
                acc += G[(j, t)] @ r[t * b:(t + 1) * b]
            z[j * b:(j + 1) * b] = v[j * b:(j + 1) * b] - c * acc
            # derivative taken against the previous minibatch's targets
            yy = yB[max(j - 1, 0) * b:max(j - 1, 0) * b + b]
            r[j * b:(j + 1) * b] = O.loss_derivative(z[j * b:(j + 1) * b], yy, loss)
        return z, r

    return [drop_last, wrong_sign, transposed_block, wrong_index]


def test_planted_mistakes_are_caught(monkeypatch):
    rng = np.random.default_rng(43)
    s, b, n = 4, 3, 5
    Y = rng.standard_normal((s * b, n)) * 0.5
    yB = np.where(rng.random(s * b) < 0.5, -1.0, 1.0)
    w0 = rng.standard_normal(n)
    sgd = O.sgd_steps(Y, yB, w0, s, b, 0.7, "logistic")
    good = O.outer_step_rows(Y, yB, w0, s, b, 0.7, "logistic")["w"]
    assert _rel(good, sgd) <= 1e-10
    for broken in _broken_recurrences():
        monkeypatch.setattr(O, "recurrence", broken)
        bad = O.outer_step_rows(Y, yB, w0, s, b, 0.7, "logistic")["w"]
        assert _rel(bad, sgd) > 1e-6, broken.__name__
        monkeypatch.undo()


# ---------------------------------------------------------------- bf16 margins
# bfloat16 keeps 8 significant bits: spacing 2^-7 on [1, 2), 2^-6 on [2, 4),
# 2^-8 on [1/2, 1), 1 on [128, 256).  Every expected value is placed by hand.
_MARGIN_CASES = [
    (1.0 + 2.0 ** -8, 1.0),                              # tie, even neighbour below
    (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),              # tie, even neighbour above
    (1.0 + 2.0 ** -8 + 2.0 ** -20, 1.0 + 2.0 ** -7),     # just above a tie
    (1.0 + 2.0 ** -8 - 2.0 ** -20, 1.0),                 # just below a tie
    (-(1.0 + 3 * 2.0 ** -8), -(1.0 + 2.0 ** -6)),        # sign is kept
    (1.0 - 2.0 ** -8, 1.0 - 2.0 ** -8),                  # exact below 1
    (2.0 + 2.0 ** -8, 2.0),                              # below the tie at 2 + 2^-7
    (255.5, 256.0),                                      # tie, rounds up into the next binade
    (3.0, 3.0),
    (0.0, 0.0),
    (2.0 ** -130, 2.0 ** -130),                          # subnormal, exact
    # float64 value just above a tie that float32 cannot hold: the float32
    # step lands on the tie itself, which then goes to even (the decision is
    # taken in float32, as on the GPU)
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 1.0),
]


def test_bf16_margins_hand_built():
    v = np.array([c[0] for c in _MARGIN_CASES])
    want = np.array([c[1] for c in _MARGIN_CASES])
    got = O.stored_margins(v, "bf16")
    assert np.array_equal(got, want)
    assert np.array_equal(O.stored_margins(v, "fp32"), v)
    with pytest.raises(ValueError):
        O.stored_margins(v, "fp16")


def _squared_step_fractions(Yi, yq, wq, s, b, c, vhat):
    """The squared-loss outer step in exact rationals from given margins."""
    n = len(wq)
    z = [None] * (s * b)
    r = [None] * (s * b)
    for j in range(s):
        for i in range(j * b, (j + 1) * b):
            acc = Fraction(0)
            for t in range(j):
                for k in range(t * b, (t + 1) * b):
                    acc += sum(Yi[i][q] * Yi[k][q] for q in range(n)) * r[k]
            z[i] = vhat[i] - c * acc
            r[i] = z[i] - yq[i]
    return [wq[q] - c * sum(Yi[i][q] * r[i] for i in range(s * b)) for q in range(n)]


def test_bf16_margin_step_matches_exact_rationals():
    # rows chosen so that Y w0 lands on ties and near-ties of bf16 (w0 = [1, 2^-8])
    Yi = [[1, 1], [1, 3], [1, -1], [2, 1]]
    wq = [Fraction(1), Fraction(1, 256)]
    vhat = [Fraction(1), 1 + Fraction(1, 64), 1 - Fraction(1, 256), Fraction(2)]  # by hand
    yq = [Fraction(1, 4), Fraction(-3, 4), Fraction(1, 2), Fraction(5, 4)]
    s, b = 2, 2
    c = Fraction(3, 8) / b
    Y = np.array(Yi, np.float64)
    yB = np.array([float(x) for x in yq])
    w0 = np.array([float(x) for x in wq])
    exact = np.array([float(x) for x in _squared_step_fractions(Yi, yq, wq, s, b, c, vhat)])
    out = O.outer_step_rows(Y, yB, w0, s, b, 0.375, "squared", margin="bf16")
    assert np.array_equal(out["v"], np.array([float(x) for x in vhat]))
    assert _rel(out["w"], exact) <= 1e-15
    # the same step from unrounded margins is a different answer: the pin sees the rounding
    v_plain = [sum(Yi[i][q] * wq[q] for q in range(2)) for i in range(4)]
    plain = np.array([float(x) for x in _squared_step_fractions(Yi, yq, wq, s, b, c, v_plain)])
    assert _rel(plain, exact) > 1e-4
    assert _rel(O.outer_step_rows(Y, yB, w0, s, b, 0.375, "squared")["w"], plain) <= 1e-15


@pytest.mark.parametrize("loss", LOSSES)
def test_bf16_margins_equal_fp32_when_margins_are_bf16_values(loss):
    # margins that bf16 holds exactly: the two precisions give the same step
    rng = np.random.default_rng(47)
    s, b, n = 3, 4, 6
    Y = rng.integers(-3, 4, (s * b, n)) / 4.0
    w0 = rng.integers(-3, 4, n) / 8.0
    yB = _targets(rng, s * b, loss)
    a = O.outer_step_rows(Y, yB, w0, s, b, 0.25, loss, margin="bf16")
    f = O.outer_step_rows(Y, yB, w0, s, b, 0.25, loss)
    for key in ("v", "z", "r", "w"):
        assert np.array_equal(a[key], f[key]), key


def test_bf16_margin_training_run_stays_close_to_sgd():
    # the recipe's claim in miniature: bf16 margins change the final loss little
    X = (np.random.default_rng(53).standard_normal((600, 20)) / 4.0).astype(np.float32)
    wstar = np.random.default_rng(54).standard_normal(20)
    y = np.where(X.astype(np.float64) @ wstar >= 0, 1.0, -1.0).astype(np.float32)
    w_sgd = O.train(X, y, np.zeros(20), 4, 8, 0.5, "logistic", 3, 30, storage="fp32", method="sgd")
    w_mix = O.train(X, y, np.zeros(20), 4, 8, 0.5, "logistic", 3, 30, margin="bf16")
    f_sgd = O.full_loss(X, y, w_sgd, "logistic", storage="fp32")
    f_mix = O.full_loss(X, y, w_mix, "logistic", storage="fp32")
    assert abs(f_mix - f_sgd) <= 5e-3 * f_sgd
    assert not np.array_equal(w_mix, O.train(X, y, np.zeros(20), 4, 8, 0.5, "logistic", 3, 30))


def test_margin_choices_hand_built():
    # v = 1 + 2^-8 and 1 + 3 * 2^-8 sit on boundaries: both neighbours admissible;
    # v = 1 has a single admissible value; the cancelling last row has
    # v = 2^-20 against sum |y w| of about 2, so its range spans many bf16 values
    Y = np.array([[1.0, 1.0], [1.0, 0.0], [1.0, 3.0], [1.0, -1.0]])
    w0 = np.array([1.0, 2.0 ** -8])
    nearest, lo, hi = O.margin_choices(Y, w0)
    assert list(nearest[:3]) == [1.0, 1.0, 1.0 + 2.0 ** -6]
    assert list(lo[:3]) == [1.0, 1.0, 1.0 + 2.0 ** -7]
    assert list(hi[:3]) == [1.0 + 2.0 ** -7, 1.0, 1.0 + 2.0 ** -6]
    Y2 = np.array([[1.0, -1.0]])
    w2 = np.array([1.0, 1.0 - 2.0 ** -20])
    n2, lo2, hi2 = O.margin_choices(Y2, w2)
    assert n2[0] == 2.0 ** -20
    # e = 2 * 2^-24 / (1 - 2^-23) * (2 - 2^-20) + 2^-23 * 2^-20, about 2^-22
    assert lo2[0] == 0.75 * 2.0 ** -20 and hi2[0] == 1.25 * 2.0 ** -20


def _f32_dot_orders(y, w, rng):
    """float32 dot products of one row in several summation orders."""
    p = (y.astype(np.float32) * w.astype(np.float32)).astype(np.float32)
    out = []
    for order in (np.arange(len(p)), np.arange(len(p))[::-1], rng.permutation(len(p))):
        acc = np.float32(0.0)
        for k in order:
            acc = np.float32(acc + p[k])
        out.append(acc)
    q = p.copy()  # pairwise
    while len(q) > 1:
        if len(q) % 2:
            q = np.append(q, np.float32(0.0))
        q = (q[0::2] + q[1::2]).astype(np.float32)
    out.append(q[0])
    return out


def test_margin_choices_cover_float32_orders():
    import torch
    rng = np.random.default_rng(61)
    n = 512
    X = (rng.standard_normal((300, n)) / np.sqrt(n)).astype(np.float32)
    Y = O.stored_values(X, "bf16")
    w0 = rng.standard_normal(n).astype(np.float32)
    nearest, lo, hi = O.margin_choices(Y, w0)
    assert np.all((lo <= nearest) & (nearest <= hi))
    # at this n the worst-case bound still leaves most rows one admissible value
    assert 0 < np.sum(lo != hi) < 0.5 * len(lo)
    for i in range(Y.shape[0]):
        for v32 in _f32_dot_orders(Y[i], w0, rng):
            got = float(torch.tensor([float(v32)], dtype=torch.float32).to(torch.bfloat16).to(torch.float64)[0])
            assert lo[i] <= got <= hi[i], (i, float(v32), lo[i], hi[i])


@pytest.mark.parametrize("storage", ["bf16", "fp32"])
def test_full_loss_across_its_row_chunks(storage):
    """full_loss sums in chunks of 2^21 / n rows; m spans two whole chunks and
    a ragged third.  Squared loss, w = e_0, y = 0: row i contributes
    x_i0^2 / 2 with x_i0 = (i mod 16) / 16 (exact in bf16), so the mean has an
    exact rational value; a dropped, repeated or shifted chunk changes it."""
    n = 64
    chunk = (1 << 21) // n
    m = 2 * chunk + 37
    X = np.zeros((m, n), np.float32)
    X[:, 0] = (np.arange(m) % 16) / 16.0
    X[:, 1:] = 3.0  # any other column is multiplied by w_j = 0
    y = np.zeros(m, np.float32)
    w = np.zeros(n)
    w[0] = 1.0
    exact = sum(Fraction(i % 16, 16) ** 2 / 2 for i in range(m)) / m
    got = O.full_loss(X, y, w, "squared", storage=storage)
    assert abs(got - float(exact)) <= 1e-15 * float(exact)
    # the same rows with the last chunk's rows dropped would differ by more than rounding
    short = sum(Fraction(i % 16, 16) ** 2 / 2 for i in range(2 * chunk)) / m
    assert abs(float(short) - float(exact)) > 1e-6


# --------------------------------------------------------------------------
# fp16 and fp8 storage, bf16-rounded Gram
# --------------------------------------------------------------------------
def _golden_rows(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            a, b, *_ = line.split()
            rows.append((a, b))
    return rows


def _f32_of(hexbits):
    return np.array([int(hexbits, 16)], dtype=np.uint32).view(np.float32)


def test_f16_rounding_golden_cases():
    for a, b in _golden_rows("fp16_rne_cases.txt"):
        x = _f32_of(a)
        assert int(O.f16_bits(x)[0]) == int(b, 16), (a, b, hex(int(O.f16_bits(x)[0])))
        if not np.isnan(x[0]):
            assert O.f16_to_f64(O.f16_bits(x))[0] == O.f16_round(x)[0] or np.isnan(O.f16_round(x)[0])


def test_e4m3_rounding_golden_cases():
    for a, b in _golden_rows("e4m3_rne_cases.txt"):
        x = _f32_of(a)
        assert int(O.e4m3_bits(x)[0]) == int(b, 16), (a, b, hex(int(O.e4m3_bits(x)[0])))


def test_fp8_scale_exponent_golden_cases():
    for a, b in _golden_rows("fp8_scale_cases.txt"):
        x = float(_f32_of(a)[0])
        k = O.fp8_exponent(x)
        assert k == int(b), (a, b, k)
        if x > 0:  # the defining property, checked exactly
            assert x * 2.0 ** k <= 448.0 < x * 2.0 ** (k + 1)


def _spread_f32(rng, count, lo_exp, hi_exp):
    """float32 values over many binades, both signs, plus exact ties."""
    mant = rng.uniform(1.0, 2.0, count)
    ex = rng.integers(lo_exp, hi_exp, count)
    x = (np.ldexp(mant, ex) * rng.choice([-1.0, 1.0], count)).astype(np.float32)
    return x


def test_f16_rounding_equals_numpy_conversion():
    # NumPy converts float32 to float16 with round-to-nearest-even and
    # overflow to infinity: the library routine the definition reduces to
    rng = np.random.default_rng(71)
    x = np.concatenate([_spread_f32(rng, 200000, -30, 18), np.float32([65504, 65519.996, 65520, 7e4])])
    # ties: values exactly halfway between neighbouring fp16 values
    h = rng.integers(1, 0x7BFF, 20000).astype(np.uint16).view(np.float16).astype(np.float64)
    nxt = (rng.integers(1, 0x7BFF, 20000).astype(np.uint16)).view(np.float16).astype(np.float64)
    x = np.concatenate([x, ((h + np.nextafter(h.astype(np.float16), np.float16(np.inf)).astype(np.float64)) / 2)
                        .astype(np.float32), nxt.astype(np.float32)])
    assert np.array_equal(O.f16_bits(x), x.astype(np.float16).view(np.uint16))


def test_e4m3_rounding_equals_torch_conversion_in_range():
    # torch's float8_e4m3fn conversion rounds to nearest even; it does not
    # saturate, so the comparison stays at |x| <= 464 (the largest value that
    # rounds to 448)
    import torch
    rng = np.random.default_rng(72)
    x = _spread_f32(rng, 200000, -14, 9)
    x = x[np.abs(x) <= 464.0]
    ties = (O.e4m3_to_f64(np.arange(0, 0x7E, dtype=np.uint8)) + O.e4m3_to_f64(np.arange(1, 0x7F, dtype=np.uint8))) / 2
    x = np.concatenate([x, ties.astype(np.float32), -ties.astype(np.float32)])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_bits(x), ref)


@pytest.mark.parametrize("fmt,u,lo,hi", [("fp16", 2.0 ** -11, 2.0 ** -14, 65504.0),
                                         ("e4m3", 2.0 ** -4, 2.0 ** -6, 448.0)])
def test_rounding_error_within_unit_roundoff_and_monotone(fmt, u, lo, hi):
    rng = np.random.default_rng(73)
    x = np.sort(np.exp(rng.uniform(np.log(lo), np.log(hi), 100000))).astype(np.float32).astype(np.float64)
    r = O.f16_round(x) if fmt == "fp16" else O.e4m3_round(x)
    assert np.all(np.abs(r - x) <= u * np.abs(x))
    assert np.all(np.diff(r) >= 0)
    # decoding the bits gives the rounded value back
    bits = O.f16_bits(x) if fmt == "fp16" else O.e4m3_bits(x)
    dec = O.f16_to_f64(bits) if fmt == "fp16" else O.e4m3_to_f64(bits)
    assert np.array_equal(dec, r)


def test_fp8_stored_values_are_scaled_e4m3_values():
    rng = np.random.default_rng(74)
    X = (rng.standard_normal((50, 40)) * 0.03).astype(np.float32)
    k = O.fp8_exponent_of(X)
    assert np.max(np.abs(X)) * 2.0 ** k <= 448.0 < np.max(np.abs(X)) * 2.0 ** (k + 1)
    V = O.stored_values(X, "fp8", k)
    # every stored value times 2^k is an E4M3 value: its own rounding
    assert np.array_equal(O.e4m3_round(np.ldexp(V, k)), np.ldexp(V, k))
    # within half an E4M3 spacing of x: relative 2^-4 for entries past the subnormal range
    big = np.abs(X) * 2.0 ** k >= 2.0 ** -6
    assert np.all(np.abs(V - X)[big] <= 2.0 ** -4 * np.abs(X)[big])
    with pytest.raises(ValueError):
        O.stored_values(X, "fp8")


def test_bf16_gram_rounds_float32_entries_once():
    # G_{1,0} = y1 . y0 with y0 = e_0: 1 + 2^-8 is a bf16 tie (stays 1),
    # 1 + 3 * 2^-8 a tie with an odd kept bit (rounds up to 1 + 2^-6)
    for g, want in ((1.0 + 2.0 ** -8, 1.0), (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6), (3.0, 3.0)):
        Y = np.array([[1.0, 0.0], [g, 5.0]])
        G = O.gram_blocks(Y, 2, 1)
        assert G[(1, 0)][0, 0] == g
        assert O.stored_gram(G, "bf16")[(1, 0)][0, 0] == want
        assert O.stored_gram(G, "fp32")[(1, 0)][0, 0] == g


@pytest.mark.parametrize("loss", O.LOSSES)
def test_bf16_gram_step_equals_fp32_step_when_entries_are_bf16_values(loss):
    # small integer rows: every Gram entry is an integer below 256, a bf16
    # value, so rounding G changes nothing
    rng = np.random.default_rng(75)
    s, b, n = 4, 3, 5
    Y = rng.integers(-3, 4, (s * b, n)).astype(np.float64)
    yB = np.abs(rng.integers(0, 3, s * b)).astype(np.float64) if loss == "poisson" else \
        rng.choice([-1.0, 1.0], s * b)
    w0 = rng.standard_normal(n) * 0.1
    a = O.outer_step_rows(Y, yB, w0, s, b, 0.05, loss, gram="fp32")
    c = O.outer_step_rows(Y, yB, w0, s, b, 0.05, loss, gram="bf16")
    for key in ("z", "r", "w"):
        assert np.array_equal(a[key], c[key])
    # and a Gram that is not bf16-exact changes the step
    Y2 = Y + 2.0 ** -9
    a2 = O.outer_step_rows(Y2, yB, w0, s, b, 0.05, loss, gram="fp32")
    c2 = O.outer_step_rows(Y2, yB, w0, s, b, 0.05, loss, gram="bf16")
    assert not np.array_equal(a2["w"], c2["w"])


def test_gram_choices_cover_float32_orders():
    rng = np.random.default_rng(76)
    s, b, n = 3, 8, 384
    Y = O.stored_values((rng.standard_normal((s * b, n)) / np.sqrt(n)).astype(np.float32), "bf16")
    near, lo, hi = O.gram_choices(Y, s, b)
    for (j, t), g in near.items():
        assert np.all((lo[(j, t)] <= g) & (g <= hi[(j, t)]))
        for i in range(b):
            for k in range(b):
                for v32 in _f32_dot_orders(Y[j * b + i], Y[t * b + k], rng):
                    r = O.stored_margins(np.array([float(v32)]), "bf16")[0]
                    assert lo[(j, t)][i, k] <= r <= hi[(j, t)][i, k]
