"""Edge cases of the GPU path through the C ABI: degenerate shapes, ragged
tiles, the largest s*b, explicit and duplicated indices, orthogonal rows,
argument errors, determinism, resume, and streams."""

import numpy as np
import pytest

from communication_avoiding_mixed_amd import binding as B
from communication_avoiding_mixed_amd import synth
from oracle import casgd_oracle as O

from gpu_common import REL_TOL, check_gram, rel_l2, torch_dev

pytestmark = pytest.mark.gpu


def _targets(loss, m, seed):
    rng = np.random.default_rng(seed)
    if loss == "logistic":
        return np.where(rng.random(m) < 0.5, -1.0, 1.0).astype(np.float32)
    if loss == "squared":
        return rng.standard_normal(m).astype(np.float32)
    return rng.poisson(1.0, m).astype(np.float32)


def run_and_compare(X, y, loss, s, b, eta, w0, seed=123, storage="bf16", idx=None, rec=None):
    import torch
    h = B.CASGD(torch_dev(X), torch_dev(y), loss, storage)
    if rec is not None:
        h.set_option(B.OPT_RECURRENCE, rec)
    w = torch_dev(w0)
    if idx is None:
        h.outer_step(s, b, eta, seed, w)
    else:
        h.outer_step_indices(s, b, eta, torch.from_numpy(np.asarray(idx, np.int32)).cuda(), w)
    ref = O.outer_step(X, y, w0.astype(np.float64), s, b, eta, seed, loss, storage=storage, idx=idx)
    assert np.array_equal(h.export(B.EXPORT_IDX).astype(np.int64), ref["idx"])
    errs = {
        "G": check_gram(h.export(B.EXPORT_G), ref["Y"], s, b, X.shape[1]),
        "v": rel_l2(h.export(B.EXPORT_V), ref["v"]),
        "z": rel_l2(h.export(B.EXPORT_Z), ref["z"]),
        "r": rel_l2(h.export(B.EXPORT_R), ref["r"]),
        "w": rel_l2(w.cpu().numpy(), ref["w"]),
    }
    for k, e in errs.items():
        assert e <= REL_TOL, (k, e, s, b, X.shape)
    return h, w, ref


@pytest.mark.parametrize("loss", ["logistic", "squared", "poisson"])
@pytest.mark.parametrize("m,n,s,b", [
    (500, 70, 3, 48),    # b not a multiple of the 64-row tile, ld 96
    (300, 33, 4, 100),   # ragged tiles on both sides, ld 64
    (200, 1, 5, 7),      # one feature, tiny blocks
    (1000, 130, 2, 130),  # tiles crossing the block edge, ld 160 (K tail)
    (64, 32, 1, 64),     # s = 1: no Gram at all
    (1, 16, 3, 5),       # one row: every index is 0
    (700, 200, 9, 1),    # b = 1: 1 x 1 blocks
])
def test_ragged_and_degenerate_shapes(loss, m, n, s, b):
    X = synth.make_uniform((m, n), seed=m + n, lo=-0.5, hi=0.5)
    y = _targets(loss, m, seed=s)
    w0 = synth.make_uniform((n,), seed=7, lo=-0.3, hi=0.3)
    h, w, ref = run_and_compare(X, y, loss, s, b, 0.3, w0)
    if s == 1:
        assert h.export(B.EXPORT_G).size == 0
        assert np.array_equal(h.export(B.EXPORT_Z), h.export(B.EXPORT_V))


@pytest.mark.parametrize("rec", [B.RECURRENCE_ALL_TO_ALL, B.RECURRENCE_LOOKAHEAD])
@pytest.mark.parametrize("loss", ["logistic", "squared", "poisson"])
@pytest.mark.parametrize("m,n,s,b", [
    (2000, 40, 2, 16),    # one near block per step
    (3000, 100, 5, 32),   # three near blocks, ragged K
    (5000, 64, 20, 64),   # helpers own 2 rows each (LDS), far sums over 16 steps
    (4000, 72, 30, 48),   # helpers own 1 row each
    (3000, 50, 9, 64),    # b at the lookahead limit, ld 64
    (3000, 1800, 3, 128),  # 8 rows per lane per block: update after the recurrence
    (1500, 3000, 2, 32),   # ld 3008: weights read from global memory in the margins
])
def test_lookahead_and_all_to_all_recurrences(loss, m, n, s, b, rec):
    X = synth.make_uniform((m, n), seed=m + s, lo=-0.4, hi=0.4)
    y = _targets(loss, m, seed=b)
    w0 = synth.make_uniform((n,), seed=3, lo=-0.3, hi=0.3)
    run_and_compare(X, y, loss, s, b, 0.2 if loss != "poisson" else 0.05, w0, rec=rec)


def test_fp32_storage_ragged():
    X = synth.make_uniform((400, 45), seed=3)
    y = _targets("logistic", 400, 1)
    run_and_compare(X, y, "logistic", 5, 24, 0.5, synth.make_uniform((45,), seed=4), storage="fp32")


@pytest.mark.parametrize("s,b", [(2, 8192), (128, 128)])
def test_largest_minibatch_set(s, b):
    # s*b = 16384, the library's limit
    X = synth.make_uniform((5000, 24), seed=11, lo=-0.2, hi=0.2)
    y = _targets("squared", 5000, 2)
    run_and_compare(X, y, "squared", s, b, 0.01, np.zeros(24, np.float32))


def test_orthogonal_rows_give_zero_gram():
    n = 64
    X = np.eye(n, dtype=np.float32)
    y = _targets("logistic", n, 5)
    idx = np.random.default_rng(0).permutation(n)[:48]
    w0 = synth.make_uniform((n,), seed=9)
    h, w, ref = run_and_compare(X, y, "logistic", 3, 16, 0.5, w0, idx=idx)
    assert not np.any(h.export(B.EXPORT_G))
    c = float(np.float32(0.5)) / 16
    expect = w0.astype(np.float64).copy()
    for i in idx:
        expect[i] -= c * O.loss_derivative(float(w0[i]), float(y[i]), "logistic")[0]
    assert rel_l2(w.cpu().numpy(), expect) <= 1e-6


def test_duplicated_indices():
    X = synth.make_uniform((50, 40), seed=12)
    y = _targets("poisson", 50, 3)
    idx = np.array([7] * 32 + [3] * 32)
    run_and_compare(X, y, "poisson", 4, 16, 0.05, synth.make_uniform((40,), seed=1, lo=-.2, hi=.2), idx=idx)


def test_invalid_arguments_leave_w_untouched():
    import torch
    X = synth.make_uniform((100, 10), seed=1)
    y = _targets("logistic", 100, 1)
    h = B.CASGD(torch_dev(X), torch_dev(y), "logistic")
    w = torch.ones(10, device="cuda")
    lib = B.load()
    hh = h._handle()
    wp = B.ctypes.c_void_p(w.data_ptr())
    assert lib.casgd_outer_step(hh, 0, 4, 0.1, 0, wp) == B.EINVAL
    assert lib.casgd_outer_step(hh, 4, 0, 0.1, 0, wp) == B.EINVAL
    assert lib.casgd_outer_step(hh, 129, 128, 0.1, 0, wp) == B.EINVAL
    assert lib.casgd_outer_step(hh, 2, 2, 0.1, 0, None) == B.EINVAL
    bad = torch.tensor([0, 1, 100, 2], dtype=torch.int32, device="cuda")
    assert lib.casgd_outer_step_indices(hh, 2, 2, 0.1, B.ctypes.c_void_p(bad.data_ptr()), wp) == B.EINVAL
    neg = torch.tensor([0, -1, 1, 2], dtype=torch.int32, device="cuda")
    assert lib.casgd_outer_step_indices(hh, 2, 2, 0.1, B.ctypes.c_void_p(neg.data_ptr()), wp) == B.EINVAL
    assert lib.casgd_debug_export(hh, B.EXPORT_V, None, 0) == B.EINVAL
    assert lib.casgd_export_rows(hh, 99, 2, B.ctypes.c_void_p(1), 10) == B.EINVAL
    assert lib.casgd_get_timing(hh, 9, None, None, 0) == B.EINVAL
    torch.cuda.synchronize()
    assert torch.equal(w, torch.ones(10, device="cuda"))
    # the handle still works afterwards
    h.outer_step(2, 2, 0.1, 0, w)
    assert np.all(np.isfinite(w.cpu().numpy()))
    with pytest.raises(B.CasgdError):
        h.export_rows(0, 101)
    assert not lib.casgd_create(B.ctypes.c_void_p(w.data_ptr()), B.ctypes.c_void_p(w.data_ptr()), 0, 5, 0, 0)
    assert not lib.casgd_create(B.ctypes.c_void_p(w.data_ptr()), B.ctypes.c_void_p(w.data_ptr()), 2, 5, 7, 0)
    assert not lib.casgd_create(B.ctypes.c_void_p(w.data_ptr()), B.ctypes.c_void_p(w.data_ptr()), 2, 5, 0, 9)


def test_nonfinite_values_propagate_without_failure():
    import torch
    X = synth.make_uniform((200, 16), seed=2, lo=0.5, hi=1.0)
    y = _targets("poisson", 200, 4)
    h = B.CASGD(torch_dev(X), torch_dev(y), "poisson")
    w = torch.full((16,), 50.0, device="cuda")
    h.outer_step(4, 8, 1e4, 1, w)
    val = h.loss_value(w)
    assert not np.isfinite(val) or val > 1e10


def test_repeatable_and_resumable():
    import torch
    name = "poisson-synth"
    wl = synth.WORKLOADS[name]
    X, y = synth.make_data(name, m=30_000)
    h = B.CASGD(torch_dev(X), torch_dev(y), wl.loss)
    w1 = torch.zeros(wl.n, device="cuda")
    h.train(wl.s, wl.b, wl.eta, 0, 0, 20, w1)
    w2 = torch.zeros(wl.n, device="cuda")
    h.train(wl.s, wl.b, wl.eta, 0, 0, 20, w2)
    assert torch.equal(w1, w2)
    w3 = torch.zeros(wl.n, device="cuda")
    h.train(wl.s, wl.b, wl.eta, 0, 0, 10, w3)
    saved = w3.clone()
    w4 = saved.clone()
    h.train(wl.s, wl.b, wl.eta, 0, 10, 10, w4)
    assert torch.equal(w4, w1)
    w5 = torch.zeros(wl.n, device="cuda")
    for k in range(20):
        h.outer_step(wl.s, wl.b, wl.eta, O.step_seed(0, k), w5)
    assert torch.equal(w5, w1)


def test_lookahead_repeatable_and_resumable():
    import torch
    name = "epsilon"
    wl = synth.WORKLOADS[name]
    X, y = synth.make_data(name, m=20_000)
    h = B.CASGD(torch_dev(X), torch_dev(y), wl.loss)
    w1 = torch.zeros(wl.n, device="cuda")
    h.train(wl.s, wl.b, wl.eta, 0, 0, 12, w1)
    w2 = torch.zeros(wl.n, device="cuda")
    h.train(wl.s, wl.b, wl.eta, 0, 0, 6, w2)
    h.train(wl.s, wl.b, wl.eta, 0, 6, 6, w2)
    assert torch.equal(w1, w2)


@pytest.mark.parametrize("form", [B.TRAIN_PERSISTENT, B.TRAIN_PER_STEP])
def test_side_stream_and_timing(form):
    import torch
    name = "logistic-4096x64"
    wl = synth.WORKLOADS[name]
    X, y = synth.make_data(name)
    h = B.CASGD(torch_dev(X), torch_dev(y), wl.loss)
    h.set_option(B.OPT_TRAIN_FORM, form)
    w_ref = torch.zeros(wl.n, device="cuda")
    h.train(wl.s, wl.b, wl.eta, 0, 0, 5, w_ref)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        w = torch.zeros(wl.n, device="cuda")
        h.set_timing(True)
        h.train(wl.s, wl.b, wl.eta, 0, 0, 5, w)
        ms, cnt = h.timing(B.K_PIPE)
        g_ms, g_cnt = h.timing(B.K_GRAM)
        t_ms, t_cnt = h.timing(B.K_TRAIN)
        h.set_timing(False)
    side.synchronize()
    assert torch.equal(w, w_ref)
    if form == B.TRAIN_PERSISTENT:
        # one launch for all five steps
        assert t_cnt == 1 and t_ms > 0 and cnt == 0 and g_cnt == 0
    else:
        # one stand-alone Gram (the first step's), then one launch per step
        assert cnt == 5 and ms > 0
        assert g_cnt == 1 and g_ms > 0 and t_cnt == 0


def test_train_forms_bit_identical():
    """The persistent launch and one launch per step give the same bits, and
    both equal outer steps queued one by one, for every lean variant."""
    import torch
    for s, b, Q_note in ((4, 16, "1 row"), (6, 64, "2 rows"), (5, 128, "2 rows, 2 columns"),
                         (3, 256, "4 rows, 4 columns")):
        n = 300
        X = synth.make_uniform((5000, n), seed=s * 100 + b, lo=-0.1, hi=0.1)
        y = np.sign(synth.make_uniform(5000, seed=b)).astype(np.float32)
        y[y == 0] = 1.0
        h = B.CASGD(torch_dev(X), torch_dev(y), "logistic")
        outs = []
        for form in (B.TRAIN_PERSISTENT, B.TRAIN_PER_STEP):
            h.set_option(B.OPT_TRAIN_FORM, form)
            w = torch_dev(synth.make_w0("epsilon", 3, n=n) * 0.05)
            h.train(s, b, 0.5, 11, 2, 7, w)
            outs.append((w.clone(), h.export(B.EXPORT_R), h.export(B.EXPORT_V), h.export(B.EXPORT_G),
                         h.export(B.EXPORT_IDX)))
        w = torch_dev(synth.make_w0("epsilon", 3, n=n) * 0.05)
        for k in range(2, 9):
            h.outer_step(s, b, 0.5, B.step_seed(11, k), w)
        outs.append((w.clone(), h.export(B.EXPORT_R), h.export(B.EXPORT_V), h.export(B.EXPORT_G),
                     h.export(B.EXPORT_IDX)))
        for o in outs[1:]:
            assert torch.equal(outs[0][0], o[0]), (s, b, Q_note)
            for a, c in zip(outs[0][1:], o[1:]):
                assert np.array_equal(a, c), (s, b, Q_note)
        h.close()


@pytest.mark.parametrize("rec", [B.RECURRENCE_ALL_TO_ALL, B.RECURRENCE_LOOKAHEAD])
def test_expired_waits_are_reported_and_cleared(rec):
    """With a bound of one poll the waits between workgroups expire: every
    kernel still ends, the next loss call reports the failure once, and with
    the default bound the handle gives the same results as a fresh one."""
    import torch
    X = synth.make_uniform((6000, 256), seed=21, lo=-0.3, hi=0.3)
    y = _targets("logistic", 6000, 8)
    s, b, eta = 16, 64, 0.5
    h = B.CASGD(torch_dev(X), torch_dev(y), "logistic")
    h.set_option(B.OPT_RECURRENCE, rec)
    h.set_option(B.OPT_SPIN_LIMIT, 1)
    w = torch.zeros(256, device="cuda")
    h.outer_step(s, b, eta, 5, w)
    with pytest.raises(B.CasgdError, match="timed out"):
        h.loss_value(w)
    if rec == B.RECURRENCE_ALL_TO_ALL:
        h.train(s, b, eta, 0, 0, 3, w)  # the pipelined launches end as well
        with pytest.raises(B.CasgdError, match="timed out"):
            h.loss_value(w)
    h.set_option(B.OPT_SPIN_LIMIT, 0)
    w1 = torch.zeros(256, device="cuda")
    h.train(s, b, eta, 0, 0, 4, w1)
    val = h.loss_value(w1)
    fresh = B.CASGD(torch_dev(X), torch_dev(y), "logistic")
    fresh.set_option(B.OPT_RECURRENCE, rec)
    w2 = torch.zeros(256, device="cuda")
    fresh.train(s, b, eta, 0, 0, 4, w2)
    assert torch.equal(w1, w2)
    assert val == fresh.loss_value(w2)
    with pytest.raises(B.CasgdError):
        h.set_option(B.OPT_SPIN_LIMIT, -1)


# Every loss-kernel path: rows of at most 4 and at most 8 16-byte chunks (the
# narrow kernels), 9-15 chunks, 16 or more; both storages (bf16: 8 values per
# chunk, float32: 4); row counts that leave a partial pass, and a single row.
@pytest.mark.parametrize("storage", ["bf16", "fp32"])
@pytest.mark.parametrize("loss", ["logistic", "squared", "poisson"])
@pytest.mark.parametrize("m,n", [
    (1, 5),         # one row
    (1000, 1),      # ld 32: 4 chunks (bf16), 8 (float32)
    (4099, 28),     # HIGGS width: 4 / 8 chunks
    (777, 33),      # ld 64: 8 / 16 chunks
    (2050, 70),     # ld 96: 12 / 24 chunks
    (513, 130),     # ld 160: 20 / 40 chunks
    (300, 520),     # ld 544: 68 / 136 chunks
])
def test_loss_every_row_width(storage, loss, m, n):
    rng = np.random.default_rng(m * 1000 + n)
    X = (rng.standard_normal((m, n)) / np.sqrt(n)).astype(np.float32)
    y = _targets(loss, m, seed=n)
    h = B.CASGD(torch_dev(X), torch_dev(y), loss, storage)
    for w0 in (np.zeros(n, np.float32), (0.5 * rng.standard_normal(n)).astype(np.float32)):
        got = h.loss_value(torch_dev(w0))
        ref = O.full_loss(X, y, w0.astype(np.float64), loss, storage=storage)
        assert abs(got - ref) <= REL_TOL * abs(ref), (storage, loss, m, n, got, ref)
    h.close()
