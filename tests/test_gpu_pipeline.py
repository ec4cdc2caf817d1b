"""casgd_train in both of its forms (one persistent launch for all steps, and
one launch per outer step: recurrence of step k, Gram of step k+1, gather of
step k+2) against the same steps queued one by one with casgd_outer_step:
weights and every exported intermediate must be bit-identical, since all run
the same device code on the same inputs."""

import numpy as np
import pytest

from communication_avoiding_mixed_amd import binding as B
from communication_avoiding_mixed_amd import synth
from oracle import casgd_oracle as O

from gpu_common import REL_TOL, rel_l2, torch_dev

pytestmark = pytest.mark.gpu

EXPORTS = (B.EXPORT_IDX, B.EXPORT_Y, B.EXPORT_YB, B.EXPORT_G, B.EXPORT_V, B.EXPORT_Z, B.EXPORT_R)
FORMS = [B.TRAIN_PERSISTENT, B.TRAIN_PER_STEP]


def _data(loss, m, n, seed):
    X = synth.make_uniform((m, n), seed=seed, lo=-0.4, hi=0.4)
    rng = np.random.default_rng(seed + 1)
    if loss == "logistic":
        y = np.where(rng.random(m) < 0.5, -1.0, 1.0).astype(np.float32)
    elif loss == "squared":
        y = rng.standard_normal(m).astype(np.float32)
    else:
        y = rng.poisson(1.0, m).astype(np.float32)
    return X, y


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("loss", ["logistic", "squared", "poisson"])
@pytest.mark.parametrize("m,n,s,b,n_outer", [
    (3000, 300, 4, 64, 5),    # several tiles, whole pipeline
    (2000, 70, 3, 48, 4),     # Q = 48: the Gram role starts at workgroup 48
    (1500, 33, 5, 100, 3),    # ragged tiles, two 64-row tiles per block edge
    (800, 200, 1, 32, 4),     # s = 1: no Gram at all
    (900, 40, 6, 16, 1),      # prologue only, then one launch
    (900, 40, 6, 16, 2),      # no gather role in either launch
    (4000, 2000, 16, 64, 3),  # the epsilon step shape
    (3000, 1800, 3, 128, 3),  # update after the recurrence (8 rows per lane per block)
    (2000, 3000, 2, 32, 3),   # ld 3008: weights read from global memory in the margins
    (3000, 28, 32, 128, 2),   # HIGGS-like: G rows too large for LDS, 2 rows per workgroup
    (4000, 512, 8, 256, 2),   # synth-like: 4 rows per workgroup, 4 columns per lane
    (2000, 64, 40, 64, 2),    # one row per workgroup with G too large for LDS
    (4000, 3000, 4, 64, 3),   # update after the recurrence in the persistent launch (16 rows per lane)
])
def test_train_equals_outer_steps(form, loss, m, n, s, b, n_outer):
    import torch
    X, y = _data(loss, m, n, seed=m + s)
    eta = 0.3 if loss != "poisson" else 0.05
    base, first = 11, 5
    h = B.CASGD(torch_dev(X), torch_dev(y), loss)
    h.set_option(B.OPT_TRAIN_FORM, form)
    w_pipe = torch_dev(synth.make_uniform((n,), seed=2, lo=-0.2, hi=0.2))
    w_step = w_pipe.clone()
    h.train(s, b, eta, base, first, n_outer, w_pipe)
    got = {k: h.export(k) for k in EXPORTS}
    for k in range(n_outer):
        h.outer_step(s, b, eta, O.step_seed(base, first + k), w_step)
    torch.cuda.synchronize()
    assert torch.equal(w_pipe, w_step)
    for k in EXPORTS:
        assert np.array_equal(got[k], h.export(k)), k


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("m,n,s,b,n_outer", [(1500, 45, 5, 24, 4), (1000, 300, 3, 64, 3), (600, 20, 1, 32, 5)])
def test_train_equals_outer_steps_fp32(form, m, n, s, b, n_outer):
    import torch
    X, y = _data("logistic", m, n, seed=m)
    h = B.CASGD(torch_dev(X), torch_dev(y), "logistic", "fp32")
    h.set_option(B.OPT_TRAIN_FORM, form)
    w_pipe = torch_dev(synth.make_uniform((n,), seed=4, lo=-0.2, hi=0.2))
    w_step = w_pipe.clone()
    h.train(s, b, 0.4, 3, 0, n_outer, w_pipe)
    got = {k: h.export(k) for k in EXPORTS}
    for k in range(n_outer):
        h.outer_step(s, b, 0.4, O.step_seed(3, k), w_step)
    torch.cuda.synchronize()
    assert torch.equal(w_pipe, w_step)
    for k in EXPORTS:
        assert np.array_equal(got[k], h.export(k)), k


@pytest.mark.parametrize("form", FORMS)
def test_train_then_steps_interleave(form):
    import torch
    name = "logistic-4096x64"
    wl = synth.WORKLOADS[name]
    X, y = synth.make_data(name)
    h = B.CASGD(torch_dev(X), torch_dev(y), wl.loss)
    h.set_option(B.OPT_TRAIN_FORM, form)
    w1 = torch.zeros(wl.n, device="cuda")
    h.outer_step(wl.s, wl.b, wl.eta, O.step_seed(0, 0), w1)
    h.train(wl.s, wl.b, wl.eta, 0, 1, 6, w1)
    h.outer_step(wl.s, wl.b, wl.eta, O.step_seed(0, 7), w1)
    h.train(wl.s, wl.b, wl.eta, 0, 8, 4, w1)
    w2 = torch.zeros(wl.n, device="cuda")
    for k in range(12):
        h.outer_step(wl.s, wl.b, wl.eta, O.step_seed(0, k), w2)
    torch.cuda.synchronize()
    assert torch.equal(w1, w2)


@pytest.mark.parametrize("form", FORMS)
def test_pipelined_step_against_oracle(form):
    """The last step of a training run, from the GPU's own w0, to the bar."""
    import torch
    name = "epsilon"
    wl = synth.WORKLOADS[name]
    X, y = synth.make_data(name, m=20_000)
    h = B.CASGD(torch_dev(X), torch_dev(y), wl.loss)
    h.set_option(B.OPT_TRAIN_FORM, form)
    w = torch.zeros(wl.n, device="cuda")
    h.train(wl.s, wl.b, wl.eta, 0, 0, 3, w)
    w0 = w.clone()
    h.train(wl.s, wl.b, wl.eta, 0, 3, 1, w)
    ref = O.outer_step(X, y, w0.cpu().numpy().astype(np.float64), wl.s, wl.b, wl.eta,
                       O.step_seed(0, 3), wl.loss)
    assert np.array_equal(h.export(B.EXPORT_IDX).astype(np.int64), ref["idx"])
    for k, key in ((B.EXPORT_V, "v"), (B.EXPORT_Z, "z"), (B.EXPORT_R, "r")):
        assert rel_l2(h.export(k), ref[key]) <= REL_TOL, key
    assert rel_l2(w.cpu().numpy(), ref["w"]) <= REL_TOL


def test_pipe_timer_counts_launches():
    import torch
    name = "logistic-4096x64"
    wl = synth.WORKLOADS[name]
    X, y = synth.make_data(name)
    h = B.CASGD(torch_dev(X), torch_dev(y), wl.loss)
    h.set_option(B.OPT_TRAIN_FORM, B.TRAIN_PER_STEP)
    w = torch.zeros(wl.n, device="cuda")
    h.set_timing(True)
    h.train(wl.s, wl.b, wl.eta, 0, 0, 7, w)
    ms, cnt = h.timing(B.K_PIPE)
    g_ms, g_cnt = h.timing(B.K_GATHER)
    h.set_timing(False)
    assert cnt == 7 and ms > 0
    assert g_cnt == 2  # prologue: steps 0 and 1


def test_train_timer_counts_one_launch():
    import torch
    name = "logistic-4096x64"
    wl = synth.WORKLOADS[name]
    X, y = synth.make_data(name)
    h = B.CASGD(torch_dev(X), torch_dev(y), wl.loss)
    w = torch.zeros(wl.n, device="cuda")
    h.set_timing(True)
    h.train(wl.s, wl.b, wl.eta, 0, 0, 7, w)
    ms, cnt = h.timing(B.K_TRAIN)
    p_ms, p_cnt = h.timing(B.K_PIPE)
    h.set_timing(False)
    assert cnt == 1 and ms > 0 and p_cnt == 0


def test_sampled_timing_stamps_every_kth_launch():
    import torch
    name = "logistic-4096x64"
    wl = synth.WORKLOADS[name]
    X, y = synth.make_data(name)
    h = B.CASGD(torch_dev(X), torch_dev(y), wl.loss)
    h.set_option(B.OPT_TRAIN_FORM, B.TRAIN_PER_STEP)
    w = torch.zeros(wl.n, device="cuda")
    h.set_timing(True, every=3)
    h.train(wl.s, wl.b, wl.eta, 0, 0, 10, w)
    ms, cnt = h.timing(B.K_PIPE, reset=True)
    h.set_timing(False)
    assert cnt == 4 and ms > 0  # launches 0, 3, 6, 9
    with pytest.raises(B.CasgdError):
        h.set_timing(True, every=-1)
