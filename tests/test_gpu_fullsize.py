"""The five workloads at their full sizes, in the launch configuration the
benchmark times, through the C ABI.

Per workload: sampled indices and gathered rows bit-exact; one outer step from
seeded weights within relative L2 1e-4 of the oracle for G, v, z, r and w
(the oracle only needs the s*b sampled rows, so this is exact at any m); the
loss at w = 0 against its closed form and at the seeded weights against the
oracle; and the whole run (20 or 200 outer steps from w = 0) ending within
0.5% of the loss of float64 SGD on the float32 data over the same minibatches.
The same step and run are repeated with bf16-stored margins (the recipe's
low-precision margin vector), held to the same bars.
"""

import math
import time

import numpy as np
import pytest

from communication_avoiding_mixed_amd import binding as B
from communication_avoiding_mixed_amd import synth
from oracle import casgd_oracle as O

from gpu_common import LOSS_GAP, REL_TOL, check_bf16_margins, check_gram, rel_l2, torch_dev

pytestmark = pytest.mark.gpu


def closed_form_loss_at_zero(loss, y):
    if loss == "logistic":
        return math.log(2.0)
    if loss == "squared":
        return 0.5 * float(np.mean(np.asarray(y, np.float64) ** 2))
    return 1.0


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_full_size_workload(name):
    import torch
    t0 = time.time()
    wl = synth.WORKLOADS[name]
    X, y = synth.make_data(name)
    h = B.CASGD(torch_dev(X), torch_dev(y), wl.loss, wl.storage)
    t_gen = time.time() - t0

    # one outer step from seeded weights
    w0 = synth.make_w0(name, 3)
    w = torch_dev(w0)
    seed = O.step_seed(0, 11)
    h.outer_step(wl.s, wl.b, wl.eta, seed, w)
    ref = O.outer_step(X, y, w0.astype(np.float64), wl.s, wl.b, wl.eta, seed, wl.loss)
    assert np.array_equal(h.export(B.EXPORT_IDX).astype(np.int64), ref["idx"])
    Yg = h.export(B.EXPORT_Y)
    expect = np.zeros_like(Yg)
    expect[:, :wl.n] = O.bf16_bits(X[ref["idx"]])
    assert np.array_equal(Yg, expect)
    errs = {
        "G": check_gram(h.export(B.EXPORT_G), ref["Y"], wl.s, wl.b, wl.n),
        "v": rel_l2(h.export(B.EXPORT_V), ref["v"]),
        "z": rel_l2(h.export(B.EXPORT_Z), ref["z"]),
        "r": rel_l2(h.export(B.EXPORT_R), ref["r"]),
        "w": rel_l2(w.cpu().numpy(), ref["w"]),
    }
    for k, e in errs.items():
        assert e <= REL_TOL, (k, e)

    # loss: closed form at zero, oracle at the seeded weights
    zero = torch.zeros(wl.n, device="cuda")
    f0 = h.loss_value(zero)
    assert abs(f0 - closed_form_loss_at_zero(wl.loss, y)) <= REL_TOL * abs(f0)
    f_seeded = h.loss_value(torch_dev(w0))
    f_seeded_ref = O.full_loss(X, y, w0.astype(np.float64), wl.loss, storage="bf16")
    assert abs(f_seeded - f_seeded_ref) <= REL_TOL * abs(f_seeded_ref)

    # whole run from zero vs float64 SGD on the float32 data
    wt = torch.zeros(wl.n, device="cuda")
    h.train(wl.s, wl.b, wl.eta, 0, 0, wl.outer, wt)
    f_gpu = h.loss_value(wt)
    w_sgd = O.train(X, y, np.zeros(wl.n), wl.s, wl.b, wl.eta, wl.loss, base_seed=0,
                    n_outer=wl.outer, storage="fp32", method="sgd")
    f_ref = O.full_loss(X, y, w_sgd, wl.loss, storage="fp32")
    gap = abs(f_gpu - f_ref) / abs(f_ref)
    print(f"{name}: step errs {({k: f'{v:.1e}' for k, v in errs.items()})} "
          f"final loss gpu {f_gpu:.6f} sgd64 {f_ref:.6f} gap {gap:.2e} "
          f"(start {f0:.4f}); data {t_gen:.0f}s total {time.time() - t0:.0f}s", flush=True)
    assert f_gpu < f0
    assert gap <= LOSS_GAP

    # the recipe's bf16-stored margins: the same step and the same run
    h.set_option(B.OPT_MARGIN_BF16, 1)
    w = torch_dev(w0)
    h.outer_step(wl.s, wl.b, wl.eta, seed, w)
    merrs, flips = check_bf16_margins(h, ref["Y"], ref["yB"], w0, wl.s, wl.b, wl.eta, wl.loss,
                                      w.cpu().numpy())
    for k, (e, bar) in merrs.items():
        assert e <= bar, ("bf16 margins", k, e, bar, flips)
    wm = torch.zeros(wl.n, device="cuda")
    h.train(wl.s, wl.b, wl.eta, 0, 0, wl.outer, wm)
    f_mix = h.loss_value(wm)
    gap_mix = abs(f_mix - f_ref) / abs(f_ref)
    print(f"{name}: bf16 margins: step {({k: f'{e:.1e}/{bar:.1e}' for k, (e, bar) in merrs.items()})} "
          f"({flips} rows off the nearest rounding), final loss {f_mix:.6f} gap {gap_mix:.2e}", flush=True)
    assert gap_mix <= LOSS_GAP
    h.close()


def test_fp32_sgd_baseline_at_epsilon_shape():
    """The plain SGD the benchmark's speedup divides by: casgd_train with
    s = 1 on float32-stored data, epsilon shape (400000 x 2000, b = 64,
    eta = 1), base seed 7, in the launch configuration the benchmark times.
    Each of the first steps, from the GPU's own weights, against the
    oracle's step on the float32 values (v, r and w within relative L2
    1e-4); then the benchmark's whole run (5 x 16 warm-up steps, then
    200 x 16 steps) ending within 0.5% of the loss of the oracle's float64
    SGD over the same minibatches."""
    import torch
    name = "epsilon"
    wl = synth.WORKLOADS[name]
    X, y = synth.make_data(name)
    h = B.CASGD(torch_dev(X), torch_dev(y), wl.loss, "fp32")
    w = torch.zeros(wl.n, device="cuda")
    for k in range(12):
        w0 = w.cpu().numpy().astype(np.float64)
        h.train(1, wl.b, wl.eta, 7, k, 1, w)
        ref = O.outer_step(X, y, w0, 1, wl.b, wl.eta, O.step_seed(7, k), wl.loss, storage="fp32")
        assert np.array_equal(h.export(B.EXPORT_IDX).astype(np.int64), ref["idx"]), k
        errs = {"v": rel_l2(h.export(B.EXPORT_V), ref["v"]), "r": rel_l2(h.export(B.EXPORT_R), ref["r"]),
                "w": rel_l2(w.cpu().numpy(), ref["w"])}
        for key, e in errs.items():
            assert e <= REL_TOL, (k, key, e)

    warm, timed = 5 * wl.s, 200 * wl.s
    wt = torch.zeros(wl.n, device="cuda")
    h.train(1, wl.b, wl.eta, 7, 0, warm, wt)
    h.train(1, wl.b, wl.eta, 7, warm, timed, wt)
    f_gpu = h.loss_value(wt)
    w_sgd = O.train(X, y, np.zeros(wl.n), 1, wl.b, wl.eta, wl.loss, base_seed=7, n_outer=warm + timed,
                    storage="fp32", method="sgd")
    f_ref = O.full_loss(X, y, w_sgd, wl.loss, storage="fp32")
    gap = abs(f_gpu - f_ref) / abs(f_ref)
    print(f"fp32 SGD baseline: last step errs {({k: f'{v:.1e}' for k, v in errs.items()})}, "
          f"final loss gpu {f_gpu:.6f} sgd64 {f_ref:.6f} gap {gap:.2e}", flush=True)
    assert f_gpu < math.log(2.0)
    assert gap <= LOSS_GAP
    h.close()


VARIANTS = {"fp16": ("fp16", 0), "fp8": ("fp8", 0), "gram-bf16": (None, 1)}


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_full_size_precision_variant(name, variant):
    """fp16 storage, fp8 storage and the bf16-communicated Gram at full size:
    one outer step from seeded weights against the oracle (G, v, z, r, w
    within 1e-4; for the bf16 Gram, z, r and w on the GPU's own admissible
    G), then the whole run from w = 0 against float64 SGD on the float32
    data over the same minibatches (final loss within 0.5%)."""
    import torch
    wl = synth.WORKLOADS[name]
    storage, gbf16 = VARIANTS[variant]
    storage = storage or wl.storage
    X, y = synth.make_data(name)
    h = B.CASGD(torch_dev(X), torch_dev(y), wl.loss, storage)
    h.set_option(B.OPT_GRAM_BF16, gbf16)
    k = O.fp8_exponent_of(X) if storage == "fp8" else None
    if k is not None:
        assert h.fp8_exponent == k
    w0 = synth.make_w0(name, 3)
    w = torch_dev(w0)
    seed = O.step_seed(0, 11)
    h.outer_step(wl.s, wl.b, wl.eta, seed, w)
    gram = "bf16" if gbf16 else "fp32"
    ref = O.outer_step(X, y, w0.astype(np.float64), wl.s, wl.b, wl.eta, seed, wl.loss, storage=storage,
                       gram=gram, fp8_exp=k)
    if gbf16:
        G = {key: g.astype(np.float64) for key, g in B.unpack_gram(h.export(B.EXPORT_G), wl.s, wl.b).items()}
        near, lo, hi = O.gram_choices(ref["Y"], wl.s, wl.b)
        for key, g in G.items():
            assert np.all((lo[key] <= g) & (g <= hi[key])), key
        ref = O.outer_step_rows(ref["Y"], ref["yB"], w0.astype(np.float64), wl.s, wl.b, wl.eta, wl.loss, G=G)
        errs = {}
    else:
        errs = {"G": check_gram(h.export(B.EXPORT_G), ref["Y"], wl.s, wl.b, wl.n),
                "v": rel_l2(h.export(B.EXPORT_V), ref["v"])}
    errs.update({"z": rel_l2(h.export(B.EXPORT_Z), ref["z"]), "r": rel_l2(h.export(B.EXPORT_R), ref["r"]),
                 "w": rel_l2(w.cpu().numpy(), ref["w"])})
    for key, e in errs.items():
        assert e <= REL_TOL, (key, e)

    wt = torch.zeros(wl.n, device="cuda")
    h.train(wl.s, wl.b, wl.eta, 0, 0, wl.outer, wt)
    f_gpu = h.loss_value(wt)
    w_sgd = O.train(X, y, np.zeros(wl.n), wl.s, wl.b, wl.eta, wl.loss, base_seed=0,
                    n_outer=wl.outer, storage="fp32", method="sgd")
    f_ref = O.full_loss(X, y, w_sgd, wl.loss, storage="fp32")
    gap = abs(f_gpu - f_ref) / abs(f_ref)
    print(f"{name} {variant}: step errs {({key: f'{v:.1e}' for key, v in errs.items()})} "
          f"final loss {f_gpu:.6f} vs float64 SGD {f_ref:.6f}, gap {gap:.2e}", flush=True)
    assert gap <= LOSS_GAP
    h.close()
