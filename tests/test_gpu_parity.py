"""GPU parity of one outer iteration against the FP64 oracle, per workload at
reduced row counts (same n, s, b, eta and loss as the full workloads), through
the C ABI.

Bars: sampled indices, stored bf16 bits and gathered rows bit-exact; G, v, z,
r and w within relative L2 1e-4 of the oracle after one outer step from the
same seeded w0; every Gram entry within the float32 dot-product bound."""

import numpy as np
import pytest

from communication_avoiding_mixed_amd import binding as B
from communication_avoiding_mixed_amd import synth
from oracle import casgd_oracle as O

from gpu_common import REL_TOL, check_gram, make_handle, rel_l2, torch_dev

pytestmark = pytest.mark.gpu

# row counts at which the oracle finishes in seconds
SMALL = {
    "logistic-4096x64": None,
    "epsilon": 20_000,
    "higgs": 200_000,
    "susy": 200_000,
    "synth-lsq": 50_000,
    "poisson-synth": 50_000,
}

_cache = {}


def handle(name, storage=None):
    key = (name, storage)
    if key not in _cache:
        _cache[key] = make_handle(name, m=SMALL[name], storage=storage)
    return _cache[key]


def expected_rows(X, idx, ld, storage):
    rows = np.asarray(X)[idx]
    if storage == "bf16":
        out = np.zeros((len(idx), ld), np.uint16)
        out[:, :rows.shape[1]] = O.bf16_bits(rows)
    else:
        out = np.zeros((len(idx), ld), np.float32)
        out[:, :rows.shape[1]] = rows
    return out


@pytest.mark.parametrize("name", list(SMALL))
def test_stored_rows_bit_exact(name):
    h, X, y, wl = handle(name)
    rows = np.unique(np.r_[0, 1, 2, np.arange(h.m - 3, h.m),
                           np.random.default_rng(1).integers(0, h.m, 200)])
    for r in rows[:20]:
        got = h.export_rows(int(r), 1)
        assert np.array_equal(got, expected_rows(X, [r], h.ld, "bf16")), r
    block = h.export_rows(0, 256)
    assert np.array_equal(block, expected_rows(X, np.arange(256), h.ld, "bf16"))


def test_fp32_storage_exact():
    h, X, y, wl = handle("logistic-4096x64", storage="fp32")
    got = h.export_rows(0, h.m)
    assert np.array_equal(got, expected_rows(X, np.arange(h.m), h.ld, "fp32"))


@pytest.mark.parametrize("name", list(SMALL))
def test_sample_and_gather_bit_exact(name):
    h, X, y, wl = handle(name)
    import torch
    w = torch.zeros(wl.n, device="cuda")
    seed = O.step_seed(0, 3)
    h.outer_step(wl.s, wl.b, wl.eta, seed, w)
    idx = h.export(B.EXPORT_IDX)
    ref_idx = O.sample_indices(seed, h.m, wl.s * wl.b)
    assert np.array_equal(idx.astype(np.int64), ref_idx)
    Y = h.export(B.EXPORT_Y)
    assert np.array_equal(Y, expected_rows(X, ref_idx, h.ld, "bf16"))
    yB = h.export(B.EXPORT_YB)
    assert np.array_equal(yB, y[ref_idx])


RECURRENCES = {"auto": B.RECURRENCE_AUTO, "all-to-all": B.RECURRENCE_ALL_TO_ALL,
               "lookahead": B.RECURRENCE_LOOKAHEAD}


@pytest.mark.parametrize("w0kind", ["zero", "seeded"])
@pytest.mark.parametrize("name,storage,rec", [(n, None, "auto") for n in SMALL] +
                         [("logistic-4096x64", "fp32", "auto"),
                          ("logistic-4096x64", None, "all-to-all"),
                          ("epsilon", None, "all-to-all"),
                          ("epsilon", None, "lookahead")])
def test_outer_step_parity(name, storage, rec, w0kind):
    h, X, y, wl = handle(name, storage)
    h.set_option(B.OPT_RECURRENCE, RECURRENCES[rec])
    st = storage or wl.storage
    w0 = np.zeros(wl.n, np.float32) if w0kind == "zero" else synth.make_w0(name, 1)
    w = torch_dev(w0)
    seed = O.step_seed(0, 7)
    h.outer_step(wl.s, wl.b, wl.eta, seed, w)
    ref = O.outer_step(X, y, w0.astype(np.float64), wl.s, wl.b, wl.eta, seed, wl.loss, storage=st)

    G = h.export(B.EXPORT_G)
    errs = {"G": check_gram(G, ref["Y"], wl.s, wl.b, wl.n)}
    errs["v"] = rel_l2(h.export(B.EXPORT_V), ref["v"])
    errs["z"] = rel_l2(h.export(B.EXPORT_Z), ref["z"])
    errs["r"] = rel_l2(h.export(B.EXPORT_R), ref["r"])
    errs["w"] = rel_l2(w.cpu().numpy(), ref["w"])
    h.set_option(B.OPT_RECURRENCE, B.RECURRENCE_AUTO)
    print(name, st, rec, w0kind, {k: f"{v:.2e}" for k, v in errs.items()})
    for k, e in errs.items():
        assert e <= REL_TOL, (k, e)


@pytest.mark.parametrize("name", list(SMALL))
def test_loss_parity(name):
    h, X, y, wl = handle(name)
    for w0 in (np.zeros(wl.n, np.float32), synth.make_w0(name, 2)):
        got = h.loss_value(torch_dev(w0))
        ref = O.full_loss(X, y, w0.astype(np.float64), wl.loss, storage="bf16")
        assert abs(got - ref) <= REL_TOL * abs(ref), (got, ref)
