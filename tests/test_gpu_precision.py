"""The precision choices beyond bf16 storage (Abstract of "Mixed-Precision
Communication-Avoiding SGD for Generalized Linear Models on GPUs": the data
stored in any low-precision format, the Gram communicated in low precision)
against the oracle, through the C ABI.

- fp16 storage (Gram on fp16 MFMA) and fp8 storage (OCP E4M3 of x * 2^k,
  widened exactly to bf16 by the gather): stored bits and the scale exponent
  bit-exact; gathered rows bit-exact; one outer step within relative L2 1e-4
  for G, v, z, r and w; the loss; casgd_train equal to its outer steps.
- G rounded once to bf16: every entry a bf16 value inside the oracle's range
  of admissible roundings of a float32 sum; z, r and w within 1e-4 of the
  oracle run on the GPU's own G and of the oracle's nearest rounding.
Inputs carry a few entries small enough to be fp16 subnormals.
"""

import numpy as np
import pytest
import torch

from communication_avoiding_mixed_amd import binding as B
from oracle import casgd_oracle as O

from gpu_common import REL_TOL, check_gram, rel_l2, torch_dev

pytestmark = pytest.mark.gpu

ETA = {"logistic": 0.5, "squared": 0.05, "poisson": 0.01}


def data(m, n, loss, seed):
    rng = np.random.default_rng(seed)
    X = (rng.standard_normal((m, n)) / np.sqrt(n)).astype(np.float32)
    tiny = rng.random((m, n)) < 0.01
    X[tiny] *= np.float32(1e-4)  # about 2^-17 * |x|: fp16 subnormals
    if loss == "logistic":
        y = rng.choice([-1.0, 1.0], m).astype(np.float32)
    elif loss == "squared":
        y = rng.standard_normal(m).astype(np.float32)
    else:
        y = rng.poisson(1.0, m).astype(np.float32)
    w0 = (rng.standard_normal(n) * 0.5).astype(np.float32)
    return X, y, w0


def stored_bits(X, storage, k):
    return O.f16_bits(X) if storage == "fp16" else O.e4m3_bits(np.ldexp(X.astype(np.float64), k))


@pytest.mark.parametrize("storage", ["fp16", "fp8"])
@pytest.mark.parametrize("m,n", [(777, 45), (300, 2000), (513, 18)])
def test_stored_bits_and_scale(storage, m, n):
    X, y, _ = data(m, n, "logistic", 1)
    h = B.CASGD(torch_dev(X), torch_dev(y), "logistic", storage)
    k = O.fp8_exponent_of(X) if storage == "fp8" else 0
    assert h.fp8_exponent == k
    rows = h.export_rows(0, m)
    ref = np.zeros_like(rows)
    ref[:, :n] = stored_bits(X, storage, k)
    assert np.array_equal(rows, ref)
    h.close()


SHAPES = [(3000, 300, 4, 64), (2500, 45, 5, 24), (4000, 2000, 3, 70), (1500, 20, 2, 100)]


@pytest.mark.parametrize("storage", ["fp16", "fp8"])
@pytest.mark.parametrize("loss", O.LOSSES)
@pytest.mark.parametrize("m,n,s,b", SHAPES)
def test_one_step_against_oracle(storage, loss, m, n, s, b):
    X, y, w0 = data(m, n, loss, 2)
    eta = ETA[loss]
    h = B.CASGD(torch_dev(X), torch_dev(y), loss, storage)
    w = torch_dev(w0)
    seed = O.step_seed(5, 2)
    h.outer_step(s, b, eta, seed, w)
    ref = O.outer_step(X, y, w0.astype(np.float64), s, b, eta, seed, loss, storage=storage)
    assert np.array_equal(h.export(B.EXPORT_IDX).astype(np.int64), ref["idx"])
    Yg = h.export(B.EXPORT_Y)
    expect = np.zeros_like(Yg)
    Yv = ref["Y"].astype(np.float32)  # stored values: exact in float32
    expect[:, :n] = O.f16_bits(Yv) if storage == "fp16" else O.bf16_bits(Yv)
    assert np.array_equal(Yg, expect)
    errs = {"G": check_gram(h.export(B.EXPORT_G), ref["Y"], s, b, n),
            "v": rel_l2(h.export(B.EXPORT_V), ref["v"]), "z": rel_l2(h.export(B.EXPORT_Z), ref["z"]),
            "r": rel_l2(h.export(B.EXPORT_R), ref["r"]), "w": rel_l2(w.cpu().numpy(), ref["w"])}
    for key, e in errs.items():
        assert e <= REL_TOL, (key, e)
    # the loss over every stored row
    f = h.loss_value(w)
    f_ref = O.full_loss(X, y, w.cpu().numpy().astype(np.float64), loss, storage=storage)
    assert abs(f - f_ref) <= REL_TOL * abs(f_ref)
    h.close()


@pytest.mark.parametrize("storage", ["fp16", "fp8"])
def test_train_equals_its_outer_steps(storage):
    X, y, w0 = data(2000, 300, "logistic", 3)
    h = B.CASGD(torch_dev(X), torch_dev(y), "logistic", storage)
    w1, w2 = torch_dev(w0), torch_dev(w0)
    h.train(4, 64, 0.5, 9, 2, 5, w1)
    for k in range(2, 7):
        h.outer_step(4, 64, 0.5, B.step_seed(9, k), w2)
    torch.cuda.synchronize()
    assert torch.equal(w1, w2)
    h.close()


def _blocks(G_packed, s, b):
    return {k: v.astype(np.float64) for k, v in B.unpack_gram(G_packed, s, b).items()}


@pytest.mark.parametrize("storage", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("loss", O.LOSSES)
@pytest.mark.parametrize("m,n,s,b", [(3000, 300, 4, 64), (4000, 2000, 3, 70), (1500, 45, 6, 20)])
def test_bf16_gram_step(storage, loss, m, n, s, b):
    X, y, w0 = data(m, n, loss, 4)
    eta = ETA[loss]
    h = B.CASGD(torch_dev(X), torch_dev(y), loss, storage)
    h.set_option(B.OPT_GRAM_BF16, 1)
    w = torch_dev(w0)
    seed = O.step_seed(6, 1)
    h.outer_step(s, b, eta, seed, w)
    ref = O.outer_step(X, y, w0.astype(np.float64), s, b, eta, seed, loss, storage=storage, gram="bf16")
    G = _blocks(h.export(B.EXPORT_G), s, b)
    near, lo, hi = O.gram_choices(ref["Y"], s, b)
    differ = 0
    for key, g in G.items():
        assert np.all((g.astype(np.float32).view(np.uint32) & 0xFFFF) == 0), ("not bf16 values", key)
        ok = (lo[key] <= g) & (g <= hi[key])
        assert np.all(ok), (key, np.argwhere(~ok)[:4])
        differ += int(np.sum(g != near[key]))
    total = sum(g.size for g in G.values())
    assert differ <= 0.01 * total, (differ, total)
    # the recurrence and update on the GPU's own G, and on the nearest rounding
    own = O.outer_step_rows(ref["Y"], ref["yB"], w0.astype(np.float64), s, b, eta, loss, G=G)
    for want in (own, ref):
        for key, got in (("z", h.export(B.EXPORT_Z)), ("r", h.export(B.EXPORT_R)), ("w", w.cpu().numpy())):
            assert rel_l2(got, want[key]) <= REL_TOL, key
    h.close()


@pytest.mark.parametrize("form", [B.TRAIN_PERSISTENT, B.TRAIN_PER_STEP])
@pytest.mark.parametrize("storage", ["bf16", "fp16", "fp8", "fp32"])
@pytest.mark.parametrize("m,n,s,b", [(2000, 300, 4, 64), (3000, 45, 6, 20)])
def test_bf16_gram_train_equals_its_outer_steps(storage, form, m, n, s, b):
    # every launch form of casgd_train rounds G like the single outer step
    # (the pipelined launch's Gram role included)
    X, y, w0 = data(m, n, "logistic", 5)
    h = B.CASGD(torch_dev(X), torch_dev(y), "logistic", storage)
    h.set_option(B.OPT_GRAM_BF16, 1)
    h.set_option(B.OPT_TRAIN_FORM, form)
    w1, w2 = torch_dev(w0), torch_dev(w0)
    h.train(s, b, 0.5, 9, 2, 5, w1)
    for k in range(2, 7):
        h.outer_step(s, b, 0.5, B.step_seed(9, k), w2)
    torch.cuda.synchronize()
    assert torch.equal(w1, w2)
    h.close()


def test_fp16_rows_decode_exactly_subnormals_included():
    # column 3 holds binary16 subnormals k * 2^-24 (and -k * 2^-24); with w
    # the unit vector of that column every margin is one decoded value
    # (the other products are exact zeros), so it must equal the oracle's
    # stored value bit for bit
    rng = np.random.default_rng(10)
    m, n, s, b = 900, 40, 3, 64
    X = (rng.standard_normal((m, n)) / np.sqrt(n)).astype(np.float32)
    X[:, 3] = (rng.integers(1, 1024, m) * 2.0 ** -24 * rng.choice([-1.0, 1.0], m)).astype(np.float32)
    X[::7, 3] = np.float32(2.0 ** -14 * 1.5)  # and a few normals
    y = rng.choice([-1.0, 1.0], m).astype(np.float32)
    h = B.CASGD(torch_dev(X), torch_dev(y), "logistic", "fp16")
    w0 = np.zeros(n, np.float32)
    w0[3] = 1.0
    w = torch_dev(w0)
    h.outer_step(s, b, 0.5, O.step_seed(3, 0), w)
    idx = h.export(B.EXPORT_IDX).astype(np.int64)
    v = h.export(B.EXPORT_V).astype(np.float64)
    assert np.array_equal(v, O.f16_round(X[idx, 3]))
    assert np.any(np.abs(v) < 2.0 ** -14)  # subnormals were among the sampled rows
    h.close()
