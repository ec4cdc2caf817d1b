"""Host-side checks of the seeded workload generators (no method arithmetic)."""

import numpy as np
import pytest

from communication_avoiding_mixed_amd import synth


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_shapes_dtypes_and_determinism(name):
    X, y = synth.make_data(name, seed=0, m=3000)
    wl = synth.WORKLOADS[name]
    assert X.shape == (3000, wl.n) and X.dtype == np.float32 and X.flags.c_contiguous
    assert y.shape == (3000,) and y.dtype == np.float32
    X2, y2 = synth.make_data(name, seed=0, m=3000)
    assert np.array_equal(X, X2) and np.array_equal(y, y2)
    X3, _ = synth.make_data(name, seed=1, m=3000)
    assert not np.array_equal(X, X3)


def test_value_structure():
    X, y = synth.make_data("epsilon", m=4000)
    assert np.allclose(np.linalg.norm(X.astype(np.float64), axis=1), 1.0, atol=1e-6)
    assert set(np.unique(y)) == {-1.0, 1.0}
    X, y = synth.make_data("higgs", m=20000)
    assert np.allclose(X.astype(np.float64).mean(0), 0.0, atol=1e-5)
    assert np.allclose(X.astype(np.float64).std(0), 1.0, atol=1e-4)
    # odd columns came from a lognormal: skewed to the right
    assert np.all(np.mean(X[:, 1::2] ** 3, axis=0) > 0.5)
    X, y = synth.make_data("susy", m=20000)
    assert X.shape == (20000, 18)
    assert np.allclose(X.astype(np.float64).mean(0), 0.0, atol=1e-5)
    assert np.allclose(X.astype(np.float64).std(0), 1.0, atol=1e-4)
    # columns 8-17 came from a lognormal (skewed right), columns 0-7 are symmetric
    assert np.all(np.mean(X[:, 8:] ** 3, axis=0) > 0.5)
    assert np.all(np.abs(np.mean(X[:, :8] ** 3, axis=0)) < 0.1)
    X, y = synth.make_data("poisson-synth", m=20000)
    assert np.all(y >= 0) and np.all(y == np.round(y))
    assert abs(X.std() - 1 / 32) < 1e-3
    X, y = synth.make_data("logistic-4096x64")
    assert X.shape == (4096, 64) and abs(X.std() - 1 / 8) < 2e-3


def test_label_flip_rate():
    X, y = synth.make_data("higgs", m=200000)
    rng = np.random.Generator(np.random.PCG64(0))
    # replay the draws: X first, then w*, then the flip uniforms
    _ = rng.standard_normal((200000, 14), dtype=np.float32)
    _ = rng.lognormal(0.0, 0.5, (200000, 14))
    w_star = rng.standard_normal(28)
    clean = np.where(X.astype(np.float64) @ w_star >= 0, 1.0, -1.0)
    assert abs(np.mean(clean != y) - 0.25) < 0.01


def test_susy_label_flip_rate():
    X, y = synth.make_data("susy", m=200000)
    rng = np.random.Generator(np.random.PCG64(0))
    _ = rng.standard_normal((200000, 8), dtype=np.float32)
    _ = rng.lognormal(0.0, 0.5, (200000, 10))
    w_star = rng.standard_normal(18)
    clean = np.where(X.astype(np.float64) @ w_star >= 0, 1.0, -1.0)
    assert abs(np.mean(clean != y) - 0.20) < 0.01
