"""Shared helpers of the GPU parity tests (comparison metrics and set-up)."""

from __future__ import annotations

import numpy as np

from communication_avoiding_mixed_amd import binding as B
from communication_avoiding_mixed_amd import synth
from oracle import casgd_oracle as O

# Relative L2 bound for G, v, z, r and w after one outer step, and for the
# loss value on the same stored data.
REL_TOL = 1e-4
# Final loss of a whole run against float64 SGD on the float32 data.
LOSS_GAP = 5e-3
# Unit roundoff used in the elementwise Gram bound: 2^-23 covers float32 sums
# rounded to nearest and those truncated toward zero, in any order.
U32 = 2.0 ** -23


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    nr = np.linalg.norm(ref)
    if nr == 0.0:
        return 0.0 if np.array_equal(got, ref) else float("inf")
    return float(np.linalg.norm(got - ref) / nr)


def gamma(k: int) -> float:
    return k * U32 / (1.0 - k * U32)


def torch_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def make_handle(name: str, m: int | None = None, storage: str | None = None, seed: int = 0):
    """(handle, X, y, workload) for a workload at m rows (default: full size)."""
    wl = synth.WORKLOADS[name]
    X, y = synth.make_data(name, seed=seed, m=m)
    h = B.CASGD(torch_dev(X), torch_dev(y), wl.loss, storage or wl.storage)
    return h, X, y, wl


def check_gram(G_packed, Y, s, b, n, tol=REL_TOL):
    """Compare the GPU's packed Gram with the oracle's blocks of Y (float64).

    Returns the worst relative L2 over blocks; asserts the elementwise bound
    |G - G_ref| <= gamma_n * (|Y_j| |Y_t|^T) everywhere.
    """
    ref = O.gram_blocks(Y, s, b)
    got = B.unpack_gram(G_packed, s, b)
    A = np.abs(Y)
    gam = gamma(n)
    all_got, all_ref = [], []
    for (j, t), blk in ref.items():
        g = got[(j, t)].astype(np.float64)
        bound = gam * (A[j * b:(j + 1) * b] @ A[t * b:(t + 1) * b].T) + 1e-30
        excess = np.abs(g - blk) - bound
        assert np.all(excess <= 0), f"block ({j},{t}) breaks the elementwise bound by {excess.max():.3e}"
        all_got.append(g.ravel())
        all_ref.append(blk.ravel())
    if not all_ref:
        assert G_packed.size == 0
        return 0.0
    return rel_l2(np.concatenate(all_got), np.concatenate(all_ref))


def check_bf16_margins(h, Y, yB, w0, s, b, eta, loss, w_after, exact=False):
    """One outer step run with bf16-stored margins, against the oracle.

    exact: the inputs make every float32 margin exact, so each device margin
    must be the oracle's rounding of it (ties to even) and z, r, w are held
    to REL_TOL.  Otherwise each device margin must be a bf16 value in the
    oracle's admissible range; where it differs from the rounding of the exact
    margin by dv, the bar for z, r, w grows by the first-order effect of dv,
    bounded block by block: |dz_j| <= |dv_j| + c L sum_{t<j} ||G_jt||_2 |dz_t|,
    |dr_t| <= L_t |dz_t|, |dw| <= c ||Y||_2 |dr|, with L_t the bound of |l''|
    on block t between the two runs (1/4 logistic, 1 squared, exp of the
    block's largest z for Poisson).
    Returns ({name: (error, bar)}, rows that differ from the nearest rounding).
    """
    w0 = np.asarray(w0, np.float64)
    v = h.export(B.EXPORT_V).astype(np.float64)
    z = h.export(B.EXPORT_Z).astype(np.float64)
    r = h.export(B.EXPORT_R).astype(np.float64)
    nearest, lo, hi = O.margin_choices(Y, w0)
    assert np.all((v.astype(np.float32).view(np.uint32) & 0xFFFF) == 0), "margins are not bf16 values"
    if exact:
        assert np.array_equal(v, nearest), np.flatnonzero(v != nearest)[:8]
    else:
        ok = (lo <= v) & (v <= hi)
        assert np.all(ok), np.flatnonzero(~ok)[:8]
    ref = O.outer_step_rows(Y, yB, w0, s, b, eta, loss, margin="bf16")
    dv = v - ref["v"]
    dz = dr = dw = 0.0
    if np.any(dv != 0):
        c = O.step_size(eta, b)
        if loss == "logistic":
            L = np.full(s, 0.25)
        elif loss == "squared":
            L = np.ones(s)
        else:
            L = np.exp(np.maximum(z, ref["z"]).reshape(s, b).max(axis=1))
        G = O.gram_blocks(Y, s, b)
        D = np.zeros(s)
        for j in range(s):
            D[j] = np.linalg.norm(dv[j * b:(j + 1) * b])
            for t in range(j):
                D[j] += c * np.linalg.norm(G[(j, t)], 2) * L[t] * D[t]
        dz = float(np.linalg.norm(D))
        dr = float(np.linalg.norm(L * D))
        dw = c * float(np.linalg.norm(Y, 2)) * dr
    out = {}
    for name, got, want, d in (("z", z, ref["z"], dz), ("r", r, ref["r"], dr),
                               ("w", w_after, ref["w"], dw)):
        nrm = np.linalg.norm(want)
        out[name] = (rel_l2(got, want), REL_TOL + (d / nrm if nrm > 0 else 0.0))
    return out, int(np.sum(dv != 0))
