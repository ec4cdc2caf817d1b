"""casgd_loss_noalloc (partial sums in the library's static scratch, result
in a caller's device double, no allocation, no wait) against casgd_loss on
the same handle and weights: the same kernels in the same order, so the same
bits.  Two calls in a row share the scratch; the second has a smaller input
(and a reduction with fewer partial sums)."""

import ctypes

import numpy as np
import pytest
import torch

from communication_avoiding_mixed_amd import binding as B
from gpu_common import make_handle, torch_dev
from communication_avoiding_mixed_amd import synth

pytestmark = pytest.mark.gpu


def _noalloc(h, w):
    out = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda:0")
    rc = B.load().casgd_loss_noalloc(h._handle(), ctypes.c_void_p(w.data_ptr()), ctypes.c_void_p(out.data_ptr()))
    assert rc == B.OK, B.load().casgd_last_error()
    torch.cuda.synchronize()
    return float(out.item())


# (workload, rows, storage): a wide bf16 reduction over every loss block,
# then a smaller fp32 one on the narrow kernel with fewer partial sums
CASES = [("epsilon", 30000, "bf16"), ("logistic-4096x64", 1000, "fp32")]


def test_noalloc_loss_equals_casgd_loss_on_two_calls_in_a_row():
    for name, m, storage in CASES:
        wl = synth.WORKLOADS[name]
        print(f"[no-alloc] {name} m={m} {storage}", flush=True)
        h, X, y, _ = make_handle(name, m=m, storage=storage)
        w = torch_dev(synth.make_w0(name, 5) * 0.1)
        ref = h.loss_value(w)
        got = _noalloc(h, w)
        assert np.isfinite(ref)
        assert got == ref, (name, got, ref)
        h.close()


def test_noalloc_loss_other_losses_and_stream_order():
    # squared and Poisson losses, each call queued on a side stream right
    # after the weights are written on it
    for name, m in (("synth-lsq", 4000), ("poisson-synth", 3000)):
        h, X, y, wl = make_handle(name, m=m)
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            w = torch_dev(synth.make_w0(name, 9) * 0.05)
            got = _noalloc(h, w)
            ref = h.loss_value(w)
        assert got == ref, (name, got, ref)
        h.close()


def test_noalloc_loss_refuses_null_pointers():
    h, X, y, wl = make_handle("logistic-4096x64", m=500)
    w = torch.zeros(wl.n, device="cuda:0")
    lib = B.load()
    hp = h._handle()
    assert lib.casgd_loss_noalloc(hp, None, ctypes.c_void_p(w.data_ptr())) == B.EINVAL
    assert lib.casgd_loss_noalloc(hp, ctypes.c_void_p(w.data_ptr()), None) == B.EINVAL
    assert lib.casgd_loss_noalloc(None, ctypes.c_void_p(w.data_ptr()), ctypes.c_void_p(w.data_ptr())) == B.EINVAL
    h.close()
