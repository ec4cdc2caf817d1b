"""The calibration kernels behind the measured peaks: the copy moves every
byte, and the MFMA loop does every MFMA it is counted for."""

import ctypes

import pytest
import torch

from communication_avoiding_mixed_amd import binding as B

pytestmark = pytest.mark.gpu


def test_calibration_copy_is_exact_and_checks_its_arguments():
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(3)
    src = torch.randn((1 << 20) + 4, generator=g).to(dev)  # a ragged tail past the unrolled loop
    dst = torch.zeros_like(src)
    assert B.peak_copy(src, dst) == src.numel() * 4
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    with pytest.raises(B.CasgdError):
        B.peak_copy(src[:3], dst[:3])  # 12 bytes: not a multiple of 16
    with pytest.raises(B.CasgdError):
        B.peak_copy(src[:8], src[4:12])  # overlapping


def test_calibration_mfma_sum_has_its_closed_form():
    # Lane L of a wave feeds A's k-slice with ((L + e) & 7) / 8 and B's with
    # ((3L + e) & 7) / 16, e < 8: over any 32 consecutive lanes each residue
    # appears 4 times, so every column of A sums to 4 * 28 / 8 = 14 and every
    # row of B to 4 * 28 / 16 = 7, and one 32x32x16 MFMA adds 16 * 14 * 7 =
    # 1568 to the sum of C's entries.  4 waves x 4 chains x iters MFMAs per
    # workgroup; every partial sum is a small multiple of 2^-7 (exact).
    wgs, iters = 6, 100
    out = torch.full((wgs * 256,), float("nan"), device="cuda:0")
    flops = B.peak_mfma(out, wgs, iters)
    torch.cuda.synchronize()
    assert flops == wgs * 16 * iters * 32768
    per_wg = out.view(wgs, 256).double().sum(dim=1).cpu()
    assert torch.all(per_wg == 16 * iters * 1568), per_wg
    # the C entry point refuses an empty grid and a zero trip count
    lib = B.load()
    ptr = ctypes.c_void_p(out.data_ptr())
    assert lib.casgd_peak_mfma(ptr, 0, iters, None) == B.EINVAL
    assert lib.casgd_peak_mfma(ptr, wgs, 0, None) == B.EINVAL


def test_calibration_read_lands_the_data():
    # 1 MiB of 1.0 over 16 workgroups: every slice spans 4096 chunks, so all
    # 8 ring slots a workgroup reports were filled from src
    src = torch.ones(1 << 18, device="cuda:0")
    out = torch.zeros(16 * 8, device="cuda:0")
    assert B.peak_read(src, out, 16) == src.numel() * 4
    torch.cuda.synchronize()
    assert torch.all(out == 1.0)
    lib = B.load()
    assert lib.casgd_peak_read(ctypes.c_void_p(src.data_ptr()), 12, ctypes.c_void_p(out.data_ptr()), 16,
                               None) == B.EINVAL
