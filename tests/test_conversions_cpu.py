"""The kernels' storage conversions (casgd_device.h, compiled for the host)
against the oracle, bit for bit: fp16 and E4M3 rounding of the golden cases
and of random values across every binade, and the exact decoding back."""

import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

from oracle import casgd_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "communication_avoiding_mixed_amd", "csrc")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def conv():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    d = tempfile.mkdtemp()
    exe = os.path.join(d, "conv_host")
    subprocess.run([hipcc, "-O2", "-std=c++17", f"-I{CSRC}", "-o", exe,
                    os.path.join(os.path.dirname(__file__), "csrc", "conv_host.cpp")],
                   check=True, capture_output=True)

    def run(x_f32):
        bits = np.ascontiguousarray(x_f32, np.float32).view(np.uint32)
        out = subprocess.run([exe], input="\n".join(f"{b:08X}" for b in bits), capture_output=True,
                             text=True, check=True).stdout.split("\n")
        rows = [r.split() for r in out if r]
        h = np.array([int(r[0], 16) for r in rows], np.uint16)
        q = np.array([int(r[1], 16) for r in rows], np.uint8)
        hd = np.array([int(r[2], 16) for r in rows], np.uint32).view(np.float32)
        qd = np.array([int(r[3], 16) for r in rows], np.uint32).view(np.float32)
        return h, q, hd, qd
    yield run
    shutil.rmtree(d, ignore_errors=True)


def _golden_inputs(name):
    out = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            out.append(int(line.split()[0], 16))
    return np.array(out, np.uint32).view(np.float32)


def test_kernel_conversions_equal_oracle(conv):
    rng = np.random.default_rng(81)
    x = np.concatenate([
        _golden_inputs("fp16_rne_cases.txt"), _golden_inputs("e4m3_rne_cases.txt"),
        (np.ldexp(rng.uniform(1, 2, 100000), rng.integers(-32, 20, 100000)) *
         rng.choice([-1.0, 1.0], 100000)).astype(np.float32),
        rng.integers(0, 2 ** 32, 100000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    h, q, hd, qd = conv(x)
    assert np.array_equal(h, O.f16_bits(x))
    assert np.array_equal(q, O.e4m3_bits(x))
    fin = ~np.isnan(x)
    assert np.array_equal(hd[fin].astype(np.float64), O.f16_to_f64(h)[fin])
    assert np.array_equal(qd[fin].astype(np.float64), O.e4m3_to_f64(q)[fin])
