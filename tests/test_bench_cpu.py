"""Host logic of bench.py (no GPU): the one-GPU contract and the algorithmic
work per outer step that the roofline figures are built on."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from communication_avoiding_mixed_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_algorithmic_work_per_outer_step(name):
    wl = synth.WORKLOADS[name]
    s, b, n = wl.s, wl.b, wl.n
    alg = bench.algorithmic(wl)
    # strictly-lower block triangle: s(s-1)/2 blocks of b x b dot products of length n, 2 flop each
    blocks = s * (s - 1) // 2
    assert alg["gram_flops"] == blocks * b * b * n * 2
    # packed float32 G: the same blocks, 4 bytes per entry, written once and read once
    g_bytes = blocks * b * b * 4
    rows = s * b * n * 2  # the gathered bf16 rows, read once for G and v, once for the update
    assert alg["B_A"] == rows + g_bytes
    assert alg["B_B"] == g_bytes
    assert alg["B_C"] == rows + 2 * n * 4


def test_epsilon_figures():
    alg = bench.algorithmic(synth.WORKLOADS["epsilon"])
    assert alg["gram_flops"] == 1_966_080_000
    assert alg["B_A"] + alg["B_B"] + alg["B_C"] == 12_140_160
