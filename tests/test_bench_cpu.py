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


def test_summary_of_a_persistent_launch():
    """Rates and fractions follow from the step count, the launch time and
    the algorithmic work: 200 steps in one 5.8 ms launch at epsilon."""
    wl = synth.WORKLOADS["epsilon"]
    r = {"ms": 6.0, "loss": 0.5, "n_break": 50,
         "launch": {"kernel": "train_kernel", "form": "persistent", "steps_per_launch": 200,
                    "us_per_launch": 5800.0, "stamped_launches": 1},
         "per": {"gather": 5.0, "gram": 13.0, "chain": 30.0, "pipe": None, "train": None}}
    peaks = {"hbm_copy_GB/s": 6000.0, "mfma_bf16_TFLOP/s": 2000.0}
    sm = bench.summarize(wl, r, 200, peaks)
    step_bytes = 12_140_160
    assert sm["us_per_step"] == pytest.approx(30.0)
    assert sm["value"] == pytest.approx(16 * 200 / 6e-3)
    assert sm["dominant"]["us_per_step"] == pytest.approx(29.0)
    assert sm["dominant"]["GB/s"] == pytest.approx(step_bytes / 29e-6 / 1e9)
    assert sm["dominant"]["hbm_frac"] == pytest.approx(step_bytes / 29e-6 / 8e12)
    assert sm["dominant"]["hbm_frac_of_measured_copy"] == pytest.approx(step_bytes / 29e-6 / 6e12)
    assert sm["gram"]["TFLOP/s"] == pytest.approx(1_966_080_000 / 13e-6 / 1e12)
    assert sm["gram"]["mfma_frac_of_measured"] == pytest.approx(1_966_080_000 / 13e-6 / 2e15)
    assert sm["gram"]["bound"] == "mfma"
    # the dependency-aware step roofline over the measured step time
    assert sm["step_roofline_frac"] == pytest.approx(sm["t_roof_us"] / 30.0)
    assert "pipe" not in sm["breakdown"]


def test_cpu_baseline_states_cores_threads_and_model():
    wl = synth.WORKLOADS["logistic-4096x64"]
    X, y = synth.make_data(wl.name)
    c = bench.cpu_baseline(X, y, wl, 0.5)
    assert c["kind"] == "oracle"
    assert c["cores"] == len(os.sched_getaffinity(0))
    assert c["one_thread"]["blas_threads"] == 1
    assert c["value"] > 0 and c["one_thread"]["value"] > 0
    assert "model name" not in (c["cpu_model"] or "")


def test_train_kernel_sources_exist():
    for f in bench.TRAIN_SOURCES:
        assert os.path.exists(os.path.join(bench.CSRC, f)), f
    assert len(bench.train_source_sha256()) == 64
