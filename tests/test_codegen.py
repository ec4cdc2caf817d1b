"""Code-generation guards for the gfx950 kernels (CPU only: hipcc cross-compiles).

Every kernel must run without scratch memory (register spills or local arrays
placed in memory turn each access into a round trip to HBM), and kernels that
are not written to use LDS must not get LDS from the compiler promoting local
arrays there."""

import concurrent.futures
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from communication_avoiding_mixed_amd import build as B

NO_LDS = ("gather_kernel", "store_bf16_kernel", "store_f32_kernel")
# host code only: the C-ABI and the dispatcher over the recurrence variants
HOST_ONLY = ("casgd_api.hip", "k_step.hip")


def _kernels(src):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        flags = [f for f in B.FLAGS if f not in ("-fPIC",)]
        subprocess.run([hipcc, *flags, "--cuda-device-only", "-S", "-o", out,
                        os.path.join(B.CSRC, src)], check=True, capture_output=True)
        text = open(out).read()
    meta = {}
    for block in re.findall(r"- \.agpr_count:.*?\.wavefront_size:\s+\d+", text, flags=re.S):
        name = re.search(r"\.name:\s+(\S+)", block).group(1)
        meta[name] = {
            "lds": int(re.search(r"\.group_segment_fixed_size:\s+(\d+)", block).group(1)),
            "scratch": int(re.search(r"\.private_segment_fixed_size:\s+(\d+)", block).group(1)),
        }
    return meta


@pytest.fixture(scope="module")
def compiled():
    """Device assembly metadata of every source, compiled in parallel."""
    if not os.path.exists(shutil.which("hipcc") or "/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    workers = max(1, min(len(B.SOURCES), os.cpu_count() or 4, 8))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        return dict(zip(B.SOURCES, ex.map(_kernels, B.SOURCES)))


@pytest.mark.parametrize("src", B.SOURCES)
def test_no_scratch_and_no_stray_lds(src, compiled):
    meta = compiled[src]
    if src in HOST_ONLY:
        return
    assert meta, f"no kernels found in {src}"
    for name, m in meta.items():
        assert m["scratch"] == 0, f"{name} uses {m['scratch']} bytes of scratch"
        if any(k in name for k in NO_LDS):
            assert m["lds"] == 0, f"{name} got {m['lds']} bytes of LDS"
