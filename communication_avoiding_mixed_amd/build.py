"""Build libcasgd.so (HIP, gfx950) in-tree with hipcc.

    python -m communication_avoiding_mixed_amd.build

Every source is compiled to an object under _build/ (in parallel), then
linked into communication_avoiding_mixed_amd/libcasgd.so.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcasgd.so")

SOURCES = ["casgd_api.hip", "k_gather.hip", "k_gram.hip", "k_chain.hip", "k_chain_la.hip", "k_loss.hip",
           "k_step.hip", "k_step_1x1.hip", "k_step_2x1.hip", "k_step_2x2.hip", "k_step_4x2.hip",
           "k_step_4x4.hip", "k_peak.hip"]
HEADERS = ["casgd_device.h", "casgd_internal.h", "casgd_chain.h"]

ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed-fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libcasgd.so")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"build step failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    jobs = []
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 8, 16)) as ex:
        for src in SOURCES:
            obj = os.path.join(BUILD, src.replace(".hip", ".o"))
            objs.append(obj)
            cmd = [hipcc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
            jobs.append(ex.submit(_run, cmd))
        for j in jobs:
            out = j.result()
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
