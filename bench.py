"""Throughput of mixed-precision CA-SGD outer iterations on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload epsilon]

A step is one outer iteration (s inner SGD steps): sample + gather + margins,
strictly-lower Gram on bf16 MFMA, inner recurrence, weight update.  The data
(seeded, synthetic, epsilon-shaped by default) is resident in HBM before the
timed region.  casgd_train runs the steps as one pipelined launch each (the
recurrence of step k beside the Gram of step k+1 and the gather of step k+2);
that launch is the dominant kernel, timed by HIP events its own dispatch
stamps, on the library's stream, over the timed region.  A second pass queues
the same steps one by one (separate gather, Gram and chain kernels) for a
per-kernel breakdown, including the Gram's MFMA throughput.  Prints one JSON
line; the CPU oracle is timed on the host on a bounded sample.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E

METRIC = "inner SGD steps/s and Gram TFLOP/s (% of roofline) at epsilon-shape, 1 GPU"
STAMP_EVERY = 8  # launches per dispatch-stamped launch in the timed region


def algorithmic(wl):
    """Algorithmic work of one outer step (no padding, no staging copies)."""
    s, b, n = wl.s, wl.b, wl.n
    sb = s * b
    gram_flops = n * b * b * s * (s - 1)          # strictly-lower blocks only
    g_bytes = 2 * b * b * s * (s - 1)              # packed float32 G
    return {
        "gram_flops": gram_flops,
        "gather_bytes": sb * n * 2 + sb * 12,           # rows read, idx/yB
        "gram_bytes": sb * n * 2 + g_bytes,             # Y read, G written
        # margins (Y read), recurrence (G read), update (Y read), vectors
        "chain_bytes": 2 * sb * n * 2 + g_bytes + sb * 20 + 3 * n * 4,
        "B_A": sb * n * 2 + g_bytes,
        "B_B": g_bytes,
        "B_C": sb * n * 2 + 2 * n * 4,
    }


PMC_SUMMARY = os.path.join(ROOT, "profiles", "pipe_kernel-epsilon-pmc.md")
CSRC = os.path.join(ROOT, "communication_avoiding_mixed_amd", "csrc")
# every source the pipelined step kernel is compiled from
PIPE_SOURCES = ("k_chain.hip", "casgd_chain.h", "casgd_gram.h", "casgd_gather.h", "casgd_device.h",
                "casgd_internal.h")


def pipe_source_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in PIPE_SOURCES:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()


def pipe_traffic(workload: str):
    """Scaled HBM bytes per pipelined step launch from the committed rocprofv3
    --pmc summary, or None if there is none for this workload or the kernel's
    sources have changed since it was taken."""
    if workload != "epsilon" or not os.path.exists(PMC_SUMMARY):
        return None
    vals = {}
    for line in open(PMC_SUMMARY):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip().strip("-* `")] = v.strip().strip("`")
    try:
        if vals["kernel_source_sha256"] != pipe_source_sha256():
            return None
        return (float(vals["fetch_kib_per_dispatch"]) * 1024 * float(vals["fetch_scale"])
                + float(vals["write_kib_per_dispatch"]) * 1024 * float(vals["write_scale"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(X, y, wl, budget_s: float):
    """The oracle's outer step, as it stands, on the host: inner steps/s."""
    import numpy as np
    from oracle import casgd_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    w = np.zeros(wl.n)
    t0 = time.perf_counter()
    k = 0
    while True:
        w = O.outer_step(X, y, w, wl.s, wl.b, wl.eta, O.step_seed(0, k), wl.loss)["w"]
        k += 1
        el = time.perf_counter() - t0
        if (el >= budget_s and k >= 2) or k >= wl.outer:
            break
    return {
        "value": wl.s * k / el,
        "unit": "inner SGD steps/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"first {k} outer steps (s={wl.s}, b={wl.b}) of the same {wl.name} run from w=0, "
                  f"float64 NumPy, {el:.1f} s",
    }


def sgd_baselines(h_bf16, X, y, wl, steps: int, warmup: int, dev):
    """Plain minibatch SGD with the same library: s = 1 outer steps (margins
    and update of one minibatch, no Gram), b and eta as the workload, the
    same number of inner steps as the timed CA-SGD run.  float32 storage is
    the baseline the method is compared with; bf16 storage separates the
    effect of the s-step formulation from that of the storage type."""
    import torch
    from communication_avoiding_mixed_amd import binding as B
    n_inner = wl.s * steps
    out = {}
    stream = torch.cuda.Stream()
    for storage in ("fp32", "bf16"):
        h = h_bf16 if storage == "bf16" else B.CASGD(torch.from_numpy(X).to(dev), torch.from_numpy(y).to(dev),
                                                     wl.loss, "fp32")
        w = torch.zeros(wl.n, device=dev)
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            h.train(1, wl.b, wl.eta, 7, 0, warmup * wl.s, w)
            start = torch.cuda.Event(enable_timing=True)
            stop = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            start.record(stream)
            h.train(1, wl.b, wl.eta, 7, warmup * wl.s, n_inner, w)
            stop.record(stream)
            torch.cuda.synchronize()
        ms = start.elapsed_time(stop)
        out[storage] = {"value": n_inner / (ms / 1e3), "unit": "inner SGD steps/s", "steps": n_inner,
                        "us_per_step": ms * 1e3 / n_inner}
        if h is not h_bf16:
            h.close()
            del h
            torch.cuda.empty_cache()
    return out


def copy_calibration(nbytes: int):
    """One plain device copy of nbytes (reads nbytes, writes nbytes), timed."""
    import torch
    n = nbytes // 4
    src = torch.ones(n, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    dst.copy_(src)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "seconds": el}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="epsilon")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sgd-baseline", action="store_true",
                    help="skip the plain minibatch SGD runs (s = 1) of the same library")
    ap.add_argument("--layout", type=int, default=0, choices=(0, 1, 2, 3),
                    help="placement of the recurrence's workgroups (CASGD_OPT_CHAIN_LAYOUT): "
                         "0 automatic, 1 spread over the XCDs, 2 on one XCD, one per CU, "
                         "3 on one XCD, up to two per CU")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only copy BYTES between two device buffers (a plain copy kernel of "
                         "known traffic, to scale the HBM byte counters) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the multi-GPU "
              "column-partitioned path is not built", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from communication_avoiding_mixed_amd import binding as B
    from communication_avoiding_mixed_amd import synth

    wl = synth.WORKLOADS[args.workload]
    t0 = time.time()
    X, y = synth.make_data(wl.name)
    print(f"[bench] data {wl.name} {X.shape} ready in {time.time() - t0:.0f}s", file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    h = B.CASGD(torch.from_numpy(X).to(dev), torch.from_numpy(y).to(dev), wl.loss, wl.storage)
    h.set_option(B.OPT_CHAIN_LAYOUT, args.layout)
    stream = torch.cuda.Stream()
    w = torch.zeros(wl.n, device=dev)
    # the zero fill above runs on the default stream; the timed stream waits for it
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        # warm-up
        h.train(wl.s, wl.b, wl.eta, 0, 0, args.warmup, w)
        stream.synchronize()
        # timed region: exactly K outer steps; every STAMP_EVERY-th launch of
        # each kernel is stamped by its own dispatch (start and end events)
        for kid in B.KERNEL_NAMES:
            h.timing(kid, reset=True)
        h.set_timing(True, every=STAMP_EVERY)
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        h.train(wl.s, wl.b, wl.eta, 0, args.warmup, args.steps, w)
        stop.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(stop)
        tot, pipe_cnt = h.timing(B.K_PIPE, reset=True)
        pipe_us = tot / max(pipe_cnt, 1) * 1e3
        h.set_timing(False)
        loss = h.loss_value(w)
        # the same K steps without the dispatch events, for comparison
        w2 = torch.zeros(wl.n, device=dev)
        h.train(wl.s, wl.b, wl.eta, 0, 0, args.warmup, w2)
        torch.cuda.synchronize()
        start.record(stream)
        h.train(wl.s, wl.b, wl.eta, 0, args.warmup, args.steps, w2)
        stop.record(stream)
        torch.cuda.synchronize()
        ms_plain = start.elapsed_time(stop)
        # the recipe's bf16-stored margins: the same K steps, unstamped
        h.set_option(B.OPT_MARGIN_BF16, 1)
        w4 = torch.zeros(wl.n, device=dev)
        h.train(wl.s, wl.b, wl.eta, 0, 0, args.warmup, w4)
        torch.cuda.synchronize()
        start.record(stream)
        h.train(wl.s, wl.b, wl.eta, 0, args.warmup, args.steps, w4)
        stop.record(stream)
        torch.cuda.synchronize()
        ms_mix = start.elapsed_time(stop)
        loss_mix = h.loss_value(w4)
        h.set_option(B.OPT_MARGIN_BF16, 0)
        # breakdown: the steps queued one by one as separate kernels
        for kid in B.KERNEL_NAMES:
            h.timing(kid, reset=True)
        h.set_timing(True)
        w3 = torch.zeros(wl.n, device=dev)
        n_break = min(args.steps, 100)
        for k in range(n_break):
            h.outer_step(wl.s, wl.b, wl.eta, B.step_seed(0, k), w3)
        per = {}
        for kid, kname in B.KERNEL_NAMES.items():
            tot, cnt = h.timing(kid, reset=True)
            per[kname] = (tot / max(cnt, 1)) * 1e3  # microseconds per launch
        h.set_timing(False)
    ms_per_step = ms / args.steps
    value = wl.s * args.steps / (ms / 1e3)
    sgd = None if args.no_sgd_baseline else sgd_baselines(h, X, y, wl, args.steps, args.warmup, dev)

    alg = algorithmic(wl)
    gram_tflops = alg["gram_flops"] / (per["gram"] * 1e-6) / 1e12
    step_bytes = alg["B_A"] + alg["B_B"] + alg["B_C"]
    kernels = {
        "pipe": {"us": pipe_us, "GB/s": step_bytes / (pipe_us * 1e-6) / 1e9,
                 "TFLOP/s": alg["gram_flops"] / (pipe_us * 1e-6) / 1e12},
        "gather": {"us": per["gather"], "GB/s": alg["gather_bytes"] / (per["gather"] * 1e-6) / 1e9},
        "gram": {"us": per["gram"], "TFLOP/s": gram_tflops,
                 "GB/s": alg["gram_bytes"] / (per["gram"] * 1e-6) / 1e9},
        "chain": {"us": per["chain"], "GB/s": alg["chain_bytes"] / (per["chain"] * 1e-6) / 1e9},
    }
    for name, k in kernels.items():
        if name == "gram" and wl.n >= 512:
            k["frac"] = k["TFLOP/s"] / PEAK_BF16_TFLOPS
        else:
            k["frac"] = k["GB/s"] / PEAK_HBM_GBS
    kernels["breakdown_steps"] = n_break
    t_roof = (max(alg["gram_flops"] / (PEAK_BF16_TFLOPS * 1e12), alg["B_A"] / (PEAK_HBM_GBS * 1e9))
              + alg["B_B"] / (PEAK_HBM_GBS * 1e9) + alg["B_C"] / (PEAK_HBM_GBS * 1e9))
    # The pipelined launch moves one step's algorithmic bytes (B_A + B_B + B_C)
    # and does one step's Gram flops; its own roofline time is bytes / HBM
    # (at epsilon 1.5 us) against flops / MFMA (0.8 us), so it is HBM-bound.
    pipe_gbs = kernels["pipe"]["GB/s"]
    roof = {"bound": "hbm", "achieved": pipe_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": pipe_gbs / PEAK_HBM_GBS, "traffic": pipe_traffic(wl.name),
            "kernel": "pipe_kernel", "algorithmic_bytes": step_bytes}

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "inner SGD steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_without_dispatch_events": ms_plain / args.steps,
        "stamped_launches": pipe_cnt,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "m": wl.m, "n": wl.n, "s": wl.s, "b": wl.b, "eta": wl.eta,
                   "loss": wl.loss, "storage": wl.storage, "accumulate": "f32",
                   "gram_bytes_full": B.gram_bytes(wl.s, wl.b, packed=False),
                   "gram_bytes_packed": B.gram_bytes(wl.s, wl.b, packed=True)},
        "roofline": roof,
        "step_roofline": {"t_roof_us": t_roof * 1e6, "t_meas_us": ms_per_step * 1e3,
                          "frac": t_roof * 1e6 / (ms_per_step * 1e3)},
        "kernels": kernels,
        "final_loss": loss,
        "margin_bf16": {"value": wl.s * args.steps / (ms_mix / 1e3), "unit": "inner SGD steps/s",
                        "ms_per_step": ms_mix / args.steps, "final_loss": loss_mix},
    }
    if sgd:
        out["sgd_baseline"] = {"kind": "minibatch SGD, s = 1, same library and b, eta", **sgd}
        out["speedup_vs_fp32_sgd"] = value / sgd["fp32"]["value"]
        out["speedup_vs_bf16_sgd"] = value / sgd["bf16"]["value"]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(X, y, wl, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
