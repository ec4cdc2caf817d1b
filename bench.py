"""Throughput of mixed-precision CA-SGD outer iterations on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload epsilon]

A step is one outer iteration (s inner SGD steps): sample + gather + margins,
strictly-lower Gram on bf16 MFMA, inner recurrence, weight update.  The data
(seeded, synthetic, epsilon-shaped by default) is resident in HBM before the
timed region.  casgd_train runs all K timed steps as one persistent launch
(the recurrence's workgroups, margin workgroups and Gram workgroups resident
together; where that launch does not fit, one pipelined launch per step);
that launch is the dominant kernel, timed by HIP events its own dispatch
stamps, on the library's stream, over the timed region.  A second pass queues
the same steps one by one (separate gather, Gram and recurrence kernels) for
a per-kernel breakdown, including the Gram's MFMA throughput.  Every other
synthetic workload is then run the same way (the `workloads` field), the
achievable HBM and MFMA rates are measured with calibration kernels, and the
CPU oracle is timed on the host on a bounded sample, with one BLAS thread and
with every usable core.  Prints one JSON line.
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


CSRC = os.path.join(ROOT, "communication_avoiding_mixed_amd", "csrc")
# every source the persistent training kernel is compiled from
TRAIN_SOURCES = ("casgd_train.h", "casgd_step.h", "casgd_chain.h", "casgd_gram.h", "casgd_gather.h",
                 "casgd_device.h", "casgd_internal.h", "k_step.hip", "k_step_1x1.hip", "k_step_2x1.hip",
                 "k_step_2x2.hip", "k_step_4x2.hip", "k_step_4x4.hip")
PMC_SUMMARY = os.path.join(ROOT, "profiles", "train_kernel-epsilon-pmc.md")


def train_source_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in TRAIN_SOURCES:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()


def train_traffic(workload: str, steps_per_launch: int):
    """Scaled HBM bytes per persistent training launch of steps_per_launch
    steps, from the committed rocprofv3 --pmc summary (bytes per step of a
    measured launch), or None if there is none for this workload or the
    kernel's sources have changed since it was taken."""
    if workload != "epsilon" or not os.path.exists(PMC_SUMMARY):
        return None
    vals = {}
    for line in open(PMC_SUMMARY):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip().strip("-* `")] = v.strip().strip("`")
    try:
        if vals["kernel_source_sha256"] != train_source_sha256():
            return None
        per_launch = (float(vals["fetch_kib_per_dispatch"]) * 1024 * float(vals["fetch_scale"])
                      + float(vals["write_kib_per_dispatch"]) * 1024 * float(vals["write_scale"]))
        return per_launch / float(vals["steps_per_dispatch"]) * steps_per_launch
    except (KeyError, ValueError, ZeroDivisionError):
        return None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _time_oracle(X, y, wl, budget_s: float):
    import numpy as np
    from oracle import casgd_oracle as O
    w = np.zeros(wl.n)
    t0 = time.perf_counter()
    k = 0
    while True:
        w = O.outer_step(X, y, w, wl.s, wl.b, wl.eta, O.step_seed(0, k), wl.loss)["w"]
        k += 1
        el = time.perf_counter() - t0
        if (el >= budget_s and k >= 2) or k >= wl.outer:
            return k, el


def cpu_baseline(X, y, wl, budget_s: float):
    """The oracle's outer step, as it stands, on the host: inner steps/s, with
    every usable core (the value) and with one BLAS thread, each on about
    budget_s / 2 seconds of the same run from w = 0."""
    from threadpoolctl import threadpool_info, threadpool_limits
    cores = len(os.sched_getaffinity(0))
    runs = {}
    for label, limit in (("one_thread", 1), ("all_cores", cores)):
        with threadpool_limits(limits=limit):
            blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
            k, el = _time_oracle(X, y, wl, budget_s / 2)
        runs[label] = {"value": wl.s * k / el, "unit": "inner SGD steps/s", "blas_threads": int(blas),
                       "sample": f"first {k} outer steps (s={wl.s}, b={wl.b}) of the {wl.name} run from w=0, "
                                 f"{el:.1f} s"}
    return {
        "value": runs["all_cores"]["value"],
        "unit": "inner SGD steps/s",
        "cores": cores,
        "blas_threads": runs["all_cores"]["blas_threads"],
        "kind": "oracle",
        "sample": runs["all_cores"]["sample"] + ", float64 NumPy, BLAS on every usable core",
        "one_thread": runs["one_thread"],
        "cpu_model": cpu_model(),
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
                        "us_per_step": ms * 1e3 / n_inner, "final_loss": h.loss_value(w)}
        if h is not h_bf16:
            h.close()
            del h
            torch.cuda.empty_cache()
    return out


def copy_calibration(nbytes: int):
    """One calibration copy of nbytes (reads nbytes, writes nbytes), timed."""
    import torch
    from communication_avoiding_mixed_amd import binding as B
    n = nbytes // 4
    src = torch.ones(n, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    B.peak_copy(src, dst)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "seconds": el}), flush=True)


def measure_peaks():
    """Achievable rates on this GPU: the calibration copy kernel over 1 GiB
    (read + written bytes per second) and the bf16 MFMA loop (flops per
    second), each the best of several timed launches."""
    import torch
    from communication_avoiding_mixed_amd import binding as B
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def best(fn, reps):
        fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(reps):
            ev[0].record(stream)
            fn()
            ev[1].record(stream)
            torch.cuda.synchronize()
            t.append(ev[0].elapsed_time(ev[1]) * 1e-3)
        return min(t)

    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, device="cuda:0")
    dst = torch.empty_like(src)
    t_copy = best(lambda: B.peak_copy(src, dst), 10)
    ok = bool(torch.equal(src, dst))
    del dst
    rwgs = torch.cuda.get_device_properties(0).multi_processor_count * 4
    rout = torch.zeros(rwgs * 8, device="cuda:0")
    t_read = best(lambda: B.peak_read(src, rout, rwgs), 10)
    ok_read = bool(torch.all(rout == 1.0))
    del src, rout
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs, iters = 2 * cus, 20000
    out = torch.empty(wgs * 256, device="cuda:0")
    flops = wgs * 4 * 4 * iters * 2 * 32 * 32 * 16
    t_mfma = best(lambda: B.peak_mfma(out, wgs, iters), 5)
    del out
    torch.cuda.empty_cache()
    return {
        "hbm_copy_GB/s": 2 * nbytes / t_copy / 1e9,
        "hbm_copy_frac_of_datasheet": 2 * nbytes / t_copy / 1e9 / PEAK_HBM_GBS,
        "copy": f"calibration copy kernel, 1 GiB read + 1 GiB written, best of 10, result checked: {ok}",
        "hbm_read_GB/s": nbytes / t_read / 1e9,
        "hbm_read_frac_of_datasheet": nbytes / t_read / 1e9 / PEAK_HBM_GBS,
        "read": f"read calibration kernel (direct-to-LDS, {rwgs} workgroups), 1 GiB, best of 10, "
                f"data checked: {ok_read}",
        "mfma_bf16_TFLOP/s": flops / t_mfma / 1e12,
        "mfma_bf16_frac_of_datasheet": flops / t_mfma / 1e12 / PEAK_BF16_TFLOPS,
        "mfma": f"{wgs} workgroups x 4 waves x 4 independent chains x {iters} "
                "v_mfma_f32_32x32x16_bf16, best of 5",
    }


def run_workload(wl, X, y, args, dev, detailed: bool):
    """Time K outer steps of casgd_train on one workload (warm-up first),
    with the dominant launch timed by its own dispatch stamps, then a
    per-kernel breakdown of steps queued one by one.  detailed adds an
    unstamped rerun, the bf16-stored-margin variant and the plain SGD runs."""
    import torch
    from communication_avoiding_mixed_amd import binding as B

    K, W = args.steps, args.warmup
    h = B.CASGD(torch.from_numpy(X).to(dev), torch.from_numpy(y).to(dev), wl.loss, wl.storage)
    h.set_option(B.OPT_CHAIN_LAYOUT, args.layout)
    stream = torch.cuda.Stream()
    w = torch.zeros(wl.n, device=dev)
    # the zero fill above runs on the default stream; the timed stream waits for it
    stream.wait_stream(torch.cuda.current_stream())
    res = {}
    with torch.cuda.stream(stream):
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)

        def timed_train(wv, stamp):
            h.train(wl.s, wl.b, wl.eta, 0, 0, W, wv)
            stream.synchronize()
            if stamp:
                for kid in B.KERNEL_NAMES:
                    h.timing(kid, reset=True)
                h.set_timing(True, every=STAMP_EVERY)
            torch.cuda.synchronize()
            start.record(stream)
            h.train(wl.s, wl.b, wl.eta, 0, W, K, wv)
            stop.record(stream)
            torch.cuda.synchronize()
            return start.elapsed_time(stop)

        ms = timed_train(w, True)
        tr_ms, tr_cnt = h.timing(B.K_TRAIN, reset=True)
        pp_ms, pp_cnt = h.timing(B.K_PIPE, reset=True)
        h.set_timing(False)
        if tr_cnt:
            launch = {"kernel": "train_kernel", "form": "persistent", "steps_per_launch": K,
                      "us_per_launch": tr_ms / tr_cnt * 1e3, "stamped_launches": tr_cnt}
        else:
            launch = {"kernel": "pipe_kernel", "form": "one pipelined launch per step", "steps_per_launch": 1,
                      "us_per_launch": pp_ms / max(pp_cnt, 1) * 1e3, "stamped_launches": pp_cnt}
        res["loss"] = h.loss_value(w)
        if detailed:
            res["ms_plain"] = timed_train(torch.zeros(wl.n, device=dev), False)
            # the recipe's bf16-stored margins: the same K steps, unstamped
            h.set_option(B.OPT_MARGIN_BF16, 1)
            w4 = torch.zeros(wl.n, device=dev)
            res["ms_mix"] = timed_train(w4, False)
            res["loss_mix"] = h.loss_value(w4)
            h.set_option(B.OPT_MARGIN_BF16, 0)
        # breakdown: the steps queued one by one as separate kernels
        for kid in B.KERNEL_NAMES:
            h.timing(kid, reset=True)
        h.set_timing(True)
        w3 = torch.zeros(wl.n, device=dev)
        n_break = min(K, 50)
        for k in range(n_break):
            h.outer_step(wl.s, wl.b, wl.eta, B.step_seed(0, k), w3)
        per = {}
        for kid, kname in B.KERNEL_NAMES.items():
            tot, cnt = h.timing(kid, reset=True)
            per[kname] = (tot / cnt) * 1e3 if cnt else None  # microseconds per launch
        h.set_timing(False)
    res.update(ms=ms, launch=launch, per=per, n_break=n_break, h=h)
    return res


def precision_variants(h_main, X, y, wl, args, dev):
    """The precision choices beyond the recipe, timed like the main run (K
    steps after W warm-up steps, unstamped): fp16 and fp8 storage of X (their
    rows go through the gather kernel each step) and G rounded once to bf16
    (on the main handle).  Final loss of each, for the gap to float32 SGD."""
    import torch
    from communication_avoiding_mixed_amd import binding as B
    K, W = args.steps, args.warmup
    out = {}
    stream = torch.cuda.Stream()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)

    def timed(h):
        w = torch.zeros(wl.n, device=dev)
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            h.train(wl.s, wl.b, wl.eta, 0, 0, W, w)
            torch.cuda.synchronize()
            start.record(stream)
            h.train(wl.s, wl.b, wl.eta, 0, W, K, w)
            stop.record(stream)
            torch.cuda.synchronize()
            loss = h.loss_value(w)
        ms = start.elapsed_time(stop)
        return {"value": wl.s * K / (ms / 1e3), "unit": "inner SGD steps/s", "ms_per_step": ms / K,
                "final_loss": loss}

    for storage in ("fp16", "fp8"):
        h = B.CASGD(torch.from_numpy(X).to(dev), torch.from_numpy(y).to(dev), wl.loss, storage)
        out[f"storage_{storage}"] = timed(h)
        if storage == "fp8":
            out["storage_fp8"]["scale_exponent"] = h.fp8_exponent
        h.close()
        torch.cuda.empty_cache()
    h_main.set_option(B.OPT_GRAM_BF16, 1)
    out["gram_bf16"] = timed(h_main)
    out["gram_bf16"]["gram_bytes_packed"] = B.gram_bytes(wl.s, wl.b, packed=True) // 2
    h_main.set_option(B.OPT_GRAM_BF16, 0)
    return out


def summarize(wl, r, K, peaks):
    """Throughput, roofline fractions and the per-kernel breakdown of one run."""
    alg = algorithmic(wl)
    step_bytes = alg["B_A"] + alg["B_B"] + alg["B_C"]
    ms_per_step = r["ms"] / K
    t_roof = (max(alg["gram_flops"] / (PEAK_BF16_TFLOPS * 1e12), alg["B_A"] / (PEAK_HBM_GBS * 1e9))
              + alg["B_B"] / (PEAK_HBM_GBS * 1e9) + alg["B_C"] / (PEAK_HBM_GBS * 1e9))
    L = r["launch"]
    launch_gbs = step_bytes * L["steps_per_launch"] / (L["us_per_launch"] * 1e-6) / 1e9
    per = r["per"]
    out = {
        "workload": wl.name, "m": wl.m, "n": wl.n, "s": wl.s, "b": wl.b, "eta": wl.eta, "loss": wl.loss,
        "storage": wl.storage, "steps": K,
        "value": wl.s * K / (r["ms"] / 1e3), "unit": "inner SGD steps/s",
        "us_per_step": ms_per_step * 1e3,
        "t_roof_us": t_roof * 1e6,
        "step_roofline_frac": t_roof / (ms_per_step * 1e-3),
        "final_loss": r["loss"],
        "dominant": {**L, "us_per_step": L["us_per_launch"] / L["steps_per_launch"],
                     "algorithmic_bytes_per_step": step_bytes, "GB/s": launch_gbs,
                     "hbm_frac": launch_gbs / PEAK_HBM_GBS,
                     "hbm_frac_of_measured_copy": launch_gbs / peaks["hbm_copy_GB/s"]},
    }
    if per.get("gram"):
        gt = alg["gram_flops"] / (per["gram"] * 1e-6) / 1e12
        gb = alg["gram_bytes"] / (per["gram"] * 1e-6) / 1e9
        out["gram"] = {"us": per["gram"], "TFLOP/s": gt, "mfma_frac": gt / PEAK_BF16_TFLOPS,
                       "mfma_frac_of_measured": gt / peaks["mfma_bf16_TFLOP/s"],
                       "GB/s": gb, "hbm_frac": gb / PEAK_HBM_GBS,
                       "bound": "mfma" if wl.n >= 512 else "hbm"}
    bk = {"steps": r["n_break"]}
    for name, key in (("gather", "gather_bytes"), ("chain", "chain_bytes")):
        if per.get(name):
            gb = alg[key] / (per[name] * 1e-6) / 1e9
            bk[name] = {"us": per[name], "GB/s": gb, "hbm_frac": gb / PEAK_HBM_GBS}
    out["breakdown"] = bk
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="epsilon")
    ap.add_argument("--others", default="all",
                    help="comma-separated further workloads for the `workloads` field, 'all' or 'none'")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sgd-baseline", action="store_true",
                    help="skip the plain minibatch SGD runs (s = 1) of the same library")
    ap.add_argument("--no-peaks", action="store_true", help="skip the calibration kernels")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the fp16 / fp8 storage and bf16-Gram runs of the main workload")
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

    import torch

    from communication_avoiding_mixed_amd import binding as B
    from communication_avoiding_mixed_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.no_peaks:
        peaks = {"hbm_copy_GB/s": PEAK_HBM_GBS, "mfma_bf16_TFLOP/s": PEAK_BF16_TFLOPS,
                 "note": "not measured (--no-peaks): datasheet values"}
    else:
        peaks = measure_peaks()
        print(f"[bench] peaks {json.dumps(peaks)}", file=sys.stderr, flush=True)

    wl = synth.WORKLOADS[args.workload]
    t0 = time.time()
    X, y = synth.make_data(wl.name)
    print(f"[bench] data {wl.name} {X.shape} ready in {time.time() - t0:.0f}s", file=sys.stderr, flush=True)
    r = run_workload(wl, X, y, args, dev, detailed=True)
    main_sum = summarize(wl, r, args.steps, peaks)
    print(f"[bench] {wl.name}: {main_sum['us_per_step']:.2f} us/step", file=sys.stderr, flush=True)
    sgd = None if args.no_sgd_baseline else sgd_baselines(r["h"], X, y, wl, args.steps, args.warmup, dev)
    variants = None if args.no_variants else precision_variants(r["h"], X, y, wl, args, dev)
    r["h"].close()
    del r["h"]
    torch.cuda.empty_cache()
    cpu = None if args.no_cpu_baseline else cpu_baseline(X, y, wl, args.cpu_budget)
    del X, y

    if args.others == "all":
        others = [n for n in synth.WORKLOADS if n != wl.name]
    elif args.others == "none":
        others = []
    else:
        others = [n for n in args.others.split(",") if n and n != wl.name]
    workloads = [main_sum]
    for name in others:
        owl = synth.WORKLOADS[name]
        t0 = time.time()
        Xo, yo = synth.make_data(name)
        ro = run_workload(owl, Xo, yo, args, dev, detailed=False)
        ro["h"].close()
        del ro["h"], Xo, yo
        torch.cuda.empty_cache()
        so = summarize(owl, ro, args.steps, peaks)
        workloads.append(so)
        print(f"[bench] {name}: {so['us_per_step']:.2f} us/step ({time.time() - t0:.0f}s with data)",
              file=sys.stderr, flush=True)

    K = args.steps
    D = main_sum["dominant"]
    step_bytes = D["algorithmic_bytes_per_step"]
    roof = {"bound": "hbm", "achieved": D["GB/s"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": D["GB/s"] / PEAK_HBM_GBS,
            "traffic": train_traffic(wl.name, K) if D["kernel"] == "train_kernel" else None,
            "kernel": D["kernel"], "algorithmic_bytes": step_bytes * D["steps_per_launch"],
            "steps_per_launch": D["steps_per_launch"], "us_per_launch": D["us_per_launch"],
            "frac_of_measured_copy": D["hbm_frac_of_measured_copy"]}
    out = {
        "metric": METRIC,
        "value": main_sum["value"],
        "unit": "inner SGD steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": r["ms"] / K,
        "ms_per_step_without_dispatch_events": r["ms_plain"] / K,
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
        "step_roofline": {"t_roof_us": main_sum["t_roof_us"], "t_meas_us": main_sum["us_per_step"],
                          "frac": main_sum["step_roofline_frac"]},
        "gram": main_sum.get("gram"),
        "kernels": main_sum["breakdown"],
        "measured_peaks": peaks,
        "final_loss": r["loss"],
        "margin_bf16": {"value": wl.s * K / (r["ms_mix"] / 1e3), "unit": "inner SGD steps/s",
                        "ms_per_step": r["ms_mix"] / K, "final_loss": r["loss_mix"]},
        "workloads": workloads,
    }
    if variants:
        ref = sgd["fp32"]["final_loss"] if sgd else None
        for v in variants.values():
            v["gap_vs_fp32_sgd"] = abs(v["final_loss"] - ref) / abs(ref) if ref else None
        out["precision_variants"] = variants
    if sgd:
        out["sgd_baseline"] = {"kind": "minibatch SGD, s = 1, same library and b, eta", **sgd}
        out["speedup_vs_fp32_sgd"] = main_sum["value"] / sgd["fp32"]["value"]
        out["final_loss_gap_vs_fp32_sgd"] = abs(r["loss"] - sgd["fp32"]["final_loss"]) / abs(sgd["fp32"]["final_loss"])
        out["speedup_vs_bf16_sgd"] = main_sum["value"] / sgd["bf16"]["value"]
    if cpu:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
