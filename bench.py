#!/usr/bin/env python3
"""Throughput of one selective-batched Orca iteration on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one orca_iteration over the whole mixed batch: every layer's
LayerNorms, the four flattened Linear layers with their fused epilogues,
the K/V append, and split attention (initiation prompts and increment
tokens).  Inputs (weights, K/V caches, hidden rows) are seeded synthetic
draws already resident in HBM when the timed region starts.

Prints ONE JSON line: tokens processed per second (sum L per iteration over
the timed iterations), the roofline of the dominant kernel (the FFN1 GEMM:
MFMA-bound) and of decode attention (HBM-bound), both timed live with HIP
events on the stream they run on, and the CPU oracle timed on one layer of
the same batch on the host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published

DEFAULT_WORKLOAD = "gpt13b-40l"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD,
                   choices=["tiny-fp32", "h1024-2l", "gpt13b-40l", "gpt175b-8l",
                            "gpt13b-40l-decode64"])
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--kernel-reps", type=int, default=20)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only", choices=["iteration", "gemm", "decode", "copy"], default=None,
                   help="run one timed region only (for profiling)")
    p.add_argument("--summarize-traffic", metavar="DIR", default=None,
                   help="no GPU: turn the rocprofv3 FETCH_SIZE / WRITE_SIZE runs under DIR "
                        "(pmc_{gemm,decode,copy}_{FETCH_SIZE,WRITE_SIZE}/run_counter_collection"
                        ".csv) into profiles/hbm_traffic_<workload>.json")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def time_events(fn, reps, stream):
    """Average milliseconds of fn() over `reps` back-to-back calls, bracketed
    by HIP events recorded on `stream`."""
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(reps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / reps


def source_hash(files):
    import hashlib
    m = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "orca_selective_iteration_amd", "csrc", f), "rb") as fh:
            m.update(fh.read())
    return m.hexdigest()[:16]


def measured_mfma_util(workload):
    """MFMA utilisation (%) of the FFN1 launch from the committed rocprofv3
    MfmaUtil run; None when absent or the GEMM source changed since."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get("mfma_util_percent")
    if not rec or rec.get("source_hash") != source_hash(["gemm.hip", "device.h", "kernels.h"]):
        return None
    vals = list(rec.get("gemm", {}).values())
    return round(sum(vals) / len(vals), 2) if vals else None


def measured_traffic(workload, key, files):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs, scaled by the plain-copy calibration; None when no
    counters exist for this workload or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(key)
    if not rec or rec.get("source_hash") != source_hash(files):
        return None
    return {"bytes": int(rec["fetch_bytes"] + rec["write_bytes"]),
            "read_bytes": int(rec["fetch_bytes"]), "write_bytes": int(rec["write_bytes"]),
            "kernel": rec["kernel"]}


# kernels each timed region launches, as rocprofv3 names them
TRAFFIC_KERNELS = {"gemm": ("gemm_bf16", "gemm_w4", "gemm_ws", "gemm_f32", "skinny_reduce"),
                   "decode": ("attn_split", "attn_combine"), "copy": ("copyBuffer",)}


def _counter_means(path, prefixes):
    """Mean counter value (KiB) per dispatch of every kernel whose name holds
    one of `prefixes`, keyed by the kernel's short name."""
    import csv
    vals = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if not any(p in name for p in prefixes):
                continue
            short = name.split("(")[0].replace("void ", "")
            vals.setdefault(short, []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}


def summarize_traffic(src, workload):
    """HBM bytes per launch of the FFN1 GEMM and the decode attention from
    the counter runs, each counter scaled by what it reads for a plain copy
    of 1 GiB read + 1 GiB written (bench.py --only copy)."""
    def run(what, counter):
        return _counter_means(os.path.join(src, f"pmc_{what}_{counter}",
                                           "run_counter_collection.csv"), TRAFFIC_KERNELS[what])
    gib_kib = float(1 << 20)
    copy_f = max(run("copy", "FETCH_SIZE").values())
    copy_w = max(run("copy", "WRITE_SIZE").values())
    fs, ws = gib_kib / copy_f, gib_kib / copy_w
    out = {"workload": workload, "fetch_scale": fs, "write_scale": ws}
    for key, what, files in (("gemm_ffn1", "gemm", ["gemm.hip", "device.h", "kernels.h"]),
                             ("decode", "decode", ["attn.hip", "device.h", "kernels.h"])):
        f, w = run(what, "FETCH_SIZE"), run(what, "WRITE_SIZE")
        if not f:
            continue
        out[key] = {"kernel": " + ".join(sorted(f)), "source_hash": source_hash(files),
                    "fetch_kib": {k: round(v, 1) for k, v in f.items()},
                    "write_kib": {k: round(v, 1) for k, v in w.items()},
                    "fetch_bytes": sum(f.values()) * 1024 * fs,
                    "write_bytes": sum(w.values()) * 1024 * ws}
    # MFMA utilisation (rocprofv3's MfmaUtil: MFMA busy cycles over GPU-active
    # cycles times SIMDs), per GEMM kernel, for the FFN1 launch and the
    # GEMMs of a whole iteration
    util = {}
    for what in ("gemm", "iteration"):
        path = os.path.join(src, f"pmc_{what}_MfmaUtil", "run_counter_collection.csv")
        if os.path.exists(path):
            util[what] = {k: round(v, 2) for k, v in
                          _counter_means(path, TRAFFIC_KERNELS["gemm"]).items()}
    if util:
        out["mfma_util_percent"] = {"source_hash": source_hash(["gemm.hip", "device.h",
                                                                  "kernels.h"]), **util}
    dst = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")
    with open(dst, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def cpu_baseline(model, work, x_dev, layers_total, min_seconds=10.0):
    """The CPU oracle on the same batch (all rows, all requests), fp32 numpy
    on the host: layers 0, 1, ... in order (each layer's output feeds the
    next) until at least `min_seconds` of work or every layer is done;
    tokens/s extrapolated to the model's depth."""
    import numpy as np
    from oracle import model as om
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    x = x_dev.float().cpu().numpy()
    reqs, off = [], 0
    for q, kv in zip(work.q_len, work.kv_len):
        reqs.append(om.Req(off, q, kv))
        off += q
    spent, done = 0.0, 0
    while done < layers_total and spent < min_seconds:
        p = {k: v.float().cpu().numpy() for k, v in model.weights[done].items()}
        caches = [model.cache_rows(done, i, 0, work.kv_len[i]) for i in range(work.n_reqs)]
        t0 = time.perf_counter()
        x = om.selective_layer(p, reqs, x, caches, work.heads, work.eps)[0]
        spent += time.perf_counter() - t0
        done += 1
    per_layer = spent / done
    return {"value": work.rows / (per_layer * layers_total), "unit": "tokens/s",
            "cores": threads, "kind": "oracle",
            "sample": f"layers 0-{done - 1} of {layers_total} ({work.rows} rows, {work.n_reqs} "
                      f"requests), numpy fp32, {spent:.1f} s; extrapolated to {layers_total} "
                      f"layers"}


def main():
    args = parse()
    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic, args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the iteration has no multi-GPU path in this build)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from orca_selective_iteration_amd import lib as L
    from orca_selective_iteration_amd import synth
    from orca_selective_iteration_amd.runner import DeviceModel

    torch.cuda.set_device(0)
    if args.only == "copy":
        # reference for the profiler's byte counters: a plain device copy of
        # exactly 1 GiB read + 1 GiB written per launch
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.kernel_reps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.kernel_reps} x 1 GiB")
        return
    work = synth.workload(args.workload, args.seed)
    t0 = time.time()
    host = synth.host_inputs(work, args.seed) if work.layers * work.hidden <= 4096 else None
    model = DeviceModel(work, host=host, device="cuda", seed=args.seed, log=log)
    if host is not None:
        x = torch.from_numpy(host.x).to("cuda", model.tdt)
    else:
        x = synth.device_normal_(torch.empty((work.rows, work.hidden), dtype=model.tdt,
                                             device="cuda"), args.seed * 31 + 5)
    y = torch.empty_like(x)
    reqs = model.descriptors()
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    log(f"setup {time.time() - t0:.1f}s: {work.name} rows={work.rows} reqs={work.n_reqs} "
        f"kv_tokens={sum(work.kv_len)} pool_slots={model.cap}")

    def step():
        model.iteration(reqs, x, y, stream)

    res = {}
    ms = None
    if args.only in (None, "iteration"):
        for _ in range(args.warmup):
            step()
        ms = time_events(step, args.steps, stream)
        log(f"iteration: {ms:.3f} ms, {work.rows / ms * 1e3:.0f} tokens/s")

    H, F, M = work.hidden, work.ffn, work.rows
    bf16 = work.dtype == "bf16"
    # dominant kernel: the FFN1 GEMM (M = sum L, N = F, K = H) with GeLU epilogue
    gemm = None
    if args.only in (None, "gemm"):
        a = synth.device_normal_(torch.empty((M, H), dtype=model.tdt, device="cuda"), 11)
        f = torch.empty((M, F), dtype=model.tdt, device="cuda")
        w = model.weights[0]
        gws_bytes = L.orca_op_linear_workspace_bytes(model.odt, M, F, H)
        gws = torch.empty(max(gws_bytes, 1), dtype=torch.uint8, device="cuda")

        def ffn1():
            L.orca_op_linear(model.odt, L.ORCA_EPI_BIAS_GELU, a, w["w_1"], w["b_1"], f, M, F, H,
                             gws, gws_bytes, stream=stream)
        for _ in range(3):
            ffn1()
        gms = time_events(ffn1, args.kernel_reps, stream)
        flops = 2.0 * M * F * H
        esz = 2 if bf16 else 4
        # algorithmic bytes: W, A and the output once each
        alg_bytes = esz * (F * H + M * H + M * F)
        peak = PEAK_BF16_TFLOPS if bf16 else PEAK_FP32_TFLOPS
        ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)            # FLOP per byte
        split = gws_bytes > 0
        tr = measured_traffic(work.name, "gemm_ffn1", ["gemm.hip", "device.h", "kernels.h"])
        if tr:
            kname = tr["kernel"]
        elif bf16:
            # the launch planner's choice: split-K for few rows, otherwise
            # the four-wave 256 x 256 or 256 x 192 tile
            kname = ("gemm_bf16_kernel<gelu> split-K + skinny_reduce_kernel<gelu>" if split
                     else "gemm_w4_kernel<gelu>")
        else:
            kname = "gemm_f32_kernel<gelu>"
        common = {"kernel": kname + " (FFN1)", "shape": [M, F, H],
                  "mfma_util_percent_counter": measured_mfma_util(work.name),
                  "traffic": tr["bytes"] if tr else None,
                  "traffic_unit": "bytes per launch (HBM read + write, rocprofv3 counters)",
                  "algorithmic_flops": int(flops), "algorithmic_bytes": int(alg_bytes),
                  "arithmetic_intensity": round(flops / alg_bytes, 1),
                  "ms_per_launch": round(gms, 4)}
        tflops = flops / (gms * 1e-3) / 1e12
        if flops / alg_bytes >= ridge:
            gemm = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(tflops / peak, 4), **common}
        else:
            # few rows: the weights stream once and the MFMAs idle
            gbs = alg_bytes / (gms * 1e-3) / 1e9
            gemm = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                    "achieved_tflops": round(tflops, 2), **common}
        log(f"FFN1 GEMM {M}x{F}x{H}: {gms:.3f} ms, {tflops:.1f} TFLOP/s, "
            f"{alg_bytes / (gms * 1e-3) / 1e9:.0f} GB/s algorithmic")
        del a, f

    decode = None
    incr = [i for i in range(work.n_reqs) if work.kv_len[i] > 0]
    if args.only in (None, "decode") and incr:
        d_reqs = L.req_array(model.descriptors(reqs=incr))
        n = len(incr)
        q = synth.device_normal_(torch.empty((n, H), dtype=model.tdt, device="cuda"), 13)
        o = torch.empty_like(q)

        def dec():
            L.orca_op_attention(model.ctx, 0, d_reqs, q, o, model.ws, model.ws_bytes, stream)
        for _ in range(3):
            dec()
        dms = time_events(dec, args.kernel_reps, stream)
        esz = 2 if bf16 else 4
        nbytes = sum(2 * (work.kv_len[i] + 1) * H * esz for i in incr)
        gbs = nbytes / (dms * 1e-3) / 1e9
        tr = measured_traffic(work.name, "decode", ["attn.hip", "device.h", "kernels.h"])
        decode = {"bound": "hbm", "kernel": "attn_split_kernel + attn_combine_kernel "
                  "(increment rows, one layer)", "achieved": round(gbs, 1),
                  "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                  "traffic": tr["bytes"] if tr else None, "ms_per_launch": round(dms, 4),
                  "algorithmic_bytes": nbytes}
        log(f"decode attention ({n} requests, one layer): {dms:.3f} ms, {gbs:.0f} GB/s")

    cpu = None
    if args.only is None and not args.no_cpu_baseline:
        t1 = time.time()
        cpu = cpu_baseline(model, work, x, work.layers)
        log(f"cpu baseline: {cpu['value']:.1f} tokens/s ({time.time() - t1:.1f}s)")

    model.close()
    if ms is None:
        return
    value = work.rows / (ms * 1e-3)
    line = {
        "metric": "processed tokens/s per mixed iteration (1 GPU)",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic (seeded random-init weights, K/V caches and hidden rows)",
        "config": {"workload": work.name, "layers": work.layers, "hidden": H,
                   "heads": work.heads, "ffn": F, "sum_L": M, "requests": work.n_reqs,
                   "initiation_requests": sum(1 for v in work.kv_len if v == 0),
                   "increment_requests": len(incr), "cached_kv_tokens": sum(work.kv_len),
                   "parallelism": "single GPU"},
        "roofline": gemm,
        "decode_attention": decode,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
