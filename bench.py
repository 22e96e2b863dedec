#!/usr/bin/env python3
"""Throughput of one selective-batched Orca iteration on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--extra a,b]

A step is one orca_iteration over the whole mixed batch: every layer's
LayerNorms, the four flattened Linear layers with their fused epilogues,
the K/V append, and split attention (initiation prompts and increment
tokens).  Inputs (weights, K/V caches, hidden rows) are seeded synthetic
draws already resident in HBM when the timed region starts.

The headline workload is the largest one that fits one GPU: eight layers of
the GPT-3 175B layer shape over a mixed batch of 256 requests (8 prompts,
248 increments).  The 13B-shaped 40-layer batch and the two-layer H1024
batch (whose iteration time is the per-iteration latency at low load) run
after it in the same process and are reported under "also".

Prints ONE JSON line: tokens processed per second (sum L per iteration over
the timed iterations); the roofline of the flattened GEMMs, timed live with
timing events the engine records on its stream around each Linear step of
every layer inside real iterations; decode attention's HBM rate (HIP events
around the increment rows' attention launch); and the CPU oracle timed on a
sample of the same batch on the host's cores.
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

DEFAULT_WORKLOAD = "gpt175b-8l"
DEFAULT_EXTRA = "gpt13b-40l,h1024-2l"
WORKLOADS = ["tiny-fp32", "h1024-2l", "gpt13b-40l", "gpt175b-8l", "gpt13b-40l-decode64"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=WORKLOADS)
    p.add_argument("--extra", default=None,
                   help="comma-separated workloads timed after the headline one "
                        f"(default with the default workload: {DEFAULT_EXTRA}; 'none' for none)")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--kernel-reps", type=int, default=20)
    p.add_argument("--step-reps", type=int, default=3,
                   help="iterations per Linear step timed in-iteration")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only", choices=["iteration", "gemm", "decode", "copy"], default=None,
                   help="run one timed region only (for profiling)")
    p.add_argument("--summarize-traffic", metavar="DIR", default=None,
                   help="no GPU: turn the rocprofv3 FETCH_SIZE / WRITE_SIZE runs under DIR "
                        "(pmc_{iteration,decode,copy}_{FETCH_SIZE,WRITE_SIZE}/"
                        "run_counter_collection.csv) into profiles/hbm_traffic_<workload>.json")
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


GEMM_FILES = ["gemm.hip", "device.h", "kernels.h"]
ATTN_FILES = ["attn.hip", "device.h", "kernels.h"]


def committed_counters(workload):
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        return json.load(f)


def measured_traffic(workload, key, files):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs, scaled by the plain-copy calibration; None when no
    counters exist for this workload or the kernel source changed since."""
    rec = committed_counters(workload).get(key)
    if not rec or rec.get("source_hash") != source_hash(files):
        return None
    return {"bytes": int(rec["fetch_bytes"] + rec["write_bytes"]),
            "read_bytes": int(rec["fetch_bytes"]), "write_bytes": int(rec["write_bytes"])}


def measured_mfma_util(workload):
    """MFMA utilisation (%) of the GEMM launches of an iteration from the
    committed rocprofv3 MfmaUtil run; None when absent or stale."""
    rec = committed_counters(workload).get("mfma_util_percent")
    if not rec or rec.get("source_hash") != source_hash(GEMM_FILES):
        return None
    vals = rec.get("iteration", {})
    return {k: v for k, v in vals.items()} or None


# kernels each timed region launches, as rocprofv3 names them (from_f32 runs
# once per iteration: it counts the iterations of a profiled run)
TRAFFIC_KERNELS = {"iteration": ("gemm_bf16", "gemm_w4", "gemm_d4", "gemm_ws", "skinny_reduce",
                                 "tail_reduce"),
                   "decode": ("attn_split", "attn_combine"), "copy": ("copyBuffer",),
                   "marker": ("from_f32",)}


def _counter_sums(path, prefixes):
    """(sum of the counter over the dispatches, dispatch count) of every
    kernel whose name holds one of `prefixes`, keyed by the short name."""
    import csv
    vals = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if not any(p in name for p in prefixes):
                continue
            short = name.split("(")[0].replace("void ", "")
            s, n = vals.get(short, (0.0, 0))
            vals[short] = (s + float(r["Counter_Value"]), n + 1)
    return vals


XCDS, SIMDS = 8, 1024
MFMA_FLOP_PER_SIMD_CLOCK = 1024   # v_mfma_f32_32x32x16_bf16: 32*32*16*2 FLOP in 32 cycles


def clock_counters(path):
    """Shader clock and MFMA busy fraction of each GEMM kernel from one
    rocprofv3 pass of GRBM_GUI_ACTIVE and SQ_VALU_MFMA_BUSY_CYCLES: rocprofv3
    sums GRBM_GUI_ACTIVE over the XCDs, so the clock is that sum / XCDs / the
    dispatch's duration.  Kernels averaging under 0.2 ms are left out (the
    counter window outlasts the dispatch by a few microseconds)."""
    import csv
    if not os.path.exists(path):
        return {}
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if not any(p in name for p in TRAFFIC_KERNELS["iteration"]):
                continue
            d = per.setdefault((r["Dispatch_Id"], name.split("(")[0].replace("void ", "")), {})
            d[r["Counter_Name"]] = float(r["Counter_Value"])
            d["dur"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    agg = {}
    for (_, k), v in per.items():
        a = agg.setdefault(k, [0.0, 0.0, 0.0, 0])
        a[0] += v.get("GRBM_GUI_ACTIVE", 0.0)
        a[1] += v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        a[2] += v["dur"]
        a[3] += 1
    out = {}
    for k, (gui, mfma, dur, n) in agg.items():
        if n == 0 or dur / n < 2e-4 or gui <= 0:
            continue
        ghz = gui / XCDS / dur / 1e9
        out[k] = {"clock_ghz": round(ghz, 3),
                  "mfma_busy_percent": round(100 * mfma / (gui / XCDS * SIMDS), 1),
                  "mfma_ceiling_tflops_at_clock":
                      round(ghz * 1e9 * SIMDS * MFMA_FLOP_PER_SIMD_CLOCK / 1e12, 1)}
    return out


def measured_clock(workload):
    """The committed clock pass of the GEMM kernels; None when absent or
    stale."""
    rec = committed_counters(workload).get("clock")
    if not rec or rec.get("source_hash") != source_hash(GEMM_FILES):
        return None
    return rec.get("iteration") or None


def summarize_traffic(src, workload):
    """HBM bytes per launch of the iteration's GEMM launches and of the
    decode attention from the counter runs, each counter scaled by what it
    reads for a plain copy of 1 GiB read + 1 GiB written (bench.py --only
    copy)."""
    def run(what, counter):
        return _counter_sums(os.path.join(src, f"pmc_{what}_{counter}",
                                          "run_counter_collection.csv"), TRAFFIC_KERNELS[what])
    gib_kib = float(1 << 20)
    cf = run("copy", "FETCH_SIZE")
    cw = run("copy", "WRITE_SIZE")
    copy_f = max(s / n for s, n in cf.values())
    copy_w = max(s / n for s, n in cw.values())
    fs, ws = gib_kib / copy_f, gib_kib / copy_w
    out = {"workload": workload, "fetch_scale": fs, "write_scale": ws}
    from orca_selective_iteration_amd import synth
    layers = synth.workload(workload).layers
    for key, what, files in (("gemm", "iteration", GEMM_FILES), ("decode", "decode", ATTN_FILES)):
        f, w = run(what, "FETCH_SIZE"), run(what, "WRITE_SIZE")
        if not f:
            continue
        if key == "gemm":
            # per Linear step (QKV, output projection, FFN1 or FFN2 of one
            # layer, with the split kernels and reduces it launches): every
            # GEMM dispatch of the run over 4 x layers x iterations
            iters = sum(n for _, n in _counter_sums(
                os.path.join(src, f"pmc_{what}_FETCH_SIZE", "run_counter_collection.csv"),
                TRAFFIC_KERNELS["marker"]).values())
            units = 4 * layers * max(iters, 1)
            unit = "Linear step"
        else:
            # per decode-attention call: one attn_split launch each
            units = sum(n for k, (_, n) in f.items() if "attn_split" in k)
            unit = "call"
        out[key] = {"kernels": sorted(f), "source_hash": source_hash(files),
                    "unit": unit, "units": units,
                    "fetch_kib_per_dispatch": {k: round(s / n, 1) for k, (s, n) in f.items()},
                    "write_kib_per_dispatch": {k: round(s / n, 1) for k, (s, n) in w.items()},
                    "fetch_bytes": sum(s for s, _ in f.values()) * 1024 * fs / units,
                    "write_bytes": sum(s for s, _ in w.values()) * 1024 * ws / units}
    util = {}
    path = os.path.join(src, "pmc_iteration_MfmaUtil", "run_counter_collection.csv")
    if os.path.exists(path):
        util = {k: round(s / n, 2) for k, (s, n) in
                _counter_sums(path, TRAFFIC_KERNELS["iteration"]).items()}
    if util:
        out["mfma_util_percent"] = {"source_hash": source_hash(GEMM_FILES), "iteration": util}
    clock = clock_counters(os.path.join(src, "pmc_iteration_clock", "run_counter_collection.csv"))
    if clock:
        out["clock"] = {"source_hash": source_hash(GEMM_FILES), "iteration": clock}
    dst = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")
    with open(dst, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def cpu_baseline(model, work, prompt_rows=4096, increments=32):
    """The CPU oracle (fp32 numpy on the host's cores) on a sample of the
    same batch: layer 0 over the batch's prompts (up to `prompt_rows` rows)
    and its first `increments` increment requests with their real caches;
    tokens/s = sample rows / that layer's time / the model's depth."""
    import torch
    from oracle import model as om
    from orca_selective_iteration_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    incr = [i for i in range(work.n_reqs) if work.kv_len[i] > 0]
    pick, rows = [], 0
    for i in range(work.n_reqs):
        if work.kv_len[i] == 0 and rows + work.q_len[i] <= prompt_rows:
            pick.append(i)
            rows += work.q_len[i]
    n_prompts = len(pick)
    pick += incr[:increments]
    rows += len(incr[:increments])
    pick.sort()
    x = synth.device_normal_(torch.empty((rows, work.hidden), dtype=model.tdt, device="cuda"), 91)
    xh = x.float().cpu().numpy()
    reqs, off = [], 0
    for i in pick:
        reqs.append(om.Req(off, work.q_len[i], work.kv_len[i]))
        off += work.q_len[i]
    p = {k: v.float().cpu().numpy() for k, v in model.weights[0].items()}
    caches = [model.cache_rows(0, i, 0, work.kv_len[i]) for i in pick]
    t0 = time.perf_counter()
    om.selective_layer(p, reqs, xh, caches, work.heads, work.eps)
    spent = time.perf_counter() - t0
    return {"value": rows / (spent * work.layers), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"layer 0 of {work.layers} over {len(pick)} of the batch's {work.n_reqs} "
                      f"requests ({n_prompts} prompts, {len(pick) - n_prompts} increments with "
                      f"their caches; {rows} of {work.rows} rows), numpy fp32, {spent:.1f} s; "
                      f"tokens/s = rows / layer time / {work.layers} layers"}


STEPS = (("qkv", 0), ("out_proj", 2), ("ffn1", 3), ("ffn2", 4))


def gemm_roofline(L, model, work, reps, log):
    """The four flattened Linear steps timed inside real iterations (the
    engine's timing events around each step of every layer), as one roofline
    over all of them plus the figure of each step."""
    H, F, M = work.hidden, work.ffn, work.rows
    bf16 = work.dtype == "bf16"
    esz = 2 if bf16 else 4
    shapes = {"qkv": (3 * H, H, False), "out_proj": (H, H, True), "ffn1": (F, H, False),
              "ffn2": (H, F, True)}
    per = {}
    x = model.x_bench
    y = torch_empty_like(x)
    reqs = model.reqs_bench
    for tag, sid in STEPS:
        L.orca_time_step(model.ctx, sid)
        vals = []
        for _ in range(reps):
            model.iteration(reqs, x, y, model.stream)
            vals.append(sum(L.orca_step_times(model.ctx, work.layers)) / work.layers)
        L.orca_time_step(model.ctx, -1)
        vals.sort()
        ms = vals[len(vals) // 2]
        n, k, resid = shapes[tag]
        flops = 2.0 * M * n * k
        # algorithmic bytes: W and A once, the output once (the fp32 residual
        # read and written for the residual epilogues)
        nbytes = esz * (n * k + M * k) + (8 if resid else esz) * M * n
        variant = L.orca_op_linear_variant(model.odt, M, n, k)
        per[tag] = {"shape": [M, n, k], "variant": variant, "ms_per_launch": round(ms, 4),
                    "tflops": round(flops / (ms * 1e-3) / 1e12, 1), "flops": flops,
                    "bytes": nbytes}
        log(f"  in-iteration {tag}: {ms:.4f} ms per layer, {per[tag]['tflops']} TFLOP/s "
            f"(variant {variant})")
    flops = sum(v["flops"] for v in per.values())
    nbytes = sum(v["bytes"] for v in per.values())
    ms = sum(v["ms_per_launch"] for v in per.values())
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_FP32_TFLOPS
    ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    tflops = flops / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    for v in per.values():
        v["frac_of_peak"] = round(v["tflops"] / peak, 4)
        v.pop("flops")
        v.pop("bytes")
    tr = measured_traffic(work.name, "gemm", GEMM_FILES)
    common = {"kernel": ("the flattened Linear launches (QKV, output projection, FFN1, FFN2) of "
                         "every layer, timed inside the iteration"),
              "launches_per_iteration": 4 * work.layers,
              "launch_unit": ("one Linear step of one layer (QKV, output projection, FFN1 or "
                              "FFN2, with the split-K kernels and reduces it launches)"),
              "algorithmic_flops_per_launch": int(flops / 4),
              "algorithmic_bytes_per_launch": int(nbytes / 4),
              "ms_per_launch": round(ms / 4, 4),
              "traffic": tr["bytes"] if tr else None,
              "traffic_unit": "bytes per Linear step (HBM read + write, rocprofv3 counters)",
              "mfma_util_percent_counter": measured_mfma_util(work.name),
              "clock_counter": measured_clock(work.name),
              "per_step": per}
    if flops / nbytes >= ridge:
        return {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(tflops / peak, 4), **common}
    # few rows: the weights stream once and the MFMAs idle
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "achieved_tflops": round(tflops, 2), **common}


def torch_empty_like(x):
    import torch
    return torch.empty_like(x)


def decode_roofline(L, model, work, reps, log):
    """Decode attention of the batch's increment rows at layer 0, HIP events
    around the launch on its stream."""
    import torch
    from orca_selective_iteration_amd import synth
    incr = [i for i in range(work.n_reqs) if work.kv_len[i] > 0]
    if not incr:
        return None
    H = work.hidden
    bf16 = work.dtype == "bf16"
    d_reqs = L.req_array(model.descriptors(reqs=incr))
    q = synth.device_normal_(torch.empty((len(incr), H), dtype=model.tdt, device="cuda"), 13)
    o = torch.empty_like(q)

    def dec():
        L.orca_op_attention(model.ctx, 0, d_reqs, q, o, model.ws, model.ws_bytes, model.stream)
    for _ in range(3):
        dec()
    dms = time_events(dec, reps, model.stream)
    esz = 2 if bf16 else 4
    nbytes = sum(2 * (work.kv_len[i] + 1) * H * esz for i in incr)
    gbs = nbytes / (dms * 1e-3) / 1e9
    tr = measured_traffic(work.name, "decode", ATTN_FILES)
    log(f"  decode attention ({len(incr)} requests, one layer): {dms:.3f} ms, {gbs:.0f} GB/s")
    return {"bound": "hbm", "kernel": "attn_split_kernel + attn_combine_kernel "
            "(increment rows, one layer)", "achieved": round(gbs, 1),
            "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": tr["bytes"] if tr else None, "ms_per_launch": round(dms, 4),
            "algorithmic_bytes": nbytes}


def prefill_roofline(L, model, work, reps, log):
    """Causal attention of the batch's prompts, timed inside iterations over
    the initiation requests alone (their rows of the same input): the
    engine's timing events around the attention step of every layer, which
    then runs the prefill kernel only."""
    import torch
    pre = [i for i in range(work.n_reqs) if work.kv_len[i] == 0 and work.q_len[i] > 0]
    if not pre or work.dtype != "bf16":
        return None
    H = work.hidden
    full = model.descriptors()
    rows = torch.cat([torch.arange(full[i][0], full[i][0] + work.q_len[i]) for i in pre])
    x = model.x_bench.index_select(0, rows.to(model.x_bench.device))
    y = torch.empty_like(x)
    reqs = model.descriptors(reqs=pre)
    model.iteration(reqs, x, y, model.stream)
    L.orca_time_step(model.ctx, 1)      # ORCA_STEP_ATTENTION
    vals = []
    for _ in range(reps):
        model.iteration(reqs, x, y, model.stream)
        vals.append(sum(L.orca_step_times(model.ctx, work.layers)) / work.layers)
    L.orca_time_step(model.ctx, -1)
    vals.sort()
    ms = vals[len(vals) // 2]
    # causal Q K^T and P V: sum over prompts of 2 L (L + 1) H FLOP per layer
    flops = sum(2.0 * work.q_len[i] * (work.q_len[i] + 1) * H for i in pre)
    tflops = flops / (ms * 1e-3) / 1e12
    tiles = sum((work.q_len[i] + 127) // 128 for i in pre) * work.heads
    form = L.orca_op_prefill_keys(work.heads, tiles // work.heads)
    log(f"  prefill attention ({len(pre)} prompts, {tiles} tiles, {form}-key steps): "
        f"{ms * 1e3:.1f} us per layer, {tflops:.0f} TFLOP/s")
    return {"bound": "mfma", "kernel": "attn_prefill_kernel (the batch's prompts, one layer, "
            "timed inside iterations over the prompts alone)", "achieved": round(tflops, 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "ms_per_launch": round(ms, 4),
            "algorithmic_flops": flops, "tiles": tiles, "keys_per_step": form}


def setup(name, seed):
    import torch
    from orca_selective_iteration_amd import synth
    from orca_selective_iteration_amd.runner import DeviceModel
    work = synth.workload(name, seed)
    t0 = time.time()
    host = synth.host_inputs(work, seed) if work.layers * work.hidden <= 4096 else None
    model = DeviceModel(work, host=host, device="cuda", seed=seed, log=log)
    if host is not None:
        x = torch.from_numpy(host.x).to("cuda", model.tdt)
    else:
        x = synth.device_normal_(torch.empty((work.rows, work.hidden), dtype=model.tdt,
                                             device="cuda"), seed * 31 + 5)
    model.x_bench = x
    model.reqs_bench = model.descriptors()
    model.stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    log(f"setup {time.time() - t0:.1f}s: {work.name} rows={work.rows} reqs={work.n_reqs} "
        f"kv_tokens={sum(work.kv_len)} pool_slots={model.cap}")
    return work, model


def config_of(work):
    return {"workload": work.name, "layers": work.layers, "hidden": work.hidden,
            "heads": work.heads, "ffn": work.ffn, "sum_L": work.rows, "requests": work.n_reqs,
            "initiation_requests": sum(1 for v in work.kv_len if v == 0),
            "increment_requests": sum(1 for v in work.kv_len if v > 0),
            "cached_kv_tokens": sum(work.kv_len), "parallelism": "single GPU"}


def run_workload(name, args, headline):
    """Setup, the timed iterations, the in-iteration GEMM and decode
    figures (and on the headline workload the CPU baseline); frees the GPU
    memory before returning."""
    import torch
    from orca_selective_iteration_amd import lib as L
    work, model = setup(name, args.seed)
    out = {}
    try:
        y = torch.empty_like(model.x_bench)

        def step():
            model.iteration(model.reqs_bench, model.x_bench, y, model.stream)
        for _ in range(args.warmup):
            step()
        ms = time_events(step, args.steps, model.stream)
        log(f"{name}: iteration {ms:.3f} ms, {work.rows / ms * 1e3:.0f} tokens/s")
        out = {"value": round(work.rows / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
               "config": config_of(work), "dtype": "bf16" if work.dtype == "bf16" else "f32"}
        if work.dtype == "bf16":
            out["roofline"] = gemm_roofline(L, model, work, args.step_reps, log)
            out["decode_attention"] = decode_roofline(L, model, work, args.kernel_reps, log)
            out["prefill_attention"] = prefill_roofline(L, model, work, args.step_reps, log)
        if headline and not args.no_cpu_baseline:
            t1 = time.time()
            out["cpu_baseline"] = cpu_baseline(model, work)
            log(f"cpu baseline: {out['cpu_baseline']['value']:.2f} tokens/s "
                f"({time.time() - t1:.1f}s)")
    finally:
        model.close()
        del model
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def run_only(args):
    """One timed region, for profilers: the iteration, the FFN1 launch alone,
    decode attention alone, or a 1 GiB copy (the counters' calibration)."""
    import torch
    from orca_selective_iteration_amd import lib as L
    from orca_selective_iteration_amd import synth
    torch.cuda.set_device(0)
    if args.only == "copy":
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.kernel_reps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.kernel_reps} x 1 GiB")
        return
    work, model = setup(args.workload, args.seed)
    try:
        if args.only == "iteration":
            y = torch.empty_like(model.x_bench)
            for _ in range(args.warmup + args.steps):
                model.iteration(model.reqs_bench, model.x_bench, y, model.stream)
            torch.cuda.synchronize()
            log(f"ran {args.warmup + args.steps} iterations")
        elif args.only == "decode":
            decode_roofline(L, model, work, args.kernel_reps, log)
        elif args.only == "gemm":
            H, F, M = work.hidden, work.ffn, work.rows
            a = synth.device_normal_(torch.empty((M, H), dtype=model.tdt, device="cuda"), 11)
            f = torch.empty((M, F), dtype=model.tdt, device="cuda")
            w = model.weights[0]
            nb = L.orca_op_linear_workspace_bytes(model.odt, M, F, H)
            ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
            for _ in range(args.kernel_reps):
                L.orca_op_linear(model.odt, L.ORCA_EPI_BIAS_GELU, a, w["w_1"], w["b_1"], f, M, F,
                                 H, ws, nb, stream=model.stream)
            torch.cuda.synchronize()
            log(f"ran {args.kernel_reps} FFN1 launches")
    finally:
        model.close()


def main():
    args = parse()
    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic, args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the iteration has no multi-GPU path in this build)", file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
    if args.only:
        run_only(args)
        return
    extra = args.extra
    if extra is None:
        extra = DEFAULT_EXTRA if args.workload == DEFAULT_WORKLOAD else "none"
    extra = [] if extra == "none" else [e for e in extra.split(",") if e and e != args.workload]
    for e in extra:
        if e not in WORKLOADS:
            sys.exit(f"unknown workload {e}")
    head = run_workload(args.workload, args, headline=True)
    also = {}
    for e in extra:
        r = run_workload(e, args, headline=False)
        if e == "h1024-2l":
            r["note"] = "two-layer H1024 batch: ms_per_step is the iteration latency at low load"
        also[e] = r
    line = {
        "metric": "processed tokens/s per mixed iteration (1 GPU)",
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded random-init weights, K/V caches and hidden rows)",
        "config": head["config"],
        "roofline": head.get("roofline"),
        "decode_attention": head.get("decode_attention"),
        "prefill_attention": head.get("prefill_attention"),
        "cpu_baseline": head.get("cpu_baseline"),
        "also": also or None,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
