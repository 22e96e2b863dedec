"""End-to-end iteration-level scheduling trace on one GPU.

    python -m orca_selective_iteration_amd.trace [--requests 1000] [--rate 32]
        [--workload gpt13b-40l] [--policy both|iteration|static] [--log FILE]

Requests arrive as a seeded Poisson stream (prompt and output lengths
uniform); the native scheduler (orca_sched_*) picks every iteration's batch
(garden.houmin.site/infra/orca 3.1.1: evict finished requests, admit waiting
ones FCFS within the batch, token and K/V budgets) and orca_iteration runs it.
The clock is the wall clock of the serving loop: each step is taken at the
time the previous iteration finished on the GPU (the engine hands back one
token per request per iteration, so the loop waits for it).  The same trace
runs under request-level (static) batching for comparison
(0h-n0.github.io digest: a static batch lasts as long as its longest member).

No embedding or LM head exists here: the hidden rows fed to every iteration
are seeded N(0,1) rows, and a request's output length is fixed in advance
(it plays the role of the end-of-sequence token).  The K/V pool is sized to
the HBM left after the weights and the workspace; every cached entry is
produced by the model's own initiation and increment iterations.
"""
from __future__ import annotations

import argparse
import json
import sys
import time
from typing import Dict, List, Optional

import numpy as np

from . import lib as L
from . import synth


POLICY_NAMES = {L.ORCA_POLICY_ITERATION: "iteration", L.ORCA_POLICY_STATIC: "static",
                L.ORCA_POLICY_CHUNKED: "chunked"}


class TraceEngine:
    """Weights, an HBM-sized K/V pool and one engine context."""

    def __init__(self, work: synth.Workload, max_batch: int, token_budget: int,
                 kv_slots: Optional[int] = None, hbm_fraction: float = 0.85, seed: int = 0,
                 log=None):
        import torch
        log = log or (lambda *a: None)
        self.work = work
        self.tdt = torch.bfloat16 if work.dtype == "bf16" else torch.float32
        self.odt = L.ORCA_BF16 if work.dtype == "bf16" else L.ORCA_F32
        esz = 2 if work.dtype == "bf16" else 4
        self.weights = [synth.device_param_tensors(work, seed * 1000003 + l, "cuda", self.tdt)
                        for l in range(work.layers)]
        self.max_rows = token_budget
        self.max_reqs = max_batch
        per_token = 2 * work.layers * work.hidden * esz
        if kv_slots is None:
            free, _ = torch.cuda.mem_get_info()
            ws_guess = 64 * work.hidden * self.max_rows + 8 * work.ffn * self.max_rows
            kv_slots = int((free * hbm_fraction - ws_guess) // per_token)
        self.cap = int(kv_slots)
        log(f"K/V pool: {self.cap} token slots ({self.cap * per_token / 1e9:.1f} GB)")
        # [layers][heads][cap][2][d]: each slot's key row, then its value row
        self.kv_pool = torch.empty((work.layers, work.heads, self.cap, 2, work.head_dim),
                                   dtype=self.tdt, device="cuda")
        self.kv = L.orca_kv_create(self.cap)
        self.ctx = L.orca_create(work.layers, work.hidden, work.heads, work.ffn, self.odt,
                                 work.eps, self.cap, self.weights, self.kv_pool,
                                 self.kv, self.max_rows, self.max_reqs)
        self.ws_bytes = L.orca_workspace_bytes(self.ctx)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        self.x = synth.device_normal_(torch.empty((self.max_rows, work.hidden), dtype=self.tdt,
                                                  device="cuda"), seed * 17 + 3)
        self.y = torch.empty_like(self.x)

    def run(self, requests: List[synth.TraceRequest], max_batch: int, token_budget: int,
            policy: int, log=None, max_wall: float = 1e9, depth: int = 1,
            cancels: Optional[Dict[int, List[int]]] = None, record: bool = False) -> dict:
        """Serve `requests` under `policy`.  depth = iterations the loop keeps
        queued on the stream: 1 waits for every iteration before the next
        scheduling step; 2 or more schedule and launch iteration k+1 while k
        still runs, so the host's step, validation and launches hide behind
        the GPU (garden.houmin.site/infra/orca 3.1.3: the scheduler keeps up
        to n_workers batches in the engine without waiting for one to
        return; unpurerationalist.github.io ORCA notes 4.1: a controller
        hands its kernels to the GPU and goes on without waiting).  The step
        clock is the host clock either way; an iteration's end time is read
        from a timing event.

        cancels: {scheduling call index: request ids} withdrawn just before
        that call (garden.houmin.site/infra/orca 3.1.1: a cancelled request
        should leave promptly and free its memory); a withdrawal the
        scheduler refuses (already released) is logged as refused.
        record: also return every iteration's descriptors and a copy of its
        output rows (taken on the stream, in order, without waiting)."""
        import torch
        from collections import deque
        log = log or (lambda *a: None)
        assert 1 <= depth <= 4, "the engine's metadata ring holds 4 batches in flight"
        s = L.orca_sched_create(self.kv, max_batch, token_budget, policy)
        stream = torch.cuda.current_stream()
        try:
            for r in requests:
                L.orca_sched_submit(s, r.id, r.arrival, r.prompt_len, r.max_tokens, r.out_len)
            torch.cuda.synchronize()
            start = torch.cuda.Event(enable_timing=True)
            start.record(stream)
            t0 = time.perf_counter()
            now = 0.0
            steps: List[tuple] = []      # non-empty iterations: (now, ids)
            calls: List[tuple] = []      # every scheduling step, for replay
            batches: List[tuple] = []    # record: descriptors of each iteration
            outputs: List = []           # record: output rows of each iteration
            withdrawn: List[tuple] = []  # (call index, id, accepted)
            cancels = cancels or {}
            ends: List = []              # timing event after each iteration
            flight = deque()
            iters = rows = busy = 0
            last_print = t0
            while not L.orca_sched_idle(s):
                for rid in cancels.get(len(calls), ()):
                    try:
                        L.orca_sched_cancel(s, rid)
                        withdrawn.append((len(calls), rid, True))
                    except L.OrcaError:
                        withdrawn.append((len(calls), rid, False))
                descs, ids = L.orca_sched_step(s, now, max_batch)
                calls.append((now, tuple(ids)))
                if not descs:
                    if L.orca_sched_idle(s):
                        break
                    nxt = L.orca_sched_next_arrival(s)
                    if nxt is None:
                        raise RuntimeError("scheduler idle with active requests")
                    # nothing to run until the next arrival: wait for it
                    stream.synchronize()
                    flight.clear()
                    time.sleep(max(0.0, nxt - (time.perf_counter() - t0)))
                    now = max(time.perf_counter() - t0, nxt)
                    continue
                n_rows = descs[-1].q_offset + descs[-1].q_len
                L.orca_iteration(self.ctx, descs, self.x, self.y, self.ws, self.ws_bytes, stream)
                if record:
                    batches.append(tuple((d.q_offset, d.q_len, d.kv_len, d.phase, d.kv_base)
                                         for d in descs))
                    outputs.append(self.y[:n_rows].clone())
                ev = torch.cuda.Event(enable_timing=True)
                ev.record(stream)
                ends.append(ev)
                flight.append(ev)
                steps.append((now, tuple(ids)))
                iters += 1
                rows += n_rows
                busy += len(descs)
                # keep at most depth - 1 iterations queued behind the next step
                while len(flight) >= depth:
                    flight.popleft().synchronize()
                now = time.perf_counter() - t0
                if now > max_wall:
                    raise RuntimeError(f"trace exceeded {max_wall} s")
                if time.perf_counter() - last_print > 20:
                    log(f"  t={now:.1f}s iterations={iters} rows={rows}")
                    last_print = time.perf_counter()
            stream.synchronize()
            wall = time.perf_counter() - t0
            # per-request latency: time the iteration holding its last token ended
            iter_end = [start.elapsed_time(e) * 1e-3 for e in ends]
            lats = []
            gen = 0
            info = {}
            for r in requests:
                adm, fin, rel = L.orca_sched_request_info(s, r.id)
                info[r.id] = (adm, fin, rel)
                if fin < 0:
                    continue          # withdrawn before its last token
                gen += r.out_len
                if policy == L.ORCA_POLICY_STATIC:
                    # request-level: the response leaves with the whole batch,
                    # after the iteration before the step that released it
                    t_end = iter_end[rel - 1] if 0 < rel <= len(iter_end) else wall
                else:
                    t_end = iter_end[fin]
                lats.append(t_end - r.arrival)
            lats = np.array(lats) if lats else np.zeros(1)
            return {
                "policy": POLICY_NAMES[policy], "depth": depth,
                "wall_s": round(wall, 3), "iterations": iters, "rows_processed": rows,
                "generated_tokens": gen,      # of the requests that finished
                "generated_tokens_per_s": round(gen / wall, 1),
                "processed_tokens_per_s": round(rows / wall, 1),
                "requests_per_s": round(len(requests) / wall, 3),
                "mean_batch": round(busy / max(iters, 1), 2),
                "latency_s": {"mean": round(float(lats.mean()), 3),
                              "p50": round(float(np.percentile(lats, 50)), 3),
                              "p99": round(float(np.percentile(lats, 99)), 3)},
                "steps": steps,
                "calls": calls,
                "cancelled": withdrawn,
                "request_info": info,         # id -> (admitted, finished, released)
                "batches": batches if record else None,
                "outputs": outputs if record else None,
            }
        finally:
            L.orca_sched_destroy(s)

    def close(self):
        """Destroys the context and the allocator and drops the device
        tensors (weights, pools, workspace), so their memory can be reused."""
        if self.ctx:
            L.orca_destroy(self.ctx)
            self.ctx = None
        if self.kv:
            L.orca_kv_destroy(self.kv)
            self.kv = None
        self.weights = []
        self.kv_pool = self.ws = self.x = self.y = None
        try:
            import torch
            torch.cuda.empty_cache()
        except Exception:
            pass


def main(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--workload", default="gpt13b-40l")
    p.add_argument("--requests", type=int, default=1000)
    p.add_argument("--rate", type=float, default=32.0, help="arrivals per second (inf: all at 0)")
    p.add_argument("--max-batch", type=int, default=64)
    p.add_argument("--token-budget", type=int, default=4096)
    p.add_argument("--policy", choices=["both", "iteration", "static", "chunked", "all"],
                   default="both", help="both: iteration and static; all: the three")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--log", default=None, help="write the per-step (now, ids) log as JSON")
    p.add_argument("--max-wall", type=float, default=600.0)
    p.add_argument("--depth", type=int, default=1,
                   help="iterations kept queued on the stream (2+: schedule ahead)")
    a = p.parse_args(argv)
    import torch
    log = lambda *m: print(*m, file=sys.stderr, flush=True)
    work = synth.workload(a.workload, a.seed)
    reqs = synth.poisson_trace(a.requests, a.rate, a.seed)
    eng = TraceEngine(work, a.max_batch, a.token_budget, seed=a.seed, log=log)
    out = {"workload": a.workload, "requests": a.requests, "rate": a.rate,
           "max_batch": a.max_batch, "token_budget": a.token_budget, "kv_slots": eng.cap,
           "depth": a.depth, "runs": []}
    try:
        # warm the kernels once
        warm = [synth.TraceRequest(10**9, 0.0, 64, 8, 2)]
        eng.run(warm, a.max_batch, a.token_budget, L.ORCA_POLICY_ITERATION)
        pols = {"both": [L.ORCA_POLICY_ITERATION, L.ORCA_POLICY_STATIC],
                "all": [L.ORCA_POLICY_ITERATION, L.ORCA_POLICY_CHUNKED, L.ORCA_POLICY_STATIC],
                "iteration": [L.ORCA_POLICY_ITERATION], "static": [L.ORCA_POLICY_STATIC],
                "chunked": [L.ORCA_POLICY_CHUNKED]}[a.policy]
        for pol in pols:
            log(f"policy {POLICY_NAMES[pol]}: {a.requests} requests at {a.rate}/s")
            res = eng.run(reqs, a.max_batch, a.token_budget, pol, log=log, max_wall=a.max_wall,
                          depth=a.depth)
            for k in ("steps", "batches", "outputs", "request_info"):
                res.pop(k)
            calls = res.pop("calls")
            log(json.dumps(res))
            res["log"] = calls if a.log else None
            out["runs"].append(res)
    finally:
        eng.close()
    if a.log:
        with open(a.log, "w") as f:
            json.dump(out, f)
    for r in out["runs"]:
        r.pop("log", None)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
