"""Parity at the full benchmark sizes (the 13B-shaped 40-layer model and the
175B-layer-shaped 8-layer model), in the launch configuration bench.py
times, on outputs the oracle can compute one request at a time.

Rows of different requests never interact, so any subset of requests can be
checked exactly:
  * full depth: the real all-layer iteration over the whole batch; for a few
    sampled increment requests the oracle (float64) replays every layer on
    that request alone, from the same seeded weights and caches, and the
    output rows and the K/V rows appended at every layer are compared;
  * one layer: a single-layer engine over layer l of the same pool runs the
    whole batch from seeded input rows; the oracle checks the complete first
    initiation prompt (or its first rows, whose causal attention needs no
    later row) and sampled increment requests.
The decode batch (64 increment rows, no prompt) runs every Linear on the
split-K path, with the residual reduces fused into the LayerNorms.
These need ~160 GB of device memory and minutes of host time: marked `big`.
"""
import numpy as np
import pytest

from oracle import model as om
from orca_selective_iteration_amd import lib as L
from orca_selective_iteration_amd import synth
from orca_selective_iteration_amd.runner import DeviceModel
from tests.util import TOL, rel_err

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu, pytest.mark.big]
DEV = "cuda"


def host64(t):
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def layer64(model, l):
    return {k: host64(v) for k, v in model.weights[l].items()}


def cache64(model, l, i, lo, hi):
    k, v = model.cache_rows(l, i, lo, hi)
    return k.astype(np.float64), v.astype(np.float64)


def run_fullsize(name, n_full_depth, init_rows, layers_checked, seed=0):
    work = synth.workload(name, seed)
    print(f"case fullsize {name}: rows={work.rows} reqs={work.n_reqs}", flush=True)
    model = DeviceModel(work, device=DEV, seed=seed, log=lambda *a: print(*a, flush=True))
    rng = np.random.default_rng(1234 + seed)
    incr = [i for i in range(work.n_reqs) if work.kv_len[i] > 0]
    init = [i for i in range(work.n_reqs) if work.kv_len[i] == 0]
    offs = work.q_offset
    try:
        x = synth.device_normal_(torch.empty((work.rows, work.hidden), dtype=model.tdt,
                                             device=DEV), 4242 + seed)
        y = torch.empty_like(x)
        reqs = model.descriptors()
        # ---- full depth over the whole batch
        model.iteration(reqs, x, y)
        torch.cuda.synchronize()
        sample = sorted(rng.choice(incr, size=n_full_depth, replace=False).tolist())
        got_y = {i: host64(y[offs[i]:offs[i] + 1]) for i in sample}
        got_kv = {(l, i): cache64(model, l, i, work.kv_len[i], work.kv_len[i] + 1)
                  for l in range(work.layers) for i in sample}
        xs = {i: host64(x[offs[i]:offs[i] + 1]) for i in sample}
        worst = 0.0
        for l in range(work.layers):
            p = layer64(model, l)
            for i in sample:
                kc = cache64(model, l, i, 0, work.kv_len[i])
                xs[i], app = om.selective_layer(p, [om.Req(0, 1, work.kv_len[i])], xs[i], [kc],
                                                work.heads, work.eps)
                ek = rel_err(got_kv[(l, i)][0], app[0][0])
                ev = rel_err(got_kv[(l, i)][1], app[0][1])
                worst = max(worst, ek, ev)
                assert ek < TOL["bf16"] and ev < TOL["bf16"], (l, i, ek, ev)
            del p
            if l % 8 == 7:
                print(f"  full depth: layer {l + 1}/{work.layers} ok (worst K/V {worst:.2e})",
                      flush=True)
        for i in sample:
            e = rel_err(got_y[i], xs[i])
            print(f"  full depth y of request {i} (kv {work.kv_len[i]}): {e:.2e}", flush=True)
            assert e < TOL["bf16"], (i, e)

        # ---- single layers over the whole batch
        size = model.kv_pool[0].numel() * model.kv_pool.element_size()
        for l in layers_checked:
            ctx = L.orca_create(1, work.hidden, work.heads, work.ffn, model.odt, work.eps,
                                model.cap, [model.weights[l]], model.kv_pool.data_ptr() + l * size,
                                model.kv, model.max_rows,
                                model.max_reqs)
            try:
                ws_bytes = L.orca_workspace_bytes(ctx)
                ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
                xl = synth.device_normal_(torch.empty_like(x), 777 + l)
                yl = torch.empty_like(x)
                L.orca_iteration(ctx, reqs, xl, yl, ws, ws_bytes)
                torch.cuda.synchronize()
                del ws
            finally:
                L.orca_destroy(ctx)
            p = layer64(model, l)
            picks = [(i, 1) for i in sorted(rng.choice(incr, size=8, replace=False).tolist())]
            if init:
                i0 = init[0]
                n0 = min(work.q_len[i0], init_rows)
                picks = [(i0, n0)] + picks
            for i, n in picks:
                kv = work.kv_len[i]
                kc = cache64(model, l, i, 0, kv)
                xr = host64(xl[offs[i]:offs[i] + n])
                yr, app = om.selective_layer(p, [om.Req(0, n, kv)], xr, [kc], work.heads,
                                             work.eps)
                gk, gv = cache64(model, l, i, kv, kv + n)
                errs = (rel_err(host64(yl[offs[i]:offs[i] + n]), yr), rel_err(gk, app[0][0]),
                        rel_err(gv, app[0][1]))
                assert max(errs) < TOL["bf16"], (l, i, n, errs)
            print(f"  layer {l}: " + (f"initiation rows 0..{n0 - 1} of request {i0} and "
                                       if init else "") + "8 increments ok", flush=True)
            del p
    finally:
        model.close()
        del model
        torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_gpt13b_40_layers_full_size():
    run_fullsize("gpt13b-40l", n_full_depth=3, init_rows=1024, layers_checked=[0, 39])


@pytest.mark.timeout(900)
def test_gpt175b_layer_shape_8_layers_full_size():
    run_fullsize("gpt175b-8l", n_full_depth=2, init_rows=384, layers_checked=[0, 7])


@pytest.mark.timeout(900)
def test_gpt13b_decode_batch_40_layers_full_size():
    run_fullsize("gpt13b-40l-decode64", n_full_depth=3, init_rows=0, layers_checked=[0, 39])
