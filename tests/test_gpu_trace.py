"""The scheduling trace on the GPU: the native scheduler drives real
iterations with wall-clock arrivals; replaying the logged step times through
the oracle scheduler must reproduce every batch exactly."""
import pytest

from oracle import sched as osch
from orca_selective_iteration_amd import lib as L
from orca_selective_iteration_amd import synth
from orca_selective_iteration_amd.trace import TraceEngine

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


NAMES = {L.ORCA_POLICY_ITERATION: "iteration", L.ORCA_POLICY_STATIC: "static",
         L.ORCA_POLICY_CHUNKED: "chunked"}


@pytest.mark.parametrize("policy,depth", [
    (L.ORCA_POLICY_ITERATION, 1), (L.ORCA_POLICY_STATIC, 1), (L.ORCA_POLICY_CHUNKED, 1),
    # the host schedules iteration k+1 while k still runs on the GPU
    (L.ORCA_POLICY_ITERATION, 3), (L.ORCA_POLICY_CHUNKED, 2)])
def test_trace_replays_through_the_oracle(policy, depth):
    print(f"case trace policy={policy} depth={depth}", flush=True)
    work = synth.custom_workload(2, 256, 2, 512, "bf16", [1], [0])
    reqs = synth.poisson_trace(60, 400.0, seed=3, prompt=(4, 60), out=(1, 24), max_tokens=24)
    # chunked prefill: a budget below the longest prompt, so prompts split
    max_batch, budget = 8, (128 if policy != L.ORCA_POLICY_CHUNKED else 40)
    eng = TraceEngine(work, max_batch, budget, kv_slots=4000)
    try:
        res = eng.run(reqs, max_batch, budget, policy, depth=depth)
    finally:
        eng.close()
    o = osch.Scheduler(max_batch, budget, 4000, NAMES[policy])
    for r in reqs:
        assert o.submit(r.id, r.arrival, r.prompt_len, r.max_tokens, r.out_len)
    for now, ids in res["calls"]:
        assert tuple(e.id for e in o.step(now)) == ids
    assert o.step(res["calls"][-1][0] + 1.0) == [] and o.idle()
    assert res["generated_tokens"] == sum(r.out_len for r in reqs)
    assert res["iterations"] == len(res["steps"])
    assert res["latency_s"]["mean"] > 0


def _replay_one_request(eng, res, rid):
    """The oracle (float64) runs request `rid` alone over its whole history:
    each iteration that held it, with the rows it had in that batch and the
    K/V its own earlier iterations appended.  Returns the worst relative
    error of its output rows against the GPU's, iteration by iteration."""
    import numpy as np
    from oracle import model as om
    from tests.util import rel_err
    work = eng.work
    params = [{k: v.float().cpu().numpy().astype(np.float64) for k, v in w.items()}
              for w in eng.weights]
    x = eng.x.float().cpu().numpy().astype(np.float64)
    kc = [np.zeros((0, work.hidden)) for _ in range(work.layers)]
    vc = [np.zeros((0, work.hidden)) for _ in range(work.layers)]
    worst, seen = 0.0, 0
    for k, ((_, ids), batch) in enumerate(zip(res["steps"], res["batches"])):
        if rid not in ids:
            continue
        q_off, q_len, kv_len, _, _ = batch[ids.index(rid)]
        assert kc[0].shape[0] == kv_len, (rid, k, kv_len)
        xr = x[q_off:q_off + q_len]
        caches = [[(kc[l], vc[l])] for l in range(work.layers)]
        yr, app = om.selective_iteration(params, [om.Req(0, q_len, kv_len)], xr, caches,
                                         work.heads, work.eps)
        for l in range(work.layers):
            kc[l] = np.concatenate([kc[l], app[l][0][0]])
            vc[l] = np.concatenate([vc[l], app[l][0][1]])
        got = res["outputs"][k][q_off:q_off + q_len].float().cpu().numpy()
        worst = max(worst, rel_err(got, yr))
        seen += 1
    assert seen > 0
    return worst


@pytest.mark.parametrize("policy,depth", [
    (L.ORCA_POLICY_ITERATION, 1), (L.ORCA_POLICY_ITERATION, 2), (L.ORCA_POLICY_ITERATION, 3),
    (L.ORCA_POLICY_STATIC, 2), (L.ORCA_POLICY_CHUNKED, 2)])
def test_trace_with_cancellations(policy, depth):
    """Requests withdrawn while queued and while running (at depth 2 and 3
    while the iteration that holds them may still be on the GPU): the logged
    steps, with the same withdrawals, replay exactly through the oracle
    scheduler; a request admitted into K/V slots a withdrawn request freed
    gets outputs that match the oracle model running it alone over its own
    history."""
    import numpy as np
    print(f"case trace cancel policy={policy} depth={depth}", flush=True)
    work = synth.custom_workload(2, 256, 2, 512, "bf16", [1], [0])
    # every request queued at t = 0, so which requests run at each call does
    # not depend on the wall clock
    reqs = synth.poisson_trace(48, float("inf"), seed=5, prompt=(4, 60), out=(6, 24),
                               max_tokens=24)
    max_batch, budget = 6, (128 if policy != L.ORCA_POLICY_CHUNKED else 40)
    # early calls withdraw requests that are running; high ids are still
    # queued when withdrawn
    cancels = {3: [1, 45], 6: [3], 9: [2, 46], 14: [8], 22: [13, 47], 30: [20]}
    eng = TraceEngine(work, max_batch, budget, kv_slots=600)
    try:
        res = eng.run(reqs, max_batch, budget, policy, depth=depth, cancels=cancels, record=True)
        o = osch.Scheduler(max_batch, budget, 600, NAMES[policy])
        for r in reqs:
            assert o.submit(r.id, r.arrival, r.prompt_len, r.max_tokens, r.out_len)
        log = {}
        for c, rid, ok in res["cancelled"]:
            log.setdefault(c, []).append((rid, ok))
        for c, (now, ids) in enumerate(res["calls"]):
            for rid, ok in log.get(c, ()):
                assert o.cancel(rid) == ok, (c, rid)
            assert tuple(e.id for e in o.step(now)) == ids, c
        assert o.step(res["calls"][-1][0] + 1.0) == [] and o.idle()
        accepted = [rid for _, rid, ok in res["cancelled"] if ok]
        assert len(accepted) >= 6, res["cancelled"]
        # withdrawn while running: admitted, never finished
        running = [rid for rid in accepted if o.requests[rid].admitted_at >= 0
                   and o.requests[rid].finished_at < 0]
        assert running, "no request was withdrawn while running"
        # a later request reusing the K/V slots a running withdrawal freed
        base_of = {}
        for (_, ids), batch in zip(res["steps"], res["batches"]):
            for rid, d in zip(ids, batch):
                base_of.setdefault(rid, d[4])
        reused = []
        for w in running:
            lo, hi = base_of[w], base_of[w] + reqs[w].prompt_len + reqs[w].max_tokens
            for rid, b in base_of.items():
                if (rid not in accepted and o.requests[rid].admitted_at >
                        o.requests[w].released_at - 1 and lo <= b < hi):
                    reused.append(rid)
        assert reused, "no request reused the slots of a withdrawn one"
        for rid in sorted(set(reused))[:2]:
            e = _replay_one_request(eng, res, rid)
            print(f"  request {rid} (in freed slots) vs the oracle alone: {e:.2e}", flush=True)
            assert e < 2e-2, (rid, e)
    finally:
        eng.close()


@pytest.mark.big
@pytest.mark.timeout(900)
@pytest.mark.parametrize("policy", [L.ORCA_POLICY_ITERATION, L.ORCA_POLICY_CHUNKED])
def test_gpt13b_serving_trace_replays_through_the_oracle(policy):
    """The serving trace's shape on the real engine: the 13B-shaped 40-layer
    model, a K/V pool sized to the HBM left, at most 64 requests and 4096
    tokens per iteration, 200 requests arriving as a Poisson stream with
    prompts U[32,512] and outputs U[1,512], the host scheduling one
    iteration ahead (depth 2).  Every logged step replays exactly through
    the oracle scheduler, and every request's admission, last-token and
    release iterations agree."""
    print(f"case gpt13b serving trace policy={policy}", flush=True)
    work = synth.workload("gpt13b-40l")
    reqs = synth.poisson_trace(200, 32.0, seed=7)
    eng = TraceEngine(work, 64, 4096, log=lambda *a: print(*a, flush=True))
    try:
        res = eng.run(reqs, 64, 4096, policy, depth=2, max_wall=600,
                      log=lambda *a: print(*a, flush=True))
        cap = eng.cap
    finally:
        eng.close()
    assert cap > 200_000      # the HBM left after the weights, not a smaller pool
    print(f"  {res['iterations']} iterations, {res['generated_tokens']} tokens, "
          f"{res['generated_tokens_per_s']} tok/s, K/V slots {cap}", flush=True)
    o = osch.Scheduler(64, 4096, cap, NAMES[policy])
    for r in reqs:
        assert o.submit(r.id, r.arrival, r.prompt_len, r.max_tokens, r.out_len)
    for c, (now, ids) in enumerate(res["calls"]):
        assert tuple(e.id for e in o.step(now)) == ids, c
    assert o.step(res["calls"][-1][0] + 1.0) == [] and o.idle()
    for r in reqs:
        q = o.requests[r.id]
        assert res["request_info"][r.id] == (q.admitted_at, q.finished_at, q.released_at), r.id
    assert res["generated_tokens"] == sum(r.out_len for r in reqs)
