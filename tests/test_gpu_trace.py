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
