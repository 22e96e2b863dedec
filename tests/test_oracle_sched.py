"""Pins for the oracle scheduler and allocator (CPU only)."""
import heapq
import itertools

import numpy as np
import pytest

from oracle import sched as osch
from tests.util import golden


def run(out_lens, slots, policy, arrivals=None, prompt=1, budget=10**9, kv=10**12,
        max_tokens=None):
    s = osch.Scheduler(slots, budget, kv, policy)
    for i, n in enumerate(out_lens):
        a = 0.0 if arrivals is None else arrivals[i]
        assert s.submit(i, a, prompt, max_tokens or max(out_lens), n)
    res = osch.run_trace(s)
    return s, res


# ------------------------------------------------- the pages' worked examples

def test_ultralytics_eight_requests_four_slots():
    """ultralytics.com glossary "Continuous Batching": the eight requests of
    its simulation on four slots, with the step counts and slot use the page
    states (tests/golden/glossary_eight_requests.txt)."""
    g = golden("glossary_eight_requests")
    lens, slots = g["output_lengths"], g["slots"]
    _, st = run(lens, slots, "static")
    _, co = run(lens, slots, "iteration")
    assert st.iterations == g["static_steps"] and co.iterations == g["continuous_steps"]
    assert st.busy_rows == co.busy_rows == sum(lens)
    assert round(100 * st.busy_rows / (st.iterations * slots)) == g["static_busy_percent"]
    assert round(100 * co.busy_rows / (co.iterations * slots)) == g["continuous_busy_percent"]


def test_estelledc_three_slot_timeline():
    """estelledc.github.io notes, case 1: A, B, C on three slots with D, E, F
    queued (tests/golden/notes_case1_three_slots.txt; D-F's lengths are not
    given: 200 each, longer than A).  Continuous: D, E, F start at the steps
    the page gives (1-based).  Static: B's slot, then C's, idles over the
    spans it gives, and D waits for the whole first batch."""
    g = golden("notes_case1_three_slots")
    lens = g["lengths_abc"] + [200, 200, 200]        # A B C D E F
    s, _ = run(lens, g["slots"], "iteration")
    starts = [s.requests[i].admitted_at + 1 for i in (3, 4, 5)]
    assert starts == g["continuous_start_def"]
    s2, res = run(lens, g["slots"], "static")
    b0, b1 = g["static_b_idle"]
    c0, c1 = g["static_c_idle"]
    for step in range(b0, b1 + 1):
        assert res.log[step - 1][1] == (0, 2)
    for step in range(c0, c1 + 1):
        assert res.log[step - 1][1] == (0,)
    assert s2.requests[3].admitted_at + 1 == c1 + 1


def test_static_batch_lasts_longest_member():
    """0h-n0 digest: T_batch = max_i T_gen(r_i)."""
    rng = np.random.default_rng(0)
    for _ in range(20):
        lens = list(rng.integers(1, 30, size=int(rng.integers(1, 6))))
        _, res = run(lens, len(lens), "static")
        assert res.iterations == max(lens)


def test_equal_lengths_make_policies_agree():
    """0h-n0 digest, results: with equal generation lengths the gap to static
    batching closes."""
    for n, slots, L in [(8, 4, 10), (12, 3, 7), (5, 5, 9)]:
        _, st = run([L] * n, slots, "static")
        _, co = run([L] * n, slots, "iteration")
        assert st.iterations == co.iterations


def heap_slot_starts(out_lens, slots):
    """The ultralytics description: each request, in order, takes the slot
    that frees first (a heap of slot-free times)."""
    free = [0] * slots
    starts = []
    for n in out_lens:
        t = heapq.heappop(free)
        starts.append(t)
        heapq.heappush(free, t + n)
    return starts, max(free)


@pytest.mark.parametrize("seed", range(10))
def test_continuous_matches_slot_heap(seed):
    rng = np.random.default_rng(seed)
    lens = [int(v) for v in rng.integers(1, 60, size=int(rng.integers(1, 25)))]
    slots = int(rng.integers(1, 7))
    s, res = run(lens, slots, "iteration")
    starts, total = heap_slot_starts(lens, slots)
    assert res.iterations == total
    assert [s.requests[i].admitted_at for i in range(len(lens))] == starts


# ------------------------------------------------------------- invariants

def _random_trace(rng, n=40):
    arr = np.cumsum(rng.exponential(2.0, size=n))
    prompts = rng.integers(1, 20, size=n)
    outs = rng.integers(1, 25, size=n)
    return arr, prompts, outs


@pytest.mark.parametrize("policy", ["iteration", "static"])
@pytest.mark.parametrize("seed", range(6))
def test_scheduler_invariants(policy, seed):
    rng = np.random.default_rng(seed)
    arr, prompts, outs = _random_trace(rng)
    max_batch, budget, kv = 5, 40, 150
    s = osch.Scheduler(max_batch, budget, kv, policy)
    for i in range(len(arr)):
        assert s.submit(i, float(arr[i]), int(prompts[i]), 25, int(outs[i]))
    seen = {i: 0 for i in range(len(arr))}
    now = 0.0
    admitted_order = []
    while True:
        batch = s.step(now)
        assert s.used == sum(r.reserved for r in s.active) <= kv
        assert s.alloc.used() == s.used
        if not batch:
            if s.idle():
                break
            now = s.next_arrival()
            continue
        assert len(batch) <= max_batch and len({e.id for e in batch}) == len(batch)
        assert sum(e.q_len for e in batch) <= budget
        off = 0
        for e in batch:
            assert e.q_offset == off
            off += e.q_len
            r = s.requests[e.id]
            assert r.arrival <= now
            if e.phase == osch.INITIATION:
                admitted_order.append(e.id)
                assert e.kv_len == 0 and e.q_len == r.prompt_len
            else:
                assert e.q_len == 1 and e.kv_len == r.prompt_len + r.generated - 1
            assert e.kv_len + e.q_len <= r.reserved
            seen[e.id] += 1
        phases = [e.phase for e in batch]
        assert phases == sorted(phases, reverse=True)     # increments first
        now += 1.0
    assert s.used == 0 and s.alloc.used() == 0
    assert admitted_order == sorted(admitted_order)       # FCFS
    for i in range(len(arr)):
        assert seen[i] == outs[i]                         # exactly n iterations


def test_increment_kv_length_grows_by_one():
    s = osch.Scheduler(2, 100, 1000, "iteration")
    s.submit(0, 0.0, 5, 10, 4)
    lens = []
    while True:
        b = s.step(0.0)
        if not b:
            break
        lens.append((b[0].phase, b[0].q_len, b[0].kv_len))
    assert lens == [(0, 5, 0), (1, 1, 5), (1, 1, 6), (1, 1, 7)]


def test_kv_shortage_breaks_fcfs():
    """0h-n0 scheduler algorithm: when the head of the queue does not fit the
    remaining K/V slots, admission stops (no skipping ahead)."""
    s = osch.Scheduler(4, 1000, 30, "iteration")
    s.submit(0, 0.0, 10, 10, 5)      # reserves 20
    s.submit(1, 0.0, 10, 10, 5)      # needs 20 > 10 left
    s.submit(2, 0.0, 1, 2, 1)        # would fit, must wait (FCFS)
    b = s.step(0.0)
    assert [e.id for e in b] == [0]


def test_token_budget_breaks_fcfs():
    s = osch.Scheduler(8, 16, 10**6, "iteration")
    s.submit(0, 0.0, 10, 10, 3)
    s.submit(1, 0.0, 7, 10, 3)       # 10 + 7 > 16
    s.submit(2, 0.0, 1, 10, 3)
    assert [e.id for e in s.step(0.0)] == [0]
    assert [e.id for e in s.step(1.0)] == [0, 1, 2]   # 1 + 7 + 1 <= 16
    assert not s.submit(9, 0.0, 17, 10, 3)            # longer than the budget


# ------------------------------------------------------------------ allocator

class Bitmap:
    def __init__(self, cap):
        self.bits = [False] * cap
        self.live = {}

    def alloc(self, n):
        for b in range(len(self.bits) - n + 1):
            if not any(self.bits[b:b + n]):
                for i in range(b, b + n):
                    self.bits[i] = True
                self.live[b] = n
                return b
        return None

    def free(self, b):
        n = self.live.pop(b)
        for i in range(b, b + n):
            self.bits[i] = False


@pytest.mark.parametrize("seed", range(20))
def test_first_fit_matches_bitmap(seed):
    rng = np.random.default_rng(seed)
    cap = int(rng.integers(1, 40))
    a, ref = osch.FirstFitAllocator(cap), Bitmap(cap)
    for _ in range(200):
        if a.live and rng.random() < 0.45:
            b = list(a.live)[int(rng.integers(len(a.live)))]
            a.free(b)
            ref.free(b)
        else:
            n = int(rng.integers(1, 12))
            assert a.alloc(n) == ref.alloc(n)
        assert a.used() == sum(ref.bits)
        # free list is coalesced: no two adjacent intervals touch
        for (s1, l1), (s2, _) in zip(a.free_list, a.free_list[1:]):
            assert s1 + l1 < s2


def test_double_free_raises():
    a = osch.FirstFitAllocator(10)
    b = a.alloc(3)
    a.free(b)
    with pytest.raises(KeyError):
        a.free(b)


# ------------------------------------------------ cancel and chunked prefill

Scheduler, INITIATION, INCREMENT = osch.Scheduler, osch.INITIATION, osch.INCREMENT

def _steps(s, now=0.0, limit=1000):
    out = []
    for _ in range(limit):
        b = s.step(now)
        if not b:
            if s.idle():
                return out
            now = s.next_arrival()
            continue
        out.append([(e.id, e.q_offset, e.q_len, e.kv_len, e.phase) for e in b])
        now += 1.0
    raise AssertionError("did not drain")


def test_chunked_hand_example():
    # budget 4: A's 6-token prompt goes 4 + 2, B's 3-token prompt 2 + 1; A's
    # first token comes with its last chunk, then it decodes; worked by hand
    # from the policy (increments, continuing chunks, admissions)
    s = Scheduler(max_batch=4, token_budget=4, kv_slots=100, policy="chunked")
    assert s.submit(0, 0.0, 6, 2, 2) and s.submit(1, 0.0, 3, 1, 1)
    got = _steps(s)
    I, D = INITIATION, INCREMENT
    assert got == [
        [(0, 0, 4, 0, I)],
        [(0, 0, 2, 4, I), (1, 2, 2, 0, I)],
        [(0, 0, 1, 6, D), (1, 1, 1, 2, I)],
    ]
    a, b = s.requests[0], s.requests[1]
    assert (a.admitted_at, a.finished_at, a.released_at) == (0, 2, 3)
    assert (b.admitted_at, b.finished_at, b.released_at) == (1, 2, 3)
    assert s.used == 0 and s.alloc.used() == 0


def test_chunked_equals_iteration_when_budget_never_binds():
    rng = np.random.default_rng(5)
    reqs = []
    for i in range(40):
        mt = int(rng.integers(1, 20))
        reqs.append((i, float(rng.uniform(0, 30)), int(rng.integers(1, 50)), mt,
                     int(rng.integers(1, mt + 1))))
    logs = []
    for pol in ("iteration", "chunked"):
        s = Scheduler(max_batch=5, token_budget=10**6, kv_slots=10**6, policy=pol)
        for r in reqs:
            assert s.submit(*r)
        logs.append(_steps(s))
    assert logs[0] == logs[1]


@pytest.mark.parametrize("seed", range(6))
def test_chunked_invariants(seed):
    rng = np.random.default_rng(40 + seed)
    budget = int(rng.integers(3, 30))
    s = Scheduler(max_batch=int(rng.integers(1, 8)), token_budget=budget, kv_slots=2000,
                  policy="chunked")
    reqs = {}
    for i in range(50):
        mt = int(rng.integers(1, 20))
        r = (i, float(rng.uniform(0, 40)), int(rng.integers(1, 80)), mt,
             int(rng.integers(1, mt + 1)))
        assert s.submit(*r)
        reqs[i] = r
    prompt_rows = {i: 0 for i in reqs}
    incr = {i: 0 for i in reqs}
    for batch in _steps(s):
        assert sum(q for _, _, q, _, _ in batch) <= budget
        phases = [ph for *_, ph in batch]
        assert phases == sorted(phases, reverse=True)      # increments first
        off = 0
        for rid, q_off, q, kv, ph in batch:
            assert q_off == off
            off += q
            if ph == INITIATION:
                assert kv == prompt_rows[rid]                  # chunks follow each other
                prompt_rows[rid] += q
            else:
                assert q == 1 and prompt_rows[rid] == reqs[rid][2]
                assert kv == reqs[rid][2] + incr[rid]
                incr[rid] += 1
    for i, (_, _, prompt, _, out) in reqs.items():
        assert prompt_rows[i] == prompt and incr[i] == out - 1


def test_cancel_hand_example():
    # 20 slots: A reserves 15, B (10) must wait; cancelling A frees its slots
    # at the next step, where B is admitted in its place
    s = Scheduler(max_batch=2, token_budget=100, kv_slots=20, policy="iteration")
    assert s.submit(0, 0.0, 5, 10, 10) and s.submit(1, 0.0, 3, 7, 2)
    assert s.submit(2, 50.0, 2, 2, 1)
    assert [e.id for e in s.step(0.0)] == [0]
    assert s.cancel(0)
    assert not s.cancel(0)                     # twice
    assert not s.cancel(7)                     # unknown
    assert s.cancel(2)                         # not arrived yet: dropped at once
    b = s.step(1.0)
    assert [(e.id, e.phase, e.kv_base) for e in b] == [(1, INITIATION, 0)]
    assert [(e.id, e.phase, e.kv_len) for e in s.step(2.0)] == [(1, INCREMENT, 3)]
    assert s.step(3.0) == [] and s.idle()
    a, bb, c = s.requests[0], s.requests[1], s.requests[2]
    assert (a.admitted_at, a.finished_at, a.released_at) == (0, -1, 1)
    assert (bb.admitted_at, bb.finished_at, bb.released_at) == (1, 2, 3)
    assert (c.admitted_at, c.released_at) == (-1, -1)
    assert not s.cancel(1)                     # already released
    assert s.used == 0


def test_cancel_static_leaves_the_rest_of_the_batch_running():
    s = Scheduler(max_batch=3, token_budget=100, kv_slots=100, policy="static")
    for i, out in enumerate([5, 5, 5]):
        assert s.submit(i, 0.0, 2, 5, out)
    assert s.submit(3, 0.0, 2, 5, 1)
    assert [e.id for e in s.step(0.0)] == [0, 1, 2]
    assert s.cancel(1)
    b = s.step(1.0)
    assert [e.id for e in b] == [0, 2]          # the cancelled member left at once
    assert s.requests[1].released_at == 1 and s.used == 14
    while True:
        b = s.step(2.0)
        if not b or 3 in [e.id for e in b]:
            break
    assert [e.id for e in b] == [3]             # next batch only after 0 and 2 end
