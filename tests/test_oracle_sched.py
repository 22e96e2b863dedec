"""Pins for the oracle scheduler and allocator (CPU only)."""
import heapq
import itertools

import numpy as np
import pytest

from oracle import sched as osch


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
    """ultralytics.com glossary "Continuous Batching": output lengths
    [5,50,8,12,40,3,30,7] on 4 slots: static 90 steps with 43% of slots busy,
    continuous 50 steps with 78% busy."""
    lens = [5, 50, 8, 12, 40, 3, 30, 7]
    _, st = run(lens, 4, "static")
    _, co = run(lens, 4, "iteration")
    assert st.iterations == 90 and co.iterations == 50
    assert st.busy_rows == co.busy_rows == 155
    assert round(100 * st.busy_rows / (st.iterations * 4)) == 43
    assert round(100 * co.busy_rows / (co.iterations * 4)) == 78


def test_estelledc_three_slot_timeline():
    """estelledc.github.io case 1: A=100, B=10, C=50 tokens on 3 slots.
    Continuous: D starts at step 11, E at 51, F at 101 (1-based steps).
    Static: B's slot idles over steps 11-50, C's over 51-100."""
    lens = [100, 10, 50, 200, 200, 200]        # A B C D E F
    s, _ = run(lens, 3, "iteration")
    starts = {i: s.requests[i].admitted_at + 1 for i in range(6)}
    assert starts[3] == 11 and starts[4] == 51 and starts[5] == 101
    s2, res = run(lens, 3, "static")
    for step in range(11, 51):
        assert res.log[step - 1][1] == (0, 2)
    for step in range(51, 101):
        assert res.log[step - 1][1] == (0,)
    assert s2.requests[3].admitted_at + 1 == 101


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
