"""Host-side checks of liborca.so (no GPU): the library loads and exports
every entry point include/orca.h declares; the native allocator and
scheduler make exactly the oracle's decisions; argument validation fails
before anything reaches the GPU."""
import ctypes

import numpy as np
import pytest

from oracle import sched as osch
from orca_selective_iteration_amd import lib as L


def test_library_exports_every_declared_function():
    names = L.header_functions()
    assert len(names) >= 25
    so = ctypes.CDLL(L.LIB_PATH)
    missing = [n for n in names if not hasattr(so, n)]
    assert not missing, missing
    assert L.orca_status_str(L.ORCA_ERR_NOSPACE) == "ORCA_ERR_NOSPACE"


# ------------------------------------------------------------------ allocator

@pytest.mark.parametrize("seed", range(12))
def test_native_allocator_matches_oracle(seed):
    rng = np.random.default_rng(100 + seed)
    cap = int(rng.integers(1, 300))
    kv = L.orca_kv_create(cap)
    ref = osch.FirstFitAllocator(cap)
    try:
        for _ in range(400):
            if ref.live and rng.random() < 0.45:
                b = list(ref.live)[int(rng.integers(len(ref.live)))]
                ref.free(b)
                L.orca_kv_free(kv, b)
            else:
                n = int(rng.integers(1, 40))
                want = ref.alloc(n)
                if want is None:
                    with pytest.raises(L.OrcaError) as e:
                        L.orca_kv_alloc(kv, n)
                    assert e.value.status == L.ORCA_ERR_NOSPACE
                else:
                    assert L.orca_kv_alloc(kv, n) == want
                    assert L.orca_kv_reservation(kv, want) == n
            assert L.orca_kv_used(kv) == ref.used()
    finally:
        L.orca_kv_destroy(kv)


def test_allocator_errors():
    kv = L.orca_kv_create(10)
    try:
        with pytest.raises(L.OrcaError) as e:
            L.orca_kv_alloc(kv, 0)
        assert e.value.status == L.ORCA_ERR_INVALID
        b = L.orca_kv_alloc(kv, 4)
        L.orca_kv_free(kv, b)
        with pytest.raises(L.OrcaError) as e:
            L.orca_kv_free(kv, b)
        assert e.value.status == L.ORCA_ERR_INVALID and "no reservation" in str(e.value)
        assert L.orca_kv_reservation(kv, 3) == -1
    finally:
        L.orca_kv_destroy(kv)
    with pytest.raises(L.OrcaError):
        L.orca_kv_create(-1)


# ------------------------------------------------------------------ scheduler

POLICIES = {"iteration": L.ORCA_POLICY_ITERATION, "static": L.ORCA_POLICY_STATIC,
            "chunked": L.ORCA_POLICY_CHUNKED}


def replay_both(reqs, max_batch, budget, kv_slots, policy, dt=1.0, cancels=None):
    """Drive the native and the oracle scheduler with the same clock; assert
    identical batches at every step; return the oracle result.  cancels maps
    a step index (steps taken so far, empty ones included) to the ids
    withdrawn just before that step."""
    pol = POLICIES[policy]
    cancels = cancels or {}
    kv = L.orca_kv_create(kv_slots)
    s = L.orca_sched_create(kv, max_batch, budget, pol)
    o = osch.Scheduler(max_batch, budget, kv_slots, policy)
    try:
        for (rid, arr, prompt, mt, out) in reqs:
            ok = o.submit(rid, arr, prompt, mt, out)
            if ok:
                L.orca_sched_submit(s, rid, arr, prompt, mt, out)
            else:
                with pytest.raises(L.OrcaError):
                    L.orca_sched_submit(s, rid, arr, prompt, mt, out)
        now, steps, calls = 0.0, 0, 0
        while True:
            for rid in cancels.get(calls, ()):
                if o.cancel(rid):
                    L.orca_sched_cancel(s, rid)
                else:
                    with pytest.raises(L.OrcaError):
                        L.orca_sched_cancel(s, rid)
            calls += 1
            want = o.step(now)
            got, ids = L.orca_sched_step(s, now, max_batch)
            assert ids == [e.id for e in want]
            assert [(g.q_offset, g.q_len, g.kv_len, g.phase, g.kv_base) for g in got] == \
                   [(e.q_offset, e.q_len, e.kv_len, e.phase, e.kv_base) for e in want]
            assert L.orca_sched_used(s) == o.used
            if not want:
                assert L.orca_sched_idle(s) == o.idle()
                if o.idle():
                    break
                nxt = o.next_arrival()
                assert L.orca_sched_next_arrival(s) == nxt
                now = nxt
                continue
            steps += 1
            now += dt
        for r in o.requests.values():
            assert L.orca_sched_request_info(s, r.id) == (r.admitted_at, r.finished_at,
                                                          r.released_at)
        assert L.orca_kv_used(kv) == 0
        return o, steps
    finally:
        L.orca_sched_destroy(s)
        L.orca_kv_destroy(kv)


def test_native_scheduler_page_examples():
    lens = [5, 50, 8, 12, 40, 3, 30, 7]
    reqs = [(i, 0.0, 1, 50, n) for i, n in enumerate(lens)]
    _, steps = replay_both(reqs, 4, 10**6, 10**6, "static")
    assert steps == 90
    _, steps = replay_both(reqs, 4, 10**6, 10**6, "iteration")
    assert steps == 50
    lens = [100, 10, 50, 200, 200, 200]
    o, _ = replay_both([(i, 0.0, 1, 200, n) for i, n in enumerate(lens)], 3, 10**6, 10**6,
                       "iteration")
    assert [o.requests[i].admitted_at + 1 for i in (3, 4, 5)] == [11, 51, 101]


@pytest.mark.parametrize("policy", ["iteration", "static", "chunked"])
@pytest.mark.parametrize("seed", range(8))
def test_native_scheduler_matches_oracle_random(policy, seed):
    rng = np.random.default_rng(200 + seed)
    n = 60
    arr = np.cumsum(rng.exponential(1.5, size=n))
    reqs = []
    for i in range(n):
        prompt = int(rng.integers(1, 40))
        mt = int(rng.integers(1, 30))
        out = int(rng.integers(1, mt + 1))
        reqs.append((i, float(arr[i]), prompt, mt, out))
    reqs.append((n, 1.0, 500, 10, 5))            # longer than the budget: rejected
    reqs.append((n + 1, 1.0, 5, 10, 11))         # out_len > max_tokens: rejected
    max_batch = int(rng.integers(1, 9))
    budget = int(rng.integers(40, 120)) if policy != "chunked" else int(rng.integers(4, 50))
    kv = int(rng.integers(80, 400))
    if policy == "chunked":
        reqs.append((n + 2, 2.0, 300, 10, 5))    # prompt far above the budget: chunked
    replay_both(reqs, max_batch, budget, kv, policy, dt=float(rng.uniform(0.2, 2.0)))


@pytest.mark.parametrize("policy", ["iteration", "static", "chunked"])
@pytest.mark.parametrize("seed", range(6))
def test_native_scheduler_cancel_matches_oracle(policy, seed):
    rng = np.random.default_rng(900 + seed)
    n = 50
    arr = np.cumsum(rng.exponential(1.0, size=n))
    reqs = []
    for i in range(n):
        mt = int(rng.integers(1, 30))
        reqs.append((i, float(arr[i]), int(rng.integers(1, 40)), mt, int(rng.integers(1, mt + 1))))
    # withdraw random ids at random steps: queued, running, finished, twice, unknown
    cancels = {}
    for _ in range(40):
        cancels.setdefault(int(rng.integers(0, 120)), []).append(int(rng.integers(0, n + 3)))
    budget = int(rng.integers(40, 120)) if policy != "chunked" else int(rng.integers(4, 50))
    replay_both(reqs, int(rng.integers(1, 9)), budget, int(rng.integers(80, 400)), policy,
                dt=float(rng.uniform(0.2, 2.0)), cancels=cancels)


# the serving trace's own parameters: 1000 requests arriving as a Poisson
# stream, prompts U[32,512], outputs U[1,512] (max_tokens 512), at most 64
# requests and 4096 tokens per iteration; K/V slots sized to HBM (300,000
# token slots on the 13B shape, never binding) or tight enough to bind
@pytest.mark.parametrize("policy", ["iteration", "static", "chunked"])
@pytest.mark.parametrize("kv_slots", [300_000, 40_000])
def test_native_scheduler_matches_oracle_serving_trace(policy, kv_slots):
    from orca_selective_iteration_amd import synth
    trace = synth.poisson_trace(1000, 32.0, seed=0)
    reqs = [(r.id, r.arrival, r.prompt_len, r.max_tokens, r.out_len) for r in trace]
    # a synthetic clock of 25 ms per iteration (the decode-dominated 13B
    # iteration is 10-25 ms)
    o, steps = replay_both(reqs, 64, 4096, kv_slots, policy, dt=0.025)
    assert all(r.finished_at >= 0 for r in o.requests.values())
    assert steps >= 512


def test_native_scheduler_cancel_matches_oracle_serving_trace():
    from orca_selective_iteration_amd import synth
    trace = synth.poisson_trace(1000, 32.0, seed=1)
    reqs = [(r.id, r.arrival, r.prompt_len, r.max_tokens, r.out_len) for r in trace]
    rng = np.random.default_rng(5)
    cancels = {}
    for _ in range(150):
        cancels.setdefault(int(rng.integers(0, 3000)), []).append(int(rng.integers(0, 1000)))
    replay_both(reqs, 64, 4096, 300_000, "iteration", dt=0.025, cancels=cancels)


def test_scheduler_argument_errors():
    kv = L.orca_kv_create(100)
    try:
        with pytest.raises(L.OrcaError):
            L.orca_sched_create(kv, 0, 10, 0)
        with pytest.raises(L.OrcaError):
            L.orca_sched_create(kv, 4, 10, 7)
        s = L.orca_sched_create(kv, 4, 10, 0)
        L.orca_sched_submit(s, 1, 0.0, 3, 5, 5)
        with pytest.raises(L.OrcaError):
            L.orca_sched_submit(s, 1, 0.0, 3, 5, 5)       # duplicate id
        with pytest.raises(L.OrcaError):
            L.orca_sched_step(s, 0.0, 3)                   # cap < max_batch
        with pytest.raises(L.OrcaError):
            L.orca_sched_submit(s, 2, 0.0, 11, 5, 5)       # prompt above the budget
        with pytest.raises(L.OrcaError):
            L.orca_sched_cancel(s, 99)                     # unknown id
        L.orca_sched_cancel(s, 1)
        with pytest.raises(L.OrcaError):
            L.orca_sched_cancel(s, 1)                      # twice
        L.orca_sched_destroy(s)
        s = L.orca_sched_create(kv, 4, 10, L.ORCA_POLICY_CHUNKED)
        L.orca_sched_submit(s, 2, 0.0, 11, 5, 5)           # chunked: accepted
        L.orca_sched_destroy(s)
    finally:
        L.orca_kv_destroy(kv)


# ------------------------------------------ validation before any GPU call

def test_engine_validation_fails_before_gpu():
    w = {k: 16 for k in L.LAYER_KEYS}                      # fake addresses: never read
    with pytest.raises(L.OrcaError) as e:
        L.orca_create(1, 64, 4, 256, L.ORCA_F32, 1e-5, 0, [w], 16, None, 8, 4)
    assert e.value.status == L.ORCA_ERR_INVALID
    with pytest.raises(L.OrcaError) as e:                  # d = 32 not supported in bf16
        L.orca_create(1, 128, 4, 256, L.ORCA_BF16, 1e-5, 64, [w], 16, None, 8, 4)
    assert e.value.status == L.ORCA_ERR_UNSUPPORTED
    kv = L.orca_kv_create(50)
    try:
        with pytest.raises(L.OrcaError) as e:              # capacity mismatch
            L.orca_create(1, 64, 4, 256, L.ORCA_F32, 1e-5, 64, [w], 16, kv, 8, 4)
        assert "capacity" in str(e.value)
    finally:
        L.orca_kv_destroy(kv)


def test_op_validation_fails_before_gpu():
    with pytest.raises(L.OrcaError) as e:
        L.orca_op_linear(L.ORCA_BF16, L.ORCA_EPI_BIAS, 16, 16, 16, 16, 8, 100, 64)
    assert e.value.status == L.ORCA_ERR_UNSUPPORTED
    with pytest.raises(L.OrcaError) as e:
        L.orca_op_linear(L.ORCA_BF16, 9, 16, 16, 16, 16, 8, 128, 64)
    assert e.value.status == L.ORCA_ERR_INVALID
    with pytest.raises(L.OrcaError) as e:
        L.orca_op_layernorm(L.ORCA_F32, 16, 16, 16, 16, 4, 12292, 1e-5)
    assert e.value.status == L.ORCA_ERR_INVALID
    with pytest.raises(L.OrcaError) as e:
        L.orca_op_qkv(L.ORCA_BF16, 16, 16, 16, 16, 16, 16, 4, 256, 8, 100)
    assert e.value.status == L.ORCA_ERR_UNSUPPORTED          # head dim 32 in bf16


# the launch planner's kernel form (orca_op_linear_variant, host only): the
# forms measured fastest on MI355X at these shapes (12 / 13: four-wave
# 256 x 256 / 256 x 192; 10: split-K; 7: eight-wave 128 x 128), and the
# fallbacks of an odd K-step count (13 -> 8, 12 -> 6 -> 3)
@pytest.mark.parametrize("m,n,k,variant", [
    (2176, 15360, 5120, 13), (2176, 5120, 5120, 13),        # 13B QKV, output projection
    (2176, 20480, 5120, 12), (2176, 5120, 20480, 13),       # 13B FFN1, FFN2
    (3698, 36864, 12288, 12), (3698, 12288, 12288, 12),     # 175B layer shapes
    (3698, 49152, 12288, 12), (3698, 12288, 49152, 12),
    (64, 15360, 5120, 10), (64, 20480, 5120, 10),           # few rows: split-K
    (1100, 15360, 5120, 13), (1100, 20480, 5120, 12), (1100, 5120, 5120, 10),
    (1600, 15360, 5120, 12), (1600, 20480, 5120, 13), (1600, 5120, 20480, 13),
    (2176, 15360, 5184, 8), (2176, 20480, 5184, 3),         # 81 K steps
])
def test_planner_variant(m, n, k, variant, monkeypatch):
    monkeypatch.delenv("ORCA_GEMM_VARIANT", raising=False)
    assert L.orca_op_linear_variant(L.ORCA_BF16, m, n, k) == variant


# the prefill form (host only): 64-key steps, two workgroups per CU, up to two
# rounds of tiles; 32-key steps, three per CU, above (13B: two 1,024-token
# prompts over 40 heads, 16 tiles; the 175B-layer seed-0 mix: 31 tiles over
# 96 heads)
def test_prefill_form(monkeypatch):
    monkeypatch.delenv("ORCA_PF_KEYS", raising=False)
    assert L.orca_op_prefill_keys(40, 16) == 64
    assert L.orca_op_prefill_keys(96, 31) == 32
    assert L.orca_op_prefill_keys(16, 4) == 64
    assert L.orca_op_prefill_keys(1024, 1) == 64 and L.orca_op_prefill_keys(1025, 1) == 32
    monkeypatch.setenv("ORCA_PF_KEYS", "64")
    assert L.orca_op_prefill_keys(96, 31) == 64
    monkeypatch.setenv("ORCA_PF_KEYS", "32")
    assert L.orca_op_prefill_keys(40, 16) == 32
    assert L.orca_op_prefill_keys(0, 1) == -2 and L.orca_op_prefill_keys(4, -1) == -2


# the prefill launch's workgroup order (host only).  Every (tile, head) of
# the batch's initiation requests appears once.  Up to two rounds of
# two-per-CU workgroups the tiles run longest-first (by cached prefix + last
# query row) with the heads of one tile adjacent; beyond, each (request,
# head)'s tiles sit on one XCD (workgroup j on XCD j % 8), the XCDs take
# equal workgroup counts, and their work (sum of tile ends) is balanced.
def _prefill_batch(rng, n):
    reqs, off = [], 0
    for _ in range(n):
        phase = L.ORCA_INITIATION if rng.random() < 0.7 else L.ORCA_INCREMENT
        q = int(rng.integers(1, 1100)) if phase == L.ORCA_INITIATION else 1
        kv = int(rng.integers(0, 600)) if rng.random() < 0.3 else 0
        reqs.append((off, q, kv, phase, 0))
        off += q
    return reqs


def _prefill_tiles(reqs):
    return [(i, q0, r[2] + min(r[1], q0 + 128)) for i, r in enumerate(reqs)
            if r[3] == L.ORCA_INITIATION for q0 in range(0, r[1], 128)]


@pytest.mark.parametrize("seed", range(8))
def test_prefill_order(seed, monkeypatch):
    monkeypatch.delenv("ORCA_PF_ORDER", raising=False)
    rng = np.random.default_rng(300 + seed)
    reqs = _prefill_batch(rng, int(rng.integers(1, 12)))
    tiles = _prefill_tiles(reqs)
    end = {(r, q0): e for r, q0, e in tiles}
    heads = int(rng.integers(1, 130))
    got = L.orca_op_prefill_order(reqs, heads)
    assert sorted(got) == sorted((r, q0, h) for r, q0, _ in tiles for h in range(heads))
    if len(tiles) * heads <= 1024:
        ends = [end[(r, q0)] for r, q0, h in got]
        assert ends == sorted(ends, reverse=True)
        assert [h for _, _, h in got] == [j % heads for j in range(len(got))]
        return
    n = len(got)
    xcd = {}
    for j, (r, q0, h) in enumerate(got):
        xcd.setdefault((r, h), set()).add(j % 8)
    # only the tiles moved to even out the counts leave their group's XCD
    split = sum(len(v) > 1 for v in xcd.values())
    assert split <= 8, split
    work = [0] * 8
    for j, (r, q0, h) in enumerate(got):
        work[j % 8] += end[(r, q0)]
    biggest = max(sum(end[(r, q0)] for q0 in range(0, reqs[r][1], 128)) for r, _, _ in tiles)
    assert max(work) - min(work) <= 2 * biggest


def test_prefill_order_forms(monkeypatch):
    monkeypatch.delenv("ORCA_PF_ORDER", raising=False)
    # the 175B-layer seed-0 prompt mix over 96 heads: grouped; two
    # 1,024-token prompts over 40 heads: longest-first
    mix = [891, 699, 586, 369, 404, 164, 195, 142]
    reqs = [(0, q, 0, L.ORCA_INITIATION, 0) for q in mix]
    got = L.orca_op_prefill_order(reqs, 96)
    assert len(got) == 31 * 96
    assert {j % 8 for j, (r, q0, h) in enumerate(got) if (r, h) == (0, 5)} == {got.index((0, 0, 5)) % 8}
    two = [(0, 1024, 0, L.ORCA_INITIATION, 0), (1024, 1024, 0, L.ORCA_INITIATION, 0)]
    got = L.orca_op_prefill_order(two, 40)
    assert got[:3] == [(0, 896, 0), (0, 896, 1), (0, 896, 2)] and got[40] == (1, 896, 0)
    monkeypatch.setenv("ORCA_PF_ORDER", "1")
    got = L.orca_op_prefill_order(two, 40)
    assert len({j % 8 for j, (r, q0, h) in enumerate(got) if (r, h) == (1, 7)}) == 1
    monkeypatch.setenv("ORCA_PF_ORDER", "0")
    got = L.orca_op_prefill_order(reqs, 96)
    assert got[:2] == [(0, 768, 0), (0, 768, 1)]
    # increments take no prefill tile; invalid arguments
    assert L.orca_op_prefill_order([(0, 1, 5, L.ORCA_INCREMENT, 0)], 8) == []
    with pytest.raises(L.OrcaError):
        L.orca_op_prefill_order(two, 0)
    with pytest.raises(L.OrcaError):
        L.orca_op_prefill_order([(0, -1, 0, L.ORCA_INITIATION, 0)], 4)


def test_planner_variant_pin_and_rejects(monkeypatch):
    monkeypatch.setenv("ORCA_GEMM_VARIANT", "7")
    assert L.orca_op_linear_variant(L.ORCA_BF16, 2176, 20480, 5120) == 7
    monkeypatch.setenv("ORCA_GEMM_VARIANT", "12")
    assert L.orca_op_linear_variant(L.ORCA_BF16, 300, 1024, 192) == 3   # 3 K steps: 6, then 3
    # the LDS-DMA forms take any K step count; past 2^31 elements they fall
    # back like the register-staged ones
    monkeypatch.setenv("ORCA_GEMM_VARIANT", "14")
    assert L.orca_op_linear_variant(L.ORCA_BF16, 300, 1024, 192) == 14
    assert L.orca_op_linear_variant(L.ORCA_BF16, 300, 1 << 19, 4096) == 6
    monkeypatch.setenv("ORCA_GEMM_VARIANT", "15")
    assert L.orca_op_linear_variant(L.ORCA_BF16, 300, 1024, 192) == 15
    assert L.orca_op_linear_variant(L.ORCA_BF16, 300, 1 << 19, 4096) == 8
    # split-K pinned where no split applies (an odd K-step count, too short a
    # K for the 256 x 256 split): a tiled form and no workspace
    monkeypatch.setenv("ORCA_GEMM_VARIANT", "10")
    assert L.orca_op_linear_variant(L.ORCA_BF16, 300, 1024, 192) in (7, 12, 13)
    assert L.orca_op_linear_workspace_bytes(L.ORCA_BF16, 300, 1024, 192) == 0
    assert L.orca_op_linear_variant(L.ORCA_BF16, 2176, 20480, 5184) in (3, 7, 8, 12, 13)
    assert L.orca_op_linear_workspace_bytes(L.ORCA_BF16, 2176, 20480, 5184) == 0
    monkeypatch.delenv("ORCA_GEMM_VARIANT")
    assert L.orca_op_linear_variant(L.ORCA_F32, 64, 128, 64) == -1
    assert L.orca_op_linear_variant(L.ORCA_BF16, 64, 100, 64) == -2
    assert L.orca_op_linear_variant(L.ORCA_BF16, 0, 128, 64) == -2


# the launch planner's split-K choice, seen through the workspace it asks for
# (split-K planes are fp32 [splits][m][n]; 0 bytes means a tiled launch)
@pytest.mark.parametrize("m,n,k,splits", [
    (64, 15360, 5120, 2),    # 13B QKV at 64 rows: 120 column tiles, one round at 2 splits
    (64, 5120, 5120, 6),     # output projection: 40 tiles x 6 splits = 240 workgroups
    (64, 20480, 5120, 3),    # FFN1: 160 tiles; 3 splits beat 2 (imbalanced) and 4 (two rounds)
    (64, 5120, 20480, 6),    # FFN2
    (16, 15360, 5120, 2),
    (2176, 20480, 5120, 0),  # the 13B mixed batch: tiles fill the GPU, no split
    (4096, 5120, 5120, 0),
])
def test_planner_split_counts(m, n, k, splits):
    assert L.orca_op_linear_workspace_bytes(L.ORCA_BF16, m, n, k) == splits * m * n * 4
    assert L.orca_op_linear_workspace_bytes(L.ORCA_F32, m, n, k) == 0


# the split tail of the four-wave launches, seen through its workspace
# (fp32 partial tiles of 256 x 256 or 256 x 192): when the last round of 256
# workgroups is at most half full, tail tiles x splits of them; fuller, a
# main-and-helper tail leaves two per tail tile, where it saves 64 K steps
# or more
@pytest.mark.parametrize("m,n,k,slots,bn", [
    (3698, 36864, 12288, 112 * 2, 256),   # 175B layer QKV: 2,160 tiles = 8 rounds + 112
    (3698, 49152, 12288, 64 * 4, 256),    # FFN1: 2,880 = 11 rounds + 64
    (3698, 12288, 12288, 0, 256),         # output projection: 720 = 2 rounds + 208, 192 steps
    (3698, 12288, 49152, 2 * 208, 256),   # FFN2: the same tiles, 768 steps: 644 a main
    (2176, 15360, 5120, 0, 192),          # 13B: 720 tiles, 2 rounds + 208, 80 steps
    (1100, 15360, 4096, 44 * 4, 256),     # the GPU tests' shapes
])
def test_planner_split_tail(m, n, k, slots, bn, monkeypatch):
    monkeypatch.delenv("ORCA_GEMM_TAIL", raising=False)
    monkeypatch.delenv("ORCA_GEMM_SK_MIN", raising=False)
    if (m, n, k) == (1100, 15360, 4096):
        monkeypatch.setenv("ORCA_GEMM_VARIANT", "12")
    else:
        monkeypatch.delenv("ORCA_GEMM_VARIANT", raising=False)
    assert L.orca_op_linear_workspace_bytes(L.ORCA_BF16, m, n, k) == slots * 256 * bn * 4
    monkeypatch.setenv("ORCA_GEMM_TAIL", "0")
    assert L.orca_op_linear_workspace_bytes(L.ORCA_BF16, m, n, k) == 0


# main-and-helper tails below the default threshold (ORCA_GEMM_SK_MIN=0)
@pytest.mark.parametrize("m,n,k,variant,slots,bn", [
    (1100, 20480, 2048, "12", 2 * 144, 256),   # 400 tiles = 256 + 144, 32 steps a tile
    (1100, 15168, 2560, "13", 2 * 139, 192),   # 395 = 256 + 139, 40 steps
    (1100, 20032, 2048, "12", 2 * 139, 256),   # 395 (last column tile 64 wide)
])
def test_planner_main_helper_tail(m, n, k, variant, slots, bn, monkeypatch):
    monkeypatch.delenv("ORCA_GEMM_TAIL", raising=False)
    monkeypatch.setenv("ORCA_GEMM_VARIANT", variant)
    monkeypatch.setenv("ORCA_GEMM_SK_MIN", "0")
    assert L.orca_op_linear_workspace_bytes(L.ORCA_BF16, m, n, k) == slots * 256 * bn * 4
    monkeypatch.delenv("ORCA_GEMM_SK_MIN")
    assert L.orca_op_linear_workspace_bytes(L.ORCA_BF16, m, n, k) == 0
