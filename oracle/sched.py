"""Oracle: iteration-level scheduling, the request-level baseline, and the
token allocator of the Attention K/V manager.  Plain Python, CPU only.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
  [houmin]   garden.houmin.site/infra/orca, 3.1.1 (iteration-level
             scheduling): after every iteration the scheduler removes finished
             requests and may admit new ones, so a new request waits at most
             one iteration; a request's K/V cache is released as soon as it
             finishes ("algorithm" paragraph).
  [0h-n0]    0h-n0.github.io Orca digest, "Scheduler algorithm": FCFS
             admission while the batch is below max_batch, reserving
             prompt_length + max_tokens K/V slots per admitted request and
             stopping (break, no skipping) at the first request that does not
             fit; "Request-Level vs Iteration-Level Scheduling": a static
             batch lasts max_i T_gen(r_i) iterations.
  [arcsin2]  unpurerationalist.github.io ORCA notes 4.2: the scheduler weighs
             max batch size, free K/V capacity and FCFS order; max_tokens is a
             per-request attribute used to pre-allocate K/V.
  [ultralytics] ultralytics.com glossary "Continuous Batching": engines also
             cap the tokens processed per step (max_num_batched_tokens); the
             8-request, 4-slot example (static 90 steps / 43% busy,
             continuous 50 steps / 78% busy).
  [estelledc] estelledc.github.io Orca notes, case 1: A=100, B=10, C=50 on
             three slots; D joins at step 11, E at 51, F at 101.
  [houmin-cancel] garden.houmin.site/infra/orca 3.1.1, scheduling workflow:
             Orca leaves cancelled requests unhandled; they should leave the
             batch promptly and their memory be released.
  [ultralytics-chunk] ultralytics.com glossary "Continuous Batching", limits
             and combined techniques: chunked prefill splits long prompts so
             a newcomer's prefill does not stall the others' decoding.

Readings where the pages leave a step open:
  * release exactly what was reserved (prompt + max_tokens); the digest's
    release of the current length would leak slots;
  * the token budget counts q_len over the batch: the prompt of each admitted
    request plus one row per continuing request; a prompt longer than the
    budget is rejected at submit because FCFS would block on it forever;
  * admission needs the slot count to fit AND a contiguous first-fit range;
    either miss ends admission for this iteration (break);
  * the batch lists continuing requests (increments) in admission order,
    then this iteration's admissions, as the figure lists x1, x2 | x3, x4;
  * a request with output length n is active for exactly n iterations; its
    first output token comes from its initiation iteration;
  * request-level (static) policy: a new batch forms only when the engine
    holds none; members that finished keep their slot idle (not computed)
    until the last member finishes, then all are released together;
  * time is an explicit argument: step(now) admits requests with
    arrival <= now;
  * cancel(id) drops a queued request at once; an admitted one leaves at the
    next step's eviction like a finished one (K/V released then, under every
    policy), so the batch the engine may still be running is never changed
    under it;
  * "chunked" policy (iteration-level with chunked prefill): a prompt is
    split across iterations so every batch fills the token budget; rows are
    ordered increments, then continuing prompt chunks, then this step's
    admissions (each group in admission order); a continuing prompt takes
    what the budget leaves after the increments, in admission order; a new
    request is admitted while any budget is left (its first chunk may be a
    single token), the K/V checks and the break on a miss unchanged; a chunk
    after the first is an initiation whose kv_len is the prompt tokens
    already cached; a prompt longer than the budget is accepted;
  * one accounting rule for every policy: after an iteration a member's
    kv_len grows by its q_len, and it has produced a token iff its prompt is
    then complete (its first token comes with its last prompt chunk).
"""
from __future__ import annotations

import heapq
from collections import deque
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

INITIATION = 0
INCREMENT = 1


class FirstFitAllocator:
    """Token-granular allocator over [0, capacity): lowest-base first fit,
    free coalesces with both neighbours.

    [0h-n0] Implementation notes: the K/V pool is allocated once at start-up
    (dynamic device malloc/free is too slow) and an index table records where
    every request's entries live.
    """

    def __init__(self, capacity: int):
        assert capacity >= 0
        self.capacity = capacity
        self.free_list: List[Tuple[int, int]] = [(0, capacity)] if capacity else []
        self.live: Dict[int, int] = {}

    def alloc(self, n: int) -> Optional[int]:
        if n <= 0:
            return None
        for i, (start, length) in enumerate(self.free_list):
            if length >= n:
                if length == n:
                    del self.free_list[i]
                else:
                    self.free_list[i] = (start + n, length - n)
                self.live[start] = n
                return start
        return None

    def free(self, base: int) -> None:
        n = self.live.pop(base)          # KeyError on unknown base / double free
        self.free_list.append((base, n))
        self.free_list.sort()
        merged: List[Tuple[int, int]] = []
        for s, l in self.free_list:
            if merged and merged[-1][0] + merged[-1][1] == s:
                merged[-1] = (merged[-1][0], merged[-1][1] + l)
            else:
                merged.append((s, l))
        self.free_list = merged

    def used(self) -> int:
        return sum(self.live.values())


@dataclass
class Request:
    id: int
    arrival: float
    prompt_len: int
    max_tokens: int
    out_len: int            # hidden from the policy: plays the role of EOS
    generated: int = 0
    kv_len: int = 0
    kv_base: int = -1
    admitted_at: int = -1   # iteration index (0-based) of its initiation
    finished_at: int = -1   # iteration index that produced its last token
    released_at: int = -1   # iteration index at whose start it was evicted
    cancelled: bool = False

    @property
    def reserved(self) -> int:
        return self.prompt_len + self.max_tokens

    @property
    def done(self) -> bool:
        return self.generated >= self.out_len

    @property
    def prefilled(self) -> bool:
        return self.kv_len >= self.prompt_len

    @property
    def gone(self) -> bool:
        """Nothing left to compute: finished or cancelled."""
        return self.done or self.cancelled


@dataclass(frozen=True)
class BatchEntry:
    id: int
    q_offset: int
    q_len: int
    kv_len: int
    phase: int
    kv_base: int


class Scheduler:
    """Iteration-level ("iteration") or request-level ("static") scheduler.

    step(now) returns the batch the engine runs next; calling step again means
    that batch has run: every member has produced one token and its K/V length
    grew by its q_len ([houmin] 3.1.1 workflow: the engine returns one output
    token per request and the scheduler appends it).
    """

    def __init__(self, max_batch: int, token_budget: int, kv_slots: int,
                 policy: str = "iteration"):
        assert policy in ("iteration", "static", "chunked")
        assert max_batch >= 1 and token_budget >= 1 and kv_slots >= 0
        self.max_batch = max_batch
        self.token_budget = token_budget
        self.kv_slots = kv_slots
        self.policy = policy
        self.alloc = FirstFitAllocator(kv_slots)
        self.used = 0
        self.pending: List[Tuple[float, int, Request]] = []   # heap by (arrival, id)
        self.waiting: deque = deque()
        self.active: List[Request] = []
        self.last: List[Tuple[Request, int]] = []            # (request, q_len)
        self.iteration = 0                                   # batches emitted
        self.requests: Dict[int, Request] = {}

    # ------------------------------------------------------------------ submit
    def submit(self, rid: int, arrival: float, prompt_len: int, max_tokens: int,
               out_len: int) -> bool:
        """Queue a request; False (rejected) if it could never be admitted."""
        if rid in self.requests or prompt_len < 1 or max_tokens < 1:
            return False
        if out_len < 1 or out_len > max_tokens:
            return False
        if prompt_len + max_tokens > self.kv_slots:
            return False
        if self.policy != "chunked" and prompt_len > self.token_budget:
            return False
        r = Request(rid, arrival, prompt_len, max_tokens, out_len)
        self.requests[rid] = r
        heapq.heappush(self.pending, (arrival, rid, r))
        return True

    # ------------------------------------------------------------------ cancel
    def cancel(self, rid: int) -> bool:
        """Withdraw a request ([houmin-cancel]).  False if it is unknown,
        already released or already cancelled."""
        r = self.requests.get(rid)
        if r is None or r.cancelled or r.released_at >= 0:
            return False
        if r.admitted_at < 0:                    # still queued: drop it now
            r.cancelled = True
            if r in self.waiting:
                self.waiting.remove(r)
            else:
                self.pending = [e for e in self.pending if e[2] is not r]
                heapq.heapify(self.pending)
            return True
        r.cancelled = True                       # admitted: leaves at the next step
        return True

    # -------------------------------------------------------------------- step
    def step(self, now: float) -> List[BatchEntry]:
        # the previous batch has run: K/V grew by q_len; a member whose prompt
        # is now complete produced one token
        for r, q_len in self.last:
            r.kv_len += q_len
            if r.prefilled:
                r.generated += 1
                if r.done:
                    r.finished_at = self.iteration - 1
        self.last = []

        # 1. evict finished and cancelled requests, release their K/V at once
        #    ([houmin] 3.1.1); the static policy keeps finished members until
        #    the whole batch is through
        if self.policy == "static":
            whole = all(r.gone for r in self.active)
            leaving = [r for r in self.active if r.cancelled or whole]
        else:
            leaving = [r for r in self.active if r.gone]
        for r in leaving:
            self.alloc.free(r.kv_base)
            self.used -= r.reserved
            r.released_at = self.iteration
        self.active = [r for r in self.active if r not in leaving]

        # 2. requests that have arrived join the FCFS queue
        while self.pending and self.pending[0][0] <= now:
            self.waiting.append(heapq.heappop(self.pending)[2])

        # 3. rows already committed: one per decoding request, then the
        #    chunks of prompts still being prefilled (chunked policy)
        running = [r for r in self.active if not r.gone and r.prefilled]
        tok = len(running)
        chunks: List[Tuple[Request, int]] = []
        for r in self.active:
            if not r.gone and not r.prefilled:
                q = min(r.prompt_len - r.kv_len, self.token_budget - tok)
                if q > 0:
                    chunks.append((r, q))
                    tok += q

        # 4. FCFS admission, stop at the first miss ([0h-n0] scheduler algorithm)
        admitted: List[Tuple[Request, int]] = []
        if self.policy != "static" or not self.active:
            while self.waiting and len(self.active) + len(admitted) < self.max_batch:
                c = self.waiting[0]
                if self.policy == "chunked":
                    q = min(c.prompt_len, self.token_budget - tok)
                    if q <= 0:
                        break
                else:
                    q = c.prompt_len
                    if tok + q > self.token_budget:
                        break
                if self.used + c.reserved > self.kv_slots:
                    break
                base = self.alloc.alloc(c.reserved)
                if base is None:
                    break
                self.waiting.popleft()
                c.kv_base = base
                c.admitted_at = self.iteration
                self.used += c.reserved
                tok += q
                admitted.append((c, q))
        self.active.extend(c for c, _ in admitted)

        # 5. emit: increments (admission order), continuing prompt chunks, then
        #    this step's initiations
        batch: List[BatchEntry] = []
        off = 0
        for r in running:
            batch.append(BatchEntry(r.id, off, 1, r.kv_len, INCREMENT, r.kv_base))
            self.last.append((r, 1))
            off += 1
        for r, q in chunks + admitted:
            batch.append(BatchEntry(r.id, off, q, r.kv_len, INITIATION, r.kv_base))
            self.last.append((r, q))
            off += q
        if batch:
            self.iteration += 1
        return batch

    def idle(self) -> bool:
        """True when nothing is queued, waiting or active."""
        return not self.pending and not self.waiting and not self.active

    def next_arrival(self) -> Optional[float]:
        return self.pending[0][0] if self.pending else None


@dataclass
class TraceResult:
    iterations: int = 0
    busy_rows: int = 0                 # increment + initiation requests computed
    tokens_processed: int = 0          # sum of q_len over all iterations
    log: List[Tuple[float, Tuple[int, ...], Tuple[int, ...]]] = field(default_factory=list)


def run_trace(sched: Scheduler, dt=lambda batch: 1.0, now: float = 0.0,
              max_iterations: int = 10**9) -> TraceResult:
    """Drive a scheduler until every submitted request has been released.

    The clock starts at `now`; each non-empty iteration advances it by
    dt(batch); an empty step with requests still to arrive jumps the clock to
    the next arrival.  The log holds (now, ids in the batch, phases).
    """
    res = TraceResult()
    while res.iterations < max_iterations:
        batch = sched.step(now)
        if not batch:
            if sched.idle():
                break
            nxt = sched.next_arrival()
            if nxt is None:
                # active requests with nothing left to compute cannot exist:
                # every active request is computed until it is done
                raise RuntimeError("scheduler stalled")
            now = max(now, nxt)
            continue
        res.iterations += 1
        res.busy_rows += len(batch)
        res.tokens_processed += sum(e.q_len for e in batch)
        res.log.append((now, tuple(e.id for e in batch), tuple(e.phase for e in batch)))
        now += dt(batch)
    return res
