// Iteration-level scheduler and the request-level (static) baseline.
//
// garden.houmin.site/infra/orca 3.1.1: after every iteration the scheduler
// drops finished requests (releasing their K/V at once) and may admit new
// ones, so a newcomer waits at most one iteration.  0h-n0.github.io digest,
// "Scheduler algorithm": FCFS admission below max_batch, reserving
// prompt_length + max_tokens K/V slots, stopping at the first request that
// does not fit.  ultralytics.com glossary, "limits": a cap on the tokens one
// step processes.  Readings: the release returns exactly the reservation;
// the token cap counts q_len over the batch; admission also needs a
// contiguous first-fit range; the batch lists increments (admission order)
// then this step's initiations.  garden.houmin.site/infra/orca 3.1.1,
// scheduling workflow: cancelled requests should leave the batch promptly
// and free their memory.  ultralytics.com glossary, limits and combined
// techniques: chunked prefill splits long prompts across iterations.
// Readings: a cancelled request leaves at the next step's eviction; with
// chunked prefill a prompt chunk takes what the token budget leaves, a chunk
// after the first is an initiation over the cached prefix, and a request
// produces a token in the iteration that completes its prompt.
#include <algorithm>
#include <deque>
#include <memory>
#include <new>
#include <set>
#include <unordered_map>
#include <utility>
#include <vector>

#include "kv.h"
#include "status.h"

namespace {

struct Req {
  int64_t id;
  double arrival;
  int32_t prompt_len, max_tokens, out_len;
  int32_t generated = 0;
  int64_t kv_len = 0;
  int64_t kv_base = -1;
  int64_t admitted_at = -1, finished_at = -1, released_at = -1;
  bool cancelled = false;

  int64_t reserved() const { return int64_t(prompt_len) + max_tokens; }
  bool done() const { return generated >= out_len; }
  bool prefilled() const { return kv_len >= prompt_len; }
  bool gone() const { return done() || cancelled; }
};

}  // namespace

struct orca_sched {
  orca_kv* kv = nullptr;
  int32_t max_batch = 0, token_budget = 0, policy = 0;
  int64_t used = 0;
  int64_t iteration = 0;
  std::unordered_map<int64_t, std::unique_ptr<Req>> reqs;
  std::set<std::pair<double, int64_t>> pending;   // (arrival, id), not yet queued
  std::deque<Req*> waiting;                        // FCFS
  std::vector<Req*> active;                        // admission order
  std::vector<std::pair<Req*, int32_t>> last;      // previous batch, with q_len
};

extern "C" {

orca_status orca_sched_create(orca_kv* kv, int32_t max_batch, int32_t token_budget,
                              int32_t policy, orca_sched** out) {
  ORCA_CHECK_ARG(kv && out, "orca_sched_create: NULL argument");
  ORCA_CHECK_ARG(max_batch >= 1 && token_budget >= 1,
                 "orca_sched_create: max_batch %d / token_budget %d must be >= 1", max_batch,
                 token_budget);
  ORCA_CHECK_ARG(policy == ORCA_POLICY_ITERATION || policy == ORCA_POLICY_STATIC ||
                     policy == ORCA_POLICY_CHUNKED,
                 "orca_sched_create: unknown policy %d", policy);
  ORCA_CHECK_ARG(kv->used == 0, "orca_sched_create: allocator already holds reservations");
  auto* s = new (std::nothrow) orca_sched;
  ORCA_CHECK_ARG(s != nullptr, "orca_sched_create: out of host memory");
  s->kv = kv;
  s->max_batch = max_batch;
  s->token_budget = token_budget;
  s->policy = policy;
  *out = s;
  return ORCA_OK;
}

void orca_sched_destroy(orca_sched* s) {
  if (!s) return;
  for (Req* r : s->active) s->kv->release(r->kv_base);
  delete s;
}

orca_status orca_sched_submit(orca_sched* s, int64_t id, double arrival, int32_t prompt_len,
                              int32_t max_tokens, int32_t out_len) {
  ORCA_CHECK_ARG(s != nullptr, "orca_sched_submit: NULL scheduler");
  ORCA_CHECK_ARG(!s->reqs.count(id), "orca_sched_submit: id %lld already submitted",
                 (long long)id);
  ORCA_CHECK_ARG(prompt_len >= 1 && max_tokens >= 1 && out_len >= 1 && out_len <= max_tokens,
                 "orca_sched_submit: lengths prompt %d max_tokens %d out %d", prompt_len,
                 max_tokens, out_len);
  ORCA_CHECK_ARG(s->policy == ORCA_POLICY_CHUNKED || prompt_len <= s->token_budget,
                 "orca_sched_submit: prompt %d exceeds the token budget %d", prompt_len,
                 s->token_budget);
  ORCA_CHECK_ARG(int64_t(prompt_len) + max_tokens <= s->kv->capacity,
                 "orca_sched_submit: reservation exceeds the K/V capacity");
  auto r = std::make_unique<Req>();
  r->id = id;
  r->arrival = arrival;
  r->prompt_len = prompt_len;
  r->max_tokens = max_tokens;
  r->out_len = out_len;
  s->pending.emplace(arrival, id);
  s->reqs.emplace(id, std::move(r));
  return ORCA_OK;
}

orca_status orca_sched_step(orca_sched* s, double now, orca_req_desc* out, int64_t* out_ids,
                            int32_t cap, int32_t* n_out) {
  ORCA_CHECK_ARG(s && out && out_ids && n_out, "orca_sched_step: NULL argument");
  ORCA_CHECK_ARG(cap >= s->max_batch, "orca_sched_step: cap %d < max_batch %d", cap,
                 s->max_batch);
  // the previous batch ran: K/V grew by q_len; a member whose prompt is now
  // complete produced one token
  for (auto& [r, q_len] : s->last) {
    r->kv_len += q_len;
    if (r->prefilled()) {
      r->generated += 1;
      if (r->done()) r->finished_at = s->iteration - 1;
    }
  }
  s->last.clear();

  // 1. eviction of finished and cancelled requests; release K/V at once
  bool whole = true;
  for (Req* r : s->active) whole &= r->gone();
  std::vector<Req*> keep;
  for (Req* r : s->active) {
    const bool leave =
        s->policy == ORCA_POLICY_STATIC ? (r->cancelled || whole) : r->gone();
    if (leave) {
      s->kv->release(r->kv_base);
      s->used -= r->reserved();
      r->released_at = s->iteration;
    } else {
      keep.push_back(r);
    }
  }
  s->active.swap(keep);

  // 2. arrivals join the FCFS queue
  while (!s->pending.empty() && s->pending.begin()->first <= now) {
    s->waiting.push_back(s->reqs.at(s->pending.begin()->second).get());
    s->pending.erase(s->pending.begin());
  }

  // 3. rows already committed: decoding requests, then the next chunk of
  //    every prompt still being prefilled
  std::vector<Req*> running;
  for (Req* r : s->active)
    if (!r->gone() && r->prefilled()) running.push_back(r);
  int64_t tok = int64_t(running.size());
  std::vector<std::pair<Req*, int32_t>> rows;   // prompt chunks, then admissions
  for (Req* r : s->active) {
    if (r->gone() || r->prefilled()) continue;
    const int64_t q = std::min<int64_t>(r->prompt_len - r->kv_len, s->token_budget - tok);
    if (q > 0) {
      rows.emplace_back(r, int32_t(q));
      tok += q;
    }
  }

  // 4. FCFS admission with break on the first miss
  size_t n_admitted = 0;
  if (s->policy != ORCA_POLICY_STATIC || s->active.empty()) {
    while (!s->waiting.empty() &&
           int64_t(s->active.size() + n_admitted) < s->max_batch) {
      Req* c = s->waiting.front();
      int64_t q = c->prompt_len;
      if (s->policy == ORCA_POLICY_CHUNKED) {
        q = std::min<int64_t>(q, s->token_budget - tok);
        if (q <= 0) break;
      } else if (tok + q > s->token_budget) {
        break;
      }
      if (s->used + c->reserved() > s->kv->capacity) break;
      const int64_t base = s->kv->alloc(c->reserved());
      if (base < 0) break;
      s->waiting.pop_front();
      c->kv_base = base;
      c->admitted_at = s->iteration;
      s->used += c->reserved();
      tok += q;
      rows.emplace_back(c, int32_t(q));
      ++n_admitted;
    }
  }
  for (size_t i = rows.size() - n_admitted; i < rows.size(); ++i)
    s->active.push_back(rows[i].first);

  // 5. emit: increments, continuing prompt chunks, then initiations
  int32_t n = 0, off = 0;
  for (Req* r : running) {
    out[n] = orca_req_desc{off, 1, int32_t(r->kv_len), ORCA_INCREMENT, r->kv_base};
    out_ids[n++] = r->id;
    s->last.emplace_back(r, 1);
    off += 1;
  }
  for (auto& [r, q] : rows) {
    out[n] = orca_req_desc{off, q, int32_t(r->kv_len), ORCA_INITIATION, r->kv_base};
    out_ids[n++] = r->id;
    s->last.emplace_back(r, q);
    off += q;
  }
  if (n > 0) s->iteration += 1;
  *n_out = n;
  return ORCA_OK;
}

orca_status orca_sched_cancel(orca_sched* s, int64_t id) {
  ORCA_CHECK_ARG(s != nullptr, "orca_sched_cancel: NULL scheduler");
  auto it = s->reqs.find(id);
  ORCA_CHECK_ARG(it != s->reqs.end(), "orca_sched_cancel: unknown id %lld", (long long)id);
  Req* r = it->second.get();
  ORCA_CHECK_ARG(!r->cancelled && r->released_at < 0,
                 "orca_sched_cancel: request %lld already %s", (long long)id,
                 r->cancelled ? "cancelled" : "released");
  r->cancelled = true;
  if (r->admitted_at < 0) {   // still queued: drop it now
    auto w = std::find(s->waiting.begin(), s->waiting.end(), r);
    if (w != s->waiting.end()) s->waiting.erase(w);
    else s->pending.erase({r->arrival, r->id});
  }
  return ORCA_OK;
}

int32_t orca_sched_idle(const orca_sched* s) {
  return s && s->pending.empty() && s->waiting.empty() && s->active.empty();
}

orca_status orca_sched_next_arrival(const orca_sched* s, double* t) {
  ORCA_CHECK_ARG(s && t, "orca_sched_next_arrival: NULL argument");
  ORCA_CHECK_ARG(!s->pending.empty(), "orca_sched_next_arrival: nothing pending");
  *t = s->pending.begin()->first;
  return ORCA_OK;
}

orca_status orca_sched_request_info(const orca_sched* s, int64_t id, int64_t* admitted_at,
                                    int64_t* finished_at, int64_t* released_at) {
  ORCA_CHECK_ARG(s && admitted_at && finished_at && released_at,
                 "orca_sched_request_info: NULL argument");
  auto it = s->reqs.find(id);
  ORCA_CHECK_ARG(it != s->reqs.end(), "orca_sched_request_info: unknown id %lld",
                 (long long)id);
  *admitted_at = it->second->admitted_at;
  *finished_at = it->second->finished_at;
  *released_at = it->second->released_at;
  return ORCA_OK;
}

int64_t orca_sched_used(const orca_sched* s) { return s ? s->used : -1; }

}  // extern "C"
