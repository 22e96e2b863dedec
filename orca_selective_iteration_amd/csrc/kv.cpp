#include "kv.h"

#include <new>

#include "status.h"

int64_t orca_kv::alloc(int64_t n) {
  for (auto it = free_ranges.begin(); it != free_ranges.end(); ++it) {
    if (it->second < n) continue;
    const int64_t base = it->first, len = it->second;
    free_ranges.erase(it);
    if (len > n) free_ranges.emplace(base + n, len - n);
    live.emplace(base, n);
    used += n;
    return base;
  }
  return -1;
}

bool orca_kv::release(int64_t base) {
  auto it = live.find(base);
  if (it == live.end()) return false;
  int64_t start = base, len = it->second;
  live.erase(it);
  used -= len;
  auto next = free_ranges.lower_bound(start);
  if (next != free_ranges.end() && start + len == next->first) {  // merge right
    len += next->second;
    next = free_ranges.erase(next);
  }
  if (next != free_ranges.begin()) {                                 // merge left
    auto prev = std::prev(next);
    if (prev->first + prev->second == start) {
      start = prev->first;
      len += prev->second;
      free_ranges.erase(prev);
    }
  }
  free_ranges.emplace(start, len);
  return true;
}

bool orca_kv::covers(int64_t lo, int64_t hi) const {
  auto it = live.upper_bound(lo);
  if (it == live.begin()) return false;
  --it;
  return it->first <= lo && hi <= it->first + it->second;
}

extern "C" {

orca_status orca_kv_create(int64_t capacity, orca_kv** out) {
  ORCA_CHECK_ARG(out != nullptr, "orca_kv_create: out is NULL");
  ORCA_CHECK_ARG(capacity >= 0, "orca_kv_create: capacity %lld < 0", (long long)capacity);
  auto* kv = new (std::nothrow) orca_kv;
  ORCA_CHECK_ARG(kv != nullptr, "orca_kv_create: out of host memory");
  kv->capacity = capacity;
  if (capacity > 0) kv->free_ranges.emplace(0, capacity);
  *out = kv;
  return ORCA_OK;
}

void orca_kv_destroy(orca_kv* kv) { delete kv; }

orca_status orca_kv_alloc(orca_kv* kv, int64_t n_tokens, int64_t* out_base) {
  ORCA_CHECK_ARG(kv && out_base, "orca_kv_alloc: NULL argument");
  ORCA_CHECK_ARG(n_tokens >= 1, "orca_kv_alloc: n_tokens %lld < 1", (long long)n_tokens);
  const int64_t base = kv->alloc(n_tokens);
  if (base < 0) {
    orca::set_error("orca_kv_alloc: no free range of %lld slots", (long long)n_tokens);
    return ORCA_ERR_NOSPACE;
  }
  *out_base = base;
  return ORCA_OK;
}

orca_status orca_kv_free(orca_kv* kv, int64_t base) {
  ORCA_CHECK_ARG(kv != nullptr, "orca_kv_free: NULL allocator");
  ORCA_CHECK_ARG(kv->release(base), "orca_kv_free: %lld starts no reservation", (long long)base);
  return ORCA_OK;
}

int64_t orca_kv_used(const orca_kv* kv) { return kv ? kv->used : -1; }
int64_t orca_kv_capacity(const orca_kv* kv) { return kv ? kv->capacity : -1; }

int64_t orca_kv_reservation(const orca_kv* kv, int64_t base) {
  if (!kv) return -1;
  auto it = kv->live.find(base);
  return it == kv->live.end() ? -1 : it->second;
}

}  // extern "C"
