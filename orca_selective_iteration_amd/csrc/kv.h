// Attention K/V manager: first-fit token allocator over one pool.
// garden.houmin.site/infra/orca 3.1.1 (release at finish); 0h-n0.github.io
// digest, implementation notes (pool allocated once; index table per request).
#pragma once
#include <cstdint>
#include <map>

struct orca_kv {
  int64_t capacity = 0;
  int64_t used = 0;
  std::map<int64_t, int64_t> free_ranges;  // start -> length, disjoint, coalesced
  std::map<int64_t, int64_t> live;         // base -> length

  // Returns -1 when no free range holds n slots.
  int64_t alloc(int64_t n);
  bool release(int64_t base);
  // Length of the reservation containing [lo, hi), or -1.
  bool covers(int64_t lo, int64_t hi) const;
};
