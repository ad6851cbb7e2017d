// Token-span allocation in the store's HBM arenas (host code, no HIP).
//
// Facts appended after creation take a span of tokens of the K and V
// arenas (both at the same offset).  Spans that removed facts leave go to a
// free list kept merged with its neighbours; a span that reaches the end of
// the used part of the arena moves that end back instead.  Allocation is
// first fit over the free list (in arena order), else from the end.
#pragma once

#include <cstdint>
#include <iterator>
#include <map>

namespace is {

// Free spans: start token -> length; no two of them touch, and none ends at
// the end of the used part (`next`).
using FreeSpans = std::map<int64_t, int64_t>;

// n tokens (n >= 1) from the free spans (first fit), else from [next, cap);
// returns the start, or -1 with nothing changed if neither has room.  Works
// on the caller's copies, so a batch of allocations can be dropped whole.
inline int64_t arena_alloc(FreeSpans& spans, int64_t& next, int64_t cap, int64_t n) {
  for (auto it = spans.begin(); it != spans.end(); ++it) {
    if (it->second < n) continue;
    const int64_t at = it->first, rest = it->second - n;
    spans.erase(it);
    if (rest > 0) spans.emplace(at + n, rest);
    return at;
  }
  if (next + n > cap) return -1;
  next += n;
  return next - n;
}

// Returns [at, at + n) (n >= 1, in use) to the arena.
inline void arena_free(FreeSpans& spans, int64_t& next, int64_t at, int64_t n) {
  auto hi = spans.lower_bound(at);
  if (hi != spans.end() && hi->first == at + n) {
    n += hi->second;
    hi = spans.erase(hi);
  }
  if (hi != spans.begin()) {
    auto lo = std::prev(hi);
    if (lo->first + lo->second == at) {
      at = lo->first;
      n += lo->second;
      spans.erase(lo);
    }
  }
  if (at + n == next) {
    next = at;
    return;
  }
  spans.emplace(at, n);
}

}  // namespace is
