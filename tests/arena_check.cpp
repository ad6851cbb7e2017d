// Randomised check of the store's token-span allocator (arena.h) against a
// brute-force model: a map of every arena token (free or the id of the span
// that holds it).  Usage: arena_check <seed> <ops>; prints "ok" or the first
// disagreement and exits non-zero.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "arena.h"

namespace {

struct Model {
  std::vector<int> owner;   // per token: -1 free, else span id
  explicit Model(int64_t cap) : owner((size_t)cap, -1) {}
  // end of the used part: one past the highest token in use
  int64_t used_end() const {
    for (int64_t t = (int64_t)owner.size(); t > 0; --t)
      if (owner[(size_t)t - 1] >= 0) return t;
    return 0;
  }
  // maximal free runs below the used end, in arena order
  is::FreeSpans runs() const {
    is::FreeSpans r;
    const int64_t end = used_end();
    for (int64_t t = 0; t < end;) {
      if (owner[(size_t)t] >= 0) { ++t; continue; }
      int64_t u = t;
      while (u < end && owner[(size_t)u] < 0) ++u;
      r.emplace(t, u - t);
      t = u;
    }
    return r;
  }
  // where first fit must place n tokens, or -1
  int64_t expect(int64_t n, int64_t cap) const {
    for (const auto& kv : runs())
      if (kv.second >= n) return kv.first;
    const int64_t end = used_end();
    return end + n <= cap ? end : -1;
  }
};

}  // namespace

int main(int argc, char** argv) {
  if (argc < 3) return 2;
  std::mt19937_64 rng(std::strtoull(argv[1], nullptr, 10));
  const int ops = std::atoi(argv[2]);
  const int64_t cap = 64 + (int64_t)(rng() % 512);
  Model m(cap);
  is::FreeSpans spans;
  int64_t next = 0;
  struct Span { int64_t at, n; };
  std::vector<Span> live;
  int id = 0;
  for (int op = 0; op < ops; ++op) {
    const bool do_alloc = live.empty() || rng() % 100 < 55;
    if (do_alloc) {
      const int64_t n = 1 + (int64_t)(rng() % 48);
      const int64_t want = m.expect(n, cap);
      const int64_t got = is::arena_alloc(spans, next, cap, n);
      if (got != want) {
        std::printf("op %d: alloc %lld -> %lld, expected %lld\n", op, (long long)n,
                    (long long)got, (long long)want);
        return 1;
      }
      if (got >= 0) {
        for (int64_t t = got; t < got + n; ++t) {
          if (m.owner[(size_t)t] >= 0) {
            std::printf("op %d: token %lld handed out twice\n", op, (long long)t);
            return 1;
          }
          m.owner[(size_t)t] = id;
        }
        live.push_back({got, n});
        ++id;
      }
    } else {
      const size_t k = (size_t)(rng() % live.size());
      const Span sp = live[k];
      live.erase(live.begin() + (long)k);
      for (int64_t t = sp.at; t < sp.at + sp.n; ++t) m.owner[(size_t)t] = -1;
      is::arena_free(spans, next, sp.at, sp.n);
    }
    if (next != m.used_end()) {
      std::printf("op %d: used end %lld, expected %lld\n", op, (long long)next,
                  (long long)m.used_end());
      return 1;
    }
    if (spans != m.runs()) {
      std::printf("op %d: free spans differ from the model's free runs\n", op);
      return 1;
    }
  }
  std::printf("ok\n");
  return 0;
}
