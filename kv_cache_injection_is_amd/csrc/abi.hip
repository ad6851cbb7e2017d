// C ABI of the library (include/inferscale.h): store placement in HBM and
// pinned host memory, per-call staging of control data, kernel launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <map>
#include <mutex>
#include <vector>

#include "inferscale.h"
#include "kernels.h"
#include "arena.h"
#include "plan.h"

#define IS_EXPORT extern "C" __attribute__((visibility("default")))

namespace is {
const char* last_error_text();
}

namespace {

using is::fail;

// Restores the caller's current device on scope exit.
struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) == hipSuccess && prev != dev) (void)hipSetDevice(dev);
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

int hip_fail(hipError_t e, const char* what) {
  return fail(IS_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// One slot of the per-store staging ring: a device buffer, its pinned host
// mirror, and an event marking the end of the last work that used them.
struct Slot {
  void* dev = nullptr;
  void* host = nullptr;
  size_t cap = 0;
  hipEvent_t done = nullptr;
};

constexpr int kSlots = 4;
constexpr int kTopkSlots = 2;
// Largest cache (in slots) the on-device overlap check covers: its bitmap
// takes slots / 8 bytes of scratch.
constexpr int64_t kDeviceCheckSlots = int64_t(1) << 32;

}  // namespace

// A pinned, device-mapped piece of the host tier holding whole facts
// [f0, f1) back to back.
struct HostChunk {
  void* k = nullptr;
  void* v = nullptr;
  int64_t f0 = 0, f1 = 0;
};

constexpr size_t kHostChunkBytes = size_t(4) << 30;

struct is_store {
  int device = 0;
  int32_t L = 0, H = 0, d = 0, dtype = 0, emb_dim = 0;
  int64_t n_facts = 0, n_hbm = 0;
  int64_t max_facts = 0;          // facts the tables and the embedding arena hold
  int64_t hbm_tokens = 0;         // tokens the HBM arenas hold
  int64_t hbm_next = 0;           // arena tokens below this are (or were) in use
  is::FreeSpans free_spans;       // freed arena token spans: start -> length
  std::vector<int32_t> len;
  // [n_facts + 1]: token offsets of the facts laid back to back in id
  // order (the layout of load sources; the host tier's layout too).  HBM
  // facts need not sit in that order once facts are removed: their
  // addresses are k_addr / v_addr.
  std::vector<int64_t> tok_off;
  size_t es = 0;
  void* k_dev = nullptr;          // HBM arenas, facts [0, n_hbm)
  void* v_dev = nullptr;
  std::vector<HostChunk> host;    // pinned tier, facts [n_hbm, n_facts)
  std::vector<uint64_t> k_addr;   // [n_facts] device-visible block addresses
  std::vector<uint64_t> v_addr;
  uint16_t* emb = nullptr;
  // Device copies of the per-fact tables, for composition on the device.
  int32_t* d_len = nullptr;
  uint64_t* d_k_addr = nullptr;
  uint64_t* d_v_addr = nullptr;
  std::mutex mu;
  Slot slots[kSlots];              // inject staging (device + pinned host)
  int next_slot = 0;
  Slot topk_slots[kTopkSlots];     // top-k scratch (device only)
  // Scratch of captured is_retrieve_inject calls: a graph replays with the
  // addresses it captured, so those calls never take a ring slot (whose
  // reuse is ordered by events that a graph cannot record); eager calls
  // size it until the first capture; from then on it never moves.
  Slot graph_slot;
  bool captured = false;          // a graph holds addresses of this store
  int next_topk_slot = 0;

  int64_t row_elems() const { return (int64_t)L * H * d; }
  // Bytes of the blocked embeddings (whole tiles, padded width).
  size_t emb_bytes() const {
    return (size_t)is::topk_padded_facts(n_facts) * is::topk_padded_dim(emb_dim) * 2;
  }
  size_t emb_alloc_bytes() const {
    return (size_t)is::topk_padded_facts(max_facts) * is::topk_padded_dim(emb_dim) * 2;
  }
  size_t fact_bytes(int64_t f0, int64_t f1) const {
    return (size_t)(tok_off[f1] - tok_off[f0]) * row_elems() * es;
  }
  // Host-side address of fact f's K or V block (for host-tier facts, the
  // pinned host pointer).
  const HostChunk& chunk_of(int64_t f) const {
    size_t lo = 0, hi = host.size() - 1;
    while (lo < hi) {
      const size_t mid = (lo + hi + 1) / 2;
      if (host[mid].f0 <= f) lo = mid; else hi = mid - 1;
    }
    return host[lo];
  }
  char* k_at(int64_t f) const {
    if (f < n_hbm) return reinterpret_cast<char*>((uintptr_t)k_addr[(size_t)f]);
    const HostChunk& c = chunk_of(f);
    return (char*)c.k + fact_bytes(c.f0, f);
  }
  char* v_at(int64_t f) const {
    if (f < n_hbm) return reinterpret_cast<char*>((uintptr_t)v_addr[(size_t)f]);
    const HostChunk& c = chunk_of(f);
    return (char*)c.v + fact_bytes(c.f0, f);
  }
  size_t token_bytes() const { return (size_t)row_elems() * es; }
  // Arena token offset of HBM fact f (K and V sit at the same offset).
  int64_t arena_token(int64_t f) const {
    return (int64_t)(((uintptr_t)k_addr[(size_t)f] - (uintptr_t)k_dev) / token_bytes());
  }
};



namespace {

void free_store(is_store* s) {
  if (s == nullptr) return;
  DeviceGuard g(s->device);
  for (Slot* ring : {s->slots, s->topk_slots}) {
    const int n = ring == s->slots ? kSlots : kTopkSlots;
    for (int i = 0; i < n; ++i) {
      Slot& sl = ring[i];
      if (sl.done) (void)hipEventSynchronize(sl.done);
      if (sl.dev) (void)hipFree(sl.dev);
      if (sl.host) (void)hipHostFree(sl.host);
      if (sl.done) (void)hipEventDestroy(sl.done);
    }
  }
  if (s->graph_slot.dev) (void)hipFree(s->graph_slot.dev);
  if (s->k_dev) (void)hipFree(s->k_dev);
  if (s->v_dev) (void)hipFree(s->v_dev);
  for (HostChunk& c : s->host) {
    if (c.k) (void)hipHostFree(c.k);
    if (c.v) (void)hipHostFree(c.v);
  }
  if (s->emb) (void)hipFree(s->emb);
  if (s->d_len) (void)hipFree(s->d_len);
  if (s->d_k_addr) (void)hipFree(s->d_k_addr);
  if (s->d_v_addr) (void)hipFree(s->d_v_addr);
  delete s;
}

// Takes the next staging slot with room for `bytes`, after the work that
// last used it has finished.  Caller holds s->mu.
// Takes the next slot of a ring once the work that last used it is done,
// growing its buffers to `bytes` (and a pinned host mirror when `host`).
int acquire(Slot* ring, int n, int* next, size_t bytes, bool host, Slot** out) {
  Slot& sl = ring[*next];
  *next = (*next + 1) % n;
  hipError_t e;
  if (sl.done == nullptr) {
    if ((e = hipEventCreateWithFlags(&sl.done, hipEventDisableTiming)) != hipSuccess)
      return hip_fail(e, "hipEventCreate");
  } else if ((e = hipEventSynchronize(sl.done)) != hipSuccess) {
    return hip_fail(e, "hipEventSynchronize");
  }
  if (sl.cap < bytes) {
    if (sl.dev) (void)hipFree(sl.dev);
    if (sl.host) (void)hipHostFree(sl.host);
    sl.dev = sl.host = nullptr;
    sl.cap = 0;
    const size_t cap = std::max<size_t>(bytes + bytes / 4, 1 << 16);
    if (hipMalloc(&sl.dev, cap) != hipSuccess) return fail(IS_ERR_OOM, "staging hipMalloc");
    if (host && hipHostMalloc(&sl.host, cap, hipHostMallocDefault) != hipSuccess) {
      (void)hipFree(sl.dev);
      sl.dev = nullptr;
      return fail(IS_ERR_OOM, "staging hipHostMalloc");
    }
    sl.cap = cap;
  }
  *out = &sl;
  return IS_OK;
}

int acquire_slot(is_store* s, size_t bytes, Slot** out) {
  return acquire(s->slots, kSlots, &s->next_slot, bytes, true, out);
}

int acquire_topk_slot(is_store* s, size_t bytes, Slot** out) {
  return acquire(s->topk_slots, kTopkSlots, &s->next_topk_slot, bytes, false, out);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

is::StoreGeom geom_of(const is_store* s) {
  is::StoreGeom g;
  g.n_layers = s->L;
  g.n_kv_heads = s->H;
  g.head_dim = s->d;
  g.dtype = s->dtype;
  g.n_facts = s->n_facts;
  g.fact_len = s->len.data();
  g.k_addr = s->k_addr.data();
  g.v_addr = s->v_addr.data();
  g.n_hbm = s->n_hbm;
  return g;
}

}  // namespace

IS_EXPORT const char* is_last_error(void) { return is::last_error_text(); }

IS_EXPORT int is_store_create(const is_store_desc* d, is_store** out) {
  is::clear_error();
  if (out == nullptr) return fail(IS_ERR_INVALID_ARG, "null output handle");
  int rc = is::check_store_desc(d);
  if (rc != IS_OK) return rc;
  is_store* s = new is_store();
  if (hipGetDevice(&s->device) != hipSuccess) {
    delete s;
    return fail(IS_ERR_HIP, "no HIP device");
  }
  s->L = d->n_layers;
  s->H = d->n_kv_heads;
  s->d = d->head_dim;
  s->dtype = d->kv_dtype;
  s->emb_dim = d->emb_dim;
  s->n_facts = d->n_facts;
  s->es = (size_t)is::elem_size(d->kv_dtype);
  s->len.assign(d->fact_len, d->fact_len + d->n_facts);
  s->tok_off.assign((size_t)d->n_facts + 1, 0);
  for (int64_t f = 0; f < d->n_facts; ++f) s->tok_off[f + 1] = s->tok_off[f] + s->len[f];
  // Facts in id order go to HBM while K+V fit the budget.
  const size_t per_tok = (size_t)s->row_elems() * s->es * 2;
  if (d->hbm_budget_bytes < 0) {
    s->n_hbm = s->n_facts;
  } else {
    const int64_t max_tok = (int64_t)((size_t)d->hbm_budget_bytes / per_tok);
    s->n_hbm = std::upper_bound(s->tok_off.begin(), s->tok_off.end(), max_tok) -
               s->tok_off.begin() - 1;
  }
  // Spare room for appended facts: HBM only, and only without a host tier.
  if ((d->spare_facts > 0 || d->spare_tokens > 0) && s->n_hbm < s->n_facts) {
    free_store(s);
    return fail(IS_ERR_UNSUPPORTED, "spare room for appends needs a store without a host tier");
  }
  s->max_facts = s->n_facts + std::max<int64_t>(d->spare_facts, 0);
  s->hbm_tokens = s->tok_off[s->n_hbm] + std::max<int64_t>(d->spare_tokens, 0);
  s->hbm_next = s->tok_off[s->n_hbm];
  const size_t hbm_bytes = (size_t)s->hbm_tokens * s->row_elems() * s->es;
  if (hbm_bytes > 0 && (hipMalloc(&s->k_dev, hbm_bytes) != hipSuccess ||
                        hipMalloc(&s->v_dev, hbm_bytes) != hipSuccess)) {
    free_store(s);
    return fail(IS_ERR_OOM, "device allocation of the fact store failed");
  }
  // Host tier: pinned chunks of at most 4 GiB (a longer fact gets its own).
  for (int64_t f0 = s->n_hbm; f0 < s->n_facts;) {
    int64_t f1 = f0 + 1;
    while (f1 < s->n_facts && s->fact_bytes(f0, f1 + 1) <= kHostChunkBytes) ++f1;
    HostChunk c;
    c.f0 = f0;
    c.f1 = f1;
    const size_t bytes = s->fact_bytes(f0, f1);
    const bool ok = hipHostMalloc(&c.k, bytes, hipHostMallocMapped) == hipSuccess &&
                    hipHostMalloc(&c.v, bytes, hipHostMallocMapped) == hipSuccess;
    s->host.push_back(c);
    if (!ok) {
      free_store(s);
      return fail(IS_ERR_OOM, "pinned host allocation of the fact store failed");
    }
    f0 = f1;
  }
  // Device-visible block address of every fact.
  s->k_addr.resize((size_t)s->n_facts);
  s->v_addr.resize((size_t)s->n_facts);
  for (int64_t f = 0; f < s->n_hbm; ++f) {
    s->k_addr[f] = (uint64_t)(uintptr_t)((char*)s->k_dev + s->fact_bytes(0, f));
    s->v_addr[f] = (uint64_t)(uintptr_t)((char*)s->v_dev + s->fact_bytes(0, f));
  }
  for (const HostChunk& c : s->host) {
    void* kd = nullptr;
    void* vd = nullptr;
    if (hipHostGetDevicePointer(&kd, c.k, 0) != hipSuccess ||
        hipHostGetDevicePointer(&vd, c.v, 0) != hipSuccess) {
      free_store(s);
      return fail(IS_ERR_HIP, "hipHostGetDevicePointer failed");
    }
    for (int64_t f = c.f0; f < c.f1; ++f) {
      s->k_addr[f] = (uint64_t)(uintptr_t)((char*)kd + s->fact_bytes(c.f0, f));
      s->v_addr[f] = (uint64_t)(uintptr_t)((char*)vd + s->fact_bytes(c.f0, f));
    }
  }
  {
    const size_t n = (size_t)s->n_facts;
    const size_t cap = (size_t)s->max_facts;
    if (hipMalloc((void**)&s->d_len, cap * 4) != hipSuccess ||
        hipMalloc((void**)&s->d_k_addr, cap * 8) != hipSuccess ||
        hipMalloc((void**)&s->d_v_addr, cap * 8) != hipSuccess) {
      free_store(s);
      return fail(IS_ERR_OOM, "device allocation of the fact tables failed");
    }
    if (hipMemcpy(s->d_len, s->len.data(), n * 4, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(s->d_k_addr, s->k_addr.data(), n * 8, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(s->d_v_addr, s->v_addr.data(), n * 8, hipMemcpyHostToDevice) != hipSuccess) {
      free_store(s);
      return fail(IS_ERR_HIP, "copy of the fact tables failed");
    }
  }
  if (s->emb_dim > 0) {
    const size_t bytes = s->emb_alloc_bytes();
    if (hipMalloc((void**)&s->emb, bytes) != hipSuccess) {
      free_store(s);
      return fail(IS_ERR_OOM, "device allocation of the embeddings failed");
    }
    if (hipMemset(s->emb, 0, bytes) != hipSuccess) {
      free_store(s);
      return fail(IS_ERR_HIP, "hipMemset of the embeddings failed");
    }
  }
  if (d->k_src || d->v_src || d->emb_src) {
    rc = is_store_load(s, 0, s->n_facts, d->k_src, d->v_src, d->emb_src, 0);
    if (rc != IS_OK) {
      std::string msg = is::last_error_text();
      free_store(s);
      return fail(rc, msg);
    }
  }
  *out = s;
  return IS_OK;
}

IS_EXPORT int is_store_load(is_store* s, int64_t first, int64_t n, const void* k,
                            const void* v, const uint16_t* emb, int src_on_device) {
  is::clear_error();
  if (s == nullptr) return fail(IS_ERR_INVALID_ARG, "null store");
  std::lock_guard<std::mutex> lock(s->mu);
  if (first < 0 || n < 0 || first + n > s->n_facts)
    return fail(IS_ERR_INVALID_ARG, "fact range outside the store");
  if (emb != nullptr && s->emb_dim == 0)
    return fail(IS_ERR_INVALID_ARG, "store has no embedding index");
  if (n == 0) return IS_OK;
  DeviceGuard guard(s->device);
  const hipMemcpyKind from_dev = src_on_device ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice;
  const hipMemcpyKind from_dev_to_host = src_on_device ? hipMemcpyDeviceToHost : hipMemcpyHostToHost;
  const int64_t end = first + n;
  // HBM part, then host part; each a contiguous span of the sources.
  struct Part { int64_t f0, f1; bool host; };
  const Part parts[2] = {{first, std::min(end, s->n_hbm), false},
                         {std::max(first, s->n_hbm), end, true}};
  size_t src_off = 0;
  for (const Part& p : parts) {
    if (p.f1 <= p.f0) continue;
    const hipMemcpyKind kind = p.host ? from_dev_to_host : from_dev;
    // HBM facts are copied by runs that are contiguous in the arena (the
    // whole range unless facts were removed), host facts chunk by chunk.
    for (int64_t f = p.f0; f < p.f1;) {
      int64_t g = f + 1;
      if (p.host) {
        g = std::min(p.f1, s->chunk_of(f).f1);
      } else {
        while (g < p.f1 && s->arena_token(g) == s->arena_token(g - 1) + s->len[(size_t)g - 1]) ++g;
      }
      const size_t bytes = s->fact_bytes(f, g);
      hipError_t e;
      if (k && (e = hipMemcpy(s->k_at(f), (const char*)k + src_off, bytes, kind)) != hipSuccess)
        return hip_fail(e, "K load");
      if (v && (e = hipMemcpy(s->v_at(f), (const char*)v + src_off, bytes, kind)) != hipSuccess)
        return hip_fail(e, "V load");
      src_off += bytes;
      f = g;
    }
  }
  if (emb) {
    // rows to device memory in pieces, then scattered into the blocked layout
    const int64_t piece_rows = 65536;
    uint16_t* tmp = nullptr;
    const size_t tmp_bytes = (size_t)std::min<int64_t>(n, piece_rows) * s->emb_dim * 2;
    if (hipMalloc((void**)&tmp, tmp_bytes) != hipSuccess) return fail(IS_ERR_OOM, "embedding staging");
    hipError_t e = hipSuccess;
    for (int64_t r0 = 0; r0 < n && e == hipSuccess; r0 += piece_rows) {
      const int64_t m = std::min(piece_rows, n - r0);
      e = hipMemcpy(tmp, emb + r0 * s->emb_dim, (size_t)m * s->emb_dim * 2, from_dev);
      if (e == hipSuccess) e = is::launch_emb_relayout(tmp, first + r0, m, s->emb_dim, s->emb, nullptr);
      if (e == hipSuccess) e = hipDeviceSynchronize();
    }
    (void)hipFree(tmp);
    if (e != hipSuccess) return hip_fail(e, "embedding load");
  }
  return IS_OK;
}

IS_EXPORT int is_store_get_info(const is_store* s, is_store_info* out) {
  is::clear_error();
  if (s == nullptr || out == nullptr) return fail(IS_ERR_INVALID_ARG, "null argument");
  std::lock_guard<std::mutex> lock(const_cast<is_store*>(s)->mu);
  out->n_facts = s->n_facts;
  out->n_hbm_facts = s->n_hbm;
  out->hbm_kv_bytes = (int64_t)s->fact_bytes(0, s->n_hbm) * 2;
  out->host_kv_bytes = (int64_t)s->fact_bytes(s->n_hbm, s->n_facts) * 2;
  out->total_tokens = s->tok_off[s->n_facts];
  out->emb_bytes = s->emb_dim > 0 ? (int64_t)s->emb_bytes() : 0;
  return IS_OK;
}

IS_EXPORT int is_store_destroy(is_store* s) {
  is::clear_error();
  free_store(s);
  return IS_OK;
}

IS_EXPORT int is_inject_check(const is_store_desc* d, int32_t n_req, const int32_t* req_off,
                              const int32_t* fact_ids, const int32_t* prefix_len,
                              const int32_t* block_tables, int32_t max_blocks,
                              const is_cache* cache, const is_rope* rope, int64_t* n_tokens) {
  is::clear_error();
  int rc = is::check_store_desc(d);
  if (rc != IS_OK) return rc;
  is::StoreGeom g;
  g.n_layers = d->n_layers;
  g.n_kv_heads = d->n_kv_heads;
  g.head_dim = d->head_dim;
  g.dtype = d->kv_dtype;
  g.n_facts = d->n_facts;
  g.fact_len = d->fact_len;
  g.n_hbm = d->n_facts;
  return is::plan_inject(g, n_req, req_off, fact_ids, prefix_len, block_tables, max_blocks,
                         cache, rope, nullptr, n_tokens);
}

IS_EXPORT int is_inject(const is_store* cs, int32_t n_req, const int32_t* req_off,
                        const int32_t* fact_ids, const int32_t* prefix_len,
                        const int32_t* block_tables, int32_t max_blocks, const is_cache* cache,
                        const is_rope* rope, void* stream) {
  is::clear_error();
  if (cs == nullptr) return fail(IS_ERR_INVALID_ARG, "null store");
  is_store* s = const_cast<is_store*>(cs);
  // planning reads the fact tables, which appends and removals change
  std::lock_guard<std::mutex> lock(s->mu);
  thread_local std::vector<is::WorkItem> items;
  thread_local std::vector<float> g;
  int64_t n_tokens = 0;
  int rc = is::plan_inject(geom_of(s), n_req, req_off, fact_ids, prefix_len, block_tables,
                           max_blocks, cache, rope, &items, &n_tokens);
  if (rc != IS_OK) return rc;
  if (items.empty()) return IS_OK;
  // Launch order only: host-tier facts first, then HBM facts, each tier by
  // fact id (stable), which is the store's layout order, so the workgroups
  // sweep each tier front to back, and the PCIe-bound host-tier reads start
  // at once with the HBM work filling in behind them.  LSD radix sort of the
  // rotated id (id - n_hbm modulo n_facts), 11-bit digits.
  thread_local std::vector<uint32_t> order, spare;
  const uint32_t n_items = (uint32_t)items.size();
  order.resize(n_items);
  spare.resize(n_items);
  for (uint32_t i = 0; i < n_items; ++i) order[i] = i;
  const uint32_t max_id = (uint32_t)(s->n_facts - 1);
  const uint32_t n_hbm = (uint32_t)s->n_hbm, n_host = (uint32_t)(s->n_facts - s->n_hbm);
  auto key = [&](uint32_t i) {
    const uint32_t f = (uint32_t)fact_ids[i];
    return f >= n_hbm ? f - n_hbm : f + n_host;
  };
  for (int shift = 0; shift == 0 || (shift < 32 && (max_id >> shift) != 0); shift += 11) {
    uint32_t hist[2049] = {};
    for (uint32_t i = 0; i < n_items; ++i) ++hist[((key(order[i]) >> shift) & 2047u) + 1];
    for (int b = 0; b < 2048; ++b) hist[b + 1] += hist[b];
    for (uint32_t i = 0; i < n_items; ++i)
      spare[hist[(key(order[i]) >> shift) & 2047u]++] = order[i];
    order.swap(spare);
  }
  is::plan_rope(s->d, rope, &g);
  const size_t items_bytes = align256(items.size() * sizeof(is::WorkItem));
  const size_t bt_bytes = align256((size_t)n_req * max_blocks * sizeof(int32_t));
  const size_t g_bytes = align256(g.size() * sizeof(float));
  const size_t total = items_bytes + bt_bytes + g_bytes;
  DeviceGuard guard(s->device);
  Slot* sl = nullptr;
  rc = acquire_slot(s, total, &sl);
  if (rc != IS_OK) return rc;
  char* h = static_cast<char*>(sl->host);
  is::WorkItem* h_items = reinterpret_cast<is::WorkItem*>(h);
  for (uint32_t i = 0; i < n_items; ++i) h_items[i] = items[order[i]];
  std::memcpy(h + items_bytes, block_tables, (size_t)n_req * max_blocks * sizeof(int32_t));
  std::memcpy(h + items_bytes + bt_bytes, g.data(), g.size() * sizeof(float));
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(sl->dev, sl->host, total, hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return hip_fail(e, "staging copy");
  is::InjectLaunch a{};
  char* dv = static_cast<char*>(sl->dev);
  a.kc = cache->k_base;
  a.vc = cache->v_base;
  a.s_layer = cache->stride_layer;
  a.s_block = cache->stride_block;
  a.s_slot = cache->stride_slot;
  a.s_head = cache->stride_head;
  a.work = reinterpret_cast<const is::WorkItem*>(dv);
  a.bt = reinterpret_cast<const int32_t*>(dv + items_bytes);
  a.g = reinterpret_cast<const float2*>(dv + items_bytes + bt_bytes);
  a.n_items = (int32_t)items.size();
  a.max_blocks = max_blocks;
  a.block_size = cache->block_size;
  a.n_layers = s->L;
  a.n_heads = s->H;
  a.head_dim = s->d;
  a.dtype = s->dtype;
  a.lanes = is::inject_lanes(s->d, s->dtype);
  a.mean_len = (float)n_tokens / (float)n_items;
  e = is::launch_inject(a, st);
  if (e != hipSuccess) return hip_fail(e, "inject launch");
  e = hipEventRecord(sl->done, st);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  return IS_OK;
}

namespace {

// Checks of a top-k call against its store (caller holds s->mu).  Sets
// *nothing = true when there is nothing to do (n_q == 0).
int check_topk_call(const is_store* s, const uint16_t* q, int32_t n_q, int32_t k,
                    const int32_t* ids, const float* scores, bool* nothing) {
  *nothing = false;
  if (s->emb_dim == 0 || s->emb == nullptr)
    return fail(IS_ERR_UNSUPPORTED, "store has no embedding index");
  if (n_q < 0) return fail(IS_ERR_INVALID_ARG, "n_q < 0");
  if (k < 1 || k > s->n_facts) return fail(IS_ERR_INVALID_ARG, "k must be in [1, n_facts]");
  if (k > 64) return fail(IS_ERR_UNSUPPORTED, "k > 64");
  if (n_q == 0) {
    *nothing = true;
    return IS_OK;
  }
  if (q == nullptr || ids == nullptr || scores == nullptr)
    return fail(IS_ERR_INVALID_ARG, "null query or output pointer");
  if (((uintptr_t)q & 15u) != 0) return fail(IS_ERR_ALIGN, "queries must be 16-byte aligned");
  return IS_OK;
}

// The launch of queries [q0, q0 + nq) (nq <= 128) with its scratch at `p`,
// laid out as `lay`.
is::TopkLaunch topk_launch_of(const is_store* s, const uint16_t* q, int32_t q0, int32_t nq,
                              int32_t k, char* p, const is::TopkScratch& lay, int32_t* ids,
                              float* scores) {
  is::TopkLaunch a{};
  a.emb = s->emb;
  a.q = q + (int64_t)q0 * s->emb_dim;
  a.n_facts = s->n_facts;
  a.emb_dim = s->emb_dim;
  a.n_q = nq;
  a.k = k;
  a.q_pad = reinterpret_cast<uint16_t*>(p + lay.q_off);
  a.gmax = reinterpret_cast<uint32_t*>(p + lay.gmax_off);
  a.tau = reinterpret_cast<float*>(p + lay.tau_off);
  a.count = reinterpret_cast<uint32_t*>(p + lay.count_off);
  a.codes = reinterpret_cast<uint32_t*>(p + lay.scode_off);
  a.scount = reinterpret_cast<uint32_t*>(p + lay.scount_off);
  a.cand = reinterpret_cast<uint64_t*>(p + lay.cand_off);
  a.ids = ids + (int64_t)q0 * k;
  a.scores = scores + (int64_t)q0 * k;
  return a;
}

}  // namespace

IS_EXPORT int is_topk(const is_store* cs, const uint16_t* q, int32_t n_q, int32_t k,
                      int32_t* ids, float* scores, void* stream) {
  is::clear_error();
  if (cs == nullptr) return fail(IS_ERR_INVALID_ARG, "null store");
  is_store* s = const_cast<is_store*>(cs);
  std::lock_guard<std::mutex> lock(s->mu);   // n_facts and the index move under removals
  bool nothing = false;
  int rc = check_topk_call(s, q, n_q, k, ids, scores, &nothing);
  if (rc != IS_OK || nothing) return rc;
  DeviceGuard guard(s->device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // Queries go in groups of up to 128 (one scan launch each).
  for (int32_t q0 = 0; q0 < n_q; q0 += 128) {
    const int32_t nq = std::min<int32_t>(128, n_q - q0);
    const is::TopkScratch lay = is::topk_scratch(s->n_facts, nq, s->emb_dim);
    Slot* sl = nullptr;
    rc = acquire_topk_slot(s, lay.bytes, &sl);
    if (rc != IS_OK) return rc;
    const is::TopkLaunch a =
        topk_launch_of(s, q, q0, nq, k, static_cast<char*>(sl->dev), lay, ids, scores);
    hipError_t e = is::launch_topk(a, st);
    if (e != hipSuccess) return hip_fail(e, "top-k launch");
    e = hipEventRecord(sl->done, st);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  }
  return IS_OK;
}

// Scratch of is_topk_noalloc: a fixed array in device memory, one copy per
// GPU, held until the process ends.  Host code never uses the array's name
// as an address (on the host it is only a stand-in for the symbol): the
// device address comes from hipGetSymbolAddress, once per device, with that
// device current.  Its size holds the largest scratch that the accepted
// stores need: 128 queries x 65,536 facts of 8-byte candidate keys (64 MiB),
// padded queries of the widest index (4 MiB), the sample's score codes
// (4 MiB) and the sample maxima, bounds and counts.
constexpr int64_t kNoAllocMaxFacts = 65536;
constexpr size_t kNoAllocScratchBytes = size_t(80) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on device `dev` (which must be current).
int scratch_on_device(int dev, char** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(IS_ERR_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return IS_OK;
}

}  // namespace

IS_EXPORT int is_topk_noalloc(const is_store* cs, const uint16_t* q, int32_t n_q, int32_t k,
                              int32_t* ids, float* scores, void* stream) {
  is::clear_error();
  if (cs == nullptr) return fail(IS_ERR_INVALID_ARG, "null store");
  is_store* s = const_cast<is_store*>(cs);
  std::lock_guard<std::mutex> lock(s->mu);
  bool nothing = false;
  int rc = check_topk_call(s, q, n_q, k, ids, scores, &nothing);
  if (rc != IS_OK || nothing) return rc;
  if (s->n_facts > kNoAllocMaxFacts)
    return fail(IS_ERR_UNSUPPORTED,
                "is_topk_noalloc covers stores of at most 65,536 facts (its fixed scratch is "
                "80 MiB per GPU); use is_topk");
  const is::TopkScratch lay = is::topk_scratch(s->n_facts, std::min<int32_t>(128, n_q), s->emb_dim);
  if (lay.bytes > kNoAllocScratchBytes)
    return fail(IS_ERR_UNSUPPORTED, "the call's scratch exceeds the fixed 80 MiB");
  DeviceGuard guard(s->device);
  char* p = nullptr;
  rc = scratch_on_device(s->device, &p);
  if (rc != IS_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // groups of 128 queries reuse the scratch one after the other on `stream`
  for (int32_t q0 = 0; q0 < n_q; q0 += 128) {
    const int32_t nq = std::min<int32_t>(128, n_q - q0);
    const is::TopkScratch lg = is::topk_scratch(s->n_facts, nq, s->emb_dim);
    const hipError_t e = is::launch_topk(topk_launch_of(s, q, q0, nq, k, p, lg, ids, scores), st);
    if (e != hipSuccess) return hip_fail(e, "top-k launch");
  }
  return IS_OK;
}

IS_EXPORT int is_retrieve_inject(const is_store* cs, const uint16_t* q, int32_t n_req, int32_t k,
                                 const int32_t* prefix_len, const int32_t* block_tables,
                                 int32_t max_blocks, const is_cache* cache, const is_rope* rope,
                                 int32_t* ids_out, int32_t* status, void* stream) {
  is::clear_error();
  if (cs == nullptr) return fail(IS_ERR_INVALID_ARG, "null store");
  is_store* s = const_cast<is_store*>(cs);
  std::lock_guard<std::mutex> lock(s->mu);   // n_facts, the index and the tables move under removals
  if (s->emb_dim == 0 || s->emb == nullptr)
    return fail(IS_ERR_UNSUPPORTED, "store has no embedding index");
  if (n_req < 0) return fail(IS_ERR_INVALID_ARG, "n_req < 0");
  if (k < 1 || k > s->n_facts) return fail(IS_ERR_INVALID_ARG, "k must be in [1, n_facts]");
  if (k > 64) return fail(IS_ERR_UNSUPPORTED, "k > 64");
  if (status == nullptr) return fail(IS_ERR_INVALID_ARG, "null status word");
  int rc = is::check_cache(s->dtype, cache);
  if (rc != IS_OK) return rc;
  rc = is::check_rope(rope);
  if (rc != IS_OK) return rc;
  if (n_req > 0 && (q == nullptr || prefix_len == nullptr || block_tables == nullptr))
    return fail(IS_ERR_INVALID_ARG, "null query, prefix or block-table pointer");
  if (max_blocks < 1) return fail(IS_ERR_INVALID_ARG, "max_blocks must be >= 1");
  if (((uintptr_t)q & 15u) != 0) return fail(IS_ERR_ALIGN, "queries must be 16-byte aligned");
  const int64_t n_slots = cache->n_blocks * (int64_t)cache->block_size;
  if (n_slots > kDeviceCheckSlots)
    return fail(IS_ERR_UNSUPPORTED, "cache too large for the on-device slot check");
  thread_local std::vector<float> g;
  is::plan_rope(s->d, rope, &g);
  const int32_t n_pairs = (int32_t)(g.size() / 2);
  if (n_pairs > is::kComposeMaxPairs) return fail(IS_ERR_UNSUPPORTED, "head_dim too large");
  DeviceGuard guard(s->device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // One scratch slot: top-k scratch (reused by each group of 128 queries),
  // then ids and scores of all requests, the work list, the rotation speeds
  // and the slot bitmap.
  const int32_t nq_group = std::min<int32_t>(128, std::max<int32_t>(n_req, 1));
  const is::TopkScratch lay = is::topk_scratch(s->n_facts, nq_group, s->emb_dim);
  const int64_t n_items = (int64_t)n_req * k;
  const int64_t slot_words = (n_slots + 63) / 64;
  const size_t off_ids = align256(lay.bytes);
  const size_t off_scores = off_ids + align256((size_t)n_items * 4);
  const size_t off_work = off_scores + align256((size_t)n_items * 4);
  // batches of more than one request are grouped by fact id on the device
  const bool sort = n_req > 1;
  const size_t off_tmp = off_work + align256((size_t)n_items * sizeof(is::WorkItem));
  const size_t off_g = off_tmp + (sort ? align256((size_t)n_items * sizeof(is::WorkItem)) : 0);
  // the bucket counters and the slot bitmap are contiguous: the first top-k
  // launch's sample scan zeroes them in one range
  const size_t off_buckets = off_g + align256((size_t)n_pairs * 8);
  const size_t off_bits = off_buckets + (sort ? align256(2 * is::kComposeBuckets * sizeof(uint32_t)) : 0);
  const size_t total = off_bits + align256((size_t)slot_words * 8);
  // Under stream capture: the graph workspace, no events, no allocation.
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(st, &capture);
  if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
  const bool capturing = capture != hipStreamCaptureStatusNone;
  Slot* sl = nullptr;
  if (capturing) {
    if (s->graph_slot.cap < total)
      return fail(IS_ERR_UNSUPPORTED,
                  "capture needs an earlier eager call of at least this size on the store "
                  "(it sizes the workspace that graph replays use)");
    sl = &s->graph_slot;
    s->captured = true;
  } else {
    rc = acquire_topk_slot(s, total, &sl);
    if (rc != IS_OK) return rc;
    Slot& gs = s->graph_slot;
    if (!s->captured && gs.cap < total) {
      if (gs.dev) (void)hipFree(gs.dev);
      gs.dev = nullptr;
      gs.cap = 0;
      if (hipMalloc(&gs.dev, total) != hipSuccess) return fail(IS_ERR_OOM, "graph workspace");
      gs.cap = total;
    }
  }
  char* p = static_cast<char*>(sl->dev);
  int32_t* ids = ids_out ? ids_out : reinterpret_cast<int32_t*>(p + off_ids);
  float* scores = reinterpret_cast<float*>(p + off_scores);
  is::ComposeLaunch c{};
  c.ids = ids;
  c.prefix = prefix_len;
  c.bt = block_tables;
  c.lens = s->d_len;
  c.k_addr = s->d_k_addr;
  c.v_addr = s->d_v_addr;
  c.n_facts = s->n_facts;
  c.n_hbm = s->n_hbm;
  c.n_blocks = cache->n_blocks;
  c.n_req = n_req;
  c.k = k;
  c.max_blocks = max_blocks;
  c.block_size = cache->block_size;
  c.slot_bits = reinterpret_cast<uint64_t*>(p + off_bits);
  c.slot_words = slot_words;
  c.work = reinterpret_cast<is::WorkItem*>(p + off_work);
  c.work_tmp = sort ? reinterpret_cast<is::WorkItem*>(p + off_tmp) : nullptr;
  c.buckets = sort ? reinterpret_cast<uint32_t*>(p + off_buckets) : nullptr;
  c.g_out = reinterpret_cast<float2*>(p + off_g);
  c.status = status;
  c.n_pairs = n_pairs;
  c.cleared = n_req > 0;
  for (int32_t i = 0; i < n_pairs; ++i) c.g[i] = make_float2(g[2 * i], g[2 * i + 1]);
  // One request: the top-k final kernel composes it (no composer launch).
  const bool fused = n_req == 1;
  for (int32_t q0 = 0; q0 < n_req; q0 += 128) {
    is::TopkLaunch a =
        topk_launch_of(s, q, q0, std::min<int32_t>(128, n_req - q0), k, p, lay, ids, scores);
    if (q0 == 0) {
      a.zero = reinterpret_cast<uint32_t*>(p + off_buckets);
      a.zero_words = (int64_t)((total - off_buckets) / 4);
      a.zero_status = status;
    }
    if ((e = is::launch_topk(a, st, fused ? &c : nullptr)) != hipSuccess)
      return hip_fail(e, "top-k launch");
  }
  if (!fused && (e = is::launch_compose(c, st)) != hipSuccess) return hip_fail(e, "compose launch");
  is::InjectLaunch a{};
  a.kc = cache->k_base;
  a.vc = cache->v_base;
  a.s_layer = cache->stride_layer;
  a.s_block = cache->stride_block;
  a.s_slot = cache->stride_slot;
  a.s_head = cache->stride_head;
  a.work = c.work;
  a.bt = block_tables;
  a.g = c.g_out;
  a.n_items = (int32_t)n_items;
  a.max_blocks = max_blocks;
  a.block_size = cache->block_size;
  a.n_layers = s->L;
  a.n_heads = s->H;
  a.head_dim = s->d;
  a.dtype = s->dtype;
  a.lanes = is::inject_lanes(s->d, s->dtype);
  a.status = status;
  // the ids are chosen on the device: the store's mean fact length stands in
  a.mean_len = (float)s->tok_off[(size_t)s->n_facts] / (float)s->n_facts;
  if ((e = is::launch_inject(a, st)) != hipSuccess) return hip_fail(e, "inject launch");
  if (!capturing && (e = hipEventRecord(sl->done, st)) != hipSuccess)
    return hip_fail(e, "hipEventRecord");
  return IS_OK;
}

IS_EXPORT int is_attend(const is_store* cs, const is_cache* cache, const is_rope* rope,
                        int32_t n_req, int32_t n_qtok, int32_t n_q_heads, const void* q,
                        const int32_t* q_pos, const int32_t* ctx_begin, const int32_t* ctx_end,
                        const int32_t* block_tables, int32_t max_blocks, float* out,
                        void* stream) {
  is::clear_error();
  if (cs == nullptr) return fail(IS_ERR_INVALID_ARG, "null store");
  is_store* s = const_cast<is_store*>(cs);
  if (s->d > 256) return fail(IS_ERR_UNSUPPORTED, "attention covers head_dim up to 256");
  int rc = is::check_cache(s->dtype, cache);
  if (rc != IS_OK) return rc;
  rc = is::check_rope(rope);
  if (rc != IS_OK) return rc;
  if (n_req < 0 || n_qtok < 0) return fail(IS_ERR_INVALID_ARG, "negative n_req or n_qtok");
  if (n_q_heads < 1 || n_q_heads % s->H != 0)
    return fail(IS_ERR_INVALID_ARG, "n_q_heads must be a positive multiple of n_kv_heads");
  if ((int64_t)n_qtok * (n_q_heads / s->H) > (1 << 20))
    return fail(IS_ERR_UNSUPPORTED, "too many query rows per kv head");
  if (n_req == 0 || n_qtok == 0) return IS_OK;
  if (q == nullptr || out == nullptr || q_pos == nullptr || ctx_begin == nullptr ||
      ctx_end == nullptr || block_tables == nullptr)
    return fail(IS_ERR_INVALID_ARG, "null pointer argument");
  if (((uintptr_t)q & 15u) != 0 || ((uintptr_t)out & 15u) != 0)
    return fail(IS_ERR_ALIGN, "q and out must be 16-byte aligned");
  if (max_blocks < 1) return fail(IS_ERR_INVALID_ARG, "max_blocks must be >= 1");
  const int64_t B = cache->block_size;
  for (int32_t r = 0; r < n_req; ++r) {
    if (q_pos[r] < 0 || (int64_t)q_pos[r] + n_qtok > ((int64_t)1 << 24))
      return fail(IS_ERR_INVALID_ARG, "query positions must lie in [0, 2^24)");
    if (ctx_begin[r] < 0 || ctx_end[r] < ctx_begin[r])
      return fail(IS_ERR_INVALID_ARG, "context range must satisfy 0 <= begin <= end");
    if (ctx_end[r] == ctx_begin[r]) continue;
    const int64_t b0 = ctx_begin[r] / B, b1 = ((int64_t)ctx_end[r] - 1) / B;
    if (b1 >= max_blocks)
      return fail(IS_ERR_BLOCK_TABLE, "block table of request " + std::to_string(r) +
                                          " is too short for its context");
    for (int64_t b = b0; b <= b1; ++b) {
      const int32_t blk = block_tables[(int64_t)r * max_blocks + b];
      if (blk < 0 || blk >= cache->n_blocks)
        return fail(IS_ERR_BLOCK_TABLE, "block table entry " + std::to_string(b) +
                                            " of request " + std::to_string(r) +
                                            " is outside [0, n_blocks)");
    }
  }
  thread_local std::vector<float> g;
  is::plan_rope(s->d, rope, &g);
  const size_t meta_bytes = align256((size_t)n_req * 3 * sizeof(int32_t));
  const size_t bt_bytes = align256((size_t)n_req * max_blocks * sizeof(int32_t));
  const size_t total = meta_bytes + bt_bytes + align256(g.size() * sizeof(float));
  DeviceGuard guard(s->device);
  std::lock_guard<std::mutex> lock(s->mu);
  Slot* sl = nullptr;
  rc = acquire_slot(s, total, &sl);
  if (rc != IS_OK) return rc;
  char* h = static_cast<char*>(sl->host);
  int32_t* meta = reinterpret_cast<int32_t*>(h);
  for (int32_t r = 0; r < n_req; ++r) {
    meta[3 * r] = q_pos[r];
    meta[3 * r + 1] = ctx_begin[r];
    meta[3 * r + 2] = ctx_end[r];
  }
  std::memcpy(h + meta_bytes, block_tables, (size_t)n_req * max_blocks * sizeof(int32_t));
  std::memcpy(h + meta_bytes + bt_bytes, g.data(), g.size() * sizeof(float));
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(sl->dev, sl->host, total, hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return hip_fail(e, "staging copy");
  const char* dv = static_cast<const char*>(sl->dev);
  is::AttendLaunch a{};
  a.kc = cache->k_base;
  a.vc = cache->v_base;
  a.s_layer = cache->stride_layer;
  a.s_block = cache->stride_block;
  a.s_slot = cache->stride_slot;
  a.s_head = cache->stride_head;
  a.q = q;
  a.out = out;
  a.meta = reinterpret_cast<const int32_t*>(dv);
  a.bt = reinterpret_cast<const int32_t*>(dv + meta_bytes);
  a.g = reinterpret_cast<const float2*>(dv + meta_bytes + bt_bytes);
  a.n_layers = s->L;
  a.n_req = n_req;
  a.n_qtok = n_qtok;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = s->H;
  a.head_dim = s->d;
  a.dtype = s->dtype;
  a.max_blocks = max_blocks;
  a.block_size = cache->block_size;
  a.rows = n_qtok * (n_q_heads / s->H);
  a.n_units = (int64_t)s->L * n_req * s->H;
  if ((e = is::launch_attend(a, st)) != hipSuccess) return hip_fail(e, "attention launch");
  if ((e = hipEventRecord(sl->done, st)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  return IS_OK;
}

namespace {

// 16-byte pieces in one layer of a fact of `len` tokens (the packing kernel
// indexes them in 32 bits).
int64_t layer_pieces(const is_store* s, int64_t len) {
  return (int64_t)s->H * len * s->d * (int64_t)s->es / 16;
}

// Stages `items` and launches the packing copy, 65535 facts per launch.
int launch_ingest_items(is_store* s, const std::vector<is::IngestItem>& items, size_t extra_bytes,
                        const void* extra, hipStream_t st, Slot** out_slot, char** extra_dev) {
  const size_t items_bytes = align256(items.size() * sizeof(is::IngestItem));
  Slot* sl = nullptr;
  int rc = acquire_slot(s, items_bytes + extra_bytes, &sl);
  if (rc != IS_OK) return rc;
  std::memcpy(sl->host, items.data(), items.size() * sizeof(is::IngestItem));
  if (extra_bytes) std::memcpy(static_cast<char*>(sl->host) + items_bytes, extra, extra_bytes);
  hipError_t e = hipMemcpyAsync(sl->dev, sl->host, items_bytes + extra_bytes,
                                hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return hip_fail(e, "staging copy");
  const is::IngestItem* dev_items = static_cast<const is::IngestItem*>(sl->dev);
  for (size_t i0 = 0; i0 < items.size(); i0 += 65535) {
    is::IngestLaunch a{};
    a.items = dev_items + i0;
    a.n_items = (int32_t)std::min<size_t>(65535, items.size() - i0);
    a.n_layers = s->L;
    a.n_heads = s->H;
    a.row_bytes = (int32_t)(s->d * s->es);
    if ((e = is::launch_ingest(a, st)) != hipSuccess) return hip_fail(e, "ingest launch");
  }
  *out_slot = sl;
  *extra_dev = static_cast<char*>(sl->dev) + items_bytes;
  return IS_OK;
}

}  // namespace

IS_EXPORT int is_store_append(is_store* s, int32_t n, const int32_t* fact_len, int32_t window,
                              const void* k_enc, const void* v_enc, const uint16_t* emb,
                              int64_t* first_id, void* stream) {
  is::clear_error();
  if (s == nullptr) return fail(IS_ERR_INVALID_ARG, "null store");
  if (first_id == nullptr) return fail(IS_ERR_INVALID_ARG, "null first_id");
  if (n < 0 || window < 0) return fail(IS_ERR_INVALID_ARG, "n and window must be >= 0");
  std::lock_guard<std::mutex> lock(s->mu);
  if (s->n_hbm < s->n_facts)
    return fail(IS_ERR_UNSUPPORTED, "appends need a store without a host tier");
  *first_id = s->n_facts;
  if (n == 0) return IS_OK;
  if (fact_len == nullptr || k_enc == nullptr || v_enc == nullptr)
    return fail(IS_ERR_INVALID_ARG, "null fact_len or encoding");
  if (s->emb_dim > 0 && emb == nullptr)
    return fail(IS_ERR_INVALID_ARG, "the store has an index: the new facts need embeddings");
  if (((uintptr_t)k_enc & 15u) || ((uintptr_t)v_enc & 15u) || ((uintptr_t)emb & 15u))
    return fail(IS_ERR_ALIGN, "encodings and embeddings must be 16-byte aligned");
  for (int32_t i = 0; i < n; ++i) {
    if (fact_len[i] < 1) return fail(IS_ERR_INVALID_ARG, "fact lengths must be >= 1");
    if ((int64_t)window + fact_len[i] > ((int64_t)1 << 24))
      return fail(IS_ERR_INVALID_ARG, "window + fact length must stay below 2^24");
    if (layer_pieces(s, fact_len[i]) >= ((int64_t)1 << 31))
      return fail(IS_ERR_INVALID_ARG, "a fact's layer must stay below 2^35 bytes");
  }
  DeviceGuard guard(s->device);
  const int64_t f0 = s->n_facts;
  if (f0 + n > s->max_facts) return fail(IS_ERR_OOM, "no spare fact slots left in the store");
  // each new fact's block: first fit in the spans that removed facts left,
  // else behind the used part of the HBM arenas
  is::FreeSpans spans = s->free_spans;
  int64_t next = s->hbm_next;
  std::vector<is::IngestItem> items((size_t)n);
  std::vector<int32_t> new_len(fact_len, fact_len + n);
  std::vector<uint64_t> new_k((size_t)n), new_v((size_t)n);
  size_t src = 0;
  const size_t row = s->token_bytes();   // one token over all layers and heads
  for (int32_t i = 0; i < n; ++i) {
    const int64_t tok = is::arena_alloc(spans, next, s->hbm_tokens, fact_len[i]);
    if (tok < 0) return fail(IS_ERR_OOM, "no spare room left in the store for these facts");
    is::IngestItem& it = items[(size_t)i];
    it.src_k = static_cast<const char*>(k_enc) + src;
    it.src_v = static_cast<const char*>(v_enc) + src;
    it.dst_k = static_cast<char*>(s->k_dev) + (size_t)tok * row;
    it.dst_v = static_cast<char*>(s->v_dev) + (size_t)tok * row;
    it.len = fact_len[i];
    it.window = window;
    new_k[(size_t)i] = (uint64_t)(uintptr_t)it.dst_k;
    new_v[(size_t)i] = (uint64_t)(uintptr_t)it.dst_v;
    src += (size_t)(window + fact_len[i]) * row;
  }
  // the device fact tables' new entries travel with the work list
  const size_t tab_bytes = (size_t)n * (4 + 8 + 8);
  std::vector<char> tables(tab_bytes);
  std::memcpy(tables.data(), new_len.data(), (size_t)n * 4);
  std::memcpy(tables.data() + (size_t)n * 4, new_k.data(), (size_t)n * 8);
  std::memcpy(tables.data() + (size_t)n * 12, new_v.data(), (size_t)n * 8);
  hipStream_t st = static_cast<hipStream_t>(stream);
  Slot* sl = nullptr;
  char* tab_dev = nullptr;
  int rc = launch_ingest_items(s, items, tab_bytes, tables.data(), st, &sl, &tab_dev);
  if (rc != IS_OK) return rc;
  hipError_t e;
  if ((e = hipMemcpyAsync(s->d_len + f0, tab_dev, (size_t)n * 4, hipMemcpyDeviceToDevice, st)) !=
          hipSuccess ||
      (e = hipMemcpyAsync(s->d_k_addr + f0, tab_dev + (size_t)n * 4, (size_t)n * 8,
                          hipMemcpyDeviceToDevice, st)) != hipSuccess ||
      (e = hipMemcpyAsync(s->d_v_addr + f0, tab_dev + (size_t)n * 12, (size_t)n * 8,
                          hipMemcpyDeviceToDevice, st)) != hipSuccess)
    return hip_fail(e, "fact table update");
  if (s->emb_dim > 0 && (e = is::launch_emb_relayout(emb, f0, n, s->emb_dim, s->emb, st)) !=
                            hipSuccess)
    return hip_fail(e, "embedding relayout");
  if ((e = hipEventRecord(sl->done, st)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  // host tables last: every step above has been enqueued
  for (int32_t i = 0; i < n; ++i) {
    s->len.push_back(fact_len[i]);
    s->tok_off.push_back(s->tok_off.back() + fact_len[i]);
    s->k_addr.push_back(new_k[(size_t)i]);
    s->v_addr.push_back(new_v[(size_t)i]);
  }
  s->n_facts += n;
  s->n_hbm += n;
  s->free_spans.swap(spans);
  s->hbm_next = next;
  return IS_OK;
}

IS_EXPORT int is_store_update(is_store* s, int64_t fact_id, int32_t window, const void* k_enc,
                              const void* v_enc, const uint16_t* emb, void* stream) {
  is::clear_error();
  if (s == nullptr) return fail(IS_ERR_INVALID_ARG, "null store");
  std::lock_guard<std::mutex> lock(s->mu);
  if (fact_id < 0 || fact_id >= s->n_facts) return fail(IS_ERR_FACT_ID, "fact id out of range");
  if (window < 0) return fail(IS_ERR_INVALID_ARG, "window must be >= 0");
  if (k_enc == nullptr || v_enc == nullptr) return fail(IS_ERR_INVALID_ARG, "null encoding");
  if (((uintptr_t)k_enc & 15u) || ((uintptr_t)v_enc & 15u) || ((uintptr_t)emb & 15u))
    return fail(IS_ERR_ALIGN, "encodings and embeddings must be 16-byte aligned");
  if (emb != nullptr && s->emb_dim == 0)
    return fail(IS_ERR_INVALID_ARG, "store has no embedding index");
  DeviceGuard guard(s->device);
  const int32_t len = s->len[(size_t)fact_id];
  if ((int64_t)window + len > ((int64_t)1 << 24))
    return fail(IS_ERR_INVALID_ARG, "window + fact length must stay below 2^24");
  if (layer_pieces(s, len) >= ((int64_t)1 << 31))
    return fail(IS_ERR_INVALID_ARG, "a fact's layer must stay below 2^35 bytes");
  std::vector<is::IngestItem> items(1);
  items[0].src_k = static_cast<const char*>(k_enc);
  items[0].src_v = static_cast<const char*>(v_enc);
  items[0].dst_k = reinterpret_cast<char*>((uintptr_t)s->k_addr[(size_t)fact_id]);
  items[0].dst_v = reinterpret_cast<char*>((uintptr_t)s->v_addr[(size_t)fact_id]);
  items[0].len = len;
  items[0].window = window;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Slot* sl = nullptr;
  char* unused = nullptr;
  int rc = launch_ingest_items(s, items, 0, nullptr, st, &sl, &unused);
  if (rc != IS_OK) return rc;
  hipError_t e;
  if (emb != nullptr &&
      (e = is::launch_emb_relayout(emb, fact_id, 1, s->emb_dim, s->emb, st)) != hipSuccess)
    return hip_fail(e, "embedding relayout");
  if ((e = hipEventRecord(sl->done, st)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  return IS_OK;
}

IS_EXPORT int is_store_remove(is_store* s, int64_t n, const int32_t* ids, void* stream) {
  is::clear_error();
  if (s == nullptr) return fail(IS_ERR_INVALID_ARG, "null store");
  if (n < 0) return fail(IS_ERR_INVALID_ARG, "n must be >= 0");
  if (n > 0 && ids == nullptr) return fail(IS_ERR_INVALID_ARG, "null ids");
  DeviceGuard guard(s->device);
  std::lock_guard<std::mutex> lock(s->mu);
  if (s->n_hbm < s->n_facts)
    return fail(IS_ERR_UNSUPPORTED, "removal needs a store without a host tier");
  if (s->captured)
    return fail(IS_ERR_UNSUPPORTED,
                "graphs were captured on this store: removal would free memory they read");
  std::vector<char> gone((size_t)s->n_facts, 0);
  for (int64_t i = 0; i < n; ++i) {
    const int32_t f = ids[i];
    if (f < 0 || (int64_t)f >= s->n_facts) return fail(IS_ERR_FACT_ID, "fact id out of range");
    if (gone[(size_t)f]) return fail(IS_ERR_INVALID_ARG, "fact id listed twice");
    gone[(size_t)f] = 1;
  }
  if (n == 0) return IS_OK;
  // survivors in id order; their blocks stay where they are
  const int64_t m = s->n_facts - n;
  std::vector<int32_t> keep;
  keep.reserve((size_t)m);
  for (int64_t f = 0; f < s->n_facts; ++f)
    if (!gone[(size_t)f]) keep.push_back((int32_t)f);
  std::vector<int32_t> len((size_t)m);
  std::vector<uint64_t> k_addr((size_t)m), v_addr((size_t)m);
  for (int64_t i = 0; i < m; ++i) {
    len[(size_t)i] = s->len[(size_t)keep[(size_t)i]];
    k_addr[(size_t)i] = s->k_addr[(size_t)keep[(size_t)i]];
    v_addr[(size_t)i] = s->v_addr[(size_t)keep[(size_t)i]];
  }
  // device work first: new fact tables, then the compacted index
  const size_t tab_bytes = align256((size_t)m * 4) + (size_t)m * 16 + (size_t)m * 4;
  Slot* sl = nullptr;
  int rc = acquire_slot(s, std::max<size_t>(tab_bytes, 16), &sl);
  if (rc != IS_OK) return rc;
  char* h = static_cast<char*>(sl->host);
  char* dv = static_cast<char*>(sl->dev);
  const size_t o_k = align256((size_t)m * 4), o_v = o_k + (size_t)m * 8, o_keep = o_v + (size_t)m * 8;
  std::memcpy(h, len.data(), (size_t)m * 4);
  std::memcpy(h + o_k, k_addr.data(), (size_t)m * 8);
  std::memcpy(h + o_v, v_addr.data(), (size_t)m * 8);
  std::memcpy(h + o_keep, keep.data(), (size_t)m * 4);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  // the new index arena first: an allocation failure must leave the store as it was
  uint16_t* emb = nullptr;
  if (s->emb_dim > 0 && hipMalloc((void**)&emb, s->emb_alloc_bytes()) != hipSuccess)
    return fail(IS_ERR_OOM, "embedding arena");
  if (m > 0) {
    if ((e = hipMemcpyAsync(dv, h, tab_bytes, hipMemcpyHostToDevice, st)) != hipSuccess ||
        (e = hipMemcpyAsync(s->d_len, dv, (size_t)m * 4, hipMemcpyDeviceToDevice, st)) != hipSuccess ||
        (e = hipMemcpyAsync(s->d_k_addr, dv + o_k, (size_t)m * 8, hipMemcpyDeviceToDevice, st)) !=
            hipSuccess ||
        (e = hipMemcpyAsync(s->d_v_addr, dv + o_v, (size_t)m * 8, hipMemcpyDeviceToDevice, st)) !=
            hipSuccess) {
      (void)hipStreamSynchronize(st);
      if (emb) (void)hipFree(emb);
      return hip_fail(e, "fact table update");
    }
  }
  if (s->emb_dim > 0) {
    const size_t bytes = s->emb_alloc_bytes();
    if ((e = hipMemsetAsync(emb, 0, bytes, st)) != hipSuccess ||
        (e = is::launch_emb_compact(s->emb, reinterpret_cast<const int32_t*>(dv + o_keep), m,
                                    s->emb_dim, emb, st)) != hipSuccess) {
      (void)hipStreamSynchronize(st);
      (void)hipFree(emb);
      return hip_fail(e, "embedding compaction");
    }
  }
  if ((e = hipEventRecord(sl->done, st)) != hipSuccess ||
      (e = hipStreamSynchronize(st)) != hipSuccess) {
    if (emb) (void)hipFree(emb);
    return hip_fail(e, "removal");
  }
  // host state last: the removed facts' spans go back to the arena
  for (int64_t f = 0; f < s->n_facts; ++f)
    if (gone[(size_t)f]) is::arena_free(s->free_spans, s->hbm_next, s->arena_token(f), s->len[(size_t)f]);
  if (emb) {
    (void)hipFree(s->emb);
    s->emb = emb;
  }
  s->len.swap(len);
  s->k_addr.swap(k_addr);
  s->v_addr.swap(v_addr);
  s->tok_off.assign((size_t)m + 1, 0);
  for (int64_t f = 0; f < m; ++f) s->tok_off[(size_t)f + 1] = s->tok_off[(size_t)f] + s->len[(size_t)f];
  s->n_facts = m;
  s->n_hbm = m;
  return IS_OK;
}
