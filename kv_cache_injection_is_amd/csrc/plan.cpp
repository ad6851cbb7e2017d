// Host half of the library: validation, composition and RoPE planning.
//
// Composition follows the "Online phase" of the InferScale explainer pages
// ("InferScale: GPU-Native KV Injection for Personalized LLM Serving",
// technical summary): the retrieved facts form one contiguous segment.
// Reading taken where the pages are silent: the segment starts right after
// the request's prefix and the facts abut in the caller's order.
#include "plan.h"

#include <algorithm>
#include <cmath>
#include <cstring>

namespace is {

namespace {
thread_local std::string g_last_error;
}

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

void clear_error() { g_last_error.clear(); }

const char* last_error_text() { return g_last_error.c_str(); }

int elem_size(int32_t dtype) {
  return dtype == IS_DTYPE_F32 ? 4 : dtype == IS_DTYPE_BF16 ? 2 : 0;
}

int inject_lanes(int32_t head_dim, int32_t dtype) {
  const int es = elem_size(dtype);
  if (es == 0 || head_dim <= 0) return 0;
  const int64_t half_bytes = (int64_t)head_dim / 2 * es;
  if (head_dim % 2 != 0 || half_bytes % 16 != 0) return 0;
  const int64_t lanes = half_bytes / 16;
  switch (lanes) {
    case 2: case 4: case 8: case 16: case 32: return (int)lanes;
    default: return 0;
  }
}

int check_store_desc(const is_store_desc* d) {
  if (d == nullptr) return fail(IS_ERR_INVALID_ARG, "null store description");
  if (d->n_layers < 1 || d->n_kv_heads < 1 || d->head_dim < 2)
    return fail(IS_ERR_INVALID_ARG, "n_layers, n_kv_heads must be >= 1, head_dim >= 2");
  if (d->n_layers > 65535 || d->n_kv_heads > 4096)
    return fail(IS_ERR_UNSUPPORTED, "n_layers must be <= 65535 and n_kv_heads <= 4096");
  if (elem_size(d->kv_dtype) == 0) return fail(IS_ERR_DTYPE, "kv_dtype must be F32 or BF16");
  if (d->head_dim % 2 != 0) return fail(IS_ERR_INVALID_ARG, "head_dim must be even");
  if ((int64_t)d->head_dim * elem_size(d->kv_dtype) % 32 != 0)
    return fail(IS_ERR_ALIGN, "head_dim * element size must be a multiple of 32 bytes");
  if (inject_lanes(d->head_dim, d->kv_dtype) == 0)
    return fail(IS_ERR_UNSUPPORTED, "head_dim outside the compiled shapes");
  if (d->n_facts < 1) return fail(IS_ERR_INVALID_ARG, "n_facts must be >= 1");
  if (d->n_facts > INT32_MAX) return fail(IS_ERR_INVALID_ARG, "n_facts must fit int32");
  if (d->fact_len == nullptr) return fail(IS_ERR_INVALID_ARG, "null fact_len");
  for (int64_t f = 0; f < d->n_facts; ++f)
    if (d->fact_len[f] < 1)
      return fail(IS_ERR_INVALID_ARG, "fact " + std::to_string(f) + " has length < 1");
  if (d->spare_facts < 0 || d->spare_tokens < 0)
    return fail(IS_ERR_INVALID_ARG, "spare_facts and spare_tokens must be >= 0");
  if (d->n_facts + d->spare_facts > INT32_MAX)
    return fail(IS_ERR_INVALID_ARG, "n_facts + spare_facts must fit int32");
  if (d->emb_dim > 16384) return fail(IS_ERR_UNSUPPORTED, "emb_dim must be <= 16384");
  if (d->emb_dim < 0 || d->emb_dim % 32 != 0)
    return fail(d->emb_dim < 0 ? IS_ERR_INVALID_ARG : IS_ERR_UNSUPPORTED,
                "emb_dim must be 0 or a positive multiple of 32");
  return IS_OK;
}

int check_rope(const is_rope* r) {
  if (r == nullptr) return fail(IS_ERR_INVALID_ARG, "null rope");
  if (!(r->theta > 1.0) || !std::isfinite(r->theta))
    return fail(IS_ERR_INVALID_ARG, "rope theta must be finite and > 1");
  if (r->scaling == IS_ROPE_NONE) return IS_OK;
  if (r->scaling != IS_ROPE_LLAMA3) return fail(IS_ERR_INVALID_ARG, "unknown rope scaling");
  if (!(r->factor > 0) || !(r->low_freq_factor > 0) ||
      !(r->high_freq_factor > r->low_freq_factor) || !(r->orig_max_pos > 0))
    return fail(IS_ERR_INVALID_ARG,
                "llama3 scaling needs factor > 0, high > low > 0, orig_max_pos > 0");
  return IS_OK;
}

void plan_rope(int32_t head_dim, const is_rope* r, std::vector<float>* g) {
  const int half = head_dim / 2;
  g->assign(2 * (size_t)half, 0.f);
  const double two_pi = 6.283185307179586476925286766559;
  for (int i = 0; i < half; ++i) {
    // theta^(-2i/d) radians per position
    double f = std::exp(-(2.0 * i / head_dim) * std::log(r->theta));
    if (r->scaling == IS_ROPE_LLAMA3) {
      const double wavelength = two_pi / f;
      const double short_edge = r->orig_max_pos / r->high_freq_factor;
      const double long_edge = r->orig_max_pos / r->low_freq_factor;
      if (wavelength > long_edge) {
        f = f / r->factor;
      } else if (wavelength >= short_edge) {
        const double w = (r->orig_max_pos / wavelength - r->low_freq_factor) /
                         (r->high_freq_factor - r->low_freq_factor);
        f = w * f + (1.0 - w) * (f / r->factor);
      }
    }
    const double turns = f / two_pi;
    const float hi = (float)turns;
    const float lo = (float)(turns - (double)hi);
    (*g)[2 * i] = hi;
    (*g)[2 * i + 1] = lo;
  }
}

namespace {

struct SlotRun {   // slots [first, last] of one physical block
  int32_t block;
  int32_t first;
  int32_t last;
  bool operator<(const SlotRun& o) const {
    return block != o.block ? block < o.block : first < o.first;
  }
};

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Slot-overlap check over a bitmap of the cache's slots (bit blk * B + s),
// for caches up to kBitmapSlots slots; larger ones sort the runs instead.
constexpr int64_t kBitmapSlots = int64_t(1) << 30;

// Sets bits [b0, b1]; returns true if one of them was set already.
bool mark_bits(std::vector<uint64_t>& bits, int64_t b0, int64_t b1) {
  bool clash = false;
  for (int64_t w = b0 >> 6; w <= (b1 >> 6); ++w) {
    const int lo = w == (b0 >> 6) ? (int)(b0 & 63) : 0;
    const int hi = w == (b1 >> 6) ? (int)(b1 & 63) : 63;
    const uint64_t m = (hi == 63 ? ~uint64_t(0) : (uint64_t(1) << (hi + 1)) - 1) & (~uint64_t(0) << lo);
    clash |= (bits[w] & m) != 0;
    bits[w] |= m;
  }
  return clash;
}

// True if two runs share a slot.  The bitmap is all zero between calls.
bool runs_overlap(const std::vector<SlotRun>& runs, int64_t B, int64_t n_blocks) {
  if (n_blocks * B > kBitmapSlots) {
    std::vector<SlotRun> sorted(runs);
    std::sort(sorted.begin(), sorted.end());
    for (size_t i = 1; i < sorted.size(); ++i)
      if (sorted[i].block == sorted[i - 1].block && sorted[i].first <= sorted[i - 1].last)
        return true;
    return false;
  }
  thread_local std::vector<uint64_t> tl_bits;
  std::vector<uint64_t>& bits = tl_bits;
  const size_t words = (size_t)((n_blocks * B + 63) >> 6);
  if (bits.size() < words) bits.resize(words, 0);
  size_t i = 0;
  bool clash = false;
  for (; i < runs.size() && !clash; ++i)
    clash = mark_bits(bits, runs[i].block * B + runs[i].first, runs[i].block * B + runs[i].last);
  for (size_t j = 0; j < i; ++j)   // clear every word touched
    for (int64_t w = (runs[j].block * B + runs[j].first) >> 6;
         w <= ((runs[j].block * B + runs[j].last) >> 6); ++w)
      bits[w] = 0;
  return clash;
}

}  // namespace

int check_cache(int32_t dtype, const is_cache* c) {
  if (c == nullptr) return fail(IS_ERR_INVALID_ARG, "null cache");
  if (c->dtype != dtype) return fail(IS_ERR_DTYPE, "cache dtype differs from the store's");
  if (c->block_size < 1 || c->n_blocks < 1)
    return fail(IS_ERR_INVALID_ARG, "cache block_size and n_blocks must be >= 1");
  if (c->n_blocks > INT32_MAX) return fail(IS_ERR_INVALID_ARG, "n_blocks must fit int32");
  if (c->k_base == nullptr || c->v_base == nullptr)
    return fail(IS_ERR_INVALID_ARG, "null cache base pointer");
  if (c->stride_layer < 0 || c->stride_block < 0 || c->stride_slot < 0 || c->stride_head < 0)
    return fail(IS_ERR_INVALID_ARG, "negative cache stride");
  const int es = elem_size(dtype);
  if (!aligned16(c->k_base) || !aligned16(c->v_base) ||
      (c->stride_layer * es) % 16 || (c->stride_block * es) % 16 ||
      (c->stride_slot * es) % 16 || (c->stride_head * es) % 16)
    return fail(IS_ERR_ALIGN, "cache rows must start on 16-byte boundaries");
  return IS_OK;
}

int plan_inject(const StoreGeom& g, int32_t n_req, const int32_t* req_off,
                const int32_t* fact_ids, const int32_t* prefix_len,
                const int32_t* block_tables, int32_t max_blocks,
                const is_cache* c, const is_rope* rope,
                std::vector<WorkItem>* items, int64_t* n_tokens) {
  if (n_req < 0) return fail(IS_ERR_INVALID_ARG, "n_req < 0");
  int rc = check_cache(g.dtype, c);
  if (rc != IS_OK) return rc;
  rc = check_rope(rope);
  if (rc != IS_OK) return rc;
  if (n_req == 0) {
    if (items) items->clear();
    if (n_tokens) *n_tokens = 0;
    return IS_OK;
  }
  if (req_off == nullptr || prefix_len == nullptr || block_tables == nullptr)
    return fail(IS_ERR_INVALID_ARG, "null req_off, prefix_len or block_tables");
  if (max_blocks < 1) return fail(IS_ERR_INVALID_ARG, "max_blocks must be >= 1");
  if (req_off[0] != 0) return fail(IS_ERR_INVALID_ARG, "req_off[0] must be 0");
  for (int32_t r = 0; r < n_req; ++r)
    if (req_off[r + 1] < req_off[r])
      return fail(IS_ERR_INVALID_ARG, "req_off must be non-decreasing");
  const int32_t n_pairs = req_off[n_req];
  if (n_pairs > 0 && fact_ids == nullptr) return fail(IS_ERR_INVALID_ARG, "null fact_ids");
  for (int32_t j = 0; j < n_pairs; ++j)
    if (fact_ids[j] < 0 || fact_ids[j] >= g.n_facts)
      return fail(IS_ERR_FACT_ID, "fact id " + std::to_string(fact_ids[j]) + " at entry " +
                                      std::to_string(j) + " is outside [0, n_facts)");

  const int64_t B = c->block_size;
  thread_local std::vector<SlotRun> tl_runs;
  std::vector<SlotRun>& runs = tl_runs;
  runs.clear();
  int64_t total = 0;
  if (items) {
    items->clear();
    items->reserve((size_t)n_pairs);
  }
  for (int32_t r = 0; r < n_req; ++r) {
    if (prefix_len[r] < 0) return fail(IS_ERR_INVALID_ARG, "negative prefix_len");
    int64_t pos = prefix_len[r];
    for (int32_t j = req_off[r]; j < req_off[r + 1]; ++j) {
      const int32_t f = fact_ids[j];
      const int64_t len = g.fact_len[f];
      if (pos + len > (int64_t)1 << 24)
        return fail(IS_ERR_INVALID_ARG, "serving positions must stay below 2^24");
      if (items)
        items->push_back(WorkItem{g.k_addr[f], g.v_addr[f], (int32_t)len, (int32_t)pos, r,
                                  f >= g.n_hbm ? 1 : 0});
      pos += len;
    }
    const int64_t first = prefix_len[r], end = pos;   // segment [first, end)
    total += end - first;
    if (end == first) continue;
    const int64_t b0 = first / B, b1 = (end - 1) / B;
    if (b1 >= max_blocks)
      return fail(IS_ERR_BLOCK_TABLE, "block table of request " + std::to_string(r) +
                                          " is too short for its segment");
    const int32_t* bt = block_tables + (int64_t)r * max_blocks;
    for (int64_t b = b0; b <= b1; ++b) {
      const int32_t blk = bt[b];
      if (blk < 0 || blk >= c->n_blocks)
        return fail(IS_ERR_BLOCK_TABLE, "block table entry " + std::to_string(b) +
                                            " of request " + std::to_string(r) +
                                            " is outside [0, n_blocks)");
      const int64_t lo = std::max(first, b * B) - b * B;
      const int64_t hi = std::min(end, (b + 1) * B) - 1 - b * B;
      runs.push_back(SlotRun{blk, (int32_t)lo, (int32_t)hi});
    }
  }
  if (runs_overlap(runs, B, c->n_blocks))
    return fail(IS_ERR_SLOT_OVERLAP, "two injected tokens of the call map to the same cache slot");
  if (n_tokens) *n_tokens = total;
  return IS_OK;
}

}  // namespace is
