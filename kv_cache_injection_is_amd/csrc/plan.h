// Host half of the library: argument validation, segment composition and
// RoPE frequency planning.  Pure C++ (no HIP), so every error path can be
// exercised without a GPU.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "inferscale.h"

namespace is {

// Sets the calling thread's last-error text and returns `code`.
int fail(int code, const std::string& msg);
void clear_error();

// One (request, fact) pair of an inject call: device-visible addresses of
// the fact's K and V blocks, its token count, the serving position of its
// first token, its request, and its tier (0 = HBM, 1 = pinned host).
struct WorkItem {
  uint64_t k;
  uint64_t v;
  int32_t len;
  int32_t pos;
  int32_t req;
  int32_t tier;
};
static_assert(sizeof(WorkItem) == 32, "WorkItem layout is shared with the kernel");

// Geometry the planner needs from a store (or a store description).
struct StoreGeom {
  int32_t n_layers = 0, n_kv_heads = 0, head_dim = 0, dtype = 0;
  int64_t n_facts = 0;
  const int32_t* fact_len = nullptr;   // [n_facts]
  const uint64_t* k_addr = nullptr;    // [n_facts] device-visible K block address, or null
  const uint64_t* v_addr = nullptr;    // [n_facts] device-visible V block address, or null
  int64_t n_hbm = 0;                   // facts [0, n_hbm) in HBM
};

int elem_size(int32_t dtype);

// Checks a store description (geometry and lengths).
int check_store_desc(const is_store_desc* d);

// Lanes per half-row for the inject kernel's 16-byte chunks, or 0 if the
// head_dim / dtype pair is outside the compiled shapes.
int inject_lanes(int32_t head_dim, int32_t dtype);

// Checks a cache descriptor against the store's dtype (geometry, 16-byte
// alignment of every row).
int check_cache(int32_t dtype, const is_cache* cache);

// Validates an inject call and, if `items` is not null, builds its work
// list.  Returns IS_OK or the first error.
int plan_inject(const StoreGeom& g, int32_t n_req, const int32_t* req_off,
                const int32_t* fact_ids, const int32_t* prefix_len,
                const int32_t* block_tables, int32_t max_blocks,
                const is_cache* cache, const is_rope* rope,
                std::vector<WorkItem>* items, int64_t* n_tokens);

// Per-frequency rotation speed in turns per position, g_i = f_i / (2 pi),
// split into an fp32 head and tail (g ~= hi + lo), interleaved
// [hi0, lo0, hi1, lo1, ...].  f_i = theta^(-2i/d), Llama-3.1-scaled on
// request.
void plan_rope(int32_t head_dim, const is_rope* rope, std::vector<float>* g);

int check_rope(const is_rope* rope);

}  // namespace is
