// Device-side launch interfaces shared by the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.h"

namespace is {

struct InjectLaunch {
  void* kc;               // cache bases
  void* vc;
  int64_t s_layer, s_block, s_slot, s_head;   // cache strides (elements)
  const WorkItem* work;   // [n_items]
  const int32_t* bt;      // [n_req][max_blocks]
  const float2* g;        // [head_dim/2] (hi, lo) turns per position
  int32_t n_items;
  int32_t max_blocks;
  int32_t block_size;
  int32_t n_layers;
  int32_t n_heads;
  int32_t head_dim;
  int32_t dtype;
  int32_t lanes;          // 16-byte chunks per half row
};

hipError_t launch_inject(const InjectLaunch& a, hipStream_t stream);

struct TopkLaunch {
  const uint16_t* emb;    // [n_facts][emb_dim] fp16
  const uint16_t* q;      // [n_q][emb_dim] fp16, n_q <= 128
  int64_t n_facts;
  int64_t sample_n;       // facts [0, sample_n) give the threshold
  int32_t emb_dim;
  int32_t n_q;
  int32_t k;
  int32_t reserved0;
  float* sample;          // [n_q][sample_n] sample scores (scratch)
  float* tau;             // [n_q] bound on each query's k-th best score (scratch)
  uint32_t* count;        // [n_q] candidates found (scratch)
  uint64_t* cand;         // [n_q][n_facts] candidate (score, id) keys (scratch)
  int32_t* ids;           // [n_q][k]
  float* scores;          // [n_q][k]
};

// Embedding layout in HBM.  For emb_dim % 64 == 0 the store keeps the
// embeddings tile-blocked, [tile of 256 facts][64-dim chunk][256 rows][64],
// rows past n_facts zero, so that every 256 x 64 block the scan streams is
// one contiguous 32 KB span; otherwise row-major [n_facts][emb_dim].
inline bool topk_blocked_layout(int32_t emb_dim) { return emb_dim % 64 == 0; }
inline int64_t topk_padded_facts(int64_t n_facts) { return (n_facts + 255) / 256 * 256; }
// Scatters rows [first, first + n) given row-major in device memory into the
// blocked layout.
hipError_t launch_emb_relayout(const uint16_t* rows, int64_t first, int64_t n,
                               int32_t emb_dim, uint16_t* emb, hipStream_t stream);

// Facts in the threshold sample for a store of n_facts facts.
int64_t topk_sample_size(int64_t n_facts);
// Scratch bytes for one call of n_q (<= 128) queries.
inline size_t topk_scratch_bytes(int64_t n_facts, int32_t n_q) {
  const size_t s = (size_t)topk_sample_size(n_facts);
  return (size_t)n_q * (s * 4 + 256) + (size_t)n_q * 8 * 2 + 1024 + (size_t)n_q * n_facts * 8;
}
hipError_t launch_topk(const TopkLaunch& a, hipStream_t stream);

}  // namespace is
