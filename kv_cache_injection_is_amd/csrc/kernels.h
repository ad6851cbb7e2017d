// Device-side launch interfaces shared by the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.h"

namespace is {

struct InjectLaunch {
  const void* k_dev;      // HBM arenas
  const void* v_dev;
  const void* k_host;     // device-visible aliases of the pinned host arenas
  const void* v_host;
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
  const uint16_t* q;      // [n_q][emb_dim] fp16
  int64_t n_facts;
  int32_t emb_dim;
  int32_t n_q;
  int32_t k;
  int32_t n_wg;           // workgroups per query block in stage 1
  uint64_t* partial;      // [n_q][n_wg][k] packed (score, id) keys
  int32_t* ids;           // [n_q][k]
  float* scores;          // [n_q][k]
};

// Stage-1 workgroup count for a store of n_facts facts.
int topk_workgroups(int64_t n_facts);
hipError_t launch_topk(const TopkLaunch& a, hipStream_t stream);

}  // namespace is
