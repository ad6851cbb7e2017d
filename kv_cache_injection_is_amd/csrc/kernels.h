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

// Top-k geometry.  The store keeps the embeddings tile-blocked,
// [tile of 256 facts][64-dim chunk][256 rows][64] fp16, with the width
// padded to a multiple of 64 and rows past n_facts zero, so that every
// 256 x 64 block the scan streams is one contiguous 32 KB span.
constexpr int kTopkTile = 256;
constexpr int kTopkChunk = 64;
constexpr int kTopkMaxScanWG = 256;     // workgroups of a scan launch (one per CU)
constexpr int kTopkGroupsPerTile = 16;  // sample groups of 16 facts per tile
inline int32_t topk_padded_dim(int32_t emb_dim) { return (emb_dim + kTopkChunk - 1) / kTopkChunk * kTopkChunk; }
inline int64_t topk_padded_facts(int64_t n_facts) { return (n_facts + kTopkTile - 1) / kTopkTile * kTopkTile; }

struct TopkLaunch {
  const uint16_t* emb;    // blocked embeddings (above)
  const uint16_t* q;      // [n_q][emb_dim] fp16, n_q <= 128, 16-byte aligned
  int64_t n_facts;
  int32_t emb_dim;        // unpadded width
  int32_t n_q;
  int32_t k;
  int32_t scan_wgs;       // derived by launch_topk
  // derived by launch_topk
  int64_t n_tiles, sample_n, sample_tiles, n_groups, cand_stride;
  // scratch (see topk_scratch)
  uint16_t* q_pad;        // [n_q][padded_dim] when emb_dim % 64 != 0
  uint32_t* gmax;         // [n_q][n_groups] sample group maxima (order codes)
  float* tau;             // [n_q] bound on each query's k-th best score
  uint32_t* count;        // [n_q][kTopkMaxScanWG] candidates per scan workgroup
  uint64_t* cand;         // [n_q][cand_stride] candidate (score, id) keys
  int32_t* ids;           // [n_q][k]
  float* scores;          // [n_q][k]
};

// Scatters rows [first, first + n) given row-major (emb_dim wide) in device
// memory into the blocked layout.
hipError_t launch_emb_relayout(const uint16_t* rows, int64_t first, int64_t n,
                               int32_t emb_dim, uint16_t* emb, hipStream_t stream);

// Facts in the threshold sample for a store of n_facts facts.
int64_t topk_sample_size(int64_t n_facts);

// Byte offsets of the scratch buffers of one call of n_q (<= 128) queries.
struct TopkScratch {
  size_t q_off, gmax_off, tau_off, count_off, cand_off, bytes;
};
TopkScratch topk_scratch(int64_t n_facts, int32_t n_q, int32_t emb_dim);
hipError_t launch_topk(const TopkLaunch& a, hipStream_t stream);

}  // namespace is
