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
  const int32_t* status;  // device status word: the kernel writes nothing unless it is 0
                          // (null: no check)
  float mean_len;         // mean injected fact length (tokens): sets the workgroup shape
  int32_t layers_per_wg;  // derived by launch_inject
};

hipError_t launch_inject(const InjectLaunch& a, hipStream_t stream);

// On-device composition and validation for a batch whose fact ids come
// from top-k (the ids never visit the host).
constexpr int kComposeMaxPairs = 256;   // head_dim / 2 of the widest compiled row
constexpr int kComposeBuckets = 4096;   // fact-id ranges the work list is grouped by
struct ComposeLaunch {
  const int32_t* ids;       // [n_req][k]
  const int32_t* prefix;    // [n_req]
  const int32_t* bt;        // [n_req][max_blocks]
  const int32_t* lens;      // [n_facts]
  const uint64_t* k_addr;   // [n_facts] device-visible K block addresses
  const uint64_t* v_addr;   // [n_facts]
  int64_t n_facts, n_hbm, n_blocks;
  int32_t n_req, k, max_blocks, block_size;
  uint64_t* slot_bits;      // [slot_words] bitmap of the cache's slots (scratch)
  int64_t slot_words;
  WorkItem* work;           // [n_req * k] out
  WorkItem* work_tmp;       // [n_req * k] scratch: when not null, the list is
                            // grouped by fact id (kComposeBuckets ranges)
  uint32_t* buckets;        // [2 * kComposeBuckets] scratch for the grouping
  float2* g_out;            // [n_pairs] out: the rotation speeds, copied from `g`
  int32_t* status;          // out: IS_OK or an error code
  int32_t n_pairs;
  int32_t cleared;          // the bitmap, buckets and status are zero already (the
                            // top-k sample scan of the same call cleared them)
  float2 g[kComposeMaxPairs];
};

// Clears the bitmap and status (unless `cleared`), then composes and
// validates every request.
hipError_t launch_compose(const ComposeLaunch& a, hipStream_t stream);

// Query-only attention over the paged cache (bf16, head_dim 128).
struct AttendLaunch {
  const void* kc;           // cache bases
  const void* vc;
  int64_t s_layer, s_block, s_slot, s_head;   // cache strides (elements)
  const void* q;            // [n_layers][n_req][n_qtok][n_q_heads][head_dim], cache dtype, before RoPE
  float* out;               // same shape, fp32
  const int32_t* meta;      // [n_req][3]: position of query token 0, context begin, end
  const int32_t* bt;        // [n_req][max_blocks]
  const float2* g;          // [64] (hi, lo) turns per position
  int64_t n_units;          // n_layers * n_req * n_kv_heads
  int32_t n_layers, n_req, n_qtok, n_q_heads, n_kv_heads, max_blocks, block_size;
  int32_t rows;             // n_qtok * (n_q_heads / n_kv_heads)
  int32_t groups;           // derived by launch_attend
  int32_t head_dim;         // 128 on the matrix-core path; any even value <= 256 otherwise
  int32_t dtype;            // IS_DTYPE_BF16 or IS_DTYPE_F32 (cache, and q)
};

hipError_t launch_attend(const AttendLaunch& a, hipStream_t stream);

// Packing of a window-encoded fact into its store block.
struct IngestItem {
  const char* src_k;        // encoding [layer][kv_head][window + len][head_dim]
  const char* src_v;
  char* dst_k;              // store block [layer][kv_head][len][head_dim]
  char* dst_v;
  int32_t len, window;
  int32_t reserved[2];
};
static_assert(sizeof(IngestItem) == 48, "IngestItem layout");
struct IngestLaunch {
  const IngestItem* items;  // [n_items], at most 65535 per launch
  int32_t n_items, n_layers, n_heads, row_bytes;
};
hipError_t launch_ingest(const IngestLaunch& a, hipStream_t stream);

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
  int32_t fuse_tau;       // derived by launch_topk: the stream scan finds the bounds
  int32_t dense;          // derived by launch_topk: one scan writes every score (below)
  // derived by launch_topk; n_tiles counts stream tiles of scan_tile facts
  // and sample_tiles sample tiles of sample_tile facts (256 for the staged
  // scan; 32, 64 or 128 for the variant that keeps the queries in registers)
  int32_t scan_tile;      // facts per stream tile
  int32_t sample_tile;    // facts per sample tile
  int64_t n_tiles, sample_n, sample_tiles, n_groups, cand_stride;
  // derived by launch_topk: the stream scan covers tiles [stream_t0,
  // n_tiles).  stream_t0 > 0: the sample scan kept the codes of its facts
  // (codes, below), which are the first stream_t0 tiles, and the threshold
  // kernel put their candidates at the head of each candidate row
  int64_t stream_t0;
  // scratch (see topk_scratch)
  uint16_t* q_pad;        // [n_q][padded_dim] when emb_dim % 64 != 0
  uint32_t* gmax;         // [n_q][n_groups] sample group maxima (order codes)
  float* tau;             // [n_q] bound on each query's k-th best score
  uint32_t* count;        // [n_q][kTopkMaxScanWG] candidates per scan workgroup
  uint64_t* cand;         // [n_q][cand_stride] candidate (score, id) keys
  uint32_t* scount;       // [n_q] candidates of the sample's facts (stream_t0 > 0)
  // dense: the scan writes every fact's order code, grouped as the group
  // maxima are ([n_q][code_stride], in the cand buffer), and gmax holds the
  // maxima of all n_groups groups (after the codes, same buffer).
  // stream_t0 > 0: the sample scan writes its facts' codes the same way
  // ([n_q][code_stride], a buffer of their own)
  uint32_t* codes;
  int64_t code_stride;
  int32_t* ids;           // [n_q][k]
  float* scores;          // [n_q][k]
  // optional side job of the sample scan: words [zero, zero + zero_words)
  // and *zero_status are set to 0 (a retrieve-and-inject call's composition
  // counters, slot bitmap and status)
  uint32_t* zero;
  int64_t zero_words;
  int32_t* zero_status;
};

// Scatters rows [first, first + n) given row-major (emb_dim wide) in device
// memory into the blocked layout.
hipError_t launch_emb_relayout(const uint16_t* rows, int64_t first, int64_t n,
                               int32_t emb_dim, uint16_t* emb, hipStream_t stream);

// Copies the blocked rows of facts keep[0..n) of `from` to rows 0..n of `to`
// (both blocked, the same width); `to` must not overlap `from`.
hipError_t launch_emb_compact(const uint16_t* from, const int32_t* keep, int64_t n,
                              int32_t emb_dim, uint16_t* to, hipStream_t stream);

// Facts in the threshold sample for a store of n_facts facts.
int64_t topk_sample_size(int64_t n_facts);

// Byte offsets of the scratch buffers of one call of n_q (<= 128) queries.
struct TopkScratch {
  size_t q_off, gmax_off, tau_off, count_off, scode_off, scount_off, cand_off, bytes;
};
TopkScratch topk_scratch(int64_t n_facts, int32_t n_q, int32_t emb_dim);
// `compose` (one query only): the final kernel also composes and validates
// that request, as launch_compose would (its clearing already done by the
// sample scan's side job).
hipError_t launch_topk(const TopkLaunch& a, hipStream_t stream,
                       const ComposeLaunch* compose = nullptr);

}  // namespace is
