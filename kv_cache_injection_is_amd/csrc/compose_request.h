// Composition and validation of one request of a retrieve-and-inject call,
// by one wave (k <= 64, one selected fact per lane).  Shared by the
// composer kernel and, for a single request, by the top-k final kernel,
// which composes its one request right after choosing the ids.
//
// Composition follows the "Online phase" of the InferScale explainer pages
// ("InferScale: GPU-Native KV Injection for Personalized LLM Serving",
// technical summary): the retrieved facts of a request form one contiguous
// segment, laid out in rank order right after the request's prefix.
#pragma once

#include <hip/hip_runtime.h>

#include "kernels.h"

namespace is {

__device__ __forceinline__ void compose_record(int32_t* status, int32_t code) { atomicMin(status, code); }

// Launch-order bucket of fact f: host-tier facts (ids from n_hbm on) first,
// so the PCIe-bound part of the batch starts at once and the HBM facts fill
// in behind it; each tier in id order.
__device__ __forceinline__ int compose_bucket_of(int32_t f, int64_t n_facts, int64_t n_hbm) {
  const int64_t rot = (int64_t)f >= n_hbm ? (int64_t)f - n_hbm : (int64_t)f + (n_facts - n_hbm);
  return (int)(rot * kComposeBuckets / n_facts);
}

// Sets bits [b0, b1] of the bitmap; true if one of them was set already.
__device__ inline bool compose_mark(uint64_t* bits, int64_t b0, int64_t b1) {
  bool clash = false;
  for (int64_t w = b0 >> 6; w <= (b1 >> 6); ++w) {
    const int lo = w == (b0 >> 6) ? (int)(b0 & 63) : 0;
    const int hi = w == (b1 >> 6) ? (int)(b1 & 63) : 63;
    const uint64_t m = (hi == 63 ? ~0ull : (1ull << (hi + 1)) - 1) & (~0ull << lo);
    const uint64_t old = atomicOr(reinterpret_cast<unsigned long long*>(bits + w),
                                  (unsigned long long)m);
    clash |= (old & m) != 0;
  }
  return clash;
}

// Request r, by the calling wave (lane = its lane).  The first request's
// wave also copies the rotation speeds to their device buffer.  Loads that
// do not depend on each other are issued together: the prefix with the
// ids, a fact's length and block addresses together, and the block-table
// entries from the prefix's block on (lane i: entry b0 + i) before the
// lengths are summed, so a request costs three memory round trips and the
// slot marks.
__device__ inline void compose_request(const ComposeLaunch& a, int r, int lane) {
  if (r == 0)
    for (int i = lane; i < a.n_pairs; i += 64) a.g_out[i] = a.g[i];
  const int64_t P = a.prefix[r];
  const bool mine = lane < a.k;
  const int32_t f = mine ? a.ids[(int64_t)r * a.k + lane] : 0;
  const bool id_ok = f >= 0 && (int64_t)f < a.n_facts;
  const int64_t len = (mine && id_ok) ? a.lens[f] : 0;
  const uint64_t fk = (mine && id_ok) ? a.k_addr[f] : 0, fv = (mine && id_ok) ? a.v_addr[f] : 0;
  const int64_t B = a.block_size;
  const int32_t* bt = a.bt + (int64_t)r * a.max_blocks;
  const int64_t b0 = P >= 0 ? P / B : 0;
  const int32_t blk0 = b0 + lane < a.max_blocks ? bt[b0 + lane] : -1;   // the segment's first 64 blocks
  if (mine && !id_ok) compose_record(a.status, IS_ERR_FACT_ID);
  if (mine && id_ok && a.work_tmp != nullptr) atomicAdd(&a.buckets[compose_bucket_of(f, a.n_facts, a.n_hbm)], 1u);
  // inclusive scan of the lengths across the wave
  int64_t incl = len;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int lo = __shfl_up((int)(uint32_t)incl, off);
    const int hi = __shfl_up((int)(uint32_t)(incl >> 32), off);
    const int64_t o = (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
    if (lane >= off) incl += o;
  }
  const int lo_t = __shfl((int)(uint32_t)incl, 63);
  const int hi_t = __shfl((int)(uint32_t)(incl >> 32), 63);
  const int64_t T = (int64_t)(((uint64_t)(uint32_t)hi_t << 32) | (uint32_t)lo_t);
  if (P < 0) {
    if (lane == 0) compose_record(a.status, IS_ERR_INVALID_ARG);
    return;
  }
  if (P + T > ((int64_t)1 << 24)) {
    if (lane == 0) compose_record(a.status, IS_ERR_INVALID_ARG);
    return;
  }
  if (mine && id_ok) {
    WorkItem w;
    w.k = fk;
    w.v = fv;
    w.len = (int32_t)len;
    w.pos = (int32_t)(P + incl - len);
    w.req = r;
    w.tier = (int64_t)f >= a.n_hbm ? 1 : 0;
    (a.work_tmp ? a.work_tmp : a.work)[(int64_t)r * a.k + lane] = w;
  }
  if (T == 0) return;
  const int64_t b1 = (P + T - 1) / B;
  if (b1 >= a.max_blocks) {
    if (lane == 0) compose_record(a.status, IS_ERR_BLOCK_TABLE);
    return;
  }
  for (int64_t b = b0 + lane; b <= b1; b += 64) {
    const int32_t blk = b - b0 < 64 ? blk0 : bt[b];
    if (blk < 0 || (int64_t)blk >= a.n_blocks) {
      compose_record(a.status, IS_ERR_BLOCK_TABLE);
      continue;
    }
    const int64_t lo = (P > b * B ? P : b * B) - b * B;
    const int64_t hi = ((P + T) < (b + 1) * B ? (P + T) : (b + 1) * B) - 1 - b * B;
    if (compose_mark(a.slot_bits, (int64_t)blk * B + lo, (int64_t)blk * B + hi))
      compose_record(a.status, IS_ERR_SLOT_OVERLAP);
  }
}

}  // namespace is
