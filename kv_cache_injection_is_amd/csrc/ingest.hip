// Packing of context-window-encoded facts into the store.
//
// Offline phase of the InferScale explainer pages ("InferScale: GPU-Native
// KV Injection for Personalized LLM Serving", technical summary): a fact is
// encoded behind a window of preceding tokens, and only the fact's own
// tokens' pre-RoPE keys and raw values are stored.  An encoding holds
// [layer][kv_head][window + len][head_dim]; the fact's store block is
// [layer][kv_head][len][head_dim], rows window .. window + len - 1 of each
// (layer, kv_head), bit for bit.
//
// A pure copy, HBM-bound: each stored byte is read once and written once.
// One workgroup per (fact, layer): that layer's kv_heads are H spans of len
// rows in both tensors, so the workgroup walks the layer's H * len * row
// bytes in 16-byte pieces, K and V together, U pieces of each per thread
// loaded before any is stored (several loads in flight per lane hide the
// HBM latency; the layer is short, so there is no second sweep to overlap
// with).  Piece -> (head, offset) by 32-bit division: a layer of one fact
// holds far fewer than 2^32 pieces.
#include <hip/hip_runtime.h>

#include "kernels.h"

#ifndef IS_INGEST_U
#define IS_INGEST_U 8          // pieces of K (and of V) in flight per thread
#endif
#ifndef IS_INGEST_NT
#define IS_INGEST_NT 1         // non-temporal loads and stores
#endif
#ifndef IS_INGEST_THREADS
#define IS_INGEST_THREADS 512
#endif

namespace is {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = IS_INGEST_THREADS;
constexpr int kU = IS_INGEST_U;

__device__ __forceinline__ u32x4 ld(const char* p) {
#if IS_INGEST_NT
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#else
  return *reinterpret_cast<const u32x4*>(p);
#endif
}

__device__ __forceinline__ void st(char* p, u32x4 v) {
#if IS_INGEST_NT
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
#else
  *reinterpret_cast<u32x4*>(p) = v;
#endif
}

__global__ __launch_bounds__(kThreads) void ingest_kernel(IngestLaunch a) {
  const IngestItem it = a.items[blockIdx.y];
  const int layer = blockIdx.x;
  const uint32_t per_head = (uint32_t)it.len * (uint32_t)(a.row_bytes / 16);
  const uint32_t n = per_head * (uint32_t)a.n_heads;
  const int64_t src_head = ((int64_t)it.window + it.len) * a.row_bytes;   // bytes per source span
  const int64_t dst_head = (int64_t)it.len * a.row_bytes;
  const int64_t lh0 = (int64_t)layer * a.n_heads;
  const char* __restrict__ sk = it.src_k + lh0 * src_head + (int64_t)it.window * a.row_bytes;
  const char* __restrict__ sv = it.src_v + lh0 * src_head + (int64_t)it.window * a.row_bytes;
  char* __restrict__ dk = it.dst_k + lh0 * dst_head;
  char* __restrict__ dv = it.dst_v + lh0 * dst_head;
  for (uint32_t c0 = threadIdx.x; c0 < n; c0 += kU * kThreads) {
    u32x4 kv[kU], vv[kU];
    int64_t so[kU], doff[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint32_t c = c0 + (uint32_t)(u * kThreads);
      const uint32_t h = c / per_head, q = c - h * per_head;
      so[u] = h * src_head + (int64_t)q * 16;
      doff[u] = h * dst_head + (int64_t)q * 16;
      if (c < n) {
        kv[u] = ld(sk + so[u]);
        vv[u] = ld(sv + so[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (c0 + (uint32_t)(u * kThreads) < n) {
        st(dk + doff[u], kv[u]);
        st(dv + doff[u], vv[u]);
      }
    }
  }
}

}  // namespace

hipError_t launch_ingest(const IngestLaunch& a, hipStream_t stream) {
  if (a.n_items == 0) return hipSuccess;
  if (a.n_items > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(ingest_kernel, dim3((unsigned)a.n_layers, (unsigned)a.n_items),
                     dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace is
