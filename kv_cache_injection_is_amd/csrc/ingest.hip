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
// One workgroup per (fact, layer): for that layer the fact's kv_heads are
// len-row spans in both tensors, so the copy runs in 16-byte pieces over
// the layer's H * len rows, K and V together.  Non-temporal accesses: the
// data is neither read again soon nor written back to.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace is {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void ingest_kernel(IngestLaunch a) {
  const IngestItem it = a.items[blockIdx.y];
  const int layer = blockIdx.x;
  const int64_t row = a.row_bytes;
  const int64_t per_head = (int64_t)it.len * row / 16;      // 16-byte pieces per head span
  const int64_t n = per_head * a.n_heads;
  const int64_t src_rows = (int64_t)it.window + it.len;
  for (int64_t c = threadIdx.x; c < n; c += kThreads) {
    const int64_t hd = c / per_head, off = (c % per_head) * 16;
    const int64_t lh = (int64_t)layer * a.n_heads + hd;
    const int64_t s = (lh * src_rows + it.window) * row + off;
    const int64_t d = lh * it.len * row + off;
    const u32x4 kv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(it.src_k + s));
    const u32x4 vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(it.src_v + s));
    __builtin_nontemporal_store(kv, reinterpret_cast<u32x4*>(it.dst_k + d));
    __builtin_nontemporal_store(vv, reinterpret_cast<u32x4*>(it.dst_v + d));
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
