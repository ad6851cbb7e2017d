// On-device composition and validation of a retrieve-and-inject batch.
//
// Composition follows the "Online phase" of the InferScale explainer pages
// ("InferScale: GPU-Native KV Injection for Personalized LLM Serving",
// technical summary): the retrieved facts of a request form one contiguous
// segment, here laid out in rank order right after the request's prefix.
// The checks are the host planner's (ids in range, serving positions below
// 2^24, block table long enough and its entries in range, no cache slot
// used twice in the call); an error is recorded in a device status word
// (the smallest code wins, so the result does not depend on timing) and the
// inject kernel then writes nothing.
//
// Kernels: a clear (status, counters and the slot bitmap to zero; a
// retrieve-and-inject call has its top-k sample scan do it instead); the
// composer, one wave per request (k <= 64, one selected fact per lane; the
// first also copies the rotation speeds to their device buffer): an
// inclusive scan of the lengths gives the
// positions, and each lane marks its share of the request's block runs in
// the bitmap with 64-bit atomic ORs -- a bit that was already set is a slot
// used twice; and, for batches, a counting sort of the list into 4096
// consecutive fact-id ranges (launch order only: the inject grid then walks
// the host tier and then HBM front to back, as the host path's sorted list
// does; the order
// inside a range is whatever the atomics give, which changes no result,
// since every item writes its own slots).
#include <hip/hip_runtime.h>

#include "compose_request.h"
#include "kernels.h"

namespace is {
namespace {

constexpr int kClearThreads = 256;

__global__ __launch_bounds__(kClearThreads) void compose_clear(ComposeLaunch a) {
  const int64_t i0 = (int64_t)blockIdx.x * kClearThreads + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kClearThreads;
  for (int64_t i = i0; i < a.slot_words; i += stride) a.slot_bits[i] = 0;
  if (a.work_tmp != nullptr)
    for (int64_t i = i0; i < 2 * kComposeBuckets; i += stride) a.buckets[i] = 0;
  if (i0 == 0) *a.status = IS_OK;
}

__global__ __launch_bounds__(64) void compose(ComposeLaunch a) {
  compose_request(a, blockIdx.x, threadIdx.x);
}

constexpr int kScanThreads = 1024;

// Exclusive scan of the bucket counts into the scatter cursors.
__global__ __launch_bounds__(kScanThreads) void bucket_scan(ComposeLaunch a) {
  constexpr int kPer = kComposeBuckets / kScanThreads;
  __shared__ uint32_t wsum[kScanThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t c[kPer], sum = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    c[j] = a.buckets[tid * kPer + j];
    sum += c[j];
  }
  uint32_t incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t base = incl - sum;
  for (int w = 0; w < wave; ++w) base += wsum[w];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    a.buckets[kComposeBuckets + tid * kPer + j] = base;
    base += c[j];
  }
}

// Moves every item with a valid id to the next slot of its bucket.
__global__ __launch_bounds__(256) void bucket_scatter(ComposeLaunch a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.n_req * a.k) return;
  const int32_t f = a.ids[i];
  if (f < 0 || (int64_t)f >= a.n_facts) return;
  const uint32_t slot = atomicAdd(&a.buckets[kComposeBuckets + compose_bucket_of(f, a.n_facts, a.n_hbm)], 1u);
  a.work[slot] = a.work_tmp[i];
}

}  // namespace

hipError_t launch_compose(const ComposeLaunch& a, hipStream_t stream) {
  if (a.k < 1 || a.k > 64 || a.n_pairs > kComposeMaxPairs) return hipErrorInvalidValue;
  int64_t blocks = (a.slot_words + kClearThreads - 1) / kClearThreads;
  if (blocks < 1) blocks = 1;
  if (blocks > 1024) blocks = 1024;
  if (!a.cleared || a.n_req == 0)
    hipLaunchKernelGGL(compose_clear, dim3((unsigned)blocks), dim3(kClearThreads), 0, stream, a);
  if (a.n_req > 0) {
    hipLaunchKernelGGL(compose, dim3((unsigned)a.n_req), dim3(64), 0, stream, a);
    if (a.work_tmp != nullptr) {
      const int64_t n = (int64_t)a.n_req * a.k;
      hipLaunchKernelGGL(bucket_scan, dim3(1), dim3(kScanThreads), 0, stream, a);
      hipLaunchKernelGGL(bucket_scatter, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                         a);
    }
  }
  return hipGetLastError();
}

}  // namespace is
