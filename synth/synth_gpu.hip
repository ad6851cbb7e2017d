/*
 * Seeded synthetic-input generator, device build: fills HBM buffers with the
 * same values as the host build (synth.c) so that stores far larger than
 * host memory can be created on the GPU, while the oracle regenerates any
 * single fact on the host bit for bit.  Holds none of the method's
 * arithmetic.  Also writes and checks the cache sentinel pattern.
 */
#include <hip/hip_runtime.h>
#include <stdint.h>

#define SYNTH_FN static inline __host__ __device__
#include "synth_core.h"

#define EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 8;

/* Element e of the chunk belongs to the fact j with
 * elem_off[j] <= e < elem_off[j+1]. */
__global__ __launch_bounds__(kThreads) void fill_kv_kernel(
    uint32_t seed, uint32_t tag, int64_t first_fact, int64_t n_facts,
    const int64_t* __restrict__ elem_off, int dtype, void* __restrict__ out) {
  const int64_t total = elem_off[n_facts];
  const int64_t base = (int64_t)blockIdx.x * kThreads * kPerThread + threadIdx.x;
  for (int u = 0; u < kPerThread; ++u) {
    const int64_t e = base + (int64_t)u * kThreads;
    if (e >= total) return;
    int64_t lo = 0, hi = n_facts - 1;
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) / 2;
      if (elem_off[mid] <= e)
        lo = mid;
      else
        hi = mid - 1;
    }
    const uint32_t n = (uint32_t)(e - elem_off[lo]);
    const int32_t num = synth_normal_num(seed, tag, (uint32_t)(first_fact + lo), n);
    const float x = (float)num * (1.0f / 65536.0f);
    if (dtype == SYNTH_F32)
      static_cast<float*>(out)[e] = x;
    else
      static_cast<uint16_t*>(out)[e] = synth_f32_to_bf16(x);
  }
}

__global__ __launch_bounds__(kThreads) void sentinel_kernel(
    uint32_t seed, uint64_t first_word, int64_t n, uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += stride)
    out[i] = synth_sentinel_word(seed, first_word + (uint64_t)i);
}

/* Counts the words w in [0, n) whose value differs from the sentinel, among
 * those whose row (w / row_words) is not marked in `written` (one byte per
 * row; NULL means no row is exempt). */
__global__ __launch_bounds__(kThreads) void sentinel_check_kernel(
    uint32_t seed, uint64_t first_word, int64_t n,
    const uint32_t* __restrict__ buf, int64_t row_words,
    const uint8_t* __restrict__ written, unsigned long long* __restrict__ bad) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  unsigned long long local = 0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += stride) {
    if (written != nullptr && written[i / row_words]) continue;
    local += buf[i] != synth_sentinel_word(seed, first_word + (uint64_t)i);
  }
  if (local) atomicAdd(bad, local);
}

int grid_for(int64_t n) {
  int64_t g = (n + kThreads - 1) / kThreads;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

/* Device elem_off [n_facts + 1] (relative to `out`). */
EXPORT int synth_gpu_fill_kv(uint32_t seed, uint32_t tag, int64_t first_fact,
                             int64_t n_facts, int64_t total_elems,
                             const int64_t* elem_off, int dtype, void* out,
                             void* stream) {
  if (n_facts <= 0 || total_elems <= 0) return 0;
  const int64_t per_block = (int64_t)kThreads * kPerThread;
  const int64_t blocks = (total_elems + per_block - 1) / per_block;
  if (blocks > 0x7FFFFFFF) return -1;
  hipLaunchKernelGGL(fill_kv_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     (hipStream_t)stream, seed, tag, first_fact, n_facts,
                     elem_off, dtype, out);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

EXPORT int synth_gpu_sentinel(uint32_t seed, uint64_t first_word, int64_t n_words,
                              void* out, void* stream) {
  if (n_words <= 0) return 0;
  hipLaunchKernelGGL(sentinel_kernel, dim3(grid_for(n_words)), dim3(kThreads), 0,
                     (hipStream_t)stream, seed, first_word, n_words,
                     static_cast<uint32_t*>(out));
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

EXPORT int synth_gpu_sentinel_check(uint32_t seed, uint64_t first_word,
                                    int64_t n_words, const void* buf,
                                    int64_t row_words, const uint8_t* written,
                                    unsigned long long* bad_count,
                                    void* stream) {
  if (n_words <= 0) return 0;
  if (row_words <= 0) return -1;
  hipLaunchKernelGGL(sentinel_check_kernel, dim3(grid_for(n_words)),
                     dim3(kThreads), 0, (hipStream_t)stream, seed, first_word,
                     n_words, static_cast<const uint32_t*>(buf), row_words,
                     written, bad_count);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
