// Exact top-k inner-product search over the fp16 fact embeddings.
//
// Stands in for the GPU-resident retrieval index of the InferScale
// explainer pages ("InferScale: GPU-Native KV Injection for Personalized
// LLM Serving", technical summary, Contributions: GPU-native system design);
// the pages do not describe the index, so this is an exact brute-force
// search.  Order: score descending, ties to the lower fact id.
//
// Stage 1 (persistent, one workgroup of 8 waves per CU): scores = E . Q^T
// on the matrix cores (v_mfma_f32_32x32x16_f16, fp32 accumulation).  Each
// wave owns 32 facts of a 256-fact tile and all 128 queries of a query
// block; its A operand (embedding rows) streams from HBM straight into
// registers, double-buffered a chunk ahead, and its B operand (query rows)
// comes from an LDS copy of the current 128-dim chunk shared by the 8
// waves.  The dot product is order-free in k, so a lane loads one
// contiguous 128-byte piece of its fact row per chunk and the query side
// uses the same k order.  After a tile, scores go through LDS to one
// thread per query, which keeps a min-heap of its best k (score, id) keys.
// Each workgroup writes its per-query lists sorted.
// Stage 2 (one workgroup per query): pairwise merge of the sorted lists,
// log2(#lists) rounds, each output rank placed by a merge-path search.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace is {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kQB = 128;            // queries per block
constexpr int kFT = kWaves * 32;    // facts per tile
constexpr int kMaxK = 64;
constexpr int kHalfRows = kFT / 2;  // score rows staged per epilogue pass
constexpr int kSPitch = kQB + 1;    // floats per staged score row

// Order-preserving map of a float to uint32 (larger float -> larger code).
__device__ __forceinline__ uint32_t ord_of(float s) {
  const uint32_t u = __builtin_bit_cast(uint32_t, s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float float_of(uint32_t o) {
  const uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __builtin_bit_cast(float, u);
}

// Larger key = better: score first, then the lower id.
__device__ __forceinline__ uint64_t key_of(uint32_t ord, uint32_t id) {
  return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - id);
}

template <int KC>
struct Smem {
  static constexpr int kQPitch = KC + 8;   // halves per staged query row
  union {
    _Float16 q[2][kQB * kQPitch];
    float s[kHalfRows * kSPitch];
  } u;
  uint64_t heap[kMaxK * kQB];              // [slot][query], min-heap per query
};

__device__ __forceinline__ void heap_replace_top(uint64_t* h, int q, int k,
                                                 uint64_t key) {
  int i = 0;
  while (true) {
    const int l = 2 * i + 1;
    if (l >= k) break;
    int m = l;
    uint64_t mk = h[l * kQB + q];
    if (l + 1 < k) {
      const uint64_t rk = h[(l + 1) * kQB + q];
      if (rk < mk) { m = l + 1; mk = rk; }
    }
    if (mk >= key) break;
    h[i * kQB + q] = mk;
    i = m;
  }
  h[i * kQB + q] = key;
}

template <int KC>
__global__ __launch_bounds__(kThreads) void topk_stage1(TopkLaunch a) {
  constexpr int kQPitch = Smem<KC>::kQPitch;
  constexpr int kLaneHalves = KC / 2;        // contiguous halves per lane per chunk
  constexpr int kLoads = kLaneHalves / 8;    // 16-byte loads per lane per chunk
  constexpr int kSteps = KC / 16;            // MFMA k-steps per chunk
  __shared__ Smem<KC> sm;

  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int row = lane % 32;
  const int grp = lane / 32;
  const int qb0 = blockIdx.y * kQB;
  const int D = a.emb_dim;
  const int n_chunks = D / KC;
  const int k = a.k;
  const int64_t n_tiles = (a.n_facts + kFT - 1) / kFT;

  for (int i = tid; i < kMaxK * kQB; i += kThreads) sm.heap[i] = 0;

  // Query chunk c -> LDS buffer b (zero rows past n_q).
  auto stage_q = [&](int c, int b) {
    constexpr int kPieces = kQB * KC / 8;    // 16-byte pieces
    for (int p = tid; p < kPieces; p += kThreads) {
      const int qr = p / (KC / 8), col = (p % (KC / 8)) * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (qb0 + qr < a.n_q)
        v = *reinterpret_cast<const u32x4*>(a.q + (int64_t)(qb0 + qr) * D + (int64_t)c * KC + col);
      *reinterpret_cast<u32x4*>(&sm.u.q[b][qr * kQPitch + col]) = v;
    }
  };

  for (int64_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const int64_t fact0 = tile * kFT;
    int64_t my_fact = fact0 + wave * 32 + row;
    if (my_fact >= a.n_facts) my_fact = a.n_facts - 1;   // clamped, masked later
    const uint16_t* erow = a.emb + my_fact * D + grp * kLaneHalves;

    float16v acc[4];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[qt][e] = 0.f;

    u32x4 e0[kLoads], e1[kLoads];
    auto load_e = [&](u32x4 (&dst)[kLoads], int c) {
#pragma unroll
      for (int i = 0; i < kLoads; ++i)
        dst[i] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(erow + (int64_t)c * KC) + i);
    };
    auto compute = [&](const u32x4 (&eb)[kLoads], int b) {
      const _Float16* qs = sm.u.q[b];
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const half8 av = __builtin_bit_cast(half8, eb[s]);
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
          const half8 bv = *reinterpret_cast<const half8*>(
              qs + (qt * 32 + row) * kQPitch + grp * kLaneHalves + s * 8);
          acc[qt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, acc[qt], 0, 0, 0);
        }
      }
    };
    load_e(e0, 0);
    __syncthreads();   // previous tile's epilogue is done with the LDS union
    stage_q(0, 0);
    __syncthreads();
    for (int c = 0; c < n_chunks; c += 2) {
      // e0 / LDS buffer 0 hold chunk c
      if (c + 1 < n_chunks) {
        load_e(e1, c + 1);
        stage_q(c + 1, 1);
      }
      compute(e0, 0);
      __syncthreads();
      if (c + 1 >= n_chunks) break;
      if (c + 2 < n_chunks) {
        load_e(e0, c + 2);
        stage_q(c + 2, 0);
      }
      compute(e1, 1);
      __syncthreads();
    }

    // Epilogue: two passes of 128 fact rows through LDS to the per-query heaps.
    for (int pass = 0; pass < 2; ++pass) {
      if (wave / (kWaves / 2) == pass) {
        const int rbase = (wave % (kWaves / 2)) * 32;
#pragma unroll
        for (int qt = 0; qt < 4; ++qt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int fr = rbase + 8 * (e / 4) + 4 * grp + (e % 4);
            sm.u.s[fr * kSPitch + qt * 32 + row] = acc[qt][e];
          }
      }
      __syncthreads();
      if (tid < kQB && qb0 + tid < a.n_q) {
        const int q = tid;
        const int64_t f0 = fact0 + pass * kHalfRows;
        int rows = (int)min<int64_t>(kHalfRows, a.n_facts - f0);
        uint64_t root = sm.heap[q];
        for (int r = 0; r < rows; ++r) {
          const uint32_t o = ord_of(sm.u.s[r * kSPitch + q]);
          if (o >= (uint32_t)(root >> 32)) {
            const uint64_t key = key_of(o, (uint32_t)(f0 + r));
            if (key > root) {
              heap_replace_top(sm.heap, q, k, key);
              root = sm.heap[q];
            }
          }
        }
      }
      __syncthreads();
    }
  }

  // Sort each heap (descending) and write it out.
  if (tid < kQB && qb0 + tid < a.n_q) {
    const int q = tid;
    uint64_t* out = a.partial + ((int64_t)(qb0 + q) * a.n_wg + blockIdx.x) * k;
    for (int n = k; n > 0; --n) {
      const uint64_t top = sm.heap[q];             // smallest of the remaining n
      out[n - 1] = top;
      const uint64_t last = sm.heap[(n - 1) * kQB + q];
      heap_replace_top(sm.heap, q, n - 1, last);
    }
  }
}

// Merge of two descending lists A (na) and B (nb): element of rank i.
__device__ __forceinline__ uint64_t merged_at(const uint64_t* A, int na,
                                              const uint64_t* B, int nb, int i) {
  // find a in [max(0, i - nb), min(i, na)] with A[a-1] > B[i-a] and
  // B[i-a-1] > A[a]  (keys are distinct)
  int lo = max(0, i - nb), hi = min(i, na);
  while (lo < hi) {
    const int a = (lo + hi) / 2;
    const int b = i - a;
    // take more from A if A[a] beats B[b-1]
    if (b > 0 && a < na && A[a] > B[b - 1])
      lo = a + 1;
    else
      hi = a;
  }
  const int a = lo, b = i - lo;
  const uint64_t x = a < na ? A[a] : 0;
  const uint64_t y = b < nb ? B[b] : 0;
  return x > y ? x : y;
}

constexpr int kMergeThreads = 256;

__global__ __launch_bounds__(kMergeThreads) void topk_stage2(TopkLaunch a) {
  __shared__ uint64_t buf[2][(256 / 2) * kMaxK];
  const int q = blockIdx.x;
  const int k = a.k;
  const int tid = threadIdx.x;
  const uint64_t* src = a.partial + (int64_t)q * a.n_wg * k;
  int n_lists = a.n_wg;
  // round 0 reads global lists, later rounds ping-pong in LDS
  const uint64_t* in = src;
  int dst = 0;
  if (n_lists == 1) {
    for (int i = tid; i < k; i += kMergeThreads) buf[0][i] = src[i];
    __syncthreads();
    in = buf[0];
  }
  while (n_lists > 1) {
    const int n_out = (n_lists + 1) / 2;
    for (int t = tid; t < n_out * k; t += kMergeThreads) {
      const int m = t / k, i = t % k;
      const uint64_t* A = in + (int64_t)(2 * m) * k;
      const bool has_b = 2 * m + 1 < n_lists;
      buf[dst][t] = has_b ? merged_at(A, k, A + k, k, i) : A[i];
    }
    __syncthreads();
    in = buf[dst];
    dst ^= 1;
    n_lists = n_out;
  }
  for (int i = tid; i < k; i += kMergeThreads) {
    const uint64_t key = in[i];
    a.ids[(int64_t)q * k + i] = (int32_t)(0xFFFFFFFFu - (uint32_t)key);
    a.scores[(int64_t)q * k + i] = float_of((uint32_t)(key >> 32));
  }
}

}  // namespace

int topk_workgroups(int64_t n_facts) {
  const int64_t tiles = (n_facts + kFT - 1) / kFT;
  return (int)(tiles < 256 ? tiles : 256);
}

hipError_t launch_topk(const TopkLaunch& a, hipStream_t stream) {
  if (a.n_q == 0) return hipSuccess;
  if (a.k < 1 || a.k > kMaxK || a.n_wg < 1 || a.n_wg > 256) return hipErrorInvalidValue;
  const dim3 grid1((unsigned)a.n_wg, (unsigned)((a.n_q + kQB - 1) / kQB));
  if (a.emb_dim % 128 == 0)
    hipLaunchKernelGGL(topk_stage1<128>, grid1, dim3(kThreads), 0, stream, a);
  else if (a.emb_dim % 32 == 0)
    hipLaunchKernelGGL(topk_stage1<32>, grid1, dim3(kThreads), 0, stream, a);
  else
    return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_stage2, dim3((unsigned)a.n_q), dim3(kMergeThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace is
