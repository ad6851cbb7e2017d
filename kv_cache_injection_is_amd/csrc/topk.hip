// Exact top-k inner-product search over the fp16 fact embeddings.
//
// Stands in for the GPU-resident retrieval index of the InferScale
// explainer pages ("InferScale: GPU-Native KV Injection for Personalized
// LLM Serving", technical summary, Contributions: GPU-native system design);
// the pages do not describe the index, so this is an exact brute-force
// search.  Order: score descending, ties to the lower fact id.
//
// Stage 1 (persistent, one workgroup of 4 waves per CU, one wave per SIMD):
// scores = E . Q^T on the matrix cores (v_mfma_f32_32x32x16_f16, fp32
// accumulation).  A 256-fact tile is split over the 4 waves (64 facts each,
// two 32-row MFMA tiles) against all 128 queries of a query block.  The A
// operand (embedding rows) streams from HBM straight into registers one
// 128-dim chunk ahead; the B operand (queries) comes from a double-buffered
// LDS copy of the current chunk.  The dot product is order-free in k, so at
// k-step s lane (row, grp) holds halves [(2s+grp)*8, +8) of the chunk for
// both operands, which makes the two lanes of a row read 32 contiguous
// bytes per load.  After each half tile the scores go through LDS to the
// wave that owns the query (32 queries per wave).  Each query keeps its best
// 64 (score, id) keys sorted, one per lane, and its k-th best key in a
// lane register: the first half tile a workgroup sees is sorted outright
// (bitonic network across the wave); afterwards a ballot against the k-th
// best rejects most queries at once, and surviving keys are inserted one by
// one (ballot/popcount and a one-lane shift).  The next tile's first chunk
// is already in flight during this selection.
// Stage 2 (one workgroup per query): the sorted per-workgroup lists are
// staged in LDS and a 64-lane tournament emits the k best heads in order.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace is {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kQB = 128;            // queries per block
constexpr int kFTW = 64;            // facts per wave per tile (two MFMA row tiles)
constexpr int kFT = kWaves * kFTW;  // facts per tile
constexpr int kMaxK = 64;
constexpr int kHalfRows = kFT / 2;  // score rows staged per epilogue pass
constexpr int kSPitch = kQB + 1;    // floats per staged score row
constexpr int kQPW = kQB / kWaves;  // queries owned by a wave in selection

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
  uint64_t list[kQB * kMaxK];              // [query][64], sorted descending
};

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
  const int lo = __shfl_xor((int)(uint32_t)v, m);
  const int hi = __shfl_xor((int)(uint32_t)(v >> 32), m);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ uint64_t shfl_up64(uint64_t v, int d) {
  const int lo = __shfl_up((int)(uint32_t)v, d);
  const int hi = __shfl_up((int)(uint32_t)(v >> 32), d);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// Sorts the wave's 64*P keys descending; key r of lane l is element r*64+l.
template <int P>
__device__ __forceinline__ void wave_sort_desc(uint64_t (&a)[P]) {
  const int lane = threadIdx.x & 63;
  constexpr int N = 64 * P;
#pragma unroll
  for (int k = 2; k <= N; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= 64) {
#pragma unroll
        for (int r = 0; r < P; ++r) {
          const int rp = r ^ (j >> 6);
          if (rp > r) {
            const bool desc = (((r * 64 + lane) & k) == 0);
            const uint64_t x = a[r], y = a[rp];
            if ((x < y) == desc) {
              a[r] = y;
              a[rp] = x;
            }
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < P; ++r) {
          const uint64_t y = shfl_xor64(a[r], j);
          const bool lower = (lane & j) == 0;
          const bool desc = (((r * 64 + lane) & k) == 0);
          const uint64_t mx = a[r] > y ? a[r] : y;
          const uint64_t mn = a[r] > y ? y : a[r];
          a[r] = (lower == desc) ? mx : mn;
        }
      }
    }
  }
}

// Inserts x into the descending 64-entry list held one entry per lane.
__device__ __forceinline__ void wave_insert(uint64_t& L, uint64_t x) {
  const int lane = threadIdx.x & 63;
  const int pos = __popcll(__ballot(L > x));
  const uint64_t up = shfl_up64(L, 1);
  L = lane < pos ? L : (lane == pos ? x : up);
}

// Inserts the keys of `m` (lanes of `key`) that beat the k-th best into L.
__device__ __forceinline__ void insert_masked(uint64_t& L, uint64_t& tau, uint64_t key,
                                              uint64_t m, int k) {
  while (m) {
    const int i = __builtin_ctzll(m);
    m &= m - 1;
    const uint64_t x = readlane64(key, i);
    if (x > tau) {
      wave_insert(L, x);
      tau = readlane64(L, k - 1);
    }
  }
}

template <int KC>
__global__ __launch_bounds__(kThreads) void topk_stage1(TopkLaunch a) {
  constexpr int kQPitch = Smem<KC>::kQPitch;
  constexpr int kLoads = KC / 16;            // 16-byte loads per lane per chunk and row tile
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
  int64_t tile = blockIdx.x;
  if (tile >= n_tiles) return;

  // Query chunk staging: 16-byte pieces loaded to registers before the
  // embedding loads of the same chunk (so waiting for them leaves the
  // embedding loads in flight), written to an LDS buffer after the MFMAs.
  constexpr int kQPieces = kQB * KC / 8;
  constexpr int kQPer = kQPieces / kThreads;
  static_assert(kQPieces % kThreads == 0, "query staging shape");
  u32x4 qreg[kQPer];
  auto load_q = [&](int c) {
#pragma unroll
    for (int i = 0; i < kQPer; ++i) {
      const int p = tid + i * kThreads;
      const int qr = p / (KC / 8), col = (p % (KC / 8)) * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (qb0 + qr < a.n_q)
        v = *reinterpret_cast<const u32x4*>(a.q + (int64_t)(qb0 + qr) * D + (int64_t)c * KC + col);
      qreg[i] = v;
    }
  };
  auto store_q = [&](int b) {
#pragma unroll
    for (int i = 0; i < kQPer; ++i) {
      const int p = tid + i * kThreads;
      const int qr = p / (KC / 8), col = (p % (KC / 8)) * 8;
      *reinterpret_cast<u32x4*>(&sm.u.q[b][qr * kQPitch + col]) = qreg[i];
    }
  };
  // This lane's embedding rows in tile t (rows past the end are clamped to
  // the last row and masked in the epilogue).
  const uint16_t* erow[2];
  auto set_rows = [&](int64_t t, const uint16_t* (&dst)[2]) {
#pragma unroll
    for (int ft = 0; ft < 2; ++ft) {
      int64_t f = t * kFT + wave * kFTW + ft * 32 + row;
      if (f >= a.n_facts) f = a.n_facts - 1;
      dst[ft] = a.emb + f * D + grp * 8;
    }
  };
  u32x4 e0[2][kLoads], e1[2][kLoads];
  auto load_e = [&](u32x4 (&dst)[2][kLoads], const uint16_t* const (&rows)[2], int c) {
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
      for (int i = 0; i < kLoads; ++i)
        dst[ft][i] = *reinterpret_cast<const u32x4*>(rows[ft] + (int64_t)c * KC + i * 16);
  };
  float16v acc[2][4];
  // MFMAs of one chunk; the query fragments of k-step s+1 are read from LDS
  // while the eight MFMAs of step s run.
  auto compute = [&](const u32x4 (&eb)[2][kLoads], int b) {
    const _Float16* qs = sm.u.q[b] + row * kQPitch + grp * 8;
    half8 bq[4], bn[4];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt)
      bq[qt] = *reinterpret_cast<const half8*>(qs + qt * 32 * kQPitch);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      if (s + 1 < kSteps) {
#pragma unroll
        for (int qt = 0; qt < 4; ++qt)
          bn[qt] = *reinterpret_cast<const half8*>(qs + qt * 32 * kQPitch + (s + 1) * 16);
      }
#pragma unroll
      for (int ft = 0; ft < 2; ++ft) {
        const half8 av = __builtin_bit_cast(half8, eb[ft][s]);
#pragma unroll
        for (int qt = 0; qt < 4; ++qt)
          acc[ft][qt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bq[qt], acc[ft][qt], 0, 0, 0);
      }
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) bq[qt] = bn[qt];
    }
  };

  // Selection state: lane j < kQPW of this wave holds the k-th best key of
  // its query j (0 until the lists exist).
  uint64_t tau_reg = 0;
  bool have_lists = false;

  // One stream of chunks over this workgroup's tiles: the loads of the
  // next chunk -- the next tile's first chunk at a tile's end -- go to e1
  // before the MFMAs of the current chunk (in e0), and stay in flight
  // through the selection at a tile's end; e1 moves to e0 when the MFMAs
  // need it.  Query chunk c sits in LDS buffer c & 1.
  set_rows(tile, erow);
  load_q(0);
  load_e(e0, erow, 0);
  store_q(0);
  __syncthreads();
  auto zero_acc = [&] {
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
      for (int qt = 0; qt < 4; ++qt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[ft][qt][e] = 0.f;
  };
  zero_acc();
  int c = 0;
  while (true) {
    const bool last = c == n_chunks - 1;
    const int64_t next_tile = tile + gridDim.x;
    const bool has_next = !last || next_tile < n_tiles;
    const uint16_t* nrow[2] = {erow[0], erow[1]};
    if (last && has_next) set_rows(next_tile, nrow);
    const int next_c = last ? 0 : c + 1;
    if (has_next) {
      if (!last) load_q(next_c);
      load_e(e1, nrow, next_c);
    }
    compute(e0, c & 1);
    if (!last) {
      store_q(next_c & 1);
#pragma unroll
      for (int ft = 0; ft < 2; ++ft)
#pragma unroll
        for (int i = 0; i < kLoads; ++i) e0[ft][i] = e1[ft][i];
      __syncthreads();
      c = next_c;
      continue;
    }
    __syncthreads();   // the staged scores below reuse the query buffers

    // Selection: two passes of 128 fact rows through LDS to the query-owning waves.
    const int64_t fact0 = tile * kFT;
    for (int pass = 0; pass < 2; ++pass) {
      const int64_t f0 = fact0 + pass * kHalfRows;
      if (f0 >= a.n_facts) break;                       // uniform
      const int valid = (int)min<int64_t>(kHalfRows, a.n_facts - f0);
      if (wave / 2 == pass) {
#pragma unroll
        for (int ft = 0; ft < 2; ++ft) {
          const int rbase = (wave % 2) * kFTW + ft * 32;
#pragma unroll
          for (int qt = 0; qt < 4; ++qt)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int fr = rbase + 8 * (e / 4) + 4 * grp + (e % 4);
              sm.u.s[fr * kSPitch + qt * 32 + row] = acc[ft][qt][e];
            }
        }
      }
      __syncthreads();
      const int q0 = wave * kQPW;
      const int nq = min(kQPW, a.n_q - qb0 - q0);       // uniform per wave
      // all of this wave's staged scores at once: one LDS round trip
      float s0[kQPW], s1[kQPW];
#pragma unroll
      for (int j = 0; j < kQPW; ++j) {
        s0[j] = sm.u.s[lane * kSPitch + q0 + j];
        s1[j] = sm.u.s[(64 + lane) * kSPitch + q0 + j];
      }
      const bool ok0 = lane < valid, ok1 = 64 + lane < valid;
      const uint32_t id0 = (uint32_t)(f0 + lane), id1 = (uint32_t)(f0 + 64 + lane);
#pragma unroll
      for (int j = 0; j < kQPW; ++j) {
        if (j >= nq) break;
        const uint64_t key0 = ok0 ? key_of(ord_of(s0[j]), id0) : 0;
        const uint64_t key1 = ok1 ? key_of(ord_of(s1[j]), id1) : 0;
        const int q = q0 + j;
        uint64_t L;
        if (!have_lists) {
          uint64_t v[2] = {key0, key1};
          wave_sort_desc<2>(v);
          L = v[0];
        } else {
          uint64_t tau = readlane64(tau_reg, j);
          const uint64_t m0 = __ballot(key0 > tau);
          const uint64_t m1 = __ballot(key1 > tau);
          if ((m0 | m1) == 0) continue;
          L = sm.list[q * kMaxK + lane];
          insert_masked(L, tau, key0, m0, k);
          insert_masked(L, tau, key1, m1, k);
        }
        sm.list[q * kMaxK + lane] = L;
        const uint64_t t = readlane64(L, k - 1);
        if (lane == j) tau_reg = t;
      }
      have_lists = true;
      __syncthreads();
    }
    if (!has_next) break;
    load_q(0);
    store_q(0);
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
      for (int i = 0; i < kLoads; ++i) e0[ft][i] = e1[ft][i];
    __syncthreads();
    tile = next_tile;
    erow[0] = nrow[0];
    erow[1] = nrow[1];
    c = 0;
    zero_acc();
  }

  // Write each query's sorted list (the first k entries).
  for (int j = 0; j < kQPW; ++j) {
    const int q = wave * kQPW + j;
    if (qb0 + q >= a.n_q) break;
    if (lane < k)
      a.partial[((int64_t)(qb0 + q) * a.n_wg + blockIdx.x) * k + lane] = sm.list[q * kMaxK + lane];
  }
}

constexpr int kMergeThreads = 256;

// Stage 2: the k best of n_wg sorted lists of k keys, by a tournament over
// the list heads held by the 64 lanes of wave 0 (lane l owns lists l,
// l+64, l+128, l+192).
__global__ __launch_bounds__(kMergeThreads) void topk_stage2(TopkLaunch a) {
  __shared__ uint64_t buf[256 * kMaxK];
  const int q = blockIdx.x;
  const int k = a.k;
  const int n = a.n_wg;
  const uint64_t* src = a.partial + (int64_t)q * n * k;
  for (int i = threadIdx.x; i < n * k; i += kMergeThreads) buf[i] = src[i];
  __syncthreads();
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  int ptr[4];
  uint64_t head[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int list = lane + 64 * m;
    ptr[m] = 0;
    head[m] = list < n ? buf[list * k] : 0;
  }
  for (int s = 0; s < k; ++s) {
    uint64_t best = head[0];
#pragma unroll
    for (int m = 1; m < 4; ++m) best = head[m] > best ? head[m] : best;
    uint64_t g = best;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const uint64_t o = shfl_xor64(g, off);
      g = o > g ? o : g;
    }
    // real keys are distinct, so exactly one head equals g
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (head[m] == g) {
        const int list = lane + 64 * m;
        ++ptr[m];
        head[m] = ptr[m] < k ? buf[list * k + ptr[m]] : 0;
      }
    }
    if (lane == 0) {
      a.ids[(int64_t)q * k + s] = (int32_t)(0xFFFFFFFFu - (uint32_t)g);
      a.scores[(int64_t)q * k + s] = float_of((uint32_t)(g >> 32));
    }
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
