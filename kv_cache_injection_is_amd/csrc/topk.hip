// Exact top-k inner-product search over the fp16 fact embeddings.
//
// Stands in for the GPU-resident retrieval index of the InferScale
// explainer pages ("InferScale: GPU-Native KV Injection for Personalized
// LLM Serving", technical summary, Contributions: GPU-native system design);
// the pages do not describe the index, so this is an exact brute-force
// search.  Order: score descending, ties to the lower fact id.
//
// The selection rests on one fact: the k-th largest score within any subset
// of the facts is a lower bound on the k-th largest score overall.
//   1. scan (sample mode): MFMA scores of facts [0, S) (S = a few percent of
//      the store) for every query, written out;
//   2. threshold: per query, the exact k-th largest sample score by an
//      8-bit-digit radix select; that is the bound tau;
//   3. scan (stream mode): MFMA scores of all facts; a score >= tau is a
//      candidate, appended to the query's list with one atomic -- about
//      k*N/S of them, while every true top-k fact is among them;
//   4. final: per query, radix select of the k-th largest candidate key
//      (score, then lower id), then the k winners sorted across a wave.
// The scan (persistent, one workgroup of 4 waves per CU): a 256-fact tile is
// split over the 4 waves (64 facts each, two 32-row MFMA tiles,
// v_mfma_f32_32x32x16_f16, fp32 accumulation) against all 128 queries of a
// query block.  The A operand (embedding rows) streams from HBM straight
// into registers one 128-dim chunk ahead; the B operand (queries) comes from
// a double-buffered LDS copy of the current chunk.  The dot product is
// order-free in k, so at k-step s lane (row, grp) holds halves
// [(2s+grp)*8, +8) of the chunk for both operands, which makes the two
// lanes of a row read 32 contiguous bytes per load.  Both scan modes run the
// same instruction sequence per tile, so a sample fact scores identically
// in both.
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
  _Float16 q[2][kQB * kQPitch];
};

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
  const int lo = __shfl_xor((int)(uint32_t)v, m);
  const int hi = __shfl_xor((int)(uint32_t)(v >> 32), m);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
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

template <int KC, bool kSample>
__global__ __launch_bounds__(kThreads) void topk_scan(TopkLaunch a) {
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
  const int64_t limit = kSample ? a.sample_n : a.n_facts;
  const int64_t n_tiles = (limit + kFT - 1) / kFT;
  int64_t tile = blockIdx.x;
  if (tile >= n_tiles) return;

  // Threshold of this lane's query in each 32-query tile.
  float tau[4];
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    const int q = qb0 + qt * 32 + row;
    tau[qt] = (!kSample && q < a.n_q) ? a.tau[q] : 0.f;
  }

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
      *reinterpret_cast<u32x4*>(&sm.q[b][qr * kQPitch + col]) = qreg[i];
    }
  };
  // This lane's embedding rows in tile t (rows past the end are clamped to
  // the last row and masked when scores are emitted).
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
    const _Float16* qs = sm.q[b] + row * kQPitch + grp * 8;
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
  auto zero_acc = [&] {
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
      for (int qt = 0; qt < 4; ++qt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[ft][qt][e] = 0.f;
  };
  // Scores of tile t out: every score (sample mode) or those >= tau.
  // Accumulator element e of lane (row, grp) is fact row 8*(e/4) + 4*grp +
  // e%4 of its 32-row tile and query column `row` of its 32-query tile.
  auto emit = [&](int64_t t) {
#pragma unroll
    for (int ft = 0; ft < 2; ++ft) {
      const int64_t fbase = t * kFT + wave * kFTW + ft * 32 + 4 * grp;
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        const int q = qb0 + qt * 32 + row;
        if (q >= a.n_q) continue;
        if (kSample) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int64_t f = fbase + 8 * (e / 4) + (e % 4);
            if (f < limit) a.sample[(int64_t)q * a.sample_n + f] = acc[ft][qt][e];
          }
        } else {
          uint32_t m = 0;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int64_t f = fbase + 8 * (e / 4) + (e % 4);
            m |= (f < limit && acc[ft][qt][e] >= tau[qt]) ? (1u << e) : 0u;
          }
          if (m) {   // rare: one counter bump per lane and row tile
            uint32_t pos = atomicAdd(&a.count[q], (uint32_t)__builtin_popcount(m));
            uint64_t* dst = a.cand + (int64_t)q * a.n_facts;
#pragma unroll
            for (int e = 0; e < 16; ++e)
              if (m & (1u << e))
                dst[pos++] = key_of(ord_of(acc[ft][qt][e]),
                                    (uint32_t)(fbase + 8 * (e / 4) + (e % 4)));
          }
        }
      }
    }
  };

  // One stream of chunks over this workgroup's tiles: the loads of the
  // next chunk -- the next tile's first chunk at a tile's end -- go to e1
  // before the MFMAs of the current chunk (in e0); e1 moves to e0 when the
  // MFMAs need it.  Query chunk c sits in LDS buffer c & 1.
  set_rows(tile, erow);
  load_q(0);
  load_e(e0, erow, 0);
  store_q(0);
  __syncthreads();
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
      load_q(next_c);
      load_e(e1, nrow, next_c);
    }
    compute(e0, c & 1);
    if (last) {
      emit(tile);
      zero_acc();
      if (!has_next) break;
      tile = next_tile;
      erow[0] = nrow[0];
      erow[1] = nrow[1];
    }
    __syncthreads();   // every wave is done with query buffer next_c & 1
    store_q(next_c & 1);
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
      for (int i = 0; i < kLoads; ++i) e0[ft][i] = e1[ft][i];
    __syncthreads();
    c = next_c;
  }
}

// ---------------------------------------------------------------------------
// The scan for emb_dim % 64 == 0 (tile-blocked embeddings): each 256-fact x
// 64-dim block (32 KB, contiguous in HBM) and the matching query chunk go
// from memory straight into a 3-stage LDS ring (global_load_lds_dwordx4, no
// registers), so two chunks are in flight while the MFMAs of a third run.
// A stage holds the tile's 256 rows and the block's 128 query rows as 8
// 16-byte pieces each; piece p of row r sits at slot r*8 + (p ^ (r & 7)),
// which spreads the 32 rows an MFMA fragment read touches over all banks.
// Each DMA instruction fills 64 consecutive slots (1 KB) from 8 whole
// 128-byte row segments.  The ring's waits are explicit (vmcnt), since the
// compiler does not track these transfers.
constexpr int kStages = 3;
constexpr int kDmaKC = 64;                    // dims per chunk
constexpr int kEPieces = kFT * kDmaKC / 8;    // 16-byte pieces of a stage's rows
constexpr int kQPiecesDma = kQB * kDmaKC / 8;
constexpr int kEDma = kEPieces / 64 / kWaves; // DMA instructions per wave per stage
constexpr int kQDma = kQPiecesDma / 64 / kWaves;
constexpr int kDmaPerStage = kEDma + kQDma;

typedef __attribute__((address_space(3))) char* lds_cptr;

struct DmaSmem {
  u32x4 e[kStages][kEPieces];
  u32x4 q[kStages][kQPiecesDma];
};

// One 16-byte piece per lane from `g` into LDS bytes [lds + 16*lane, +16).
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds), "v"(g) : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <bool kSample>
__global__ __launch_bounds__(kThreads) void topk_scan_dma(TopkLaunch a) {
  __shared__ DmaSmem sm;
  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int row = lane % 32;
  const int grp = lane / 32;
  const int qb0 = blockIdx.y * kQB;
  const int D = a.emb_dim;
  const int n_chunks = D / kDmaKC;
  const int64_t limit = kSample ? a.sample_n : a.n_facts;
  const int64_t n_tiles = (limit + kFT - 1) / kFT;
  if ((int64_t)blockIdx.x >= n_tiles) return;
  const int64_t my_tiles = (n_tiles - blockIdx.x + gridDim.x - 1) / gridDim.x;
  const int64_t total = my_tiles * n_chunks;

  float tau[4];
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    const int q = qb0 + qt * 32 + row;
    tau[qt] = (!kSample && q < a.n_q) ? a.tau[q] : 0.f;
  }

  const uint32_t e_lds = (uint32_t)(size_t)(lds_cptr)(void*)&sm.e[0][0];
  const uint32_t q_lds = (uint32_t)(size_t)(lds_cptr)(void*)&sm.q[0][0];
  // Chunk g of this workgroup's stream: tile blockIdx.x + (g / n_chunks) *
  // gridDim.x, dims [(g % n_chunks) * 64, +64).
  auto issue = [&](int64_t g) {
    const int64_t t = blockIdx.x + (g / n_chunks) * gridDim.x;
    const int c = (int)(g % n_chunks);
    const int b = (int)(g % kStages);
    // the tile's 256 x 64 block of the blocked layout: 32 KB contiguous
    const uint16_t* blk = a.emb + (t * n_chunks + c) * (int64_t)(kFT * kDmaKC);
#pragma unroll
    for (int i = 0; i < kEDma; ++i) {
      const int slot = (wave * kEDma + i) * 64 + lane;
      const int r = slot / 8, piece = (slot % 8) ^ (r & 7);
      const uint32_t dst = __builtin_amdgcn_readfirstlane(
          e_lds + (uint32_t)((b * kEPieces + (wave * kEDma + i) * 64) * 16));
      dma16(blk + r * kDmaKC + piece * 8, dst);
    }
#pragma unroll
    for (int i = 0; i < kQDma; ++i) {
      const int slot = (wave * kQDma + i) * 64 + lane;
      const int r = slot / 8, piece = (slot % 8) ^ (r & 7);
      const uint16_t* src = qb0 + r < a.n_q ? a.q + (int64_t)(qb0 + r) * D + c * kDmaKC + piece * 8
                                            : a.q;
      const uint32_t dst = __builtin_amdgcn_readfirstlane(
          q_lds + (uint32_t)((b * kQPiecesDma + (wave * kQDma + i) * 64) * 16));
      dma16(src, dst);
    }
  };

  float16v acc[2][4];
  auto zero_acc = [&] {
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
      for (int qt = 0; qt < 4; ++qt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[ft][qt][e] = 0.f;
  };
  // k-step s uses logical pieces 2s + grp of every row (both operands).
  auto compute = [&](int b) {
    const u32x4* es = sm.e[b];
    const u32x4* qs = sm.q[b];
#pragma unroll
    for (int s = 0; s < kDmaKC / 16; ++s) {
      const int x = (2 * s + grp) ^ (row & 7);
      half8 av[2], bv[4];
#pragma unroll
      for (int ft = 0; ft < 2; ++ft)
        av[ft] = __builtin_bit_cast(half8, es[(wave * kFTW + ft * 32 + row) * 8 + x]);
#pragma unroll
      for (int qt = 0; qt < 4; ++qt)
        bv[qt] = __builtin_bit_cast(half8, qs[(qt * 32 + row) * 8 + x]);
#pragma unroll
      for (int ft = 0; ft < 2; ++ft)
#pragma unroll
        for (int qt = 0; qt < 4; ++qt)
          acc[ft][qt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[ft], bv[qt], acc[ft][qt], 0, 0, 0);
    }
  };
  auto emit = [&](int64_t t) {
#pragma unroll
    for (int ft = 0; ft < 2; ++ft) {
      const int64_t fbase = t * kFT + wave * kFTW + ft * 32 + 4 * grp;
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        const int q = qb0 + qt * 32 + row;
        if (q >= a.n_q) continue;
        if (kSample) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int64_t f = fbase + 8 * (e / 4) + (e % 4);
            if (f < limit) a.sample[(int64_t)q * a.sample_n + f] = acc[ft][qt][e];
          }
        } else {
          uint32_t m = 0;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int64_t f = fbase + 8 * (e / 4) + (e % 4);
            m |= (f < limit && acc[ft][qt][e] >= tau[qt]) ? (1u << e) : 0u;
          }
          if (m) {
            uint32_t pos = atomicAdd(&a.count[q], (uint32_t)__builtin_popcount(m));
            uint64_t* dst = a.cand + (int64_t)q * a.n_facts;
#pragma unroll
            for (int e = 0; e < 16; ++e)
              if (m & (1u << e))
                dst[pos++] = key_of(ord_of(acc[ft][qt][e]),
                                    (uint32_t)(fbase + 8 * (e / 4) + (e % 4)));
          }
        }
      }
    }
  };

  for (int64_t g = 0; g < kStages - 1 && g < total; ++g) issue(g);
  zero_acc();
  for (int64_t g = 0; g < total; ++g) {
    // chunk g's transfers are done once at most the later stages' are in flight
    if (g + 1 < total) wait_vm<kDmaPerStage>(); else wait_vm<0>();
    __syncthreads();   // every wave's transfers for chunk g landed; chunk g-1's buffer is free
    if (g + kStages - 1 < total) issue(g + kStages - 1);
    compute((int)(g % kStages));
    if (g % n_chunks == n_chunks - 1) {
      emit(blockIdx.x + (g / n_chunks) * gridDim.x);
      zero_acc();
    }
  }
  wait_vm<0>();
}

constexpr int kSelThreads = 256;

// The k-th largest of n values (32- or 64-bit) in global memory, by
// most-significant-digit radix select over 8-bit digits.  All threads of
// the workgroup call it; the result is returned to all.
template <typename V>
__device__ V radix_kth_largest(const V* vals, int64_t n, int k, uint32_t* hist, V* share) {
  constexpr int kBits = 8 * sizeof(V);
  V prefix = 0, mask = 0;
  int remaining = k;
  for (int shift = kBits - 8; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    for (int64_t i = threadIdx.x; i < n; i += kSelThreads) {
      const V v = vals[i];
      if ((v & mask) == prefix) atomicAdd(&hist[(uint32_t)(v >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t above = 0;
      int b = 255;
      for (; b > 0; --b) {
        if (above + hist[b] >= (uint32_t)remaining) break;
        above += hist[b];
      }
      share[0] = (V)b;
      share[1] = (V)above;
    }
    __syncthreads();
    const V b = share[0];
    remaining -= (int)share[1];
    prefix |= b << shift;
    mask |= (V)255 << shift;
    __syncthreads();
  }
  return prefix;
}

// Per query: the bound tau = k-th largest sample score (lowered by a hair
// so that a fact scoring exactly tau in the sample still passes), and the
// candidate counter cleared for the stream scan.
__global__ __launch_bounds__(kSelThreads) void topk_threshold(TopkLaunch a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t share[2];
  const int q = blockIdx.x;
  const float* v = a.sample + (int64_t)q * a.sample_n;
  // float order as uint32 order: compare the order-preserving codes
  uint32_t* codes = reinterpret_cast<uint32_t*>(a.sample) + (int64_t)q * a.sample_n;
  for (int64_t i = threadIdx.x; i < a.sample_n; i += kSelThreads) codes[i] = ord_of(v[i]);
  __syncthreads();
  const uint32_t kth = radix_kth_largest<uint32_t>(codes, a.sample_n, a.k, hist, share);
  if (threadIdx.x == 0) {
    const float t = float_of(kth);
    a.tau[q] = t - (fabsf(t) * 0x1p-20f + 0x1p-100f);
    a.count[q] = 0;
  }
}

// Per query: the k best candidates, in order.
__global__ __launch_bounds__(kSelThreads) void topk_final(TopkLaunch a) {
  __shared__ uint32_t hist[256];
  __shared__ uint64_t share[2];
  __shared__ uint64_t best[kMaxK];
  __shared__ uint32_t n_best;
  const int q = blockIdx.x;
  const int64_t n = a.count[q];
  const uint64_t* keys = a.cand + (int64_t)q * a.n_facts;
  const uint64_t kth = radix_kth_largest<uint64_t>(keys, n, a.k, hist, share);
  if (threadIdx.x == 0) n_best = 0;
  if (threadIdx.x < kMaxK) best[threadIdx.x] = 0;
  __syncthreads();
  for (int64_t i = threadIdx.x; i < n; i += kSelThreads) {
    const uint64_t v = keys[i];
    if (v >= kth) best[atomicAdd(&n_best, 1u)] = v;   // exactly k keys (keys are distinct)
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    uint64_t v[1] = {best[threadIdx.x]};
    wave_sort_desc<1>(v);
    if (threadIdx.x < a.k) {
      a.ids[(int64_t)q * a.k + threadIdx.x] = (int32_t)(0xFFFFFFFFu - (uint32_t)v[0]);
      a.scores[(int64_t)q * a.k + threadIdx.x] = float_of((uint32_t)(v[0] >> 32));
    }
  }
}

__global__ __launch_bounds__(256) void emb_relayout(const uint16_t* __restrict__ rows,
                                                   int64_t first, int64_t n, int32_t D,
                                                   uint16_t* __restrict__ emb) {
  const int pieces = D / 8;
  const int n_chunks = D / kDmaKC;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n * pieces) return;
  const int64_t r = i / pieces;
  const int p = (int)(i % pieces);
  const int64_t f = first + r;
  const int64_t dst = ((f / kFT * n_chunks + p / 8) * kFT + f % kFT) * kDmaKC + (p % 8) * 8;
  *reinterpret_cast<u32x4*>(emb + dst) = *reinterpret_cast<const u32x4*>(rows + r * D + p * 8);
}

}  // namespace

hipError_t launch_emb_relayout(const uint16_t* rows, int64_t first, int64_t n, int32_t emb_dim,
                               uint16_t* emb, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t threads = n * (emb_dim / 8);
  hipLaunchKernelGGL(emb_relayout, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                     rows, first, n, emb_dim, emb);
  return hipGetLastError();
}

int topk_workgroups(int64_t n_facts) {
  const int64_t tiles = (n_facts + kFT - 1) / kFT;
  return (int)(tiles < 256 ? tiles : 256);
}

int64_t topk_sample_size(int64_t n_facts) {
  int64_t s = n_facts / 32;
  if (s < 4096) s = 4096;
  s = (s + kFT - 1) / kFT * kFT;
  return s < n_facts ? s : n_facts;
}

hipError_t launch_topk(const TopkLaunch& a, hipStream_t stream) {
  if (a.n_q == 0) return hipSuccess;
  if (a.k < 1 || a.k > kMaxK || a.k > a.sample_n || a.n_q > kQB) return hipErrorInvalidValue;
  const unsigned qblocks = (unsigned)((a.n_q + kQB - 1) / kQB);
  const dim3 g_sample((unsigned)topk_workgroups(a.sample_n), qblocks);
  const dim3 g_stream((unsigned)topk_workgroups(a.n_facts), qblocks);
  if (a.emb_dim % kDmaKC == 0) {
    hipLaunchKernelGGL((topk_scan_dma<true>), g_sample, dim3(kThreads), 0, stream, a);
  } else if (a.emb_dim % 32 == 0) {
    hipLaunchKernelGGL((topk_scan<32, true>), g_sample, dim3(kThreads), 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(topk_threshold, dim3((unsigned)a.n_q), dim3(kSelThreads), 0, stream, a);
  if (a.emb_dim % kDmaKC == 0)
    hipLaunchKernelGGL((topk_scan_dma<false>), g_stream, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((topk_scan<32, false>), g_stream, dim3(kThreads), 0, stream, a);
  hipLaunchKernelGGL(topk_final, dim3((unsigned)a.n_q), dim3(kSelThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace is
