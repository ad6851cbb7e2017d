// Exact top-k inner-product search over the fp16 fact embeddings.
//
// Stands in for the GPU-resident retrieval index of the InferScale
// explainer pages ("InferScale: GPU-Native KV Injection for Personalized
// LLM Serving", technical summary, Contributions: GPU-native system design);
// the pages do not describe the index, so this is an exact brute-force
// search.  Order: score descending, ties to the lower fact id.
//
// The selection rests on one fact: if k distinct facts all score at least
// tau, the k-th largest score overall is at least tau, so every fact of the
// true top k scores >= tau.
//   1. scan (sample mode): MFMA scores of the facts of the first few tiles
//      (a few percent of the store) for every query; each lane reduces the
//      16 scores it holds to their maximum, so the sample is cut into
//      disjoint groups of 16 facts and each group reports its best score;
//      the scan also keeps every sample score as a 4-byte order code;
//   2. threshold: per query, the k-th largest group maximum is tau -- k
//      groups, hence k distinct facts, reach it -- and the sample's
//      candidates (codes >= tau, from the groups whose maximum reaches it)
//      go to the head of the query's candidate list (for at most four
//      queries on the shared query tile the stream scan finds tau itself,
//      over the whole store, and the sample keeps no codes);
//   3. scan (stream mode): MFMA scores of the facts after the sample; a
//      score >= tau is a candidate, appended to the workgroup's own region
//      of the query's candidate list (position from LDS or from the query's
//      own lanes, so the HBM stream is never drained to wait for a global
//      atomic);
//   4. final: per query, the candidate regions are gathered and the k best
//      (score, then lower id) keys are placed by counting, for each key, the
//      keys above it (after cutting many candidates down to those that reach
//      a bound k of them reach).  For one request of a retrieve-and-inject
//      call the final kernel then composes the request.
// Steps 2 and 4 find their bounds the same way (offer_bound): each thread
// offers its best value, each wave ranks its 64 offers, and the least of
// the waves' ceil(k/4)-th best is reached by k offers; many equal values
// fall through to a radix select.
// Small stores take one pass instead (at most 8M scores for the launch and
// 131,072 facts, any width): the scan writes every fact's score as an
// order code together with every group's maximum, and the final kernel
// takes the bound from all the groups (offer_bound over its threads' best
// group maxima), then gathers the codes that reach it from the groups whose
// maximum does (a few more than k groups).  No sample scan and no threshold
// launch; the codes cost 4 bytes per (query, fact) of writes.
// Every scan computes a fact's score as the same MFMA chain, so a sample
// fact scores identically in the sample and the stream, whatever the
// variant or tile size, and a query scores alike alone or in a batch.
//
// Scan layout.  The store keeps the embeddings tile-blocked (see kernels.h):
// every 256-fact x 64-dim block is one contiguous 32 KB span.  Persistent
// workgroups (4 waves, one per SIMD, one workgroup per CU) stream their
// tiles' blocks from memory straight into an LDS ring with
// global_load_lds_dwordx4 (no registers on the way); v_mfma_f32_32x32x16_f16
// forms the scores with fp32 accumulation.  Two variants:
//   topk_scan     other widths and 33-64-query batches: each wave owns 64
//                 facts of a 256-fact tile against every query tile the
//                 launch fills; the query chunk is staged with the fact
//                 block in a 3-stage ring, and a wave refills its own fact
//                 rows without waiting for the other waves;
//   topk_scan_rq  width 1024: each wave keeps 32 query rows in registers
//                 for the whole launch and the ring (8 or 16 stages, all
//                 but one in flight) holds fact rows only.  Full batches
//                 (65-128 queries): wave w holds query tile w and scores
//                 every fact of a 32- or 64-fact tile, candidates staged in
//                 LDS until the loop ends.  Batches of at most 32 (shared
//                 mode): every wave holds the same tile and scores its own
//                 32-fact row tile of a 128-fact stage.  Sample and stream
//                 may use different tile sizes.
#include <hip/hip_runtime.h>

#include "compose_request.h"
#include "kernels.h"

#ifndef IS_TOPK_RESIDENT
#define IS_TOPK_RESIDENT 1   // full batches at width 1024 keep their queries in registers
#endif
#ifndef IS_TOPK_STREAM_FT
#define IS_TOPK_STREAM_FT 32   // stream tile (facts) of full batches: 32 or 64 (32 measured
#endif                         // faster on the 50k and the 1M index)
static_assert(IS_TOPK_STREAM_FT == 32 || IS_TOPK_STREAM_FT == 64,
              "stream tiles of 32 or 64 facts (128-fact tiles spill with the fragment prefetch)");
#ifndef IS_TOPK_DENSE_CODES
#define IS_TOPK_DENSE_CODES (1 << 23)   // most score codes (queries x facts) the one-pass
#endif                                  // mode writes; 0 turns it off

namespace is {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kQB = 128;              // queries per launch
constexpr int kFTW = 64;              // facts per wave per tile (two MFMA row tiles)
constexpr int kFT = kWaves * kFTW;    // facts per tile
constexpr int kMaxK = 64;
constexpr int kStages = 3;
constexpr int kKC = kTopkChunk;       // dims per chunk
constexpr int kEPieces = kFT * kKC / 8;   // 16-byte pieces of a stage's fact rows
constexpr int kQPieces = kQB * kKC / 8;   // ... and of its query rows
constexpr int kEDma = kEPieces / 64 / kWaves;   // DMA instructions per wave per stage
// Query rows are staged in tiles of 32 (one MFMA column tile); a launch
// stages and scores only the tiles its queries fill, QT of them.
template <int QT>
constexpr int q_dma() { return QT * 32 * kKC / 8 / 64 / kWaves; }   // per wave per stage
static_assert(kFT == kTopkTile, "tile size");

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

// The stream bound from the k-th largest sample group maximum (an order
// code; 0 marks an empty group: fewer than k groups reached it), lowered by
// a hair so that rounding cannot drop a fact that ties it.
__device__ __forceinline__ float tau_of_code(uint32_t kth) {
  const float t = kth == 0 ? -INFINITY : float_of(kth);
  return kth == 0 ? t : t - (fabsf(t) * 0x1p-20f + 0x1p-100f);
}

// A lower bound on the k-th largest of n (<= 1024) order codes held by a
// wave, code lane + 64 j in v[j] (0 past n), exact to 20 bits below the
// prefix that all nonzero codes share: the search starts from that common
// prefix and keeps a bit when at least k codes reach the prefix with it
// set.  Any code that k codes reach is a valid bound, and the low bits it
// gives up only let a few more facts through as candidates.  0 when fewer
// than k codes are nonzero.
constexpr int kWaveKthMax = 1024;
__device__ __forceinline__ void wave_load_codes(const uint32_t* __restrict__ src, int64_t n,
                                                uint32_t (&v)[kWaveKthMax / 64]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < kWaveKthMax / 64; ++j)
    v[j] = (lane + 64 * j < n) ? src[lane + 64 * j] : 0u;
}
template <int S>
__device__ uint32_t wave_kth_code_s(const uint32_t (&v)[kWaveKthMax / 64], int k) {
  uint32_t hi = 0, lo = 0xFFFFFFFFu, nz = 0;
#pragma unroll
  for (int j = 0; j < S; ++j) {
    hi = v[j] > hi ? v[j] : hi;
    lo = (v[j] != 0u && v[j] < lo) ? v[j] : lo;
    nz += (uint32_t)__builtin_popcountll(__ballot(v[j] != 0u));
  }
  if (nz < (uint32_t)k) return 0u;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t h = (uint32_t)__shfl_xor((int)hi, off), l = (uint32_t)__shfl_xor((int)lo, off);
    hi = h > hi ? h : hi;
    lo = l < lo ? l : lo;
  }
  const int common = __builtin_clz(hi ^ lo | 1u);   // leading bits every nonzero code shares
  const int top = 31 - common;                       // highest bit left to decide
  uint32_t prefix = common == 0 ? 0u : (hi & ~(0xFFFFFFFFu >> common));
  const int last = top - 19 > 0 ? top - 19 : 0;
  for (int b = top; b >= last; --b) {
    const uint32_t cand = prefix | (1u << b);
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < S; ++j) cnt += (uint32_t)__builtin_popcountll(__ballot(v[j] >= cand));
    if (cnt >= (uint32_t)k) prefix = cand;
  }
  return prefix;
}
__device__ uint32_t wave_kth_code(const uint32_t (&v)[kWaveKthMax / 64], int64_t n, int k) {
  return n <= 512 ? wave_kth_code_s<8>(v, k) : wave_kth_code_s<16>(v, k);
}

// Side job of the sample scan (a retrieve-and-inject call): zero the words
// the composition of the same call counts and marks in, and its status
// word, so that no separate clearing launch sits on the request's path; the
// launches in between order them.
__device__ __forceinline__ void side_zero(const TopkLaunch& a) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.zero_words; i += stride)
    a.zero[i] = 0u;
  if (a.zero_status != nullptr && blockIdx.x == 0 && threadIdx.x == 0) *a.zero_status = 0;
}

// First tile of workgroup w when n_tiles tiles are dealt round-robin to G
// workgroups, counted as if each workgroup's tiles were contiguous: the
// workgroup's candidate region starts at this tile's first fact.
__device__ __forceinline__ int64_t region_tile(int w, int64_t n_tiles, int G) {
  const int64_t per = n_tiles / G, extra = n_tiles % G;
  return (int64_t)w * per + (w < extra ? w : extra);
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
  const int lo = __shfl_xor((int)(uint32_t)v, m);
  const int hi = __shfl_xor((int)(uint32_t)(v >> 32), m);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Minimum over the wave: running minima within each row of 16 lanes
// (row_shr 1, 2, 4, 8), then the rows chained (row_bcast15 into rows 1 and
// 3, row_bcast31 into rows 2 and 3), so lane 63 holds the wave's; lanes a
// shift leaves without a source keep their own value.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp_min_step(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kCtrl, kRowMask, 0xF, false);
  return o < v ? o : v;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = dpp_min_step<0x111, 0xF>(v);   // row_shr:1
  v = dpp_min_step<0x112, 0xF>(v);   // row_shr:2
  v = dpp_min_step<0x114, 0xF>(v);   // row_shr:4
  v = dpp_min_step<0x118, 0xF>(v);   // row_shr:8
  v = dpp_min_step<0x142, 0xA>(v);   // row_bcast:15
  v = dpp_min_step<0x143, 0xC>(v);   // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Sorts the wave's 64 keys descending (bitonic network across lanes).
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t a) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint64_t y = shfl_xor64(a, j);
      const bool lower = (lane & j) == 0;
      const bool desc = (lane & k) == 0;
      const uint64_t mx = a > y ? a : y;
      const uint64_t mn = a > y ? y : a;
      a = (lower == desc) ? mx : mn;
    }
  }
  return a;
}

typedef __attribute__((address_space(3))) char* lds_cptr;

// Scores of a lane's MFMA fragment whose facts lie past the store: element
// e is fact f0 + 8 * (e / 4) + e % 4, and `room` = n_facts - f0.  Only the
// tile holding the store's last fact calls it, so the other tiles' epilogue
// is a 16-way maximum and a compare.
__device__ __forceinline__ void mask_padding(float (&v)[16], int32_t room) {
#pragma unroll
  for (int e = 0; e < 16; ++e)
    if (8 * (e / 4) + (e % 4) >= room) v[e] = -INFINITY;
}

struct ScanSmem {
  u32x4 e[kStages][kEPieces];
  u32x4 q[kStages][kQPieces];
  uint32_t count[kQB];   // candidates this workgroup found per query
};

// LDS slot of 16-byte piece p (of 8) of staged row r.  The XOR spreads the
// 16 rows that one 16-lane group of an MFMA fragment read touches over all
// 64 banks: rows 2j and 2j+1 fall in the two halves of a 256-byte bank
// line, and the 8 pairs get 8 different piece positions.
__device__ __forceinline__ int piece_slot(int r, int p) { return r * 8 + (p ^ ((r >> 1) & 7)); }

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

// Workgroup barrier without a memory fence.  The ring's transfers are
// tracked by the explicit vmcnt waits, and the "memory" clobber keeps the
// compiler from moving LDS accesses across it; a fenced barrier would also
// wait for the epilogue's global stores, draining the stream.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_barrier" ::: "memory"); }

// The four k-steps of one 64-dim chunk: MFMA scores of the wave's 64 facts
// against the 128 queries.  k-step s uses logical pieces 2s + grp of every
// row of both operands (the dot product is order-free in k).  The first
// chunk of a tile starts from zero accumulators.
template <bool kFirst, int QT>
__device__ __forceinline__ void mma_chunk(const u32x4* es, const u32x4* qs, int wave, int row,
                                          int grp, float16v (&acc)[2][QT]) {
  half8 av[2][2], bv[2][QT];
  auto load = [&](int s, int buf) {
    const int p = 2 * s + grp;
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
      av[buf][ft] = __builtin_bit_cast(half8, es[piece_slot(wave * kFTW + ft * 32 + row, p)]);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
      bv[buf][qt] = __builtin_bit_cast(half8, qs[piece_slot(qt * 32 + row, p)]);
  };
  const float16v zero = {};
  load(0, 0);
#pragma unroll
  for (int s = 0; s < kKC / 16; ++s) {
    if (s + 1 < kKC / 16) load(s + 1, (s + 1) & 1);
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
        acc[ft][qt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
            av[s & 1][ft], bv[s & 1][qt], (kFirst && s == 0) ? zero : acc[ft][qt], 0, 0, 0);
  }
}

template <bool kSample, int QT, bool kDense = false>
__global__ __launch_bounds__(kThreads) void topk_scan(TopkLaunch a) {
  static_assert(!(kSample && kDense), "the one-pass scan is a stream scan");
  constexpr int kQDma = q_dma<QT>();
  __shared__ ScanSmem sm;
  if (kSample || kDense) side_zero(a);
  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int row = lane % 32;
  const int grp = lane / 32;
  const int D = a.emb_dim;
  const int n_chunks = D / kKC;
  const int G = (int)gridDim.x;
  const int w = (int)blockIdx.x;
  // the stream starts after the sample's tiles when the sample kept their codes
  const int64_t t0 = kSample ? 0 : a.stream_t0;
  const int64_t n_tiles = kSample ? a.sample_tiles : a.n_tiles - t0;
  const int my_tiles = (int)((n_tiles - w + G - 1) / G);
  const int total = my_tiles * n_chunks;
  const int64_t edge_tile = (a.n_facts - 1) / kFT;   // the tile that may hold padding rows

  float tau[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int q = qt * 32 + row;
    tau[qt] = (!kSample && !kDense && q < a.n_q) ? a.tau[q] : 0.f;
  }
  if (tid < kQB) sm.count[tid] = 0;   // first read after the loop's barriers
  const uint64_t region0 = (uint64_t)(t0 + region_tile(w, n_tiles, G)) * kFT;

  const uint32_t e_lds = (uint32_t)(size_t)(lds_cptr)(void*)&sm.e[0][0];
  const uint32_t q_lds = (uint32_t)(size_t)(lds_cptr)(void*)&sm.q[0][0];
  // Wave w's transfers fill exactly the fact rows [64w, 64w + 64) that its
  // own MFMAs read, so it may refill its part of a ring buffer as soon as it
  // has finished with it; the query rows are read by every wave and wait for
  // the barrier.
  // Fact cursor: tile et, chunk ec, ring buffer eb.
  int64_t et = t0 + w;
  int ec = 0, eb = 0;
  auto issue_e = [&]() {
    // the tile's 256 x 64 block of the blocked layout: 32 KB contiguous
    const uint16_t* blk = a.emb + (et * n_chunks + ec) * (int64_t)(kFT * kKC);
#pragma unroll
    for (int i = 0; i < kEDma; ++i) {
      const int s0 = (wave * kEDma + i) * 64;
      const int slot = s0 + lane;
      const int r = slot >> 3, p = (slot & 7) ^ ((r >> 1) & 7);
      dma16(blk + r * kKC + p * 8,
            __builtin_amdgcn_readfirstlane(e_lds + (uint32_t)((eb * kEPieces + s0) * 16)));
    }
    if (++ec == n_chunks) {
      ec = 0;
      et += G;
    }
    if (++eb == kStages) eb = 0;
  };
  // Query cursor: chunk qc, ring buffer qb.
  int qc = 0, qb = 0;
  auto issue_q = [&]() {
#pragma unroll
    for (int i = 0; i < kQDma; ++i) {
      const int s0 = (wave * kQDma + i) * 64;
      const int slot = s0 + lane;
      const int r = slot >> 3, p = (slot & 7) ^ ((r >> 1) & 7);
      // rows past n_q re-load row 0; their scores are never used
      const uint16_t* src = a.q + (int64_t)(r < a.n_q ? r : 0) * D + qc * kKC + p * 8;
      dma16(src, __builtin_amdgcn_readfirstlane(q_lds + (uint32_t)((qb * kQPieces + s0) * 16)));
    }
    if (++qc == n_chunks) qc = 0;
    if (++qb == kStages) qb = 0;
  };

  float16v acc[2][QT];
  auto emit = [&](int64_t t) {
#pragma unroll
    for (int ft = 0; ft < 2; ++ft) {
      // element e of a lane's fragment is fact f0 + 8 * (e / 4) + e % 4
      const int64_t f0 = t * kFT + wave * kFTW + ft * 32 + 4 * grp;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const int q = qt * 32 + row;
        float v[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = acc[ft][qt][e];
        if (t == edge_tile) mask_padding(v, (int32_t)(a.n_facts - f0));   // uniform branch
        float mx = v[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mx = fmaxf(mx, v[e]);
        if (kSample || kDense) {
          if (q < a.n_q) {
            const int64_t gi = ((t * kWaves + wave) * 2 + ft) * 2 + grp;
            a.gmax[(int64_t)q * a.n_groups + gi] = (mx == -INFINITY) ? 0u : ord_of(mx);
            if (kDense || a.stream_t0 > 0) {
              // the group's 16 codes, in fragment order (0: padding)
              u32x4* dst = reinterpret_cast<u32x4*>(a.codes + (int64_t)q * a.code_stride + gi * 16);
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                u32x4 c;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  c[i] = v[4 * j + i] == -INFINITY ? 0u : ord_of(v[4 * j + i]);
                dst[j] = c;
              }
            }
          }
        } else if (q < a.n_q && mx >= tau[qt]) {
          uint32_t m = 0;
#pragma unroll
          for (int e = 0; e < 16; ++e) m |= (v[e] >= tau[qt]) ? (1u << e) : 0u;
          uint32_t pos = atomicAdd(&sm.count[q], (uint32_t)__builtin_popcount(m));
          uint64_t* dst = a.cand + (int64_t)q * a.cand_stride + region0;
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (m & (1u << e))
              dst[pos++] = key_of(ord_of(v[e]), (uint32_t)(f0 + 8 * (e / 4) + (e % 4)));
        }
      }
    }
  };

  static_assert(kStages == 3, "the wait counts below assume three ring buffers");
  for (int g = 0; g < kStages - 1 && g < total; ++g) {
    issue_e();
    issue_q();
  }
  // Compute cursor: tile ct, chunk cc, ring buffer cb.
  int64_t ct = t0 + w;
  int cc = 0, cb = 0;
  for (int g = 0; g < total; ++g) {
    // Chunk g+2's fact rows go into the buffer this wave finished with in
    // chunk g-1.  Issued after chunk g's query rows: the fact rows of g+1
    // and g+2 and the query rows of g+1 (20 transfers), so chunk g has
    // landed once at most that many are in flight (loads complete in order).
    if (g + 2 < total) {
      issue_e();
      wait_vm<2 * kEDma + kQDma>();
    } else if (g + 1 < total) {
      wait_vm<kEDma + kQDma>();
    } else {
      wait_vm<0>();
    }
    ring_barrier();   // every wave's transfers for chunk g landed; chunk g-1's query rows are free
    if (g + 2 < total) issue_q();
    if (cc == 0)
      mma_chunk<true, QT>(sm.e[cb], sm.q[cb], wave, row, grp, acc);
    else
      mma_chunk<false, QT>(sm.e[cb], sm.q[cb], wave, row, grp, acc);
    if (cc == n_chunks - 1) emit(ct);
    if (++cc == n_chunks) {
      cc = 0;
      ct += G;
    }
    if (++cb == kStages) cb = 0;
  }
  wait_vm<0>();
  if (!kSample && !kDense) {
    __syncthreads();
    if (tid < a.n_q) a.count[(int64_t)tid * kTopkMaxScanWG + w] = sm.count[tid];
  }
}

// Scan variant for full query batches (65..128 queries) at width 1024.
// The query rows are the same for every tile, so instead of re-staging them
// through LDS for every chunk, each wave keeps its own 32 query rows -- all
// 1024 dims, 256 registers per lane -- for the whole launch, and the LDS
// ring holds fact rows only: stages of an FT-fact x 64-dim block (FT = 32,
// 64 or 128 facts: part of a stored 256 x 64 block), all but one of them in
// flight while one is scored.  Every wave scores all FT facts of a stage
// against its 32 queries (FT / 32 v_mfma_f32_32x32x16_f16 row tiles per
// k-step), so all waves read every stage and one barrier per chunk both
// publishes a stage and frees the one scored before it.  With 16 chunks per
// tile and 8 or 16 stages the ring slot of a chunk is fixed by its index in
// the tile, which keeps the query registers and the ring addressing static
// (a ring slot taken from a running count measured a quarter slower).
// Small tiles spread a small store (or the threshold sample) over many
// workgroups; large ones cost fewer barriers per byte.
//
// A fact's score is the same chain of MFMAs in every tile size and in
// topk_scan: k-step s of chunk c multiplies dims c*64 + (2s + grp)*8 .. +8 of
// both operands (fact as the A row, query as the B column), chunks in
// order, starting from a zero accumulator.  A sample scanned with one tile
// size and a stream scanned with another therefore score every fact bit for
// bit alike, which keeps the bound exact.
constexpr int kRChunks = 16;   // 64-dim chunks of a 1024-wide row
template <int FT>
struct Rq {
  static constexpr int kStages = FT == 128 ? 8 : 16;
  static constexpr int kPieces = FT * kKC / 8;        // 16-byte pieces of a stage
  static constexpr int kDma = kPieces / 64 / kWaves;  // transfers per wave per stage
  static constexpr int kRows = FT / 32;               // MFMA row tiles per stage
  static_assert(kRChunks % kStages == 0, "ring slot must be static per chunk");
  static_assert(kDma >= 1 && (kStages - 2) * kDma < 64, "vmcnt range");
  static_assert(kFT % FT == 0, "a tile is a part of a stored 256-fact block");
};
static_assert(kQB == kWaves * 32, "one 32-query tile per wave");

// Candidates found during the stream are staged in LDS and written out
// after the loop: a global store counts in vmcnt like the ring's transfers,
// and, issued behind the chunks in flight, it would make every ring wait of
// the next steps wait for that much more.  Each wave owns its queries, so
// it also owns their candidates: a query's running count lives in the
// registers of its two lanes, and each wave fills its own part of the
// staging area, slots taken by a ballot prefix sum (no atomics).  An
// entry's destination is (query << 25) | position in the query's region;
// a wave whose part is full stores further candidates directly.
constexpr int kCandWave = 512;   // staged candidates per wave
constexpr int kPosBits = 25;

template <int FT>
struct ScanSmemRq {
  u32x4 e[Rq<FT>::kStages][Rq<FT>::kPieces];
  uint64_t ckey[kWaves][kCandWave];
  uint32_t cdst[kWaves][kCandWave];
  uint32_t qcount[32];   // shared-query mode: candidates per query so far
  float qtau[kWaves];    // shared-query mode with fuse_tau: each query's bound
};

// Exclusive prefix sum over the wave of n (0 <= n <= 64) and the wave's
// total, bit by bit from ballots.
__device__ __forceinline__ uint32_t wave_prefix(uint32_t n, uint32_t& total) {
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int b = 0; b < 7; ++b) {
    const uint64_t bal = __ballot((n >> b) & 1u);
    const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    pre += below << b;
    tot += (uint32_t)__builtin_popcountll(bal) << b;
  }
  total = tot;
  return pre;
}

// Waits until at most D * min(n, N) of this wave's transfers are in flight
// (n is a constant once the chunk loop is unrolled).
template <int D, int N>
__device__ __forceinline__ void wait_stages(int n) {
  if constexpr (N <= 0) {
    wait_vm<0>();
  } else {
    if (n >= N) {
      wait_vm<D * N>();
      return;
    }
    wait_stages<D, N - 1>(n);
  }
}

// kShared: batches of at most 32 queries.  Every wave holds the same 32
// query rows (rows past n_q are zero and load nothing) and scores its own
// 32-fact row tile of each 128-fact stage, so one query's candidates come
// from all four waves and take their positions from an LDS counter.
template <bool kSample, int FT, bool kShared, bool kDense = false>
__global__ __launch_bounds__(kThreads) void topk_scan_rq(TopkLaunch a) {
  using R = Rq<FT>;
  static_assert(!kShared || R::kRows == kWaves, "shared queries: one row tile per wave");
  static_assert(!(kSample && kDense), "the one-pass scan is a stream scan");
  constexpr int kRowsW = kShared ? 1 : R::kRows;   // row tiles a wave scores per stage
  __shared__ ScanSmemRq<FT> sm;
  if (kSample || kDense) side_zero(a);
  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int row = lane % 32;
  const int grp = lane / 32;
  const int G = (int)gridDim.x;
  const int w = (int)blockIdx.x;
  // the stream starts after the sample's tiles when the sample kept their codes
  const int64_t t0 = kSample ? 0 : a.stream_t0;
  const int64_t n_tiles = kSample ? a.sample_tiles : a.n_tiles - t0;
  const int my_tiles = (int)((n_tiles - w + G - 1) / G);
  const int64_t edge_tile = (a.n_facts - 1) / FT;
  const int q = (kShared ? 0 : wave * 32) + row;   // this lane's query (column of every score tile)
  const bool q_ok = q < a.n_q;
  // the bound: from the threshold kernel, or (fuse_tau: at most four
  // queries, shared query tile) found below by wave q from the sample
  const bool fuse = kShared && !kSample && !kDense && a.fuse_tau;
  float tau = (!kSample && !kDense && !fuse && q_ok) ? a.tau[q] : 0.f;
  const uint64_t region0 = (uint64_t)(t0 + region_tile(w, n_tiles, G)) * FT;
  const bool stage_ok = (int64_t)my_tiles * FT <= ((int64_t)1 << kPosBits);
  uint32_t q_count = 0;    // candidates of this lane's query so far (both its lanes)
  uint32_t staged = 0;     // this wave's staging slots used (wave-uniform)

  if (kShared) {
    if (tid < 32) sm.qcount[tid] = 0;
    __syncthreads();
  }
  // fuse: wave w's query's sample group maxima, loaded ahead of the ring so
  // that waiting for them does not wait for the ring's transfers
  uint32_t gv[kWaveKthMax / 64];
  if (fuse && wave < a.n_q) wave_load_codes(a.gmax + (int64_t)wave * a.n_groups, a.n_groups, gv);
  half8 qv[kRChunks * 4];   // this lane's query row, loaded after the ring prologue

  const uint32_t e_lds = (uint32_t)(size_t)(lds_cptr)(void*)&sm.e[0][0];
  // Issue cursor: tile et (in FT-fact tiles), chunk ec.  Tile et is part
  // et % P of stored 256-fact tile et / P, whose chunk ec is one 32 KB span.
  constexpr int P = kFT / FT;
  int64_t et = t0 + w;
  int ec = 0;
  auto issue = [&](int slot_stage) {
    const uint16_t* blk =
        a.emb + (((et / P) * kRChunks + ec) * kFT + (et % P) * FT) * (int64_t)kKC;
#pragma unroll
    for (int i = 0; i < R::kDma; ++i) {
      const int s0 = (wave * R::kDma + i) * 64;
      const int slot = s0 + lane;
      const int r = slot >> 3, p = (slot & 7) ^ ((r >> 1) & 7);
      dma16(blk + r * kKC + p * 8,
            __builtin_amdgcn_readfirstlane(e_lds + (uint32_t)((slot_stage * R::kPieces + s0) * 16)));
    }
    if (++ec == kRChunks) {
      ec = 0;
      et += G;
    }
  };

  float16v acc[kRowsW];
  // The tile's epilogue, one 32-fact row tile at a time (16 scores per lane
  // live at once).  Element e of a lane's fragment of row tile ft is fact
  // f0 + 8 * (e / 4) + e % 4, f0 = t * FT + ft * 32 + 4 * grp.
  auto emit = [&](int64_t t) {
#pragma unroll
    for (int fw = 0; fw < kRowsW; ++fw) {
      const int ft = kShared ? wave : fw;   // row tile of the stage
      const int64_t f0 = t * FT + ft * 32 + 4 * grp;
      float v[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] = acc[fw][e];
      if (t == edge_tile) mask_padding(v, (int32_t)(a.n_facts - f0));   // uniform branch
      float mx = v[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mx = fmaxf(mx, v[e]);
      if (kSample || kDense) {
        if (q_ok) {
          const int64_t gi = (t * R::kRows + ft) * 2 + grp;
          a.gmax[(int64_t)q * a.n_groups + gi] = (mx == -INFINITY) ? 0u : ord_of(mx);
          if (kDense || a.stream_t0 > 0) {
            // the group's 16 codes, in fragment order (0: padding)
            u32x4* dst = reinterpret_cast<u32x4*>(a.codes + (int64_t)q * a.code_stride + gi * 16);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              u32x4 c;
#pragma unroll
              for (int i = 0; i < 4; ++i)
                c[i] = v[4 * j + i] == -INFINITY ? 0u : ord_of(v[4 * j + i]);
              dst[j] = c;
            }
          }
        }
        continue;
      }
      uint32_t m = 0;
      if (q_ok && mx >= tau) {
#pragma unroll
        for (int e = 0; e < 16; ++e) m |= (v[e] >= tau) ? (1u << e) : 0u;
      }
      if (!__any(m != 0)) continue;
      // positions in the query's region: the grp 0 lane's candidates first
      const uint32_t n = (uint32_t)__builtin_popcount(m);
      const uint32_t n_pair = __shfl_xor(n, 32);
      uint32_t base = 0;
      if (grp == 0 && n + n_pair != 0) base = atomicAdd(&sm.qcount[row], n + n_pair);
      uint32_t pos = (uint32_t)__shfl((int)base, row) + (grp ? n_pair : 0u);
      uint32_t wave_n;
      uint32_t slot = staged + wave_prefix(n, wave_n);
      staged += wave_n;
      uint64_t* direct = a.cand + (int64_t)q * a.cand_stride + region0;
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (m & (1u << e)) {
          const uint64_t key = key_of(ord_of(v[e]), (uint32_t)f0 + 8 * (e / 4) + (e % 4));
          if (stage_ok && slot < (uint32_t)kCandWave) {
            sm.ckey[wave][slot] = key;
            sm.cdst[wave][slot] = ((uint32_t)q << kPosBits) | pos;
          } else {
            direct[pos] = key;
          }
          ++slot;
          ++pos;
        }
    }
  };

  // Batch stream epilogue.  Candidates are rare (a few per 32 x 32 row
  // tile), so the wave takes one ballot per fragment element: an element no
  // lane keeps costs a compare, a kept one a few instructions.  `capture`
  // keeps a tile's scores (padding masked) and notes which row tiles hold
  // any candidate; `drain_all` appends their candidates.  A query's two
  // lanes see each other's bit in the ballot, which orders their candidates
  // (the grp 0 lane's first).
  float dv[kRowsW][16];   // scores of the captured tile
  int64_t d_t = 0;        // the captured tile
  uint32_t d_any = 0;     // bit fw: row tile fw of the captured tile has candidates
  auto capture = [&](int64_t t) {
    d_t = t;
    d_any = 0;
#pragma unroll
    for (int fw = 0; fw < kRowsW; ++fw) {
#pragma unroll
      for (int e = 0; e < 16; ++e) dv[fw][e] = acc[fw][e];
      if (t == edge_tile) mask_padding(dv[fw], (int32_t)(a.n_facts - (t * FT + fw * 32 + 4 * grp)));
      float mx = dv[fw][0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mx = fmaxf(mx, dv[fw][e]);
      if (__any(q_ok && mx >= tau)) d_any |= 1u << fw;
    }
  };
  // Every element's ballot first (no branches), then a scalar loop over
  // the elements some lane keeps, reading the score at a uniform index.
  auto drain_all = [&]() {
#pragma unroll
    for (int fw = 0; fw < kRowsW; ++fw) {
      if (!(d_any & (1u << fw))) continue;   // uniform
      uint32_t act = 0;
#pragma unroll
      for (int e = 0; e < 16; ++e) act |= __ballot(q_ok && dv[fw][e] >= tau) != 0 ? 1u << e : 0u;
      while (act != 0) {
        const int e = __builtin_ctz(act);
        act &= act - 1;
        const float x = dv[fw][e];
        const bool hit = q_ok && x >= tau;
        const uint64_t bal = __ballot(hit);
        const uint32_t b_pair = (uint32_t)(bal >> (lane ^ 32)) & 1u;
        const uint32_t pos = q_count + (grp ? b_pair : 0u);
        q_count += (uint32_t)hit + b_pair;
        if (hit) {
          const uint32_t slot = staged + __builtin_amdgcn_mbcnt_hi(
                                             (uint32_t)(bal >> 32),
                                             __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
          const uint32_t f = (uint32_t)(d_t * FT) + fw * 32 + 4 * grp + 8 * (e >> 2) + (e & 3);
          const uint64_t key = key_of(ord_of(x), f);
          if (stage_ok && slot < (uint32_t)kCandWave) {
            sm.ckey[wave][slot] = key;
            sm.cdst[wave][slot] = ((uint32_t)q << kPosBits) | pos;
          } else {
            a.cand[(int64_t)q * a.cand_stride + region0 + pos] = key;
          }
        }
        staged += (uint32_t)__builtin_popcountll(bal);
      }
    }
  };

  // One chunk: `after` = chunks of this workgroup still to come after it
  // (a constant once the chunk loop is unrolled; kRChunks for every tile
  // but the last).  All fragments of the stage are read before its MFMAs,
  // so the chunk pays one LDS latency rather than one per MFMA.
  //
  // The fragments of chunk c + 1 are read while chunk c's MFMAs run, so a
  // chunk costs a barrier and its MFMA chain, not also an LDS latency: step
  // c waits until chunk c + 1 has landed, passes the barrier (which also
  // tells that every wave is done with chunk c - 1, whose fragments were
  // read a step earlier), refills chunk c - 1's slot, reads chunk c + 1 and
  // scores chunk c from the fragments read before.
  half8 av[kKC / 16][kRowsW];   // fragments of the chunk being scored
  auto read_frags = [&](int c, half8 (&dst)[kKC / 16][kRowsW]) {
    const u32x4* es = sm.e[c % R::kStages];
#pragma unroll
    for (int s = 0; s < kKC / 16; ++s)
#pragma unroll
      for (int fw = 0; fw < kRowsW; ++fw)
        dst[s][fw] = __builtin_bit_cast(
            half8, es[piece_slot((kShared ? wave : fw) * 32 + row, 2 * s + grp)]);
  };
  auto step = [&](int c, int after) {
    half8 nx[kKC / 16][kRowsW];
    if (after >= 1) {
      wait_stages<R::kDma, R::kStages - 3>(after - 1);
      ring_barrier();   // chunk c + 1 landed for every wave; chunk c - 1's slot is free
      if (after >= R::kStages - 1) issue((c + R::kStages - 1) % R::kStages);
      read_frags((c + 1) % kRChunks, nx);
    }
    __builtin_amdgcn_sched_barrier(0);
    const float16v zero = {};
#pragma unroll
    for (int s = 0; s < kKC / 16; ++s)
#pragma unroll
      for (int fw = 0; fw < kRowsW; ++fw)
        acc[fw] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
            av[s][fw], qv[c * 4 + s], (c == 0 && s == 0) ? zero : acc[fw], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (after >= 1) {
#pragma unroll
      for (int s = 0; s < kKC / 16; ++s)
#pragma unroll
        for (int fw = 0; fw < kRowsW; ++fw) av[s][fw] = nx[s][fw];
    }
  };
  // total >= 16 >= kStages: the prologue always fills the ring.  It is
  // issued before the query rows are loaded, so the first stages stream in
  // while the queries arrive.
#pragma unroll
  for (int g = 0; g < R::kStages - 1; ++g) issue(g);
  // k-step s of chunk c multiplies dims c*64 + (2s + grp)*8 .. +8 of both
  // operands (the dot product is order-free in k).  Rows past n_q are zero,
  // load nothing, and their scores are never used.
  if (q_ok) {
    const uint16_t* src = a.q + (int64_t)q * (kRChunks * kKC) + grp * 8;
#pragma unroll
    for (int j = 0; j < kRChunks * 4; ++j)
      qv[j] = *reinterpret_cast<const half8*>(src + j * 16);
  } else {
#pragma unroll
    for (int j = 0; j < kRChunks * 4; ++j) qv[j] = half8{};
  }
  if (kShared && !kSample) {
    if (fuse) {
      // while the ring's first stages land: wave w finds query w's bound
      if (wave < a.n_q) {
        const float t = tau_of_code(wave_kth_code(gv, a.n_groups, a.k));
        if (lane == 0) sm.qtau[wave] = t;
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the bound is in LDS before the barrier
    }
  }
  // chunk 0's fragments
  wait_vm<R::kDma * (R::kStages - 2)>();
  ring_barrier();
  if (fuse && q_ok) tau = sm.qtau[row];
  read_frags(0, av);
  int64_t ct = t0 + w;
  if constexpr (!kSample && !kShared && !kDense) {
    for (int i = 0; i + 1 < my_tiles; ++i) {
#pragma unroll
      for (int c = 0; c < kRChunks; ++c) step(c, kRChunks);
      capture(ct);
      drain_all();
      ct += G;
    }
#pragma unroll
    for (int c = 0; c < kRChunks; ++c) step(c, kRChunks - 1 - c);
    capture(ct);
    drain_all();
  } else {
    for (int i = 0; i + 1 < my_tiles; ++i) {
#pragma unroll
      for (int c = 0; c < kRChunks; ++c) step(c, kRChunks);
      emit(ct);
      ct += G;
    }
#pragma unroll
    for (int c = 0; c < kRChunks; ++c) step(c, kRChunks - 1 - c);
    emit(ct);
  }
  wait_vm<0>();
  if (!kSample && !kDense) {
    if (kShared) {
      __syncthreads();   // every wave's positions are taken
      if (tid < 32 && tid < a.n_q) a.count[(int64_t)tid * kTopkMaxScanWG + w] = sm.qcount[tid];
    } else if (grp == 0 && q_ok) {
      a.count[(int64_t)q * kTopkMaxScanWG + w] = q_count;
    }
    // the wave's own staged entries (written by this wave only)
    const uint32_t used = !stage_ok ? 0u : staged < (uint32_t)kCandWave ? staged : (uint32_t)kCandWave;
    for (uint32_t i = lane; i < used; i += 64) {
      const uint32_t d = sm.cdst[wave][i];
      a.cand[(int64_t)(d >> kPosBits) * a.cand_stride + region0 + (d & ((1u << kPosBits) - 1))] =
          sm.ckey[wave][i];
    }
  }
}

constexpr int kSelThreads = 256;
constexpr int kStage32 = 8192;   // group maxima staged in LDS by the threshold kernel
constexpr int kStage64 = 4096;   // candidate keys staged in LDS by the final kernel
constexpr int kDenseGroups = 32 * kSelThreads;   // group maxima the one-pass final holds
constexpr int kBestGroups = 2;   // groups per thread the one-pass final fetches ahead

struct SelShared {
  uint32_t hist[256];
  uint32_t wsum[kSelThreads / 64];
  uint32_t pick[3];
};

// The k-th largest of n values (32- or 64-bit; duplicates allowed), by
// most-significant-digit radix select over 8-bit digits; `each(fn)` applies
// fn to every value this thread owns.  Returns t with the digits found so
// far and the rest zero: at most k - 1 values exceed the k-th largest, and
// the values >= t are exactly the k largest once the bucket holding the
// k-th largest holds no other value (then the select stops early); for
// distinct values that is reached at the last digit at the latest.
// Returns 0 when n < k.  All threads of the workgroup call it.
template <typename V, typename Each>
__device__ V kth_largest(Each each, int64_t n, int k, SelShared& sh) {
  if (n < k) return 0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  V prefix = 0, mask = 0;
  uint32_t remaining = (uint32_t)k;
  for (int shift = 8 * (int)sizeof(V) - 8; shift >= 0; shift -= 8) {
    sh.hist[tid] = 0;
    __syncthreads();
    each([&](V v) {
      if ((v & mask) == prefix) atomicAdd(&sh.hist[(uint32_t)(v >> shift) & 255u], 1u);
    });
    __syncthreads();
    // thread t owns bin t; s = number of matching values in bins >= t
    const uint32_t h = sh.hist[tid];
    uint32_t s = h;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_down(s, off);
      if (lane + off < 64) s += o;
    }
    if (lane == 0) sh.wsum[wave] = s;
    __syncthreads();
    for (int w2 = wave + 1; w2 < kSelThreads / 64; ++w2) s += sh.wsum[w2];
    const uint32_t above = s - h;
    if (s >= remaining && above < remaining) {
      sh.pick[0] = (uint32_t)tid;
      sh.pick[1] = above;
      sh.pick[2] = h;
    }
    __syncthreads();
    const uint32_t b = sh.pick[0];
    remaining -= sh.pick[1];
    const uint32_t hb = sh.pick[2];
    prefix |= (V)b << shift;
    mask |= (V)255 << shift;
    if (hb == remaining) break;
  }
  return prefix;
}

constexpr int kSel = 2 * kSelThreads;   // keys the final kernel orders by counting
constexpr int kFewRegions = 8;          // candidate regions the final gathers spread out

// Barrier over the workgroup's LDS accesses only: global loads in flight
// (the one-pass final's prefetched codes) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// A bound reached by at least k codes of the workgroup: every thread
// offers its largest code `mine` (0: none); each wave ranks its 64 offers
// (its own lanes' LDS writes, read back in order) and keeps the least offer
// ranked below ceil(k / 4), which that many of its offers reach, so the
// least of the four waves' is reached by at least k offers -- k distinct
// codes (0 when fewer threads offer one).  `offers` holds a code per
// thread, `wmin` one per wave; one barrier.
__device__ __forceinline__ uint32_t offer_bound(uint32_t mine, int k, uint32_t* offers, uint32_t* wmin) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  offers[tid] = mine;
  const uint32_t kw = (uint32_t)(k + kSelThreads / 64 - 1) / (kSelThreads / 64);
  uint32_t above = 0;
  const u32x4* v4 = reinterpret_cast<const u32x4*>(offers + wave * 64);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const u32x4 v = v4[i];
    above += (v[0] > mine ? 1u : 0u) + (v[1] > mine ? 1u : 0u) + (v[2] > mine ? 1u : 0u) +
             (v[3] > mine ? 1u : 0u);
  }
  uint32_t t = wave_min_u32(above < kw ? mine : 0xFFFFFFFFu);
  if (lane == 0) wmin[wave] = t;
  lds_barrier();
#pragma unroll
  for (int w2 = 0; w2 < kSelThreads / 64; ++w2) t = wmin[w2] < t ? wmin[w2] : t;
  return t;
}

// Per query: tau = the k-th largest group maximum of the sample (lowered by
// a hair), or -inf when the sample has fewer than k non-empty groups.  Up
// to kDenseGroups maxima (32 per thread): the maxima that reach a bound k of
// them reach (offer_bound) hold the k-th largest, with its rank among all,
// so it is the least of them ranked below k; many equal maxima, or more
// groups, take the radix select.
// When the sample kept its facts' codes (stream_t0 > 0) the stream scan
// skips those facts, and this kernel takes their candidates instead: the
// codes that reach tau, from the groups whose maximum does (about k
// groups), written at the head of the query's candidate row, their number
// in scount.  A thread's best groups that reach the first bound (up to four)
// are fetched while the rest of the selection runs.
__global__ __launch_bounds__(kSelThreads) void topk_threshold(TopkLaunch a) {
  __shared__ __attribute__((aligned(16))) uint32_t vals[kStage32];
  __shared__ SelShared sh;
  __shared__ __attribute__((aligned(16))) uint32_t offers[kSelThreads];
  __shared__ uint32_t wmin[kSelThreads / 64];
  __shared__ __attribute__((aligned(16))) uint32_t sel[kSel];
  __shared__ uint32_t n_sel;
  __shared__ uint32_t n_sc;    // the sample's candidates taken so far
  __shared__ uint32_t n_grp;   // ... their groups listed so far
  constexpr int kKeyStage = 1024;
  __shared__ __attribute__((aligned(16))) uint64_t kstage[kKeyStage];   // their keys
  __shared__ uint32_t glist[kStage32 / 16];                             // their groups
  const int q = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t n = a.n_groups;
  const uint32_t* src = a.gmax + (int64_t)q * n;
  const bool keep = a.stream_t0 > 0;
  const u32x4* codes =
      keep ? reinterpret_cast<const u32x4*>(a.codes + (int64_t)q * a.code_stride) : nullptr;
  if (tid == 0) {
    n_sc = 0;
    n_grp = 0;
  }
  uint32_t kth = 0;
  bool done = false;
  const bool fast = n <= kDenseGroups && n >= a.k;
  constexpr int kJ = kDenseGroups / kSelThreads;
  // fast: this thread's maxima (groups tid + 256 j) and its kPre best,
  // whose codes are fetched into cp while the bound is ranked (of the k or
  // so groups that reach it, a thread rarely holds more than two; kPre = 4
  // leaves a dependent load after the bound to almost no launch).
  constexpr int kPre = 4;
  // Loops over a thread's maxima stop at jn, the count of 256-wide rows the
  // groups fill (a uniform branch): at one wave per SIMD every instruction
  // of these short kernels is on the critical path.
  const int jn = fast ? (int)((n + kSelThreads - 1) / kSelThreads) : 0;
  uint32_t v[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) v[j] = 0u;
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    if (j >= jn) break;
    const int64_t i = tid + (int64_t)kSelThreads * j;
    v[j] = i < n ? src[i] : 0u;
  }
  int bj[kPre];        // the best groups' j, best first (-1: none)
  uint32_t bm[kPre];   // ... and their maxima
#pragma unroll
  for (int r = 0; r < kPre; ++r) {
    bj[r] = -1;
    bm[r] = 0;
  }
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    if (j >= jn) break;
    // insert v[j] into the descending list (ties keep the earlier j first)
    uint32_t x = v[j];
    int xj = j;
#pragma unroll
    for (int r = 0; r < kPre; ++r) {
      const bool up = x > bm[r];
      const uint32_t tm = bm[r];
      const int tj = bj[r];
      bm[r] = up ? x : tm;
      bj[r] = up ? xj : tj;
      x = up ? tm : x;
      xj = up ? tj : xj;
    }
  }
  const uint32_t mx = bm[0];
  u32x4 cp[kPre][4];
  uint32_t pf = 0;   // bit r: cp[r] holds group bj[r]'s codes
  if (fast) {
    if (tid == 0) n_sel = 0;
    for (int i = tid; i < kSel; i += kSelThreads) sel[i] = 0;   // past the selection: zero
    const uint32_t t1 = offer_bound(mx, a.k, offers, wmin);
    // The groups that reach t1 (at most kSel of them, about k) hold those
    // that reach tau, but for a hair: their codes are fetched now, while
    // the bound is ranked.  Every lane loads (a lane with nothing to fetch
    // reads group 0, one line for all of them).
    const u32x4* cbase = keep ? codes : reinterpret_cast<const u32x4*>(a.gmax);
#pragma unroll
    for (int r = 0; r < kPre; ++r) {
      const bool want = keep && bj[r] >= 0 && bm[r] >= t1;
      pf |= want ? 1u << r : 0u;
      const int64_t g = want ? tid + (int64_t)kSelThreads * bj[r] : 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) cp[r][i] = cbase[g * 4 + i];
    }
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      if (j >= jn) break;
      cnt += (v[j] != 0u && v[j] >= t1) ? 1u : 0u;
    }
    {
      // positions by a wave prefix sum, one LDS atomic per wave
      uint32_t wave_n;
      const uint32_t pre = wave_prefix(cnt, wave_n);
      uint32_t base = 0;
      if ((tid & 63) == 0 && wave_n != 0) base = atomicAdd(&n_sel, wave_n);
      uint32_t slot = (uint32_t)__shfl((int)base, 0) + pre;
#pragma unroll
      for (int j = 0; j < kJ; ++j) {
        if (j >= jn) break;
        if (v[j] != 0u && v[j] >= t1) {
          if (slot < (uint32_t)kSel) sel[slot] = v[j];
          ++slot;
        }
      }
    }
    lds_barrier();
    const uint32_t m = n_sel;
    if (m <= (uint32_t)kSel) {
      // fewer than k nonzero maxima: the k-th largest is an empty group (0)
      uint32_t least = 0xFFFFFFFFu;
      if (m >= (uint32_t)a.k) {
        // eight 16-byte reads in flight; sel is zero past m (ranks above none)
        const u32x4* s4 = reinterpret_cast<const u32x4*>(sel);
        const uint32_t n4 = ((m + 3) / 4 + 7) & ~7u;   // <= kSel / 4
        for (uint32_t i = tid; i < m; i += kSelThreads) {
          const uint32_t mine = sel[i];
          uint32_t above = 0;
          for (uint32_t j0 = 0; j0 < n4; j0 += 8) {
            u32x4 w4[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) w4[u] = s4[j0 + u];
#pragma unroll
            for (int u = 0; u < 8; ++u)
              above += (w4[u][0] > mine ? 1u : 0u) + (w4[u][1] > mine ? 1u : 0u) +
                       (w4[u][2] > mine ? 1u : 0u) + (w4[u][3] > mine ? 1u : 0u);
          }
          if (above < (uint32_t)a.k && mine < least) least = mine;
        }
      }
      least = wave_min_u32(least);
      if ((tid & 63) == 0) wmin[tid >> 6] = least;   // each wave read wmin before the last barrier
      lds_barrier();
#pragma unroll
      for (int w2 = 0; w2 < kSelThreads / 64; ++w2) least = wmin[w2] < least ? wmin[w2] : least;
      kth = m >= (uint32_t)a.k ? least : 0u;
      done = true;
    }
  }
  if (!done) {
    if (n <= kStage32) {
      for (int64_t i = tid; i < n; i += kSelThreads) vals[i] = src[i];
      __syncthreads();
      kth = kth_largest<uint32_t>([&](auto fn) {
        for (int64_t i = tid; i < n; i += kSelThreads) fn(vals[i]);
      }, n, a.k, sh);
    } else {
      kth = kth_largest<uint32_t>([&](auto fn) {
        for (int64_t i = tid; i < n; i += kSelThreads) fn(src[i]);
      }, n, a.k, sh);
    }
  }
  const float tau = tau_of_code(kth);
  if (tid == 0) a.tau[q] = tau;
  if (!keep) return;
  // The sample's candidates: group g's code e is fact
  // 32 (g / 2) + 4 (g % 2) + 8 (e / 4) + e % 4, in the order the scan stored
  // them.  A thread's groups that reach tau are its np best (the test is
  // monotone in the maximum), so the first min(np, kPre) are in registers.
  // Their codes are listed in LDS (the maxima's staging area, free once tau
  // is known), then every thread tests (group, code) pairs of the list and
  // the hits are placed by ballot prefix sums, one LDS atomic per wave;
  // keys are staged in LDS and written out together.  More groups than the
  // list holds (many equal maxima): each thread takes its own groups.
  uint64_t* head = a.cand + (int64_t)q * a.cand_stride;
  const int lane = tid & 63;
  auto pass = [&](uint32_t gm) { return gm != 0u && float_of(gm) >= tau; };
  auto put = [&](uint32_t slot, uint64_t key) {
    if (slot < (uint32_t)kKeyStage) kstage[slot] = key;
    else head[slot] = key;
  };
  auto fact = [](int64_t g, int e) {
    return (uint32_t)(32 * (g >> 1) + 4 * (g & 1) + 8 * (e >> 2) + (e & 3));
  };
  u32x4* lcodes = reinterpret_cast<u32x4*>(vals);   // group i's codes: lcodes[4 i .. 4 i + 4)
  constexpr uint32_t kListGroups = kStage32 / 16;
  uint32_t pm = 0;   // fast: this thread's groups that reach tau (bit j)
  if (fast) {
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      if (j >= jn) break;
      pm |= pass(v[j]) ? 1u << j : 0u;
    }
    const uint32_t np = (uint32_t)__builtin_popcount(pm);
    uint32_t wave_n;
    const uint32_t pre = wave_prefix(np, wave_n);
    uint32_t base = 0;
    if (lane == 0 && wave_n != 0) base = atomicAdd(&n_grp, wave_n);
    const uint32_t slot = (uint32_t)__shfl((int)base, 0) + pre;
#pragma unroll
    for (int r = 0; r < kPre; ++r) {
      if ((uint32_t)r < np && slot + r < kListGroups) {
        const int64_t g = tid + (int64_t)kSelThreads * bj[r];
        if (pf & (1u << r)) {
#pragma unroll
          for (int i = 0; i < 4; ++i) lcodes[(slot + r) * 4 + i] = cp[r][i];
        } else {   // reaches tau, not t1 (within the hair below it)
#pragma unroll
          for (int i = 0; i < 4; ++i) lcodes[(slot + r) * 4 + i] = codes[g * 4 + i];
        }
        glist[slot + r] = (uint32_t)g;
      }
    }
    if (np > (uint32_t)kPre) {
      // groups past the fetched ones, in j order after them
      uint32_t rest = pm;
#pragma unroll
      for (int r = 0; r < kPre; ++r) rest &= bj[r] >= 0 ? ~(1u << bj[r]) : ~0u;
      uint32_t at = slot + kPre;
      while (rest != 0) {
        const int j = __builtin_ctz(rest);
        rest &= rest - 1;
        const int64_t g = tid + (int64_t)kSelThreads * j;
        if (at < kListGroups) {
#pragma unroll
          for (int i = 0; i < 4; ++i) lcodes[at * 4 + i] = codes[g * 4 + i];
          glist[at] = (uint32_t)g;
        }
        ++at;
      }
    }
  }
  lds_barrier();   // the list and its length
  const uint32_t n_list = n_grp;
  if (fast && n_list <= kListGroups) {
    const uint32_t* lc = vals;
    const uint32_t pairs = 16 * n_list;
    // four pairs per thread per round (uniform trip count), one prefix sum
    // and one LDS atomic per wave per round
    for (uint32_t p0 = 0; p0 < pairs; p0 += 4 * kSelThreads) {
      uint32_t o[4], hits = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t p = p0 + tid + u * kSelThreads;
        o[u] = p < pairs ? lc[p] : 0u;
        hits |= (o[u] != 0u && float_of(o[u]) >= tau) ? 1u << u : 0u;
      }
      uint32_t wave_n;
      const uint32_t pre = wave_prefix((uint32_t)__builtin_popcount(hits), wave_n);
      uint32_t base = 0;
      if (lane == 0 && wave_n != 0) base = atomicAdd(&n_sc, wave_n);
      uint32_t slot = (uint32_t)__shfl((int)base, 0) + pre;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (hits & (1u << u)) {
          const uint32_t p = p0 + tid + u * kSelThreads;
          put(slot++, key_of(o[u], fact(glist[p >> 4], (int)(p & 15))));
        }
    }
  } else {
    // each thread its own groups that reach tau
    auto take = [&](int64_t g, const u32x4 (&c)[4]) {
      uint32_t m = 0;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t o = c[e / 4][e % 4];
        m |= (o != 0u && float_of(o) >= tau) ? 1u << e : 0u;
      }
      if (m == 0) return;
      uint32_t slot = atomicAdd(&n_sc, (uint32_t)__builtin_popcount(m));
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (m & (1u << e)) put(slot++, key_of(c[e / 4][e % 4], fact(g, e)));
    };
    for (int64_t g = tid; g < n; g += kSelThreads) {
      if (!pass(src[g])) continue;
      u32x4 c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] = codes[g * 4 + i];
      take(g, c);
    }
  }
  __syncthreads();
  const uint32_t total = n_sc;
  const uint32_t in_lds = total < (uint32_t)kKeyStage ? total : (uint32_t)kKeyStage;
  for (uint32_t i = tid; i < in_lds; i += kSelThreads) head[i] = kstage[i];
  if (tid == 0) a.scount[q] = total;
}

// Per query: the k best candidates, in order.
struct FinalShared {
  alignas(16) uint64_t keys[kStage64];   // candidate keys
  alignas(16) uint64_t sel[kSel + 8];    // the candidates that reach a bound (room for padding)
  SelShared sh;
  alignas(16) uint32_t offers[kSelThreads];   // read 16 bytes at a time
  uint32_t wtot[kSelThreads / 64];
  uint64_t best[kMaxK];
  uint32_t n_best;
  uint32_t n_cand;
  uint32_t n_sel;
  uint32_t roff[kFewRegions + 1];    // few regions: the first key of each in the list
  uint32_t rbase[kFewRegions + 1];   // ... and its offset in the candidate row
  int32_t gsel[kBestGroups * kSelThreads];   // one-pass mode: each thread's best groups
};

// Query q's k best of the m distinct keys set[0, m) (m <= kSel), written
// in order: every key counts the keys above it, which is its position.
// Positions past m (fewer than k keys: cannot happen for a consistent
// bound) are id -1, score -inf.  Pads set[m, m rounded up to 8) with zero
// keys, which rank above none; one barrier.
__device__ __forceinline__ void write_ranked(const TopkLaunch& a, int q, uint64_t* set, uint32_t m) {
  const int tid = threadIdx.x;
  if (tid < (int)((8 - m % 8) % 8)) set[m + tid] = 0;
  lds_barrier();
  const uint32_t n8 = (m + 7) / 8;
  for (uint32_t i = tid; i < m; i += kSelThreads) {
    const uint64_t mine = set[i];
    uint32_t rank = 0;
    for (uint32_t j = 0; j < n8; ++j) {
#pragma unroll
      for (int e = 0; e < 8; ++e) rank += set[8 * j + e] > mine ? 1u : 0u;
    }
    if (rank < (uint32_t)a.k) {
      a.ids[(int64_t)q * a.k + rank] = (int32_t)(0xFFFFFFFFu - (uint32_t)mine);
      a.scores[(int64_t)q * a.k + rank] = float_of((uint32_t)(mine >> 32));
    }
  }
  if (tid >= (int)m && tid < a.k) {
    a.ids[(int64_t)q * a.k + tid] = -1;
    a.scores[(int64_t)q * a.k + tid] = -INFINITY;
  }
}

// The k best of `total` candidate keys, as query q's ids and scores (the
// threads of the workgroup that hold them write them).  `staged`: the keys
// sit in fs.keys[0, total); otherwise each(fn) hands fn every key this
// thread owns, read from memory.  fs.best, fs.n_best and fs.n_sel are
// cleared, and a barrier has passed since.  Many equal scores fall through
// to the radix select.
template <typename Each>
__device__ void select_best(const TopkLaunch& a, int q, FinalShared& fs, uint32_t total,
                            bool staged, Each each) {
  const int tid = threadIdx.x;
  uint64_t* keys = fs.keys;
  auto write = [&](uint64_t v) {
    // key 0: fewer candidates than k (cannot happen for a consistent
    // bound); reported as id -1, score -inf
    if (tid < a.k) {
      a.ids[(int64_t)q * a.k + tid] = v ? (int32_t)(0xFFFFFFFFu - (uint32_t)v) : -1;
      a.scores[(int64_t)q * a.k + tid] = v ? float_of((uint32_t)(v >> 32)) : -INFINITY;
    }
  };
  if (staged && total <= (uint32_t)kSel) {
    write_ranked(a, q, keys, total);
    return;
  }
  if (staged) {
    // the keys whose score reaches a bound that k of them reach hold the
    // k best, with their positions among all the candidates
    uint64_t mx = 0;
    for (uint32_t i = tid; i < total; i += kSelThreads) mx = keys[i] > mx ? keys[i] : mx;
    const uint32_t t1 = offer_bound((uint32_t)(mx >> 32), a.k, fs.offers, fs.wtot);
    for (uint32_t i = tid; i < total; i += kSelThreads)
      if ((uint32_t)(keys[i] >> 32) >= t1) {
        const uint32_t slot = atomicAdd(&fs.n_sel, 1u);
        if (slot < (uint32_t)kSel) fs.sel[slot] = keys[i];
      }
    lds_barrier();
    const uint32_t m = fs.n_sel;
    if (m <= (uint32_t)kSel) {
      write_ranked(a, q, fs.sel, m);
      return;
    }
  }
  auto take = [&](uint64_t v, uint64_t thr) {
    if (v >= thr) {
      const uint32_t slot = atomicAdd(&fs.n_best, 1u);   // at most k keys pass
      if (slot < (uint32_t)kMaxK) fs.best[slot] = v;
    }
  };
  if (staged) {
    const uint64_t thr = kth_largest<uint64_t>([&](auto fn) {
      for (uint32_t i = tid; i < total; i += kSelThreads) fn(keys[i]);
    }, total, a.k, fs.sh);
    for (uint32_t i = tid; i < total; i += kSelThreads) take(keys[i], thr);
  } else {
    const uint64_t thr = kth_largest<uint64_t>(each, total, a.k, fs.sh);
    each([&](uint64_t v) { take(v, thr); });
  }
  __syncthreads();
  if (tid < 64) write(wave_sort_desc(fs.best[tid]));
}

// Query q's candidates from the stream scan's regions (and, when the
// stream skipped the sample's facts, the threshold kernel's candidates of
// those, at the head of the row), then its selection.  Staged: with at most
// kFewRegions stream regions (a small store's few scan workgroups, each
// region long) the keys are spread over all threads, so they cost one round
// trip; otherwise thread t loads region t, 16 keys in flight (a large
// store's regions hold a few keys each), and the head's keys are spread
// over the threads.  Not staged: thread t reads region t and every 256th
// key of the head from memory in each pass.
__device__ void final_regions(const TopkLaunch& a, int q, FinalShared& fs) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.scan_wgs;
  const int64_t t0 = a.stream_t0;      // the stream's first tile
  const int64_t nt = a.n_tiles - t0;   // ... and its tiles
  const uint32_t sc = t0 > 0 ? a.scount[q] : 0u;   // keys at the head of the row
  const uint32_t cnt = tid < G ? a.count[(int64_t)q * kTopkMaxScanWG + tid] : 0u;
  uint32_t incl = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) fs.wtot[wave] = incl;
  if (tid < kMaxK) fs.best[tid] = 0;
  if (tid == 0) {
    fs.n_best = 0;
    fs.n_sel = 0;
  }
  __syncthreads();
  // the list: the head's keys, then the regions' in workgroup order
  uint32_t excl = sc + incl - cnt, total = sc;
  for (int w2 = 0; w2 < kSelThreads / 64; ++w2) {
    if (w2 < wave) excl += fs.wtot[w2];
    total += fs.wtot[w2];
  }
  const uint64_t* cq = a.cand + (int64_t)q * a.cand_stride;
  const int64_t base = tid < G ? (t0 + region_tile(tid, nt, G)) * a.scan_tile : 0;
  const uint64_t* mine = cq + base;
  const bool staged = total <= (uint32_t)kStage64;
  if (staged) {
    if (G <= kFewRegions) {
      // a small store's few regions (region 0 the head, r + 1 workgroup
      // r's): key i of the list is gathered by thread i % 256, which finds
      // its region among the regions' starts (the last start at or before
      // i), eight loads in flight per thread
      if (tid < G) {
        fs.roff[tid + 1] = excl;
        fs.rbase[tid + 1] = (uint32_t)base;
      }
      if (tid == 0) {
        fs.roff[0] = 0;
        fs.rbase[0] = 0;
      }
      lds_barrier();
      for (uint32_t i0 = 0; i0 < total; i0 += 8 * kSelThreads) {
        uint64_t t[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t i = i0 + tid + j * kSelThreads;
          int lo = 0;
#pragma unroll
          for (int step = kFewRegions; step >= 1; step >>= 1)
            if (lo + step <= G && fs.roff[lo + step] <= i) lo += step;
          t[j] = i < total ? cq[fs.rbase[lo] + (i - fs.roff[lo])] : 0;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t i = i0 + tid + j * kSelThreads;
          if (i < total) fs.keys[i] = t[j];
        }
      }
    } else {
      // the head's first 256 keys, one per thread, in flight with the
      // regions': thread t loads scan workgroup t's region, 16 keys at a time
      const uint64_t hk = (uint32_t)tid < sc ? cq[tid] : 0;
      for (uint32_t i0 = 0; i0 < cnt; i0 += 16) {
        uint64_t t[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) t[j] = i0 + j < cnt ? mine[i0 + j] : 0;
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (i0 + j < cnt) fs.keys[excl + i0 + j] = t[j];
      }
      if ((uint32_t)tid < sc) fs.keys[tid] = hk;
      for (uint32_t i = tid + kSelThreads; i < sc; i += kSelThreads) fs.keys[i] = cq[i];
    }
    __syncthreads();
  }
  select_best(a, q, fs, total, staged, [&](auto fn) {
    for (uint32_t i = tid; i < sc; i += kSelThreads) fn(cq[i]);
    for (uint32_t i = 0; i < cnt; ++i) fn(mine[i]);
  });
}

// One-pass mode.  Thread t holds the maxima of groups t + 256 j (groups of
// 16 facts, j < 32).  The bound comes from the threads' best maxima (see
// below); k groups, hence k distinct facts, reach it, so the query's k best
// are codes that reach it in groups whose maximum does -- a few more than k
// groups, nearly all among the two best groups of some thread.  Those
// groups' codes are on their way while the bound is found, fetched four
// lanes to a group (each lane 16 bytes, a quarter of the group) so that
// one load instruction covers 16 whole groups.  Group g's 16 codes are facts
// 32 (g / 2) + 4 (g % 2) + 8 (e / 4) + e % 4, e = 0 .. 15, in the order the
// scan stored them.
__device__ void final_dense(const TopkLaunch& a, int q, FinalShared& fs) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t ng = a.n_groups;   // <= kDenseGroups
  const uint32_t* gm = a.gmax + (int64_t)q * ng;
  const uint32_t* codes = a.codes + (int64_t)q * a.code_stride;
  constexpr int kJ = kDenseGroups / kSelThreads;
  uint32_t gv[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    const int64_t i = tid + (int64_t)kSelThreads * j;
    gv[j] = i < ng ? gm[i] : 0u;
  }
  // this thread's best kBestGroups groups jb[], maxima mb[] descending
  // (0: none)
  uint32_t mb[kBestGroups] = {};
  int jb[kBestGroups] = {};
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    uint32_t v = gv[j];
    int jj = j;
#pragma unroll
    for (int b = 0; b < kBestGroups; ++b)
      if (v > mb[b]) {
        const uint32_t tv = mb[b];
        const int tj = jb[b];
        mb[b] = v;
        jb[b] = jj;
        v = tv;
        jj = tj;
      }
  }
  const uint32_t m1 = mb[0];
  // the codes of group tid + 256 j; returns the group's first fact
  auto load_group = [&](int j, u32x4 (&c)[4]) -> uint32_t {
    const int64_t g = tid + (int64_t)kSelThreads * j;
    const u32x4* src = reinterpret_cast<const u32x4*>(codes + g * 16);
#pragma unroll
    for (int h = 0; h < 4; ++h) c[h] = src[h];
    return (uint32_t)(32 * (g >> 1) + 4 * (g & 1));
  };
  // the wave's best groups (kBestGroups per thread; -1: none), exchanged
  // through LDS within the wave (its own writes, in order), then lane l
  // fetches quarter l % 4 of group slot 16 i + l / 4
  constexpr int kSlots = 64 * kBestGroups;   // the wave's
  constexpr int kPieces = kSlots * 4 / 64;   // per lane
#pragma unroll
  for (int b = 0; b < kBestGroups; ++b)
    fs.gsel[kBestGroups * tid + b] = mb[b] != 0u ? tid + kSelThreads * jb[b] : -1;
  u32x4 pc[kPieces];
  uint32_t pf[kPieces];
#pragma unroll
  for (int i = 0; i < kPieces; ++i) {
    const int g = fs.gsel[wave * kSlots + 16 * i + lane / 4];
    const int h = lane % 4;
    pc[i] = u32x4{0u, 0u, 0u, 0u};
    pf[i] = 0u;
    if (g >= 0) {
      pc[i] = *reinterpret_cast<const u32x4*>(codes + (int64_t)g * 16 + 4 * h);
      pf[i] = (uint32_t)(32 * (g >> 1) + 4 * (g & 1) + 8 * h);
    }
  }
  if (tid < kMaxK) fs.best[tid] = 0;
  if (tid == 0) {
    fs.n_best = 0;
    fs.n_cand = 0;
    fs.n_sel = 0;
  }
  // the bound: k groups reach it (0: every group holds candidates)
  const uint32_t t = offer_bound(m1, a.k, fs.offers, fs.wtot);
  auto reaches = [&](uint32_t c) { return c != 0u && c >= t; };
  uint32_t mask = 0;
#pragma unroll
  for (int j = 0; j < kJ; ++j) mask |= reaches(gv[j]) ? 1u << j : 0u;
  auto append = [&](const u32x4 (&c)[4], uint32_t f0) {
    uint32_t n = 0;
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) n += reaches(c[h][i]) ? 1u : 0u;
    uint32_t slot = atomicAdd(&fs.n_cand, n);   // the group's share of the key list
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (reaches(c[h][i])) {
          if (slot < (uint32_t)kStage64) fs.keys[slot] = key_of(c[h][i], f0 + 8 * h + i);
          ++slot;
        }
  };
  {
    // the fetched quarters: a code that reaches the bound lies in a group
    // whose maximum does
    uint32_t n = 0;
#pragma unroll
    for (int i = 0; i < kPieces; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) n += reaches(pc[i][e]) ? 1u : 0u;
    if (n != 0) {
      uint32_t slot = atomicAdd(&fs.n_cand, n);
#pragma unroll
      for (int i = 0; i < kPieces; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (reaches(pc[i][e])) {
            if (slot < (uint32_t)kStage64) fs.keys[slot] = key_of(pc[i][e], pf[i] + e);
            ++slot;
          }
    }
  }
  // the rare qualifying groups past a thread's best ones
  uint32_t fetched = 0;
#pragma unroll
  for (int b = 0; b < kBestGroups; ++b) fetched |= mb[b] != 0u ? 1u << jb[b] : 0u;
  for (uint32_t m = mask & ~fetched; m != 0; m &= m - 1) {
    u32x4 c[4];
    const uint32_t f0 = load_group(__builtin_ctz(m), c);
    append(c, f0);
  }
  lds_barrier();
  const uint32_t total = fs.n_cand;
  select_best(a, q, fs, total, total <= (uint32_t)kStage64, [&](auto fn) {
    for (uint32_t m = mask; m != 0; m &= m - 1) {
      u32x4 c[4];
      const uint32_t f0 = load_group(__builtin_ctz(m), c);
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (reaches(c[h][i])) fn(key_of(c[h][i], f0 + 8 * h + i));
    }
  });
}

// One kernel per mode, so that each holds only its own code.
template <bool kDense>
__global__ __launch_bounds__(kSelThreads) void topk_final(TopkLaunch a) {
  __shared__ FinalShared fs;
  if (kDense) final_dense(a, blockIdx.x, fs);
  else final_regions(a, blockIdx.x, fs);
}

// One request (one query): its final selection, then its composition by
// the first wave once the barrier has made every thread's ids visible, so
// the composer's launch drops out of the request's path.
template <bool kDense>
__global__ __launch_bounds__(kSelThreads) void topk_final_compose(TopkLaunch a, ComposeLaunch c) {
  __shared__ FinalShared fs;
  if (kDense) final_dense(a, 0, fs);
  else final_regions(a, 0, fs);
  __syncthreads();   // the ids are written by the threads that hold them
  if (threadIdx.x < 64) compose_request(c, 0, threadIdx.x);
}

// Scatters embedding rows [first, first + n) (row-major, `emb_dim` wide, in
// device memory) into the blocked layout, `padded_dim` wide.
__global__ __launch_bounds__(256) void emb_relayout(const uint16_t* __restrict__ rows,
                                                   int64_t first, int64_t n, int32_t emb_dim,
                                                   int32_t padded_dim,
                                                   uint16_t* __restrict__ emb) {
  const int pieces = emb_dim / 8;
  const int n_chunks = padded_dim / kKC;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n * pieces) return;
  const int64_t r = i / pieces;
  const int p = (int)(i % pieces);
  const int64_t f = first + r;
  const int64_t dst = ((f / kFT * n_chunks + p / 8) * kFT + f % kFT) * kKC + (p % 8) * 8;
  *reinterpret_cast<u32x4*>(emb + dst) = *reinterpret_cast<const u32x4*>(rows + r * emb_dim + p * 8);
}

// Moves the rows of facts keep[0..n) of the blocked layout `from` to rows
// 0..n of `to`, all `padded_dim` columns (the padding stays zero).
__global__ __launch_bounds__(256) void emb_compact(const uint16_t* __restrict__ from,
                                                  const int32_t* __restrict__ keep, int64_t n,
                                                  int32_t padded_dim, uint16_t* __restrict__ to) {
  const int pieces = padded_dim / 8;
  const int n_chunks = padded_dim / kKC;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n * pieces) return;
  const int64_t r = i / pieces;
  const int p = (int)(i % pieces);
  const int64_t f = keep[r];
  const int64_t src = ((f / kFT * n_chunks + p / 8) * kFT + f % kFT) * kKC + (p % 8) * 8;
  const int64_t dst = ((r / kFT * n_chunks + p / 8) * kFT + r % kFT) * kKC + (p % 8) * 8;
  *reinterpret_cast<u32x4*>(to + dst) = *reinterpret_cast<const u32x4*>(from + src);
}

// Copies queries [n_q][emb_dim] to [n_q][padded_dim], zero-filling the tail.
__global__ __launch_bounds__(256) void pad_queries(const uint16_t* __restrict__ q, int32_t n_q,
                                                  int32_t emb_dim, int32_t padded_dim,
                                                  uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)n_q * padded_dim) return;
  const int64_t r = i / padded_dim;
  const int c = (int)(i % padded_dim);
  out[i] = c < emb_dim ? q[r * emb_dim + c] : (uint16_t)0;
}

}  // namespace

hipError_t launch_emb_relayout(const uint16_t* rows, int64_t first, int64_t n, int32_t emb_dim,
                               uint16_t* emb, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t threads = n * (emb_dim / 8);
  hipLaunchKernelGGL(emb_relayout, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                     rows, first, n, emb_dim, topk_padded_dim(emb_dim), emb);
  return hipGetLastError();
}

hipError_t launch_emb_compact(const uint16_t* from, const int32_t* keep, int64_t n,
                              int32_t emb_dim, uint16_t* to, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int32_t padded = topk_padded_dim(emb_dim);
  const int64_t threads = n * (padded / 8);
  hipLaunchKernelGGL(emb_compact, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                     from, keep, n, padded, to);
  return hipGetLastError();
}

// A sample of S facts leaves about k * N / S candidates per query.  The
// sample scan costs about one tile per workgroup whatever S is, up to a tile
// for every CU, so small stores take 8192 facts (256 tiles of 32).
int64_t topk_sample_size(int64_t n_facts) {
  int64_t s = n_facts / 32;
  if (s < 8192) s = 8192;
  s = (s + kFT - 1) / kFT * kFT;
  return s < n_facts ? s : n_facts;
}

TopkScratch topk_scratch(int64_t n_facts, int32_t n_q, int32_t emb_dim) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const int64_t tiles = (n_facts + kFT - 1) / kFT;
  const int64_t sample_tiles = (topk_sample_size(n_facts) + kFT - 1) / kFT;
  TopkScratch s{};
  size_t off = 0;
  s.q_off = off;
  off += emb_dim % kKC ? up((size_t)n_q * topk_padded_dim(emb_dim) * 2) : 0;
  s.gmax_off = off;
  off += up((size_t)n_q * sample_tiles * kTopkGroupsPerTile * 4);
  s.tau_off = off;
  off += up((size_t)n_q * 4);
  s.count_off = off;
  off += up((size_t)n_q * kTopkMaxScanWG * 4);
  s.scode_off = off;   // the sample's facts' codes (sample_tiles x sample_tile <= this width)
  off += up((size_t)n_q * topk_padded_facts(topk_sample_size(n_facts)) * 4);
  s.scount_off = off;
  off += up((size_t)n_q * 4);
  s.cand_off = off;
  off += up((size_t)n_q * tiles * kFT * 8);
  s.bytes = off;
  return s;
}

hipError_t launch_topk(const TopkLaunch& in, hipStream_t stream, const ComposeLaunch* compose) {
  if (in.n_q == 0) return hipSuccess;
  if (in.k < 1 || in.k > kMaxK || in.k > in.n_facts || in.n_q > kQB || in.emb_dim <= 0 ||
      in.emb_dim % 8 != 0)
    return hipErrorInvalidValue;
  TopkLaunch a = in;
  a.stream_t0 = 0;
  const int32_t padded = topk_padded_dim(a.emb_dim);
  // query tiles of 32 the launch fills: 1, 2 or 4.  At width 1024, full
  // batches keep their queries in registers, sample and stream in 32-fact
  // tiles (IS_TOPK_STREAM_FT for the stream; 64-fact sample tiles measured
  // about 10% slower on the 1M index).  Batches of at most 32 queries share
  // one query tile across the waves (128-fact tiles).  Other batches and
  // widths use the staged scan.
  const int qt = a.n_q <= 32 ? 1 : a.n_q <= 64 ? 2 : 4;
  const bool wide = IS_TOPK_RESIDENT && padded == kRChunks * kKC;
  const bool resident = wide && qt == 4;
  const bool shared = wide && qt == 1;
  a.sample_n = topk_sample_size(a.n_facts);
  int ft_stream = kFT, ft_sample = kFT;
  if (shared) {
    ft_stream = ft_sample = 128;
  } else if (resident) {
    ft_stream = IS_TOPK_STREAM_FT;
    ft_sample = 32;
  }
  a.scan_tile = ft_stream;
  a.sample_tile = ft_sample;
  a.n_tiles = (a.n_facts + ft_stream - 1) / ft_stream;
  a.sample_tiles = (a.sample_n + ft_sample - 1) / ft_sample;
  a.n_groups = a.sample_tiles * (ft_sample / 16);   // groups of 16 facts
  a.cand_stride = topk_padded_facts(a.n_facts);
  a.scan_wgs = (int32_t)(a.n_tiles < kTopkMaxScanWG ? a.n_tiles : kTopkMaxScanWG);
  if (padded != a.emb_dim) {
    const int64_t n = (int64_t)a.n_q * padded;
    hipLaunchKernelGGL(pad_queries, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       a.q, a.n_q, a.emb_dim, padded, a.q_pad);
    a.q = a.q_pad;
    a.emb_dim = padded;
  }
  const int sample_wgs = (int)(a.sample_tiles < kTopkMaxScanWG ? a.sample_tiles : kTopkMaxScanWG);
  auto scan = [&](bool sample, unsigned wgs) {
    const dim3 g(wgs), b(kThreads);
    const int ft = sample ? ft_sample : ft_stream;
    if (shared) {
      if (sample) hipLaunchKernelGGL((topk_scan_rq<true, 128, true>), g, b, 0, stream, a);
      else hipLaunchKernelGGL((topk_scan_rq<false, 128, true>), g, b, 0, stream, a);
    } else if (resident) {
      if (sample) {
        hipLaunchKernelGGL((topk_scan_rq<true, 32, false>), g, b, 0, stream, a);
      } else {
        if (ft == 64) hipLaunchKernelGGL((topk_scan_rq<false, 64, false>), g, b, 0, stream, a);
        else hipLaunchKernelGGL((topk_scan_rq<false, 32, false>), g, b, 0, stream, a);
      }
    } else if (sample) {
      if (qt == 1) hipLaunchKernelGGL((topk_scan<true, 1>), g, b, 0, stream, a);
      else if (qt == 2) hipLaunchKernelGGL((topk_scan<true, 2>), g, b, 0, stream, a);
      else hipLaunchKernelGGL((topk_scan<true, 4>), g, b, 0, stream, a);
    } else {
      if (qt == 1) hipLaunchKernelGGL((topk_scan<false, 1>), g, b, 0, stream, a);
      else if (qt == 2) hipLaunchKernelGGL((topk_scan<false, 2>), g, b, 0, stream, a);
      else hipLaunchKernelGGL((topk_scan<false, 4>), g, b, 0, stream, a);
    }
  };
  // One pass when the codes of every score are few: the scan writes them
  // all with the maxima of all groups, and the final kernel takes the bound
  // from those (no sample scan, no threshold launch).
  const int64_t scanned = a.n_tiles * ft_stream;   // facts the stream scan covers
  a.dense = scanned / 16 <= kDenseGroups &&
            (int64_t)a.n_q * scanned <= (int64_t)IS_TOPK_DENSE_CODES;
  if (a.dense) {
    a.codes = reinterpret_cast<uint32_t*>(a.cand);   // n_q x scanned x 4.25 B <= the cand buffer
    a.code_stride = scanned;
    a.gmax = a.codes + (int64_t)a.n_q * scanned;
    a.n_groups = scanned / 16;
    a.fuse_tau = 0;
    const dim3 g((unsigned)a.scan_wgs), b(kThreads);
    if (shared) hipLaunchKernelGGL((topk_scan_rq<false, 128, true, true>), g, b, 0, stream, a);
    else if (resident && ft_stream == 64) hipLaunchKernelGGL((topk_scan_rq<false, 64, false, true>), g, b, 0, stream, a);
    else if (resident) hipLaunchKernelGGL((topk_scan_rq<false, 32, false, true>), g, b, 0, stream, a);
    else if (qt == 1) hipLaunchKernelGGL((topk_scan<false, 1, true>), g, b, 0, stream, a);
    else if (qt == 2) hipLaunchKernelGGL((topk_scan<false, 2, true>), g, b, 0, stream, a);
    else hipLaunchKernelGGL((topk_scan<false, 4, true>), g, b, 0, stream, a);
  } else {
    // at most four queries on the shared tile: the stream finds the bounds
    a.fuse_tau = shared && a.n_q <= kWaves && a.n_groups <= kWaveKthMax;
    // Otherwise the sample scan keeps its facts' codes, the threshold kernel
    // takes their candidates from those, and the stream scan starts after
    // the sample's tiles (the sample facts are whole stream tiles).
    const int64_t sample_facts = a.sample_tiles * ft_sample;
    if (!a.fuse_tau && a.codes != nullptr && a.scount != nullptr && sample_facts % ft_stream == 0 &&
        sample_facts / ft_stream < a.n_tiles) {
      a.stream_t0 = sample_facts / ft_stream;
      a.code_stride = sample_facts;
      const int64_t rest = a.n_tiles - a.stream_t0;
      a.scan_wgs = (int32_t)(rest < kTopkMaxScanWG ? rest : kTopkMaxScanWG);
    }
    scan(true, (unsigned)sample_wgs);
    if (!a.fuse_tau)
      hipLaunchKernelGGL(topk_threshold, dim3((unsigned)a.n_q), dim3(kSelThreads), 0, stream, a);
    scan(false, (unsigned)a.scan_wgs);
  }
  const dim3 fb(kSelThreads);
  if (compose != nullptr && a.n_q == 1) {
    if (a.dense) hipLaunchKernelGGL(topk_final_compose<true>, dim3(1), fb, 0, stream, a, *compose);
    else hipLaunchKernelGGL(topk_final_compose<false>, dim3(1), fb, 0, stream, a, *compose);
  } else {
    if (a.dense) hipLaunchKernelGGL(topk_final<true>, dim3((unsigned)a.n_q), fb, 0, stream, a);
    else hipLaunchKernelGGL(topk_final<false>, dim3((unsigned)a.n_q), fb, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace is
