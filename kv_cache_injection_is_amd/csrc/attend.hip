// Query-only attention over the paged KV cache: the step that follows the
// injection (InferScale explainer pages, technical summary, Online phase:
// the engine prefills only the query over the cache that holds the injected
// facts; Theorem 6: a re-rotated key scores like a key prefilled at the same
// position).  Synthetic queries stand in for a model's, so the injected
// cache is checked end to end on the device and its read side is measured.
//
//   out[l][r][t][hq] = sum_p softmax_p(s_p) V_l[slot_r(p)][hq / g]
//   s_p = <R(qpos_r + t) q[l][r][t][hq], K_l[slot_r(p)][hq / g]> / sqrt(d)
//   over positions p in [ctx_begin_r, ctx_end_r), g = n_q_heads / n_kv_heads.
//
// Design (gfx950; bf16 cache, head_dim 128).  One workgroup per (layer,
// request, kv head) and group of up to 64 query rows (a row is a (query
// token, query head of the group) pair).  The context is cut into 32-token
// chunks taken round-robin by the chunk streams (two when the group has
// more than 32 rows, four otherwise); each stream has one wave per 32-row
// query tile.  The two-tile kernel's four waves stay within 256 registers
// and 69 KB of LDS, so two workgroups share a CU and one's query rotation
// and final merge overlap the other's transfers.  The queries are
// rotated at their positions, pre-scaled by log2(e) / sqrt(d) and split into
// bf16 hi + lo once per workgroup; each wave keeps its tile's in registers.
//
// A chunk's K and V rows travel from the cache straight into LDS
// (global_load_lds_dwordx4, no registers on the way) in a ring of two slots
// per stream; the two waves of a stream move half of each slot (K tile / V
// tile).  In steps: every wave waits for its own transfers, a barrier makes
// all of them visible and frees the slot of the step before, the next
// step's transfers go into it, and the step is computed while they fly.
// The block table is read with scalar loads, so the ring's transfers are
// the only vector-memory operations in the loop and the waits are exact
// counts.
//
// LDS tile of one chunk (K or V): token t's 256-byte row at byte
// (t / 4) * 1024 + (t % 4) * 256, its 16-byte pieces (dims 8p .. 8p + 7)
// permuted within the row: piece p at position p ^ (t % 16) for K and
// p ^ (4 (t % 4)) for V.  One transfer instruction fills four whole rows,
// 16 lanes per row, so every load reads full 256-byte rows of the cache
// (each lane fetches the piece that belongs at its position).  The
// permutations make the K fragment reads (16 lanes = 16 tokens of one piece)
// and the transposed V reads (4 tokens x 4 pieces per 16 lanes, 32 lanes
// per cycle) free of bank conflicts.
//
// Per chunk a wave forms S^T = K Q^T and O^T += V^T P^T with
// v_mfma_f32_32x32x16_bf16; in both products the query row is the MFMA
// column, so lane l holds scores and outputs of row l % 32 only and the
// online-softmax state stays in the lane (lanes l and l ^ 32 share a row and
// exchange only the chunk maximum).  The probabilities are split into bf16
// hi + lo like the queries, so both products keep about 16 bits beyond bf16;
// accumulation is fp32.  The V^T operand comes from the transposing LDS read
// (ds_read_b64_tr_b16): within a group of 16 lanes, lane i receives element
// i % 4 of the 8 bytes that lane 4 e + i / 4 addressed, as its element e
// (e = 0..3).  The streams merge their softmax states through LDS at the
// end.  Workgroups of one (layer, request, kv head) that split its query
// rows run on the same XCD (ids congruent mod 8).
#include <hip/hip_runtime.h>

#include "kernels.h"
#include "rope_math.h"

// Chunk streams and ring slots per stream of the two-tile kernel (measured
// on the 100-request Mistral-7B-shaped batch: 2 x 2 at 5.3-5.5 ms with two
// workgroups per CU; with one workgroup per CU 4 x 2 at 6.0, 3 x 3 at 6.5,
// 2 x 4 at 7.0).
#ifndef IS_ATT_NS
#define IS_ATT_NS 2
#endif
#ifndef IS_ATT_NST
#define IS_ATT_NST 2
#endif
#ifndef IS_ATT_MINW
#define IS_ATT_MINW 2     // waves per SIMD the two-tile kernel's registers must allow
#endif

namespace is {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char* lds_cptr;
typedef __attribute__((address_space(3))) s16x4* lds_s4ptr;
typedef const __attribute__((address_space(4))) int32_t* const_i32ptr;

constexpr int kD = 128;              // head_dim
constexpr int kChunk = 32;           // context tokens per wave step
constexpr int kTileBytes = kChunk * kD * 2;       // one chunk of K (or of V): 8 KB
constexpr int kStageBytes = 2 * kTileBytes;       // K tile, then V tile
constexpr int kOPitch = kD + 4;      // floats per merged output row

__device__ __forceinline__ unsigned short bf16_bits(float x) {
  return __builtin_bit_cast(unsigned short, (__bf16)x);   // round to nearest even
}
__device__ __forceinline__ float bf16_value(unsigned short b) {
  return __uint_as_float((unsigned)b << 16);
}

// Splits 8 floats into bf16 hi and lo parts (x ~= hi + lo), two values per
// conversion (round to nearest even, as one at a time).
__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
  u32x4 hv, lv;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float2v pair = {x[2 * w], x[2 * w + 1]};
    const unsigned hp = __builtin_bit_cast(unsigned, __builtin_convertvector(pair, bf16x2));
    const float2v rest = {x[2 * w] - __uint_as_float(hp << 16),
                          x[2 * w + 1] - __uint_as_float(hp & 0xFFFF0000u)};
    hv[w] = hp;
    lv[w] = __builtin_bit_cast(unsigned, __builtin_convertvector(rest, bf16x2));
  }
  hi = __builtin_bit_cast(bf16x8, hv);
  lo = __builtin_bit_cast(bf16x8, lv);
}

// One 16-byte piece per lane from `g` into LDS bytes [lds + 16 lane, +16).
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds), "v"(g) : "memory", "m0");
}

// Waits until at most N vector-memory operations of this wave are in flight
// (they complete in order).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Barrier after this wave's LDS accesses have completed, without waiting
// for the ring's transfers (a fenced barrier would).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int QT, int NS, int NST>
struct AttendSmem {
  union {
    unsigned char ring[NST * NS * kStageBytes];      // [slot][stream][K tile | V tile]
    float o[NS][QT * 32 * kOPitch];                 // partial outputs, for the merge
  };
  float m[NS][QT * 32];
  float l[NS][QT * 32];
};

// Rotated, split query rows while they are staged (in slot 1 of the ring,
// before its first use): row r's 16-byte slice j (dims [8 j, +8)) at
// r * 16 + (j ^ (r & 15)), so the 16 rows that one 16-lane group reads land
// in 16 different bank groups.
__device__ __forceinline__ int q_slot(int r, int j) { return r * 16 + (j ^ (r & 15)); }

template <int QT, int NS, int NST, int MINW>
__global__ __launch_bounds__(QT * NS * 64, MINW) void attend_kernel(AttendLaunch a) {
  constexpr int kStreams = NS;         // chunk streams
  constexpr int kStages = NST;         // ring slots per stream
  constexpr int kThreadsWG = QT * NS * 64;
  static_assert(NST >= 2 && NST <= 4, "ring depth");
  // transfers per wave per stage: the two row-tile waves of a stream split
  // the stage (K tile / V tile); a lone wave moves both
  constexpr int kDmaWave = QT == 2 ? 8 : 16;
  __shared__ AttendSmem<QT, NS, NST> sm;
  static_assert(2 * QT * 32 * 16 * 16 <= kStreams * kStageBytes, "query staging fits one slot");
  // XCD-aware unit / row-group mapping (see above)
  const int id = (int)blockIdx.x;
  const int xcd = id & 7;
  const int kk = id >> 3;
  const int grp = kk % a.groups;
  const int64_t unit = (int64_t)(kk / a.groups) * 8 + xcd;
  if (unit >= a.n_units) return;
  const int kvh = (int)(unit % a.n_kv_heads);
  const int r = (int)((unit / a.n_kv_heads) % a.n_req);
  const int layer = (int)(unit / ((int64_t)a.n_kv_heads * a.n_req));
  const int G = a.n_q_heads / a.n_kv_heads;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sid = wave % kStreams;           // chunk stream
  const int rt = wave / kStreams;            // row tile
  const int col = lane & 31, h = lane >> 5;
  const const_i32ptr meta = (const_i32ptr)a.meta;
  const int qpos = meta[3 * r], cb = meta[3 * r + 1], ce = meta[3 * r + 2];
  const int n_ctx = ce - cb;
  const int row0 = grp * QT * 32;
  const float kScale = 1.4426950408889634f * 0.08838834764831845f;   // log2(e) / sqrt(128)

  const char* kc = static_cast<const char*>(a.kc);
  const char* vc = static_cast<const char*>(a.vc);
  const const_i32ptr btr = (const_i32ptr)(a.bt + (int64_t)r * a.max_blocks);
  const int B = a.block_size;
  const int64_t head_off = (int64_t)layer * a.s_layer + (int64_t)kvh * a.s_head;
  const uint32_t ring0 = (uint32_t)(size_t)(lds_cptr)(void*)sm.ring;

  // Element offset of this lane's token row in the chunk starting at c0.
  // Tokens past the context read the chunk's first row (a chunk wholly past
  // it, the context's first row); their scores are masked.  The chunk's
  // block-table entries are uniform loads, selected per lane.
  auto row_of = [&](int c0) -> int64_t {
    const bool live = c0 < n_ctx;
    const int p_first = live ? cb + c0 : cb;
    const int p_last = live ? min(cb + c0 + kChunk, ce) - 1 : cb;
    const int p = (live && c0 + col < n_ctx) ? cb + c0 + col : p_first;
    int blk = 0, off = 0;
    for (int b = p_first / B; b <= p_last / B; ++b) {
      const int e = btr[b];
      if (p >= b * B) {
        blk = e;
        off = p - b * B;
      }
    }
    return head_off + (int64_t)blk * a.s_block + (int64_t)off * a.s_slot;
  };
  // This wave's share of slot s <- the chunk starting at c0: the K tile
  // (row tile 0 or a lone wave) and the V tile (row tile 1 or a lone wave).
  const int pos16 = lane & 15, tq = lane >> 4;
  auto issue = [&](int s, int c0) {
    const int64_t rowe = row_of(c0);
    const int r_lo = (int)(uint32_t)rowe, r_hi = (int)(rowe >> 32);
    const uint32_t base = (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(ring0 + (uint32_t)((s * kStreams + sid) * kStageBytes)));
    // every row offset first, then the transfers: the asm transfers order
    // memory, so a shuffle placed between two of them would wait alone
    int64_t rj[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = 4 * j + tq;
      rj[j] = (int64_t)(((uint64_t)(uint32_t)__shfl(r_hi, t) << 32) | (uint32_t)__shfl(r_lo, t));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = 4 * j + tq;
      if (QT == 1 || rt == 0)
        dma16(kc + rj[j] * 2 + ((pos16 ^ (t & 15)) << 4), base + j * 1024);
      if (QT == 1 || rt == 1)
        dma16(vc + rj[j] * 2 + ((pos16 ^ (4 * tq)) << 4), base + kTileBytes + j * 1024);
    }
  };

  const int step = kStreams * kChunk;
  const int n_steps = (n_ctx + step - 1) / step;
  // the first NST - 1 steps go to slots 0 .. NST - 2; the queries are
  // staged in the last slot meanwhile
  for (int k = 0; k < kStages - 1 && k < n_steps; ++k) issue(k, (k * kStreams + sid) * kChunk);

  // Queries: rotated at their positions, pre-scaled, split into hi + lo,
  // staged in LDS (slot 1 of the ring), then loaded by every wave for its
  // row tile.  A task is a row and a pair of slices (j, j + 8): dims d and
  // d + 64 rotate together.
  u32x4* qs_hi = reinterpret_cast<u32x4*>(sm.ring + (kStages - 1) * kStreams * kStageBytes);
  u32x4* qs_lo = qs_hi + QT * 32 * 16;
  for (int task = tid; task < QT * 32 * 8; task += kThreadsWG) {
    const int rr = task >> 3, j = task & 7;
    const int R = row0 + rr;
    float x[2][8];
    if (R < a.rows) {
      const int t = R / G, hq = kvh * G + R % G;
      const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                           ((((int64_t)layer * a.n_req + r) * a.n_qtok + t) *
                                  a.n_q_heads + hq) * kD;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(qp + 8 * j + 64 * half);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const unsigned u = v[w];
          x[half][2 * w] = __uint_as_float(u << 16);
          x[half][2 * w + 1] = __uint_as_float(u & 0xFFFF0000u);
        }
      }
      const int pos = qpos + t;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 g = a.g[8 * j + e];
        const float2 cs = sincos_of_turns(pos, g.x, g.y);
        const float u = x[0][e], w = x[1][e];
        x[0][e] = __builtin_fmaf(u, cs.x, -(w * cs.y)) * kScale;
        x[1][e] = __builtin_fmaf(w, cs.x, u * cs.y) * kScale;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[0][e] = x[1][e] = 0.f;
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      bf16x8 hi, lo;
      split8(x[half], hi, lo);
      qs_hi[q_slot(rr, j + 8 * half)] = __builtin_bit_cast(u32x4, hi);
      qs_lo[q_slot(rr, j + 8 * half)] = __builtin_bit_cast(u32x4, lo);
    }
  }
  lds_barrier();
  // B operand of S^T = K Q^T per 16-dim step s: row rt * 32 + col, dims
  // 16 s + 8 h .. + 8.
  bf16x8 qh[8], ql[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int slot = q_slot(rt * 32 + col, 2 * s + h);
    qh[s] = __builtin_bit_cast(bf16x8, qs_hi[slot]);
    ql[s] = __builtin_bit_cast(bf16x8, qs_lo[slot]);
  }

  float m = -1e30f, lsum = 0.f;
  float16v o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = float16v{};

  // Per-lane parts of the LDS fragment addresses.  K: token col, piece
  // 2 s + h.  V^T (transposing read; group of 16 lanes g = lane / 16, i =
  // lane % 16, which addresses token 4 h + i / 4 (+ 16 ks + 8 half) at dims
  // 32 dt + 16 (g % 2) + 4 (i % 4): piece 4 dt + 2 (g % 2) + (i % 4) / 2,
  // byte 8 (i % 2) within it).
  const int gi = lane & 15, ge = gi >> 2;
  const int k_row = (col >> 2) * 1024 + (col & 3) * 256;
  const int k_sw = col & 15;
  const int v_lane = h * 1024 + ge * 256 + (2 * ((lane >> 4) & 1) + ((gi & 3) >> 1)) * 16 +
                     (gi & 1) * 8;
  auto process = [&](int s_idx, int c0) {
    const char* st_k = reinterpret_cast<const char*>(sm.ring) + (s_idx * kStreams + sid) * kStageBytes;
    const char* st_v = st_k + kTileBytes;
    // S^T: element (token, row) at lane col = row, reg i -> token
    // 8 (i / 4) + 4 h + i % 4
    float16v st = float16v{};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
          st_k + k_row + (((2 * s + h) ^ k_sw) << 4));
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qh[s], st, 0, 0, 0);
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, ql[s], st, 0, 0, 0);
    }
    // online softmax (base 2); P split for the second product
    float sv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) sv[i] = st[i];
    if (c0 + kChunk > n_ctx) {   // the last, partial chunk (a uniform branch)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (c0 + 8 * (i / 4) + 4 * h + (i % 4) >= n_ctx) sv[i] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sv[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // Lazy rescaling: the reference m only moves when some row's maximum
    // passes it by more than 8 (a factor 256 in the weights); until then
    // the weights exp2(s - m) may exceed 1 by up to that factor, which the
    // split operands and fp32 sums carry without loss.
    if (__builtin_amdgcn_ballot_w64(mx > m + 8.0f)) {
      const float mn = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      m = mn;
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
    }
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sv[i] = __builtin_amdgcn_exp2f(sv[i] - m);
      ps += sv[i];
    }
    lsum += ps;
    bf16x8 phi[2], plo[2];
    split8(sv, phi[0], plo[0]);
    split8(sv + 8, phi[1], plo[1]);
    // O^T += V^T P^T: A = V^T rows d = 32 dt + col, k = the lane's 8 tokens
    // 16 ks + 8 (e / 4) + 4 h + e % 4, from two transposing reads
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s4ptr)(lds_cptr)(void*)(st_v + v_lane + ((dt ^ ge) << 6) + 4 * ks * 1024));
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s4ptr)(lds_cptr)(void*)(st_v + v_lane + ((dt ^ ge) << 6) + (4 * ks + 2) * 1024));
        const s16x8 vv = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 va = __builtin_bit_cast(bf16x8, vv);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, phi[ks], o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, plo[ks], o[dt], 0, 0, 0);
      }
    }
  };

  // The ring, in steps: step n's chunks (one per stream) sit in slot n % 2.
  // At each step every wave waits for its own transfers, the barrier makes
  // all of them visible and frees the slot that step n - 1 used, the next
  // step's transfers go into that slot, and the step is computed while they
  // are in flight.  The query staging (slot 1) is free after the first
  // barrier.
  for (int n = 0; n < n_steps; ++n) {
    // this wave's transfers younger than step n's: those of the steps
    // n + 1 .. n + NST - 2 that exist
    const int younger = min(kStages - 2, n_steps - 1 - n);
    if (younger >= 2)
      wait_vm<2 * kDmaWave>();
    else if (younger == 1)
      wait_vm<kDmaWave>();
    else
      wait_vm<0>();
    lds_barrier();
    const int nx = n + kStages - 1;
    if (nx < n_steps) issue(nx % kStages, (nx * kStreams + sid) * kChunk);
    const int c0 = (n * kStreams + sid) * kChunk;
    if (c0 < n_ctx) process(n % kStages, c0);
  }
  wait_vm<0>();   // no transfer may land in the LDS once it is reused below

  // merge the streams' softmax states (per row tile)
  lsum += __shfl_xor(lsum, 32);
  lds_barrier();   // every wave is done with the ring (the union's other half)
  if (h == 0) {
    sm.m[sid][rt * 32 + col] = m;
    sm.l[sid][rt * 32 + col] = lsum;
  }
  float* ob = sm.o[sid] + (rt * 32 + col) * kOPitch;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) ob[32 * dt + 8 * (i / 4) + 4 * h + (i % 4)] = o[dt][i];
  __syncthreads();
  for (int idx = tid; idx < QT * 32 * kD; idx += kThreadsWG) {
    const int rr = idx / kD, d = idx % kD;
    const int R = row0 + rr;
    if (R >= a.rows) continue;
    float M = sm.m[0][rr];
#pragma unroll
    for (int w = 1; w < kStreams; ++w) M = fmaxf(M, sm.m[w][rr]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kStreams; ++w) {
      const float f = __builtin_amdgcn_exp2f(sm.m[w][rr] - M);
      L += sm.l[w][rr] * f;
      O += sm.o[w][rr * kOPitch + d] * f;
    }
    const int t = R / G, hq = kvh * G + R % G;
    a.out[((((int64_t)layer * a.n_req + r) * a.n_qtok + t) * a.n_q_heads + hq) * kD + d] =
        L > 0.f ? O / L : 0.f;
  }
}

// Any head_dim (even, at most 256) and cache dtype (fp32 or bf16), for the
// shapes the matrix-core kernel does not take: one wave per query row
// (layer, request, query token, query head).  Lane j holds the rotation
// pairs (j, j + d/2) and (j + 64, j + 64 + d/2) of the query and of every
// key and value row it reads; a score is a wave-wide sum; the online softmax
// (base 2) and the output accumulate in fp32.  Plain loads, one context
// token after the other: a parity path for small shapes, not a fast one.
template <typename T>
__device__ __forceinline__ float elem(const T* p, int64_t i);
template <>
__device__ __forceinline__ float elem<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float elem<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_value(p[i]);
}

template <typename T>
__global__ __launch_bounds__(64) void attend_generic(AttendLaunch a) {
  const int64_t row = blockIdx.x;
  const int hq = (int)(row % a.n_q_heads);
  const int t = (int)((row / a.n_q_heads) % a.n_qtok);
  const int r = (int)((row / ((int64_t)a.n_q_heads * a.n_qtok)) % a.n_req);
  const int layer = (int)(row / ((int64_t)a.n_q_heads * a.n_qtok * a.n_req));
  const int kvh = hq / (a.n_q_heads / a.n_kv_heads);
  const int lane = threadIdx.x;
  const int half = a.head_dim / 2;
  const int qpos = a.meta[3 * r] + t, cb = a.meta[3 * r + 1], ce = a.meta[3 * r + 2];
  const float scale = 1.4426950408889634f / sqrtf((float)a.head_dim);   // log2(e) / sqrt(d)
  const T* q = static_cast<const T*>(a.q) + row * a.head_dim;
  float qa[2], qb[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = lane + 64 * u;
    qa[u] = qb[u] = 0.f;
    if (i < half) {
      const float x = elem<T>(q, i), y = elem<T>(q, i + half);
      const float2 cs = sincos_of_turns(qpos, a.g[i].x, a.g[i].y);
      qa[u] = __builtin_fmaf(x, cs.x, -(y * cs.y)) * scale;
      qb[u] = __builtin_fmaf(y, cs.x, x * cs.y) * scale;
    }
  }
  const T* kc = static_cast<const T*>(a.kc);
  const T* vc = static_cast<const T*>(a.vc);
  const int32_t* bt = a.bt + (int64_t)r * a.max_blocks;
  const int64_t head_off = (int64_t)layer * a.s_layer + (int64_t)kvh * a.s_head;
  float m = -1e30f, l = 0.f, oa[2] = {0.f, 0.f}, ob[2] = {0.f, 0.f};
  for (int p = cb; p < ce; ++p) {
    const int64_t off = head_off + (int64_t)bt[p / a.block_size] * a.s_block +
                        (int64_t)(p % a.block_size) * a.s_slot;
    float part = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = lane + 64 * u;
      if (i < half)
        part += qa[u] * elem<T>(kc, off + i) + qb[u] * elem<T>(kc, off + i + half);
    }
#pragma unroll
    for (int w = 32; w >= 1; w >>= 1) part += __shfl_xor(part, w);
    const float mn = fmaxf(m, part);
    const float alpha = __builtin_amdgcn_exp2f(m - mn), wgt = __builtin_amdgcn_exp2f(part - mn);
    m = mn;
    l = l * alpha + wgt;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = lane + 64 * u;
      if (i < half) {
        oa[u] = oa[u] * alpha + wgt * elem<T>(vc, off + i);
        ob[u] = ob[u] * alpha + wgt * elem<T>(vc, off + i + half);
      }
    }
  }
  float* out = a.out + row * a.head_dim;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = lane + 64 * u;
    if (i < half) {
      out[i] = l > 0.f ? oa[u] / l : 0.f;
      out[i + half] = l > 0.f ? ob[u] / l : 0.f;
    }
  }
}

}  // namespace

hipError_t launch_attend(const AttendLaunch& in, hipStream_t stream) {
  if (in.n_units == 0 || in.rows == 0) return hipSuccess;
  if (in.dtype != IS_DTYPE_BF16 || in.head_dim != kD) {
    if (in.head_dim < 2 || in.head_dim % 2 != 0 || in.head_dim > 256) return hipErrorInvalidValue;
    const int64_t rows = (int64_t)in.n_layers * in.n_req * in.n_qtok * in.n_q_heads;
    if (rows > INT32_MAX) return hipErrorInvalidValue;
    if (in.dtype == IS_DTYPE_F32)
      hipLaunchKernelGGL(attend_generic<float>, dim3((unsigned)rows), dim3(64), 0, stream, in);
    else
      hipLaunchKernelGGL(attend_generic<uint16_t>, dim3((unsigned)rows), dim3(64), 0, stream, in);
    return hipGetLastError();
  }
  AttendLaunch a = in;
  const int qt = a.rows <= 32 ? 1 : 2;
  a.groups = (a.rows + qt * 32 - 1) / (qt * 32);
  const int64_t wgs = (a.n_units + 7) / 8 * 8 * a.groups;
  if (wgs > INT32_MAX) return hipErrorInvalidValue;
  if (qt == 1)
    hipLaunchKernelGGL((attend_kernel<1, 4, 2, 1>), dim3((unsigned)wgs), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((attend_kernel<2, IS_ATT_NS, IS_ATT_NST, IS_ATT_MINW>), dim3((unsigned)wgs),
                       dim3(2 * IS_ATT_NS * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace is
