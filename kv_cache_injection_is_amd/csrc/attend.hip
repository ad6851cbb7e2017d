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
// Design (gfx950; bf16 cache, head_dim 128).  One workgroup of four waves
// per (layer, request, kv head) and group of up to 64 query rows (a row is a
// (query token, query head of the group) pair; two 32-row MFMA tiles, one
// when the rows fit in 32).  The queries are rotated at their positions,
// pre-scaled by log2(e) / sqrt(d), split into bf16 hi + lo and stored once
// in LDS for all four waves (XOR-swizzled, conflict-free reads).  The waves
// take the context's 32-token chunks round-robin; each keeps a ring of
// chunks in registers (K fragments and V rows, 16-byte loads, two lanes per
// 256-byte row) so that while one chunk is computed the next are in flight.
// Per chunk a wave forms S^T = K Q^T and O^T += V^T P^T with
// v_mfma_f32_32x32x16_bf16; in both products the query row is the MFMA
// column, so lane l holds scores and outputs of row l % 32 only and the
// online-softmax state stays in the lane (lanes l and l ^ 32 share a row and
// exchange only the chunk maximum).  The probabilities are split into bf16
// hi + lo like the queries, so both products keep about 16 bits beyond bf16;
// accumulation is fp32.  V rows pass through LDS to be read transposed.  The
// four waves merge their softmax states through LDS at the end.  Workgroups
// of one (layer, request, kv head) that split its query rows run on the same
// XCD (ids congruent mod 8).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kernels.h"
#include "rope_math.h"

namespace is {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;              // head_dim
constexpr int kChunk = 32;           // context tokens per wave step
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kVPitch = kD + 8;      // bf16 per staged V row (16-byte pad: no bank conflicts)
constexpr int kOPitch = kD + 4;      // floats per merged output row

__device__ __forceinline__ unsigned short bf16_bits(float x) {
  return __builtin_bit_cast(unsigned short, (__bf16)x);   // round to nearest even
}
__device__ __forceinline__ float bf16_value(unsigned short b) {
  return __uint_as_float((unsigned)b << 16);
}

// Splits 8 floats into bf16 hi and lo parts (x ~= hi + lo).
__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
  unsigned short h[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = bf16_bits(x[e]);
    l[e] = bf16_bits(x[e] - bf16_value(h[e]));
  }
  u32x4 hv, lv;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    hv[w] = (unsigned)h[2 * w] | ((unsigned)h[2 * w + 1] << 16);
    lv[w] = (unsigned)l[2 * w] | ((unsigned)l[2 * w + 1] << 16);
  }
  hi = __builtin_bit_cast(bf16x8, hv);
  lo = __builtin_bit_cast(bf16x8, lv);
}

template <int QT>
struct AttendSmem {
  union {
    struct {
      // rotated, pre-scaled queries split in bf16 hi and lo: row r's 16-byte
      // slice j (dims [8 j, +8)) at r * 16 + (j ^ (r & 15)), so the 16 rows
      // one 16-lane group reads land in 16 different bank groups
      u32x4 qhi[QT * 32 * 16];
      u32x4 qlo[QT * 32 * 16];
      unsigned short v[kWaves][kChunk * kVPitch];   // staged V rows, per wave
    } run;
    float o[kWaves][QT * 32 * kOPitch];             // partial outputs, for the merge
  };
  float m[kWaves][QT * 32];
  float l[kWaves][QT * 32];
};

__device__ __forceinline__ int q_slot(int r, int j) { return r * 16 + (j ^ (r & 15)); }

template <int QT>
__global__ __launch_bounds__(kThreads) void attend_kernel(AttendLaunch a) {
  __shared__ AttendSmem<QT> sm;
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

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, h = lane >> 5;
  const int qpos = a.meta[3 * r], cb = a.meta[3 * r + 1], ce = a.meta[3 * r + 2];
  const int row0 = grp * QT * 32;
  const float kScale = 1.4426950408889634f * 0.08838834764831845f;   // log2(e) / sqrt(128)

  // Queries: rotated at their positions, pre-scaled, split into hi + lo,
  // written to LDS once for all four waves.  A task is a row and a pair of
  // slices (j, j + 8): dims d and d + 64 rotate together.
  for (int task = tid; task < QT * 32 * 8; task += kThreads) {
    const int rr = task >> 3, j = task & 7;
    const int R = row0 + rr;
    float x[2][8];
    if (R < a.rows) {
      const int t = R / G, hq = kvh * G + R % G;
      const uint16_t* qp = a.q + ((((int64_t)layer * a.n_req + r) * a.n_qtok + t) *
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
      sm.run.qhi[q_slot(rr, j + 8 * half)] = __builtin_bit_cast(u32x4, hi);
      sm.run.qlo[q_slot(rr, j + 8 * half)] = __builtin_bit_cast(u32x4, lo);
    }
  }
  __syncthreads();

  float m[QT], lsum[QT];
  float16v o[QT][4];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m[qt] = -1e30f;
    lsum[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[qt][dt] = float16v{};
  }

  const char* kc = static_cast<const char*>(a.kc);
  const char* vc = static_cast<const char*>(a.vc);
  const int32_t* bt = a.bt + (int64_t)r * a.max_blocks;
  unsigned short* vs = sm.run.v[wave];
  const int n_ctx = ce - cb;
  // Element offset of this lane's K/V row in the chunk starting at c0
  // (positions past the context re-read the first one; their scores are
  // masked).
  auto row_of = [&](int c0) -> int64_t {
    const int tok = c0 + col;
    const int p = cb + (tok < n_ctx ? tok : 0);
    return (int64_t)layer * a.s_layer + (int64_t)bt[p / a.block_size] * a.s_block +
           (int64_t)(p % a.block_size) * a.s_slot + (int64_t)kvh * a.s_head;
  };
  // A ring of chunks in registers: while one is computed, the others are in
  // flight (three for one row tile; two rows tiles leave room for two).
  constexpr int kDepth = QT == 1 ? 3 : 2;
  bf16x8 kf[kDepth][8];
  u32x4 vr[kDepth][8];
  auto issue = [&](auto B, int c0) {
    if (c0 >= n_ctx) return;
    const int64_t rowe = row_of(c0);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      kf[B][s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kc + (rowe + 16 * s + 8 * h) * 2));
      vr[B][s] = *reinterpret_cast<const u32x4*>(vc + (rowe + 16 * s + 8 * h) * 2);
    }
  };
  auto process = [&](auto B, int c0) {
#pragma unroll
    for (int s = 0; s < 8; ++s)
      *reinterpret_cast<u32x4*>(vs + col * kVPitch + 16 * s + 8 * h) = vr[B][s];
    // S^T for each row tile: element (token, row) at lane col = row,
    // reg i -> token 8 (i / 4) + 4 h + i % 4
    float16v st[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      st[qt] = float16v{};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int slot = q_slot(qt * 32 + col, 2 * s + h);
        const bf16x8 qh = __builtin_bit_cast(bf16x8, sm.run.qhi[slot]);
        const bf16x8 ql = __builtin_bit_cast(bf16x8, sm.run.qlo[slot]);
        st[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[B][s], qh, st[qt], 0, 0, 0);
        st[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[B][s], ql, st[qt], 0, 0, 0);
      }
    }
    // online softmax (base 2); P split for the second product
    bf16x8 phi[QT][2], plo[QT][2];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float sv[16];
      float mx = -INFINITY;
      const bool tail = c0 + kChunk > n_ctx;   // the last, partial chunk
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int ti = c0 + 8 * (i / 4) + 4 * h + (i % 4);
        sv[i] = (!tail || ti < n_ctx) ? st[qt][i] : -INFINITY;
        mx = fmaxf(mx, sv[i]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      // Lazy rescaling: the reference m only moves when some row's maximum
      // passes it by more than 8 (a factor 256 in the weights); until then
      // the weights exp2(s - m) may exceed 1 by up to that factor, which the
      // split operands and fp32 sums carry without loss.
      if (__builtin_amdgcn_ballot_w64(mx > m[qt] + 8.0f)) {
        const float mn = fmaxf(m[qt], mx);
        const float alpha = __builtin_amdgcn_exp2f(m[qt] - mn);
        m[qt] = mn;
        lsum[qt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[qt][dt][i] *= alpha;
      }
      const float mn = m[qt];
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sv[i] = __builtin_amdgcn_exp2f(sv[i] - mn);
        ps += sv[i];
      }
      lsum[qt] += ps;
      split8(sv, phi[qt][0], plo[qt][0]);
      split8(sv + 8, phi[qt][1], plo[qt][1]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's V rows are in LDS
    // O^T += V^T P^T: A = V^T rows d = 32 dt + col, k = the lane's 8 tokens
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        unsigned short vt[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int tk = 16 * ks + 8 * (e / 4) + 4 * h + (e % 4);
          vt[e] = vs[tk * kVPitch + 32 * dt + col];
        }
        u32x4 vv;
#pragma unroll
        for (int w = 0; w < 4; ++w) vv[w] = (unsigned)vt[2 * w] | ((unsigned)vt[2 * w + 1] << 16);
        const bf16x8 va = __builtin_bit_cast(bf16x8, vv);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          o[qt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, phi[qt][ks], o[qt][dt], 0, 0, 0);
          o[qt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, plo[qt][ks], o[qt][dt], 0, 0, 0);
        }
      }
    }
  };
  const int step = kWaves * kChunk;
  const std::integral_constant<int, 0> b0;
  const std::integral_constant<int, 1> b1;
  const std::integral_constant<int, kDepth - 1> b2;   // the third buffer when kDepth == 3
  int c = wave * kChunk;
  issue(b0, c);
  issue(b1, c + step);
  if constexpr (kDepth == 3) issue(b2, c + 2 * step);
  for (; c < n_ctx; c += kDepth * step) {
    process(b0, c);
    issue(b0, c + kDepth * step);
    if (c + step >= n_ctx) break;
    process(b1, c + step);
    issue(b1, c + (kDepth + 1) * step);
    if constexpr (kDepth == 3) {
      if (c + 2 * step >= n_ctx) break;
      process(b2, c + 2 * step);
      issue(b2, c + 5 * step);
    }
  }

  // merge the four waves' states
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) lsum[qt] += __shfl_xor(lsum[qt], 32);
  __syncthreads();   // every wave is done with its V staging (the union's other half)
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    if (h == 0) {
      sm.m[wave][qt * 32 + col] = m[qt];
      sm.l[wave][qt * 32 + col] = lsum[qt];
    }
    float* ob = sm.o[wave] + (qt * 32 + col) * kOPitch;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) ob[32 * dt + 8 * (i / 4) + 4 * h + (i % 4)] = o[qt][dt][i];
  }
  __syncthreads();
  for (int idx = tid; idx < QT * 32 * kD; idx += kThreads) {
    const int rr = idx / kD, d = idx % kD;
    const int R = row0 + rr;
    if (R >= a.rows) continue;
    float M = sm.m[0][rr];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm.m[w][rr]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = __builtin_amdgcn_exp2f(sm.m[w][rr] - M);
      L += sm.l[w][rr] * f;
      O += sm.o[w][rr * kOPitch + d] * f;
    }
    const int t = R / G, hq = kvh * G + R % G;
    a.out[((((int64_t)layer * a.n_req + r) * a.n_qtok + t) * a.n_q_heads + hq) * kD + d] =
        L > 0.f ? O / L : 0.f;
  }
}

}  // namespace

hipError_t launch_attend(const AttendLaunch& in, hipStream_t stream) {
  if (in.n_units == 0 || in.rows == 0) return hipSuccess;
  AttendLaunch a = in;
  const int qt = a.rows <= 32 ? 1 : 2;
  a.groups = (a.rows + qt * 32 - 1) / (qt * 32);
  const int64_t wgs = (a.n_units + 7) / 8 * 8 * a.groups;
  if (wgs > INT32_MAX) return hipErrorInvalidValue;
  if (qt == 1)
    hipLaunchKernelGGL(attend_kernel<1>, dim3((unsigned)wgs), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(attend_kernel<2>, dim3((unsigned)wgs), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace is
