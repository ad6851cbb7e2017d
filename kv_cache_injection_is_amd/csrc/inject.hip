// Fused gather -> Chunked RoPE -> paged scatter (the injection kernel).
//
// Follows the "Online phase" of the InferScale explainer pages
// ("InferScale: GPU-Native KV Injection for Personalized LLM Serving",
// technical summary): stored pre-RoPE keys receive the RoPE rotation of
// their new serving position (Theorem 6: exact under RoPE) and, with the raw
// values, are scatter-copied into the paged KV cache.  Rotation reading:
// rotate-half pairs (i, i + d/2) turn by p * f_i.
//
// Facts of the pinned host tier are read by the same code through their
// device-visible addresses (zero-copy over PCIe).
//
// Design (gfx950): one workgroup of 256 lanes per (selected fact, layer).
// The fact's [kv_head][token][head_dim] block for that layer is contiguous
// in the store, so the workgroup streams it with 16-byte loads.  A lane owns
// one 16-byte chunk of the first half of a row and the matching chunk of the
// second half, so the rotate-half partner of every element sits in its own
// registers.  cos/sin of p * f_i are computed once per (token, frequency) in
// fp32 registers -- no table in memory -- and shared through LDS by all
// kv_heads of the layer.  The angle is reduced exactly in turns: with
// g = f / 2pi split as hi + lo in fp32, p*hi is split into its rounded value
// and its exact FMA error, the integer turns are dropped, and the remaining
// fraction feeds a quadrant reduction and Taylor polynomials of degree 9
// (sine) and 10 (cosine) on |y| <= pi/4.
#include <hip/hip_runtime.h>

#include "kernels.h"
#include "rope_math.h"

// Tuning knobs (compile-time).
#ifndef IS_INJECT_NT_LOAD
#define IS_INJECT_NT_LOAD 0     // non-temporal loads of the store (plain loads measured 1.2%
#endif                          // faster on the Mistral batch: facts picked by several
                                // requests are re-read from cache)
#ifndef IS_INJECT_NT_STORE
#define IS_INJECT_NT_STORE 1    // non-temporal stores to the cache
#endif
#ifndef IS_INJECT_PREFETCH
#define IS_INJECT_PREFETCH 0    // issue the first rows' loads before computing cos/sin
#endif
#ifndef IS_INJECT_LDS_TABLE
#define IS_INJECT_LDS_TABLE 32768   // bytes of the per-chunk cos/sin table
#endif
#ifndef IS_INJECT_ROWS
#define IS_INJECT_ROWS 4        // rows in flight per lane
#endif
// Row-contiguous variant for 256-byte rows (bf16 head_dim 128, fp32 64).
#ifndef IS_R16
#define IS_R16 1                // use it where it applies
#endif
#ifndef IS_R16_THREADS
#define IS_R16_THREADS 512      // lanes per workgroup for long facts
#endif
#ifndef IS_R16_ROWS
#define IS_R16_ROWS 8           // rows in flight per lane, long facts
#endif
#ifndef IS_R16_SHORT_ROWS
#define IS_R16_SHORT_ROWS 128   // below this many rows per layer (kv_heads x mean fact length)
#endif                          // a workgroup takes several layers, with 256 lanes
#ifndef IS_R16_SHORT_THREADS
#define IS_R16_SHORT_THREADS 256  // lanes per workgroup for short facts
#endif
#ifndef IS_R16_SHORT_U
#define IS_R16_SHORT_U 4        // rows in flight per lane, short facts
#endif
#ifndef IS_R16_FIXED_LAYERS
#define IS_R16_FIXED_LAYERS 0   // > 0: that many layers per workgroup, whatever the lengths
#endif
#ifndef IS_R16_TC
#define IS_R16_TC 64            // tokens per cos/sin pass
#endif
#ifndef IS_R16_LAYER_FAST
#define IS_R16_LAYER_FAST 1     // grid x = layer group (consecutive workgroups share a fact)
#endif
#ifndef IS_R16_ONE_PER_CU
#define IS_R16_ONE_PER_CU 65536 // dynamic LDS (bytes) requested by the long-fact launch so that
#endif                          // one 512-lane workgroup runs per CU (0: as many as fit)
#ifndef IS_R16_HOST_WHOLE
#define IS_R16_HOST_WHOLE 1     // one workgroup moves all layers of a host-tier fact
#endif

namespace is {
namespace {

constexpr int kThreads = 256;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 load16(const char* p) {
#if IS_INJECT_NT_LOAD
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#else
  return *reinterpret_cast<const u32x4*>(p);
#endif
}

__device__ __forceinline__ void store16(char* p, u32x4 v) {
#if IS_INJECT_NT_STORE
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
#else
  *reinterpret_cast<u32x4*>(p) = v;
#endif
}

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  const __bf16 x = (__bf16)a;   // round to nearest even
  const __bf16 y = (__bf16)b;
  return (unsigned)__builtin_bit_cast(unsigned short, x) |
         ((unsigned)__builtin_bit_cast(unsigned short, y) << 16);
}

// Rotates the pairs (lo[e], hi[e]) by cs[e]; ES = element size.  Vector
// elements are copied to scalars before any bit reinterpretation (a bit
// cast applied to a vector-element lvalue reads the wrong element).
template <int ES>
__device__ __forceinline__ void rotate_chunk(u32x4& lo, u32x4& hi, const float2* cs) {
  u32x4 nlo, nhi;
  if constexpr (ES == 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const unsigned ua = lo[e], ub = hi[e];
      const float a = __uint_as_float(ua);
      const float b = __uint_as_float(ub);
      const float2 r = cs[e];
      nlo[e] = __float_as_uint(__builtin_fmaf(a, r.x, -(b * r.y)));
      nhi[e] = __float_as_uint(__builtin_fmaf(b, r.x, a * r.y));
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const unsigned ua = lo[w], ub = hi[w];
      const float a0 = __uint_as_float(ua << 16);
      const float a1 = __uint_as_float(ua & 0xFFFF0000u);
      const float b0 = __uint_as_float(ub << 16);
      const float b1 = __uint_as_float(ub & 0xFFFF0000u);
      const float2 r0 = cs[2 * w], r1 = cs[2 * w + 1];
      const float y0 = __builtin_fmaf(a0, r0.x, -(b0 * r0.y));
      const float y1 = __builtin_fmaf(a1, r1.x, -(b1 * r1.y));
      const float z0 = __builtin_fmaf(b0, r0.x, a0 * r0.y);
      const float z1 = __builtin_fmaf(b1, r1.x, a1 * r1.y);
      nlo[w] = pack_bf16(y0, y1);
      nhi[w] = pack_bf16(z0, z1);
    }
  }
  lo = nlo;
  hi = nhi;
}

template <int ES, int LPT>
__global__ __launch_bounds__(kThreads) void inject_kernel(InjectLaunch a) {
  constexpr int VEC = 16 / ES;                 // elements per 16-byte chunk
  constexpr int HALF = LPT * VEC;              // head_dim / 2
  constexpr int D = 2 * HALF;
  constexpr int TC = (IS_INJECT_LDS_TABLE / 8 / HALF) < 128 ? (IS_INJECT_LDS_TABLE / 8 / HALF)
                                                             : 128;  // tokens per pass
  constexpr int ROWS = kThreads / LPT;         // rows per workgroup sweep
  constexpr int U = IS_INJECT_ROWS;            // rows in flight per lane

  __shared__ float2 cs[TC * HALF];
  __shared__ int64_t slot_off[TC];

  if (a.status != nullptr && *a.status != 0) return;   // the call failed validation
  const WorkItem w = a.work[blockIdx.x];
  const int layer = blockIdx.y;
  const int len = w.len;
  const int64_t layer_off = (int64_t)layer * a.n_heads * len * D * ES;
  const char* __restrict__ ksrc = reinterpret_cast<const char*>(w.k) + layer_off;
  const char* __restrict__ vsrc = reinterpret_cast<const char*>(w.v) + layer_off;
  char* __restrict__ kc = static_cast<char*>(a.kc);
  char* __restrict__ vc = static_cast<char*>(a.vc);
  const int32_t* __restrict__ bt = a.bt + (int64_t)w.req * a.max_blocks;
  const int tid = threadIdx.x;
  const int chunk = tid % LPT;

  for (int t0 = 0; t0 < len; t0 += TC) {
    const int tc = min(TC, len - t0);
    const int rows = a.n_heads * tc;
    const float inv_tc = 1.0f / (float)tc;
    u32x4 klo[U], khi[U], vlo[U], vhi[U];
    int hh[U], tt[U];
    // Loads of rows r0 + u*ROWS, u < U (rows past `rows` are skipped).
    auto load_rows = [&](int r0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = r0 + u * ROWS;
        const int h = (int)(((float)r + 0.5f) * inv_tc);   // r / tc for r < 2^16
        hh[u] = h;
        tt[u] = r - h * tc;
        if (r < rows) {
          const int64_t e = ((int64_t)h * len + t0 + tt[u]) * D + chunk * VEC;
          klo[u] = load16(ksrc + e * ES);
          khi[u] = load16(ksrc + (e + HALF) * ES);
          vlo[u] = load16(vsrc + e * ES);
          vhi[u] = load16(vsrc + (e + HALF) * ES);
        }
      }
    };
    int r0 = tid / LPT;
#if IS_INJECT_PREFETCH
    load_rows(r0);
#endif
    for (int idx = tid; idx < tc * HALF; idx += kThreads) {
      const int t = idx / HALF, i = idx % HALF;
      const float2 g = a.g[i];
      cs[idx] = sincos_of_turns(w.pos + t0 + t, g.x, g.y);
    }
    for (int t = tid; t < tc; t += kThreads) {
      const int p = w.pos + t0 + t;
      const int64_t blk = bt[p / a.block_size];
      slot_off[t] = (int64_t)layer * a.s_layer + blk * a.s_block +
                    (int64_t)(p % a.block_size) * a.s_slot;
    }
    __syncthreads();
    for (; r0 < rows; r0 += U * ROWS) {
#if IS_INJECT_PREFETCH
      if (r0 != tid / LPT) load_rows(r0);
#else
      load_rows(r0);
#endif
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = r0 + u * ROWS;
        if (r < rows) {
          rotate_chunk<ES>(klo[u], khi[u], cs + tt[u] * HALF + chunk * VEC);
          const int64_t dst = slot_off[tt[u]] + (int64_t)hh[u] * a.s_head + chunk * VEC;
          store16(kc + dst * ES, klo[u]);
          store16(kc + (dst + HALF) * ES, khi[u]);
          store16(vc + dst * ES, vlo[u]);
          store16(vc + (dst + HALF) * ES, vhi[u]);
        }
      }
    }
    __syncthreads();
  }
}

// Row-contiguous injection for 256-byte rows: 16 lanes cover a row with one
// 16-byte chunk each, so a wave's load or store covers four whole rows.  The
// rotate-half partner of lane c (first half) is lane c + 8 (second half) of
// the same 16-lane row; the pair swap is a DPP rotate by 8 within the row.
// A workgroup handles G consecutive layers of one selected fact (G set per
// launch): those layers' [kv_head][token][head_dim] blocks are one
// contiguous span.  A workgroup's start (work item, cos/sin, slot offsets,
// barrier, then the first loads) costs about 2 us whatever it moves, so
// short facts take several layers per workgroup: with one layer each, a
// batch of 1-3 token facts is bound by workgroup starts, not by memory.  A
// fact of the host tier is moved by one workgroup, all its layers (one span
// of pinned memory); the other workgroups of its grid row exit at once.
template <int ES, int T, int U, int TC>
__global__ __launch_bounds__(T) void inject_row16(InjectLaunch a) {
  constexpr int VEC = 16 / ES;      // elements per lane
  constexpr int HALF = 8 * VEC;     // head_dim / 2
  constexpr int D = 2 * HALF;
  constexpr int RPS = T / 16;       // rows per workgroup sweep
  __shared__ float2 cs[TC * HALF];
  __shared__ int64_t slot_off[TC];

  if (a.status != nullptr && *a.status != 0) return;   // the call failed validation
#if IS_R16_LAYER_FAST
  const WorkItem w = a.work[blockIdx.y];
  const int grp = blockIdx.x;
#else
  const WorkItem w = a.work[blockIdx.x];
  const int grp = blockIdx.y;
#endif
  const int G = a.layers_per_wg;
  const bool whole = IS_R16_HOST_WHOLE && w.tier != 0;
  if (whole && grp != 0) return;
  const int l_begin = whole ? 0 : grp * G;
  const int l_end = whole ? a.n_layers : min(a.n_layers, l_begin + G);
  const int len = w.len;
  const int H = a.n_heads;
  char* __restrict__ kc = static_cast<char*>(a.kc);
  char* __restrict__ vc = static_cast<char*>(a.vc);
  const int32_t* __restrict__ bt = a.bt + (int64_t)w.req * a.max_blocks;
  const int tid = threadIdx.x;
  const int c = tid & 15;
  const int upper = c >> 3;                  // 0: first half of the row, 1: second
  const int col = upper * HALF + (c & 7) * VEC;
  const int fcol = (c & 7) * VEC;            // first frequency of this lane
  const float sgn = upper ? 1.0f : -1.0f;

  for (int t0 = 0; t0 < len; t0 += TC) {
    const int tc = min(TC, len - t0);
    for (int idx = tid; idx < tc * HALF; idx += T) {
      const int t = idx / HALF, i = idx % HALF;
      const float2 g = a.g[i];
      cs[idx] = sincos_of_turns(w.pos + t0 + t, g.x, g.y);
    }
    for (int t = tid; t < tc; t += T) {
      const int p = w.pos + t0 + t;
      slot_off[t] = (int64_t)bt[p / a.block_size] * a.s_block +
                    (int64_t)(p % a.block_size) * a.s_slot;
    }
    __syncthreads();
    const int per_layer = H * tc;
    const float inv_pl = 1.0f / (float)per_layer;
    const float inv_tc = 1.0f / (float)tc;
    // layers per pass: a pass indexes its rows below 2^16, where the row
    // decomposition by float reciprocals is exact
    const int lpp = max(1, 65535 / per_layer);
    for (int l0 = l_begin; l0 < l_end; l0 += lpp) {
      const int rows = min(lpp, l_end - l0) * per_layer;
      const int64_t base = (int64_t)l0 * H * len * D * ES;
      const char* __restrict__ ksrc = reinterpret_cast<const char*>(w.k) + base;
      const char* __restrict__ vsrc = reinterpret_cast<const char*>(w.v) + base;
      // r -> (layer g, head h, token t); exact for r < 2^16
      auto split_row = [&](int r, int& g, int& h, int& t) {
        g = (int)(((float)r + 0.5f) * inv_pl);
        const int rem = r - g * per_layer;
        h = (int)(((float)rem + 0.5f) * inv_tc);
        t = rem - h * tc;
      };
      for (int r0 = tid / 16; r0 < rows; r0 += U * RPS) {
        u32x4 kv[U], vv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int r = r0 + u * RPS;
          int g, h, t;
          split_row(r, g, h, t);
          if (r < rows) {
            const int64_t e = ((int64_t)(g * H + h) * len + t0 + t) * D + col;
            kv[u] = load16(ksrc + e * ES);
            vv[u] = load16(vsrc + e * ES);
          }
        }
        // The row's (layer, head, token) again for the stores, from an
        // opaque copy of the row index: kept from the loads, they would hold
        // 3 U registers across the wait (133 registers in all instead of 110).
        int r0s;
        asm volatile("v_mov_b32 %0, %1" : "=v"(r0s) : "v"(r0));
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int r = r0s + u * RPS;
          int gl_u, hh_u, tt_u;
          split_row(r, gl_u, hh_u, tt_u);
          if (r < rows) {   // uniform across each 16-lane row
            u32x4 other;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              other[q] = (unsigned)__builtin_amdgcn_mov_dpp((int)kv[u][q], 0x128, 0xF, 0xF, false);
            const float2* csr = cs + tt_u * HALF + fcol;
            u32x4 out;
            if constexpr (ES == 4) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const unsigned uo = kv[u][e], up = other[e];
                const float2 r2 = csr[e];
                out[e] = __float_as_uint(__builtin_fmaf(__uint_as_float(uo), r2.x,
                                                        __uint_as_float(up) * (sgn * r2.y)));
              }
            } else {
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const unsigned uo = kv[u][q], up = other[q];
                const float2 r0c = csr[2 * q], r1c = csr[2 * q + 1];
                const float y0 = __builtin_fmaf(__uint_as_float(uo << 16), r0c.x,
                                                __uint_as_float(up << 16) * (sgn * r0c.y));
                const float y1 = __builtin_fmaf(__uint_as_float(uo & 0xFFFF0000u), r1c.x,
                                                __uint_as_float(up & 0xFFFF0000u) * (sgn * r1c.y));
                out[q] = pack_bf16(y0, y1);
              }
            }
            const int64_t dst = (int64_t)(l0 + gl_u) * a.s_layer + slot_off[tt_u] +
                                (int64_t)hh_u * a.s_head + col;
            store16(kc + dst * ES, out);
            store16(vc + dst * ES, vv[u]);
          }
        }
      }
    }
    __syncthreads();
  }
}

template <int ES, int T, int U>
hipError_t launch_r16(const InjectLaunch& a, hipStream_t stream, size_t pad_lds) {
  const unsigned n_groups = (unsigned)((a.n_layers + a.layers_per_wg - 1) / a.layers_per_wg);
  // the item index is grid y: launch at most 65535 items at a time
  constexpr int32_t kMaxItems = IS_R16_LAYER_FAST ? 65535 : INT32_MAX;
  for (int32_t i0 = 0; i0 < a.n_items; i0 += kMaxItems) {
    InjectLaunch part = a;
    part.work = a.work + i0;
    part.n_items = a.n_items - i0 < kMaxItems ? a.n_items - i0 : kMaxItems;
    const dim3 grid16 = IS_R16_LAYER_FAST ? dim3(n_groups, (unsigned)part.n_items)
                                          : dim3((unsigned)part.n_items, n_groups);
    hipLaunchKernelGGL((inject_row16<ES, T, U, IS_R16_TC>), grid16, dim3(T), pad_lds, stream, part);
  }
  return hipGetLastError();
}

template <int ES>
hipError_t launch_es(const InjectLaunch& in, hipStream_t stream) {
  if (IS_R16 && in.lanes == 8) {
    // Workgroup shape from the mean fact length: rows of one layer of a
    // fact = kv_heads x length.  Long facts: one layer per 512-lane
    // workgroup (8 rows in flight per lane).  Short facts: enough layers per
    // 256-lane workgroup (4 rows in flight per lane) for about
    // IS_R16_SHORT_ROWS rows.
    InjectLaunch a = in;
    const float rows = (float)a.n_heads * (a.mean_len > 1.0f ? a.mean_len : 1.0f);
    const bool short_facts = rows < (float)IS_R16_SHORT_ROWS;
    int g = short_facts ? (int)((float)IS_R16_SHORT_ROWS / rows + 0.999f) : 1;
    if (IS_R16_FIXED_LAYERS > 0) g = IS_R16_FIXED_LAYERS;
    a.layers_per_wg = g < a.n_layers ? g : a.n_layers;
    // Long facts: one workgroup per CU.  With two (their registers allow
    // it), the Mistral-shaped batch measured 1.5% slower (more concurrent
    // DRAM streams against the memory system's mixed read/write limit) and
    // the Llama-3.1 Zipf batch, whose repeated facts hit the cache, 11%
    // faster; the batch the step is quoted on decides.
    return short_facts ? launch_r16<ES, IS_R16_SHORT_THREADS, IS_R16_SHORT_U>(a, stream, 0)
                       : launch_r16<ES, IS_R16_THREADS, IS_R16_ROWS>(a, stream, IS_R16_ONE_PER_CU);
  }
  const dim3 grid((unsigned)in.n_items, (unsigned)in.n_layers);
  switch (in.lanes) {
#define IS_CASE(L) \
    case L: hipLaunchKernelGGL((inject_kernel<ES, L>), grid, dim3(kThreads), 0, stream, in); break;
    IS_CASE(2) IS_CASE(4) IS_CASE(8) IS_CASE(16) IS_CASE(32)
#undef IS_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_inject(const InjectLaunch& a, hipStream_t stream) {
  if (a.n_items == 0) return hipSuccess;
  return a.dtype == IS_DTYPE_F32 ? launch_es<4>(a, stream) : launch_es<2>(a, stream);
}

}  // namespace is
