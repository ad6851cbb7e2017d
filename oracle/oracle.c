/*
 * ORACLE -- test infrastructure only.  A plain, slow, fp64 CPU statement of
 * what the retrieve-and-inject path computes.  It is used by the tests, by
 * the smoke check and by the bench's CPU-baseline leg, and by nothing else;
 * it shares no code with the GPU library.
 *
 * Sources: "InferScale: GPU-Native KV Injection for Personalized LLM
 * Serving" (gist.science explainer pages, technical summary):
 *   - Online phase, "Pre-RoPE storage": keys are captured before RoPE and
 *     stored together with the raw values;
 *   - Online phase, "Dynamic rotation": the retrieved facts are composed into
 *     one contiguous segment and each stored key receives the RoPE rotation
 *     of its new serving position (Theorem 6: exact under RoPE);
 *   - Online phase, "Injection": the composed K/V are scatter-copied into the
 *     paged KV cache;
 *   - Contributions, "GPU-native system design": retrieval over a
 *     GPU-resident index picks the facts (here: exact inner-product top-k);
 *   - Offline phase, context-window encoding: a fact is encoded behind a
 *     window of preceding tokens and only its own tokens are stored
 *     (or_ingest);
 *   - Online phase, query-only prefill: the engine then runs attention of
 *     the query over the cache holding the injected facts (here: synthetic
 *     queries, softmax attention with grouped kv heads, or_attend).
 * The pages give no formulas.  Readings taken here, where the pages are
 * silent: textbook RoPE (Su et al., RoFormer) with frequencies
 * theta^(-2i/d) and rotate-half pairing (i, i + d/2); the published
 * Llama-3.1 frequency-scaling rule; facts laid out back to back in the
 * caller's order starting right after the request's prefix; the rotation
 * uses the logical position, never the slot; one rounding fp64 -> cache
 * dtype; top-k ordered by score descending with ties to the lower id.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define EXPORT __attribute__((visibility("default")))

static const double OR_PI = 3.14159265358979323846;

enum { OR_F32 = 0, OR_BF16 = 1 };
enum { OR_SCALING_NONE = 0, OR_SCALING_LLAMA3 = 1 };

/* ---------------------------------------------------------------- numbers */

/* Exact value of an IEEE binary16 bit pattern. */
EXPORT double or_half_to_double(uint16_t h) {
  const int sign = h >> 15;
  const int e = (h >> 10) & 0x1F;
  const int m = h & 0x3FF;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
  return sign ? -v : v;
}

/* fp64 -> bf16 bits, one rounding to nearest, ties to even.  bf16 keeps 8
 * significant bits with fp32's exponent range (normal exponents -126..127,
 * subnormal quantum 2^-133). */
EXPORT uint16_t or_double_to_bf16(double x) {
  uint16_t sign = 0;
  if (signbit(x)) {
    sign = 0x8000;
    x = -x;
  }
  if (isnan(x)) return (uint16_t)(sign | 0x7FC0);
  if (x == 0.0) return sign;
  int e;
  (void)frexp(x, &e);
  int ex = e - 1; /* x in [2^ex, 2^(ex+1)) */
  if (ex < -126) ex = -126;
  const double quantum = ldexp(1.0, ex - 7);
  const double r = nearbyint(x / quantum) * quantum; /* ties to even */
  if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);
  float f = (float)r; /* exact: 8 significant bits in fp32's range */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(sign | (u >> 16));
}

/* ------------------------------------------------------------ frequencies */

/* Llama-3.1 rule for one frequency f (radians per position): wavelengths
 * shorter than orig/high are kept, longer than orig/low are divided by
 * `factor`, and in between the two are blended linearly in orig/wavelength. */
EXPORT double or_llama3_scale(double f, double factor, double low, double high,
                              double orig) {
  const double wavelen = 2.0 * OR_PI / f;
  if (wavelen < orig / high) return f;
  if (wavelen > orig / low) return f / factor;
  const double smooth = (orig / wavelen - low) / (high - low);
  return (1.0 - smooth) * f / factor + smooth * f;
}

/* f[i] = theta^(-2i/d), i < d/2, optionally Llama-3.1-scaled. */
EXPORT void or_rope_freqs(int d, double theta, int scaling, double factor,
                          double low, double high, double orig, double* f) {
  for (int i = 0; i < d / 2; ++i) {
    f[i] = pow(theta, -2.0 * i / d);
    if (scaling == OR_SCALING_LLAMA3)
      f[i] = or_llama3_scale(f[i], factor, low, high, orig);
  }
}

/* ---------------------------------------------------------------- RoPE */

/* Rotate-half RoPE of a d-vector x at position p: each pair (x[i], x[i+d/2])
 * turns by the angle p * f[i]. */
EXPORT void or_rotate(const double* x, int d, double p, const double* f,
                      double* y) {
  const int h = d / 2;
  for (int i = 0; i < h; ++i) {
    const double c = cos(p * f[i]), s = sin(p * f[i]);
    y[i] = x[i] * c - x[i + h] * s;
    y[i + h] = x[i + h] * c + x[i] * s;
  }
}

/* ------------------------------------------------------------------ top-k */

typedef struct {
  double s;
  int32_t id;
} scored;

static int by_score_then_id(const void* a, const void* b) {
  const scored* x = (const scored*)a;
  const scored* y = (const scored*)b;
  if (x->s != y->s) return x->s > y->s ? -1 : 1;
  return (x->id > y->id) - (x->id < y->id);
}

/* For each query q: the k facts with the largest inner product
 * <Q[q], E[f]>, computed exactly in fp64 from the fp16 values, in order of
 * score descending, ties to the lower id.  q: [n_q][dim] fp16 bits,
 * e: [n_facts][dim] fp16 bits; ids: [n_q][k]; scores: [n_q][k]. */
EXPORT int or_topk(const uint16_t* q, const uint16_t* e, int64_t n_q,
                   int64_t n_facts, int64_t dim, int k, int32_t* ids,
                   double* scores) {
  if (k < 1 || k > n_facts) return -1;
  double* lut = (double*)malloc(sizeof(double) * 65536);
  for (int i = 0; i < 65536; ++i) lut[i] = or_half_to_double((uint16_t)i);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t qi = 0; qi < n_q; ++qi) {
    scored* all = (scored*)malloc(sizeof(scored) * (size_t)n_facts);
    const uint16_t* qrow = q + (size_t)qi * dim;
    for (int64_t f = 0; f < n_facts; ++f) {
      const uint16_t* erow = e + (size_t)f * dim;
      double s = 0.0;
      for (int64_t i = 0; i < dim; ++i) s += lut[qrow[i]] * lut[erow[i]];
      all[f].s = s;
      all[f].id = (int32_t)f;
    }
    qsort(all, (size_t)n_facts, sizeof(scored), by_score_then_id);
    for (int j = 0; j < k; ++j) {
      ids[qi * k + j] = all[j].id;
      scores[qi * k + j] = all[j].s;
    }
    free(all);
  }
  free(lut);
  return 0;
}

/* ------------------------------------------------------------ composition */

/* Serving position of the first token of each selected fact: request r's
 * facts (fact_ids[req_off[r] .. req_off[r+1])) sit back to back in the given
 * order, the first one right after the request's prefix. */
EXPORT void or_positions(int n_req, const int32_t* req_off,
                         const int32_t* fact_ids, const int32_t* fact_len,
                         const int32_t* prefix_len, int64_t* start) {
  for (int r = 0; r < n_req; ++r) {
    int64_t pos = prefix_len[r];
    for (int32_t j = req_off[r]; j < req_off[r + 1]; ++j) {
      start[j] = pos;
      pos += fact_len[fact_ids[j]];
    }
  }
}

/* Cache slot of every injected token, request by request, fact by fact
 * (segment order), token by token: slot = block_table[r][p / block_size] *
 * block_size + p % block_size for serving position p.  Returns the number of
 * tokens, or -1 if a block-table lookup falls outside [0, max_blocks). */
EXPORT int64_t or_token_slots(int n_req, const int32_t* req_off,
                              const int32_t* fact_ids, const int32_t* fact_len,
                              const int32_t* prefix_len,
                              const int32_t* block_tables, int max_blocks,
                              int block_size, int64_t* slots) {
  int64_t n = 0;
  for (int r = 0; r < n_req; ++r) {
    int64_t p = prefix_len[r];
    for (int32_t j = req_off[r]; j < req_off[r + 1]; ++j)
      for (int32_t t = 0; t < fact_len[fact_ids[j]]; ++t, ++p) {
        if (p / block_size >= max_blocks) return -1;
        slots[n++] = (int64_t)block_tables[(int64_t)r * max_blocks + p / block_size] *
                         block_size + p % block_size;
      }
  }
  return n;
}

/* Exact inner product of two fp16 rows, in fp64. */
EXPORT double or_dot(const uint16_t* a, const uint16_t* b, int64_t dim) {
  double s = 0.0;
  for (int64_t i = 0; i < dim; ++i) s += or_half_to_double(a[i]) * or_half_to_double(b[i]);
  return s;
}

/* ----------------------------------------------------------------- inject */

static double load_elem(const void* base, int64_t i, int dtype) {
  if (dtype == OR_F32) return (double)((const float*)base)[i];
  uint32_t u = (uint32_t)((const uint16_t*)base)[i] << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static void store_elem(void* base, int64_t i, int dtype, double v) {
  if (dtype == OR_F32)
    ((float*)base)[i] = (float)v; /* one rounding, to nearest even */
  else
    ((uint16_t*)base)[i] = or_double_to_bf16(v);
}

static void copy_elem(void* dst, int64_t di, const void* src, int64_t si,
                      int dtype) {
  if (dtype == OR_F32)
    ((uint32_t*)dst)[di] = ((const uint32_t*)src)[si];
  else
    ((uint16_t*)dst)[di] = ((const uint16_t*)src)[si];
}

/*
 * Retrieve-and-inject for a batch of requests, written into a host cache.
 *
 * Store (host): k_store / v_store hold every fact's [layer][kv_head][token]
 * [head_dim] block back to back in id order; fact f's tokens are
 * [tok_off[f], tok_off[f+1]) of that sequence.
 * Cache (host): element (layer l, block b, slot s, head h, dim i) of the K
 * cache is k_cache[l*s_layer + b*s_block + s*s_slot + h*s_head + i]; same
 * for V.  Block tables: [n_req][max_blocks].
 * For each request r, fact j (order given), token t at serving position p:
 * slot = block_table[r][p / block_size] * block_size + p % block_size; the
 * stored key row is rotated to position p and written to the slot, the
 * stored value row is copied unchanged.  Nothing else is written.
 * Returns 0, or -1 on an index out of range (nothing is checked beyond what
 * keeps this function inside its buffers).
 */
EXPORT int or_inject(int n_layers, int n_heads, int d, int dtype,
                     const void* k_store, const void* v_store,
                     const int64_t* tok_off, int64_t n_facts, int n_req,
                     const int32_t* req_off, const int32_t* fact_ids,
                     const int32_t* prefix_len, const int32_t* block_tables,
                     int max_blocks, int block_size, int64_t n_blocks,
                     void* k_cache, void* v_cache, int64_t s_layer,
                     int64_t s_block, int64_t s_slot, int64_t s_head,
                     const double* freqs) {
  int32_t* len = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n_facts > 0 ? n_facts : 1));
  for (int64_t f = 0; f < n_facts; ++f) len[f] = (int32_t)(tok_off[f + 1] - tok_off[f]);
  const int32_t n_pairs = req_off[n_req];
  int64_t* start = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_pairs > 0 ? n_pairs : 1));
  int bad = 0;
  for (int32_t j = 0; j < n_pairs; ++j)
    if (fact_ids[j] < 0 || fact_ids[j] >= n_facts) bad = 1;
  if (!bad) or_positions(n_req, req_off, fact_ids, len, prefix_len, start);
  for (int r = 0; r < n_req && !bad; ++r)
    for (int32_t j = req_off[r]; j < req_off[r + 1]; ++j) {
      const int64_t last = start[j] + len[fact_ids[j]] - 1;
      if (last / block_size >= max_blocks) bad = 1;
    }
  if (bad) {
    free(len);
    free(start);
    return -1;
  }
  const int64_t row = (int64_t)d;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int r = 0; r < n_req; ++r) {
    double* x = (double*)malloc(sizeof(double) * (size_t)d);
    double* y = (double*)malloc(sizeof(double) * (size_t)d);
    for (int32_t j = req_off[r]; j < req_off[r + 1]; ++j) {
      const int32_t f = fact_ids[j];
      const int64_t n_tok = len[f];
      const int64_t fact_base = tok_off[f] * (int64_t)n_layers * n_heads * d;
      for (int64_t t = 0; t < n_tok; ++t) {
        const int64_t p = start[j] + t;
        const int32_t blk = block_tables[(int64_t)r * max_blocks + p / block_size];
        if (blk < 0 || blk >= n_blocks) {
          bad = 1;
          continue;
        }
        const int64_t in_blk = p % block_size;
        for (int l = 0; l < n_layers; ++l)
          for (int h = 0; h < n_heads; ++h) {
            const int64_t src =
                fact_base + (((int64_t)l * n_heads + h) * n_tok + t) * row;
            const int64_t dst =
                l * s_layer + blk * s_block + in_blk * s_slot + h * s_head;
            for (int i = 0; i < d; ++i) x[i] = load_elem(k_store, src + i, dtype);
            or_rotate(x, d, (double)p, freqs, y);
            for (int i = 0; i < d; ++i) {
              store_elem(k_cache, dst + i, dtype, y[i]);
              copy_elem(v_cache, dst + i, v_store, src + i, dtype);
            }
          }
      }
    }
    free(x);
    free(y);
  }
  free(len);
  free(start);
  return bad ? -1 : 0;
}

/* -------------------------------------------------------------- attention */

/*
 * Query-only attention over a paged host cache: the step that follows the
 * injection, when the engine prefills only the query over a cache that
 * already holds the injected facts (Online phase; Theorem 6 says the scores
 * equal those of a cache prefilled at the same positions).  For layer l,
 * request r, query token t at position qpos[r] + t and query head hq, whose
 * kv head is hq / g (g = n_q_heads / n_kv_heads):
 *   s_p = <R(qpos[r] + t) q, K_l[slot_r(p)][hq / g]> / sqrt(d),
 *         p in [cb[r], ce[r]),  slot_r(p) = bt[r][p / B] * B + p mod B
 *   out = sum_p softmax(s)_p V_l[slot_r(p)][hq / g]
 * q: [n_layers][n_req][n_qtok][n_q_heads][d] in `dtype`, before RoPE; it is
 * rotated here in fp64.  out: fp64, same shape.  An empty context gives
 * zeros.  Returns -1 if a position's block lies outside the table or the
 * cache (nothing is written for that row), else 0.
 */
EXPORT int or_attend(int n_layers, int n_kv_heads, int n_q_heads, int d, int dtype,
                     const void* q, int n_req, int n_qtok, const int32_t* qpos,
                     const int32_t* cb, const int32_t* ce, const int32_t* block_tables,
                     int max_blocks, int block_size, int64_t n_blocks, const void* k_cache,
                     const void* v_cache, int64_t s_layer, int64_t s_block, int64_t s_slot,
                     int64_t s_head, const double* f, double* out) {
  const int g = n_q_heads / n_kv_heads;
  const double scale = 1.0 / sqrt((double)d);
  int bad = 0;
#pragma omp parallel for collapse(2) schedule(dynamic) reduction(| : bad)
  for (int l = 0; l < n_layers; ++l)
    for (int r = 0; r < n_req; ++r) {
      const int64_t n_ctx = ce[r] > cb[r] ? (int64_t)ce[r] - cb[r] : 0;
      double* x = (double*)malloc(sizeof(double) * (size_t)d);
      double* qr = (double*)malloc(sizeof(double) * (size_t)d);
      double* s = (double*)malloc(sizeof(double) * (size_t)(n_ctx > 0 ? n_ctx : 1));
      int64_t* row = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_ctx > 0 ? n_ctx : 1));
      /* element offset of each context position's slot (head 0) */
      for (int64_t j = 0; j < n_ctx; ++j) {
        const int64_t p = cb[r] + j;
        const int64_t bi = p / block_size;
        const int32_t blk = bi < max_blocks ? block_tables[(int64_t)r * max_blocks + bi] : -1;
        if (blk < 0 || blk >= n_blocks) {
          bad = 1;
          row[j] = -1;
          continue;
        }
        row[j] = l * s_layer + blk * s_block + (p % block_size) * s_slot;
      }
      for (int t = 0; t < n_qtok; ++t)
        for (int hq = 0; hq < n_q_heads; ++hq) {
          const int64_t qi = ((((int64_t)l * n_req + r) * n_qtok + t) * n_q_heads + hq) * d;
          const int64_t kvh = hq / g;
          for (int i = 0; i < d; ++i) x[i] = load_elem(q, qi + i, dtype);
          or_rotate(x, d, (double)qpos[r] + t, f, qr);
          double mx = -INFINITY;
          for (int64_t j = 0; j < n_ctx; ++j) {
            if (row[j] < 0) continue;
            double acc = 0.0;
            const int64_t kb = row[j] + kvh * s_head;
            for (int i = 0; i < d; ++i) acc += qr[i] * load_elem(k_cache, kb + i, dtype);
            s[j] = acc * scale;
            if (s[j] > mx) mx = s[j];
          }
          double sum = 0.0;
          for (int64_t j = 0; j < n_ctx; ++j) {
            if (row[j] < 0) continue;
            s[j] = exp(s[j] - mx);
            sum += s[j];
          }
          for (int i = 0; i < d; ++i) out[qi + i] = 0.0;
          for (int64_t j = 0; j < n_ctx; ++j) {
            if (row[j] < 0) continue;
            const int64_t vb = row[j] + kvh * s_head;
            for (int i = 0; i < d; ++i) out[qi + i] += s[j] / sum * load_elem(v_cache, vb + i, dtype);
          }
        }
      free(x);
      free(qr);
      free(s);
      free(row);
    }
  return bad ? -1 : 0;
}

/* ----------------------------------------------------------------- ingest */

/*
 * Packing of context-window-encoded facts into the store layout (Offline
 * phase: each fact is encoded behind a window of w preceding tokens, and
 * only the fact's own tokens' pre-RoPE keys and values are kept).  Input:
 * the n facts' encodings back to back, fact i as [layer][kv_head][w +
 * len[i]][d]; output: the facts' store blocks back to back, fact i as
 * [layer][kv_head][len[i]][d] -- the token rows w .. w + len[i] - 1 of each
 * (layer, kv_head), bit for bit.  Elements of `es` bytes.
 */
EXPORT void or_ingest(int n_layers, int n_heads, int d, int es, int n, const int32_t* len,
                      int w, const void* enc, void* out) {
  const char* src = (const char*)enc;
  char* dst = (char*)out;
  for (int i = 0; i < n; ++i) {
    for (int l = 0; l < n_layers; ++l)
      for (int h = 0; h < n_heads; ++h)
        for (int t = 0; t < len[i]; ++t) {
          const int64_t s_row = ((int64_t)(l * n_heads + h) * (w + len[i]) + w + t) * d;
          const int64_t d_row = ((int64_t)(l * n_heads + h) * len[i] + t) * d;
          memcpy(dst + d_row * es, src + s_row * es, (size_t)d * es);
        }
    src += (int64_t)n_layers * n_heads * (w + len[i]) * d * es;
    dst += (int64_t)n_layers * n_heads * len[i] * d * es;
  }
}

/* Thread count of the parallel loops above (test infrastructure: the bench
 * times the oracle on all host cores and on one). */
EXPORT void or_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
EXPORT int or_max_threads(void) { return omp_get_max_threads(); }
