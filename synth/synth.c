/*
 * Seeded synthetic-input generator, host build.  Produces every input that
 * the library under test and the oracle both consume; holds none of the
 * method's arithmetic.  Exported with C linkage for ctypes.
 *
 * Input recipe (one stream per tag, all keyed by the seed):
 *   K, V        element n of fact f: normal variate (Irwin-Hall(12)) of
 *               stream (K|V, f), index n over the fact's
 *               [layer][kv_head][token][head_dim] block, stored exactly in
 *               fp32 or rounded to nearest even in bf16;
 *   embeddings  row f: normal variates of stream (EMB, f), L2-normalised in
 *               fp64, rounded to nearest even in fp16;
 *   queries     row q: normal variates of stream (QUERY, q), rounded to fp16;
 *   lengths     uniform integers, or a clipped lognormal;
 *   fact ids    Zipf(s) without replacement, in draw order;
 *   prefixes    uniform integers;
 *   blocks      a Fisher-Yates permutation of the physical blocks handed out
 *               in request order, so block tables never overlap.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SYNTH_FN static inline
#include "synth_core.h"

#define EXPORT __attribute__((visibility("default")))

EXPORT void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2],
                                uint32_t out[4]) {
  for (int i = 0; i < 4; ++i) out[i] = ctr[i];
  synth_philox_rounds(out, key[0], key[1]);
}

EXPORT int32_t synth_normal_numerator(uint32_t seed, uint32_t tag,
                                      uint32_t entity, uint32_t n) {
  return synth_normal_num(seed, tag, entity, n);
}

/* n elements of fact `fact`'s K (tag 1) or V (tag 2) block, element index
 * starting at `first`. */
EXPORT void synth_fact_kv(uint32_t seed, uint32_t tag, int64_t fact,
                          int64_t first, int64_t n, int dtype, void* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const int32_t num =
        synth_normal_num(seed, tag, (uint32_t)fact, (uint32_t)(first + i));
    const float x = (float)num * (1.0f / 65536.0f);
    if (dtype == SYNTH_F32)
      ((float*)out)[i] = x;
    else
      ((uint16_t*)out)[i] = synth_f32_to_bf16(x);
  }
}

/* K or V of facts [first_fact, first_fact + n_facts), packed back to back;
 * elem_off[j] (relative, n_facts + 1 entries) is where fact first_fact + j
 * starts in `out`. */
EXPORT void synth_kv_range(uint32_t seed, uint32_t tag, int64_t first_fact,
                           int64_t n_facts, const int64_t* elem_off, int dtype,
                           void* out) {
  const size_t es = dtype == SYNTH_F32 ? 4 : 2;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t j = 0; j < n_facts; ++j) {
    const int64_t n = elem_off[j + 1] - elem_off[j];
    char* dst = (char*)out + (size_t)elem_off[j] * es;
    for (int64_t i = 0; i < n; ++i) {
      const int32_t num = synth_normal_num(seed, tag, (uint32_t)(first_fact + j),
                                           (uint32_t)i);
      const float x = (float)num * (1.0f / 65536.0f);
      if (dtype == SYNTH_F32)
        ((float*)dst)[i] = x;
      else
        ((uint16_t*)dst)[i] = synth_f32_to_bf16(x);
    }
  }
}

/* double -> IEEE binary16 bits, round to nearest even, with subnormals,
 * overflow to infinity. */
EXPORT uint16_t synth_double_to_f16(double x) {
  uint16_t sign = 0;
  if (signbit(x)) {
    sign = 0x8000;
    x = -x;
  }
  if (isnan(x)) return (uint16_t)(sign | 0x7E00);
  if (x == 0.0) return sign;
  int e;
  (void)frexp(x, &e); /* x = m * 2^e, m in [0.5, 1) */
  int exp_unb = e - 1; /* x in [2^exp_unb, 2^(exp_unb+1)) */
  if (exp_unb < -14) exp_unb = -14; /* subnormal range: quantum 2^-24 */
  const double quantum = ldexp(1.0, exp_unb - 10);
  double q = nearbyint(x / quantum); /* x/quantum exact: power-of-two scale */
  double r = q * quantum;
  if (r >= 65520.0 || r > 65504.0) return (uint16_t)(sign | 0x7C00);
  /* encode r */
  if (r < ldexp(1.0, -14)) {
    return (uint16_t)(sign | (uint16_t)(r / ldexp(1.0, -24)));
  }
  int e2;
  double m = frexp(r, &e2); /* r = m 2^e2 */
  const int biased = e2 - 1 + 15;
  const uint16_t frac = (uint16_t)((m * 2.0 - 1.0) * 1024.0);
  return (uint16_t)(sign | (uint16_t)(biased << 10) | frac);
}

/* Fact embeddings: rows [first, first + n) of dim `dim`, L2-normalised. */
EXPORT void synth_embeddings(uint32_t seed, int64_t first, int64_t n, int dim,
                             uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    double* x = (double*)malloc(sizeof(double) * (size_t)dim);
    double ss = 0.0;
    for (int i = 0; i < dim; ++i) {
      x[i] = (double)synth_normal_num(seed, SYNTH_TAG_EMB, (uint32_t)(first + r),
                                      (uint32_t)i) /
             65536.0;
      ss += x[i] * x[i];
    }
    const double inv = 1.0 / sqrt(ss);
    for (int i = 0; i < dim; ++i)
      out[(size_t)r * dim + i] = synth_double_to_f16(x[i] * inv);
    free(x);
  }
}

/* Query embeddings, not normalised. */
EXPORT void synth_queries(uint32_t seed, int64_t n, int dim, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r)
    for (int i = 0; i < dim; ++i)
      out[(size_t)r * dim + i] = synth_double_to_f16(
          (double)synth_normal_num(seed, SYNTH_TAG_QUERY, (uint32_t)r,
                                   (uint32_t)i) /
          65536.0);
}

static uint64_t word64(uint32_t seed, uint32_t tag, uint32_t entity,
                       uint32_t counter) {
  uint32_t w[4];
  synth_words(seed, tag, entity, counter, w);
  return ((uint64_t)w[1] << 32) | w[0];
}

/* Uniform double in [0, 1) with 53 random bits. */
static double uniform53(uint32_t seed, uint32_t tag, uint32_t entity,
                        uint32_t counter) {
  return (double)(word64(seed, tag, entity, counter) >> 11) *
         (1.0 / 9007199254740992.0);
}

/* Fact lengths uniform on [lo, hi]. */
EXPORT void synth_len_uniform(uint32_t seed, int64_t n, int lo, int hi,
                              int32_t* out) {
  const uint64_t span = (uint64_t)(hi - lo + 1);
  for (int64_t f = 0; f < n; ++f)
    out[f] = lo + (int32_t)(word64(seed, SYNTH_TAG_LEN, (uint32_t)f, 0) % span);
}

/* Fact lengths round(median * exp(sigma * z)), z normal, clipped to
 * [lo, hi]. */
EXPORT void synth_len_lognormal(uint32_t seed, int64_t n, double median,
                                double sigma, int lo, int hi, int32_t* out) {
  for (int64_t f = 0; f < n; ++f) {
    const double z =
        (double)synth_normal_num(seed, SYNTH_TAG_LEN, (uint32_t)f, 0) / 65536.0;
    double len = nearbyint(median * exp(sigma * z));
    if (len < lo) len = lo;
    if (len > hi) len = hi;
    out[f] = (int32_t)len;
  }
}

static int cmp_double(const void* a, const void* b) {
  const double x = *(const double*)a, y = *(const double*)b;
  return (x > y) - (x < y);
}

/* k distinct ids per request, Zipf(s) over [0, n_ids) with
 * P(id = i) proportional to (i + 1)^-s, repeats rejected, in draw order.
 * out is [n_req][k].  Returns 0, or -1 if k > n_ids. */
EXPORT int synth_zipf_requests(uint32_t seed, int n_req, int k, int64_t n_ids,
                               double s, int32_t* out) {
  if (k > n_ids) return -1;
  double* cdf = (double*)malloc(sizeof(double) * (size_t)n_ids);
  double acc = 0.0;
  for (int64_t i = 0; i < n_ids; ++i) {
    acc += pow((double)(i + 1), -s);
    cdf[i] = acc;
  }
  (void)cmp_double;
  for (int r = 0; r < n_req; ++r) {
    int32_t* row = out + (size_t)r * k;
    int have = 0;
    uint32_t draw = 0;
    while (have < k) {
      const double u = uniform53(seed, SYNTH_TAG_ZIPF, (uint32_t)r, draw++) * acc;
      int64_t lo = 0, hi = n_ids - 1; /* first i with cdf[i] > u */
      while (lo < hi) {
        const int64_t mid = (lo + hi) / 2;
        if (cdf[mid] > u)
          hi = mid;
        else
          lo = mid + 1;
      }
      int dup = 0;
      for (int j = 0; j < have; ++j) dup |= row[j] == (int32_t)lo;
      if (!dup) row[have++] = (int32_t)lo;
    }
  }
  free(cdf);
  return 0;
}

/* Prefix lengths uniform on [lo, hi]. */
EXPORT void synth_prefix(uint32_t seed, int n_req, int lo, int hi,
                         int32_t* out) {
  const uint64_t span = (uint64_t)(hi - lo + 1);
  for (int r = 0; r < n_req; ++r)
    out[r] =
        lo + (int32_t)(word64(seed, SYNTH_TAG_PREFIX, (uint32_t)r, 0) % span);
}

/* Random permutation of [0, n) (Fisher-Yates, from the top). */
EXPORT void synth_permutation(uint32_t seed, int64_t n, int32_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (int32_t)i;
  for (int64_t i = n - 1; i > 0; --i) {
    const int64_t j = (int64_t)(word64(seed, SYNTH_TAG_PERM, (uint32_t)(i >> 32),
                                       (uint32_t)i) %
                                (uint64_t)(i + 1));
    const int32_t t = out[i];
    out[i] = out[j];
    out[j] = t;
  }
}

/* Non-overlapping block tables: request r needs ceil(need[r] / block_size)
 * blocks, taken in order from a random permutation of the n_blocks physical
 * blocks.  out is [n_req][max_blocks], unused entries -1.  Returns 0, -1 if
 * a row would exceed max_blocks, -2 if the blocks run out. */
EXPORT int synth_block_tables(uint32_t seed, int n_req, const int64_t* need,
                              int block_size, int64_t n_blocks, int max_blocks,
                              int32_t* out) {
  int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)n_blocks);
  synth_permutation(seed, n_blocks, perm);
  int64_t cursor = 0;
  int rc = 0;
  for (int r = 0; r < n_req && rc == 0; ++r) {
    const int64_t nb = (need[r] + block_size - 1) / block_size;
    if (nb > max_blocks) {
      rc = -1;
      break;
    }
    if (cursor + nb > n_blocks) {
      rc = -2;
      break;
    }
    for (int j = 0; j < max_blocks; ++j)
      out[(size_t)r * max_blocks + j] = j < nb ? perm[cursor + j] : -1;
    cursor += nb;
  }
  free(perm);
  return rc;
}

/* Sentinel words [first_word, first_word + n). */
EXPORT void synth_sentinel_host(uint32_t seed, uint64_t first_word, int64_t n,
                                uint32_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = synth_sentinel_word(seed, first_word + (uint64_t)i);
}
