/*
 * Seeded synthetic-input generator: the arithmetic shared by the host (C) and
 * device (HIP) builds of the generator.  It holds none of the method's
 * arithmetic: it only produces the inputs (stored pre-RoPE keys and raw
 * values, embeddings, queries, fact lengths, fact ids, prefixes, block tables
 * and the cache sentinel) that both the library under test and the oracle
 * consume.
 *
 * The includer defines SYNTH_FN (for example `static inline` for C, or
 * `static inline __host__ __device__` for HIP) before including this file.
 *
 * Random bits come from Philox4x32-10, the counter-based generator of
 * J. K. Salmon, M. A. Moraes, R. O. Dror and D. E. Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC'11: ten rounds of two 32x32->64-bit
 * multiplications (multipliers 0xD2511F53 and 0xCD9E8D57) with a Weyl key
 * schedule (increments 0x9E3779B9 and 0xBB67AE85).
 *
 * Normal variates are Irwin-Hall sums of twelve 16-bit uniforms, centred.
 * The sum is an integer, so the variate (an integer times 2^-16) is exact in
 * float and double and every build reproduces it bit for bit.  Its mean is 0
 * and its variance 1 - 2^-32, its support [-6, 6].
 */
#ifndef SYNTH_CORE_H
#define SYNTH_CORE_H

#include <stdint.h>

#ifndef SYNTH_FN
#error "define SYNTH_FN before including synth_core.h"
#endif

/* Stream tags: one independent counter space per kind of input. */
#define SYNTH_TAG_K 1u
#define SYNTH_TAG_V 2u
#define SYNTH_TAG_EMB 3u
#define SYNTH_TAG_QUERY 4u
#define SYNTH_TAG_LEN 5u
#define SYNTH_TAG_ZIPF 6u
#define SYNTH_TAG_PREFIX 7u
#define SYNTH_TAG_PERM 8u
#define SYNTH_TAG_SENTINEL 9u

/* Storage codes (match the library's dtype enumeration). */
#define SYNTH_F32 0
#define SYNTH_BF16 1

SYNTH_FN void synth_philox_rounds(uint32_t c[4], uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)c[2];
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t n0 = hi1 ^ c[1] ^ k0;
    const uint32_t n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

/* Four random words for (seed, tag, entity, counter). */
SYNTH_FN void synth_words(uint32_t seed, uint32_t tag, uint32_t entity,
                          uint32_t counter, uint32_t out[4]) {
  out[0] = counter;
  out[1] = entity;
  out[2] = tag;
  out[3] = 0u;
  synth_philox_rounds(out, seed, 0x5EEDu);
}

/*
 * Numerator of the n-th normal variate of stream (seed, tag, entity): an
 * integer in [-393210, 393210]; the variate is numerator * 2^-16.  Uses the
 * first six words of the Philox blocks at counters 2n and 2n+1.
 */
SYNTH_FN int32_t synth_normal_num(uint32_t seed, uint32_t tag, uint32_t entity,
                                  uint32_t n) {
  uint32_t a[4], b[4];
  synth_words(seed, tag, entity, 2u * n, a);
  synth_words(seed, tag, entity, 2u * n + 1u, b);
  uint32_t s = 0;
  for (int i = 0; i < 4; ++i) s += (a[i] & 0xFFFFu) + (a[i] >> 16);
  for (int i = 0; i < 2; ++i) s += (b[i] & 0xFFFFu) + (b[i] >> 16);
  /* sum_j (u_j + 1/2) / 65536 - 6  ==  (s + 6 - 6*65536) / 65536 */
  return (int32_t)s - 393210;
}

/* float -> bf16 bits, round to nearest even (inputs here are finite). */
SYNTH_FN uint16_t synth_f32_to_bf16(float x) {
  union {
    float f;
    uint32_t u;
  } v;
  v.f = x;
  const uint32_t bias = 0x7FFFu + ((v.u >> 16) & 1u);
  return (uint16_t)((v.u + bias) >> 16);
}

/* murmur3's 32-bit finaliser (A. Appleby), used for the cache sentinel. */
SYNTH_FN uint32_t synth_fmix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85EBCA6Bu;
  h ^= h >> 13;
  h *= 0xC2B2AE35u;
  h ^= h >> 16;
  return h;
}

/* Sentinel word at 32-bit word index w of a buffer. */
SYNTH_FN uint32_t synth_sentinel_word(uint32_t seed, uint64_t w) {
  const uint32_t hi = synth_fmix32((uint32_t)(w >> 32) ^ (seed * 0x9E3779B9u) ^
                                   SYNTH_TAG_SENTINEL);
  return synth_fmix32((uint32_t)w ^ hi);
}

#endif /* SYNTH_CORE_H */
