/* Seeded synthetic inputs: the counter-based generator core.
 *
 * This header holds no arithmetic of the decode method.  It defines how every
 * synthetic value (weights, KV-cache prefixes, start tokens) is derived from a
 * (seed, stream, index) triple, so that the host and the device produce the
 * same bytes.  It is included by the host generator (synth.c, built with gcc)
 * and by the device fill kernels (synth_dev.hip); SYNTH_FN selects the
 * function qualifiers.
 *
 * Generator: the SplitMix64 output function (Steele, Lea and Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014) applied to a Weyl
 * sequence, used counter-style: value i of a stream is mix(key + (i+1)*gamma).
 *
 * Normal variates in BF16: inverse-CDF sampling over the BF16 grid.  For a
 * normal N(0, sigma) rounded to the nearest BF16 value, the probability of each
 * non-negative BF16 magnitude is the normal mass of its rounding interval; the
 * host tabulates the cumulative masses as 63-bit fixed-point thresholds
 * (synth_table_build in synth.c).  One 64-bit hash gives the sign (bit 0) and a
 * 63-bit uniform (bits 1..63); the magnitude is the first table entry above the
 * uniform, found from a 2^16-entry guide table plus a short scan.  Only integer
 * compares run at sampling time, so host and device results are identical.
 * Positive BF16 bit patterns are ordered like their values, so the table index
 * is the BF16 bit pattern itself.
 */
#ifndef SYNTH_CORE_H
#define SYNTH_CORE_H

#include <stdint.h>

#ifndef SYNTH_FN
#define SYNTH_FN static inline
#endif

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ull
#define SYNTH_GUIDE_BITS 16
#define SYNTH_TABLE_MAX 0x7F81 /* positive finite BF16 patterns 0x0000..0x7F7F, plus one sentinel */

SYNTH_FN uint64_t synth_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* Key of one stream of a seed. */
SYNTH_FN uint64_t synth_key(uint64_t seed, uint64_t stream) {
  return synth_mix64(synth_mix64(seed + SYNTH_GAMMA) + (stream + 1) * 0xD1B54A32D192ED03ull);
}

/* 64 random bits: element `i` of the stream with key `key`. */
SYNTH_FN uint64_t synth_u64(uint64_t key, uint64_t i) { return synth_mix64(key + (i + 1) * SYNTH_GAMMA); }

/* BF16 bit pattern of a normal variate rounded to BF16, from 64 random bits.
 * thr: cumulative thresholds (thr[n-1] == 2^63); guide[j]: first k with thr[k] > j*2^47. */
SYNTH_FN uint16_t synth_bf16_from_bits(uint64_t r, const uint64_t* thr, const uint16_t* guide) {
  uint64_t u = r >> 1;
  uint32_t k = guide[u >> (63 - SYNTH_GUIDE_BITS)];
  while (u >= thr[k]) ++k;
  return (uint16_t)(k | ((uint32_t)(r & 1u) << 15));
}

/* Stream ids of the synthetic model's tensors (one stream per tensor kind and layer). */
enum {
  SYNTH_EMBED = 1,
  SYNTH_LM_HEAD = 2,
  SYNTH_WQ = 3,
  SYNTH_WK = 4,
  SYNTH_WV = 5,
  SYNTH_WO = 6,
  SYNTH_WROUTER = 7,
  SYNTH_WGATE = 8,
  SYNTH_WUP = 9,
  SYNTH_WDOWN = 10,
  SYNTH_NORM = 11  /* RMSNorm gains (layer index; n_layers = the final norm) */
};

SYNTH_FN uint64_t synth_weight_stream(int kind, int layer) { return ((uint64_t)kind << 32) | (uint32_t)layer; }

/* KV values are keyed by logical coordinates only (never by page placement):
 * stream = sequence id; index = (((layer * 2^20 + pos) * 2 + kv) * n_kv_heads + head) * d_head + dim. */
#define SYNTH_KV_POS_SPAN (1ull << 20)
SYNTH_FN uint64_t synth_kv_index(int layer, int64_t pos, int kv, int head, int dim, int n_kv_heads, int d_head) {
  return ((((uint64_t)layer * SYNTH_KV_POS_SPAN + (uint64_t)pos) * 2u + (uint64_t)kv) * (uint64_t)n_kv_heads + (uint64_t)head) *
             (uint64_t)d_head +
         (uint64_t)dim;
}

#endif
