/* Seeded synthetic inputs, host side (plain C, OpenMP).
 *
 * Shared by the CPU oracle's tests and by the GPU harness: it produces the
 * synthetic weights, KV-cache prefixes, start tokens, context lengths and page
 * orders of the workloads.  It holds no arithmetic of the decode method.  The
 * device fill kernels in synth_dev.hip use the same generator core
 * (synth_core.h) and the same tables, so both sides see identical bytes.
 */
#include "synth_core.h"
#include "../include/synth.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* Cumulative-mass thresholds of |X| for X ~ N(0, sigma) rounded to BF16.
 * Entry k is P(|X| < midpoint(v_k, v_{k+1})) * 2^63, v_k the BF16 value with bit
 * pattern k.  Masses use erf for small arguments and erfc for large ones so the
 * absolute error stays near 2^-53.  The last entry is 2^63 (a sentinel above
 * every 63-bit uniform). */
static double bf16_bits_to_double(uint32_t k) {
  uint32_t u = k << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

int synth_table_build(double sigma, uint64_t* thr, uint16_t* guide, int32_t* n_out) {
  if (!(sigma > 0) || !thr || !guide || !n_out) return -1;
  const double two63 = 9223372036854775808.0;
  const double inv = 1.0 / (sigma * sqrt(2.0));
  uint64_t prev = 0;
  int32_t n = 0;
  for (uint32_t k = 0; k < 0x7F7F; ++k) {
    double hi = 0.5 * (bf16_bits_to_double(k) + bf16_bits_to_double(k + 1)); /* exact in double */
    double z = hi * inv;
    uint64_t t;
    double e = erf(z);
    if (e < 0.5) {
      t = (uint64_t)llround(e * two63);
    } else {
      double c = erfc(z) * two63;
      t = c < 0.5 ? (uint64_t)1 << 63 : ((uint64_t)1 << 63) - (uint64_t)llround(c);
    }
    if (t < prev) t = prev; /* keep monotone across the erf/erfc switch */
    thr[k] = t;
    prev = t;
    n = (int32_t)k + 1;
    if (t >= ((uint64_t)1 << 63)) break;
  }
  if (n >= SYNTH_TABLE_MAX) return -2;
  thr[n - 1] = (uint64_t)1 << 63; /* sentinel: every 63-bit uniform is below it */
  /* guide[j] = first k with thr[k] > j * 2^47 */
  uint32_t k = 0;
  for (uint32_t j = 0; j < (1u << SYNTH_GUIDE_BITS); ++j) {
    uint64_t lo = (uint64_t)j << (63 - SYNTH_GUIDE_BITS);
    while (thr[k] <= lo) ++k;
    guide[j] = (uint16_t)k;
  }
  *n_out = n;
  return 0;
}

void synth_fill_bf16(uint16_t* dst, int64_t n, uint64_t seed, uint64_t stream, uint64_t index0, const uint64_t* thr,
                     const uint16_t* guide) {
  const uint64_t key = synth_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) dst[i] = synth_bf16_from_bits(synth_u64(key, index0 + (uint64_t)i), thr, guide);
}

int synth_fill_kv_paged(uint16_t* kv, int n_layers_buf, int layer0, int64_t n_pages, int n_kv_heads, int d_head, int page_size,
                        const int32_t* page_table, int64_t n_table, int seq_id, int64_t pos0, int64_t pos1, uint64_t seed,
                        const uint64_t* thr, const uint16_t* guide) {
  if (pos0 < 0 || pos1 < pos0 || page_size <= 0) return -1;
  if (pos1 > 0 && (pos1 - 1) / page_size >= n_table) return -1;
  for (int64_t p = pos0; p < pos1; ++p) {
    int32_t ph = page_table[p / page_size];
    if (ph < 0 || ph >= n_pages) return -2;
  }
  const uint64_t key = synth_key(seed, (uint64_t)seq_id);
  const int64_t rows = (int64_t)n_layers_buf * (pos1 - pos0) * 2 * n_kv_heads;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    int64_t t = r;
    int head = (int)(t % n_kv_heads);
    t /= n_kv_heads;
    int kvs = (int)(t % 2);
    t /= 2;
    int64_t pos = pos0 + t % (pos1 - pos0);
    int lb = (int)(t / (pos1 - pos0));
    int64_t ph = page_table[pos / page_size];
    uint16_t* row = kv + ((((int64_t)lb * n_pages + ph) * 2 + kvs) * n_kv_heads + head) * (int64_t)page_size * d_head +
                    (pos % page_size) * (int64_t)d_head;
    uint64_t i0 = synth_kv_index(layer0 + lb, pos, kvs, head, 0, n_kv_heads, d_head);
    for (int d = 0; d < d_head; ++d) row[d] = synth_bf16_from_bits(synth_u64(key, i0 + (uint64_t)d), thr, guide);
  }
  return 0;
}

void synth_splitmix64(uint64_t state, int64_t n, uint64_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = synth_mix64(state + (uint64_t)(i + 1) * SYNTH_GAMMA);
}

void synth_u64_fill(uint64_t seed, uint64_t stream, uint64_t index0, int64_t n, uint64_t* out) {
  const uint64_t key = synth_key(seed, stream);
  for (int64_t i = 0; i < n; ++i) out[i] = synth_u64(key, index0 + (uint64_t)i);
}

/* Uniform double in [0, 1) from the top 53 bits. */
static double u01(uint64_t r) { return (double)(r >> 11) * (1.0 / 9007199254740992.0); }

int32_t synth_token(uint64_t seed, int seq, int vocab) {
  uint64_t r = synth_u64(synth_key(seed, (uint64_t)seq), 0);
  return (int32_t)(r % (uint64_t)vocab);
}

void synth_loguniform_ints(uint64_t seed, uint64_t stream, int n, int64_t lo, int64_t hi, int64_t* out) {
  const uint64_t key = synth_key(seed, stream);
  const double a = log((double)lo), b = log((double)hi);
  for (int i = 0; i < n; ++i) {
    double v = floor(exp(a + (b - a) * u01(synth_u64(key, (uint64_t)i))));
    int64_t x = (int64_t)v;
    out[i] = x < lo ? lo : (x > hi ? hi : x);
  }
}

void synth_permutation(uint64_t seed, uint64_t stream, int n, int32_t* out) {
  const uint64_t key = synth_key(seed, stream);
  for (int i = 0; i < n; ++i) out[i] = i;
  for (int i = n - 1; i > 0; --i) { /* Fisher-Yates */
    int j = (int)(synth_u64(key, (uint64_t)i) % (uint64_t)(i + 1));
    int32_t t = out[i];
    out[i] = out[j];
    out[j] = t;
  }
}

void synth_skew_bias(uint64_t seed, int n_experts, double scale, float* out) {
  int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)n_experts);
  synth_permutation(seed, 0, n_experts, perm);
  for (int r = 1; r <= n_experts; ++r) out[perm[r - 1]] = (float)(-scale * log((double)r));
  free(perm);
}
