/* CPU oracle of one decode step (plain C, OpenMP).  TEST INFRASTRUCTURE ONLY:
 * only the tests, the smoke entry point and the benchmark's CPU-baseline leg
 * may load it.  It shares no code with the GPU path.  See oracle.h for what
 * each function computes and the passages it follows.
 *
 * Sources (page title, section):
 *  [AC] agenticcommons.xyz, "Cohere North Mini Code megakernel serving engine":
 *       section 為什麼 decode 慢 (BF16 MoE decode, weights + KV read per step);
 *       section 三個實際的加速來源, item 1 (parallel layer: attention and MoE read
 *       one normalised input, joined by residual add + RMSNorm), item 2 (KV
 *       groups; per-expert up then down projection), item 3 (router and QKV
 *       projections read the normalised input).
 *  [AM] aimodeling.com, "Cohere megakernel engine: one CUDA file, 1.58x vLLM on
 *       H100": section "From demo to a full serving system" (paged attention,
 *       ragged lengths, continuous batching).
 * Readings where the pages are silent: RMSNorm gains are data (unit in the
 * synthetic model), rotate-half RoPE with angle pos*base^(-2i/dh) in fp64,
 * scale 1/sqrt(dh), contiguous GQA groups, K/V stored after RoPE and rounded to
 * BF16 before the token attends to itself, softmax over the k selected router
 * logits, ties to the lower index, SwiGLU experts without biases, no
 * embedding or logit scaling.
 *
 * parity pins: every function here is checked in tests/test_oracle_*.py against
 * closed forms, library routines or brute force; the whole-step composition is
 * pinned only through its parts and the layer-algebra identity.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

float or_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

uint16_t or_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40); /* quiet NaN */
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb; /* round to nearest, ties to even */
  return (uint16_t)(u >> 16);
}

void or_matvec(const uint16_t* W, int64_t rows, int64_t cols, const float* x, float* y) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const uint16_t* w = W + r * cols;
    double acc = 0.0;
    for (int64_t c = 0; c < cols; ++c) acc += (double)or_bf16_to_f32(w[c]) * (double)x[c];
    y[r] = (float)acc;
  }
}

void or_rmsnorm(const float* x, const uint16_t* gamma, int d, double eps, float* out) {
  double ss = 0.0;
  for (int i = 0; i < d; ++i) ss += (double)x[i] * (double)x[i];
  const double inv = 1.0 / sqrt(ss / d + eps);
  for (int i = 0; i < d; ++i) out[i] = (float)((double)x[i] * (double)or_bf16_to_f32(gamma[i]) * inv);
}

void or_rope(float* v, int n_heads, int d_head, int64_t pos, double base) {
  const int half = d_head / 2;
  for (int i = 0; i < half; ++i) {
    const double theta = (double)pos * pow(base, -2.0 * i / d_head);
    const double c = cos(theta), s = sin(theta);
    for (int h = 0; h < n_heads; ++h) {
      float* a = v + (int64_t)h * d_head;
      const double x0 = a[i], x1 = a[i + half];
      a[i] = (float)(x0 * c - x1 * s);
      a[i + half] = (float)(x0 * s + x1 * c);
    }
  }
}

/* Address of the K (kv=0) or V (kv=1) row of KV head g at logical position j. */
static const uint16_t* kv_row(const or_dims* D, const uint16_t* kv_layer, const int32_t* page_table, int64_t j, int kv, int g) {
  const int64_t ph = page_table[j / D->page_size];
  return kv_layer + (((ph * 2 + kv) * D->n_kv_heads + g) * (int64_t)D->page_size + j % D->page_size) * D->d_head;
}

int or_attention(const or_dims* D, const float* q, const uint16_t* kv_layer, int64_t n_pages, const int32_t* page_table,
                 int64_t n_table, int64_t n_ctx, float* out) {
  if (!D || !q || !kv_layer || !page_table || !out || n_ctx < 1) return -1;
  if ((n_ctx - 1) / D->page_size >= n_table) return -1;
  for (int64_t p = 0; p * D->page_size < n_ctx; ++p)
    if (page_table[p] < 0 || page_table[p] >= n_pages) return -2;
  const int dh = D->d_head, Hq = D->n_q_heads, grp = D->n_q_heads / D->n_kv_heads;
  const double scale = 1.0 / sqrt((double)dh);
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int h = 0; h < Hq; ++h) {
    const int g = h / grp;
    const float* qh = q + (int64_t)h * dh;
    double* s = (double*)malloc(sizeof(double) * (size_t)n_ctx);
    double* o = (double*)calloc((size_t)dh, sizeof(double));
    if (!s || !o) {
      bad = 1;
      free(s);
      free(o);
      continue;
    }
    double m = -INFINITY;
    for (int64_t j = 0; j < n_ctx; ++j) {
      const uint16_t* k = kv_row(D, kv_layer, page_table, j, 0, g);
      double acc = 0.0;
      for (int i = 0; i < dh; ++i) acc += (double)qh[i] * (double)or_bf16_to_f32(k[i]);
      s[j] = acc * scale;
      if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < n_ctx; ++j) {
      const double w = exp(s[j] - m);
      l += w;
      const uint16_t* v = kv_row(D, kv_layer, page_table, j, 1, g);
      for (int i = 0; i < dh; ++i) o[i] += w * (double)or_bf16_to_f32(v[i]);
    }
    for (int i = 0; i < dh; ++i) out[(int64_t)h * dh + i] = (float)(o[i] / l);
    free(s);
    free(o);
  }
  return bad ? -3 : 0;
}

void or_router(const float* n, const uint16_t* w_router, const float* bias, int n_experts, int d, int k, int32_t* sel, float* gate,
               float* logits_out) {
  float* r = (float*)malloc(sizeof(float) * (size_t)n_experts);
  for (int e = 0; e < n_experts; ++e) {
    double acc = 0.0;
    const uint16_t* w = w_router + (int64_t)e * d;
    for (int i = 0; i < d; ++i) acc += (double)or_bf16_to_f32(w[i]) * (double)n[i];
    r[e] = (float)acc + (bias ? bias[e] : 0.0f);
  }
  if (logits_out) memcpy(logits_out, r, sizeof(float) * (size_t)n_experts);
  /* top-k: repeatedly take the largest remaining logit; the lower index wins a tie. */
  char* taken = (char*)calloc((size_t)n_experts, 1);
  for (int j = 0; j < k; ++j) {
    int best = -1;
    for (int e = 0; e < n_experts; ++e) {
      if (taken[e]) continue;
      if (best < 0 || r[e] > r[best]) best = e;
    }
    taken[best] = 1;
    sel[j] = best;
  }
  const double mx = r[sel[0]];
  double z = 0.0;
  for (int j = 0; j < k; ++j) z += exp((double)r[sel[j]] - mx);
  for (int j = 0; j < k; ++j) gate[j] = (float)(exp((double)r[sel[j]] - mx) / z);
  free(taken);
  free(r);
}

void or_expert(const float* n, const uint16_t* wg, const uint16_t* wu, const uint16_t* wd, int d, int F, float* y) {
  float* g = (float*)malloc(sizeof(float) * (size_t)F);
  float* u = (float*)malloc(sizeof(float) * (size_t)F);
  float* h = (float*)malloc(sizeof(float) * (size_t)F);
  or_matvec(wg, F, d, n, g);
  or_matvec(wu, F, d, n, u);
  for (int f = 0; f < F; ++f) {
    const double z = g[f];
    h[f] = (float)(z / (1.0 + exp(-z)) * (double)u[f]);
  }
  or_matvec(wd, d, F, h, y);
  free(g);
  free(u);
  free(h);
}

int or_embed(const or_dims* D, const uint16_t* embed, const int32_t* tokens, int B, float* x) {
  for (int b = 0; b < B; ++b)
    if (tokens[b] < 0 || tokens[b] >= D->vocab) return -1;
  for (int b = 0; b < B; ++b)
    for (int i = 0; i < D->d_model; ++i) x[(int64_t)b * D->d_model + i] = or_bf16_to_f32(embed[(int64_t)tokens[b] * D->d_model + i]);
  return 0;
}

int or_layer(const or_dims* D, const or_layer_w* W, int B, const int64_t* pos, const int32_t* page_tables, int64_t n_table,
             uint16_t* kv_layer, int64_t n_pages, float* x, const int32_t* sel_force, int32_t* sel_out, float* gate_out, float* n_out,
             float* attn_out, float* moe_out, float* logits_out) {
  if (!D || !W || !pos || !page_tables || !kv_layer || !x || B < 0) return -1;
  const int d = D->d_model, Hq = D->n_q_heads, Hkv = D->n_kv_heads, dh = D->d_head, E = D->n_experts, k = D->top_k, F = D->d_ffn;
  const int ps = D->page_size;
  float* n = (float*)malloc(sizeof(float) * d);
  float* q = (float*)malloc(sizeof(float) * (size_t)Hq * dh);
  float* kk = (float*)malloc(sizeof(float) * (size_t)Hkv * dh);
  float* vv = (float*)malloc(sizeof(float) * (size_t)Hkv * dh);
  float* o = (float*)malloc(sizeof(float) * (size_t)Hq * dh);
  float* a = (float*)malloc(sizeof(float) * d);
  float* y = (float*)malloc(sizeof(float) * d);
  double* m = (double*)malloc(sizeof(double) * d);
  int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * k);
  float* gate = (float*)malloc(sizeof(float) * k);
  float* lg = (float*)malloc(sizeof(float) * E);
  int rc = 0;
  for (int b = 0; b < B && rc == 0; ++b) {
    float* xb = x + (int64_t)b * d;
    const int32_t* pt = page_tables + (int64_t)b * n_table;
    const int64_t p = pos[b];
    if (p < 0 || p / ps >= n_table || pt[p / ps] < 0 || pt[p / ps] >= n_pages) {
      rc = -2;
      break;
    }
    or_rmsnorm(xb, W->attn_norm, d, D->rms_eps, n);
    /* attention branch */
    or_matvec(W->wq, (int64_t)Hq * dh, d, n, q);
    or_matvec(W->wk, (int64_t)Hkv * dh, d, n, kk);
    or_matvec(W->wv, (int64_t)Hkv * dh, d, n, vv);
    or_rope(q, Hq, dh, p, D->rope_base);
    or_rope(kk, Hkv, dh, p, D->rope_base);
    for (int g = 0; g < Hkv; ++g) {
      uint16_t* krow = (uint16_t*)kv_row(D, kv_layer, pt, p, 0, g);
      uint16_t* vrow = (uint16_t*)kv_row(D, kv_layer, pt, p, 1, g);
      for (int i = 0; i < dh; ++i) {
        krow[i] = or_f32_to_bf16(kk[g * dh + i]);
        vrow[i] = or_f32_to_bf16(vv[g * dh + i]);
      }
    }
    rc = or_attention(D, q, kv_layer, n_pages, pt, n_table, p + 1, o);
    if (rc) break;
    or_matvec(W->wo, d, (int64_t)Hq * dh, o, a);
    /* MoE branch */
    or_router(n, W->w_router, W->router_bias, E, d, k, sel, gate, lg);
    if (sel_force && sel_force[(int64_t)b * k] >= 0) {
      /* adopt a given selection; gates are the softmax of this token's own logits over it */
      for (int j = 0; j < k; ++j) sel[j] = sel_force[(int64_t)b * k + j];
      double mx = -INFINITY, z = 0.0;
      for (int j = 0; j < k; ++j)
        if (lg[sel[j]] > mx) mx = lg[sel[j]];
      for (int j = 0; j < k; ++j) z += exp((double)lg[sel[j]] - mx);
      for (int j = 0; j < k; ++j) gate[j] = (float)(exp((double)lg[sel[j]] - mx) / z);
    }
    for (int i = 0; i < d; ++i) m[i] = 0.0;
    for (int j = 0; j < k; ++j) {
      const int e = sel[j];
      if (e < 0 || e >= E || !W->w_gate[e] || !W->w_up[e] || !W->w_down[e]) {
        rc = -4;
        break;
      }
      or_expert(n, W->w_gate[e], W->w_up[e], W->w_down[e], d, F, y);
      for (int i = 0; i < d; ++i) m[i] += (double)gate[j] * (double)y[i];
    }
    if (rc) break;
    for (int i = 0; i < d; ++i) {
      const float mo = (float)m[i];
      if (attn_out) attn_out[(int64_t)b * d + i] = a[i];
      if (moe_out) moe_out[(int64_t)b * d + i] = mo;
      xb[i] = (float)((double)xb[i] + (double)a[i] + (double)mo);
    }
    if (n_out) memcpy(n_out + (int64_t)b * d, n, sizeof(float) * d);
    if (sel_out) memcpy(sel_out + (int64_t)b * k, sel, sizeof(int32_t) * k);
    if (gate_out) memcpy(gate_out + (int64_t)b * k, gate, sizeof(float) * k);
    if (logits_out) memcpy(logits_out + (int64_t)b * E, lg, sizeof(float) * E);
  }
  free(n);
  free(q);
  free(kk);
  free(vv);
  free(o);
  free(a);
  free(y);
  free(m);
  free(sel);
  free(gate);
  free(lg);
  return rc;
}

void or_head(const or_dims* D, const float* x, int B, const uint16_t* final_norm, const uint16_t* lm_head, float* logits, int32_t* next) {
  const int d = D->d_model;
  float* n = (float*)malloc(sizeof(float) * d);
  for (int b = 0; b < B; ++b) {
    or_rmsnorm(x + (int64_t)b * d, final_norm, d, D->rms_eps, n);
    float* z = logits + (int64_t)b * D->vocab;
    or_matvec(lm_head, D->vocab, d, n, z);
    int best = 0;
    for (int v = 1; v < D->vocab; ++v)
      if (z[v] > z[best]) best = v;
    next[b] = best;
  }
  free(n);
}

int or_decode_step(const or_dims* D, const or_layer_w* layers, const uint16_t* embed, const uint16_t* final_norm, const uint16_t* lm_head,
                   int B, const int32_t* tokens, const int64_t* pos, const int32_t* page_tables, int64_t n_table, uint16_t* kv,
                   int64_t n_pages, float* logits, int32_t* next, int32_t* sel_out, float* gate_out, float* n_out) {
  const int d = D->d_model, k = D->top_k;
  const int64_t layer_elems = n_pages * 2 * D->n_kv_heads * (int64_t)D->page_size * D->d_head;
  float* x = (float*)malloc(sizeof(float) * (size_t)B * d);
  int rc = or_embed(D, embed, tokens, B, x);
  for (int l = 0; l < D->n_layers && rc == 0; ++l)
    rc = or_layer(D, &layers[l], B, pos, page_tables, n_table, kv + l * layer_elems, n_pages, x, NULL,
                  sel_out ? sel_out + (int64_t)l * B * k : NULL, gate_out ? gate_out + (int64_t)l * B * k : NULL,
                  n_out ? n_out + (int64_t)l * B * d : NULL, NULL, NULL, NULL);
  if (rc == 0) or_head(D, x, B, final_norm, lm_head, logits, next);
  free(x);
  return rc;
}

int or_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
