/* CPU oracle of one decode step of the parallel-transformer MoE decoder.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke entry point and the
 * benchmark's CPU-baseline leg may load or call this library.  It shares no
 * code with the GPU path.
 *
 * What it computes (the plain definition of the decode step the megakernel
 * reschedules; "Cohere's North Mini Code Megakernel Serving Engine" write-ups):
 *  - parallel layer: attention and the MoE feed-forward both read the same
 *    RMS-normalised input and are joined by a residual add
 *    (agenticcommons.xyz, section on wave quantization: parallel transformer
 *    layer with fused residual add + RMSNorm);
 *  - GQA attention in KV groups over a paged KV cache with ragged lengths
 *    (agenticcommons.xyz, section on false dependencies; aimodeling.com,
 *    "From demo to a full serving system");
 *  - a router choosing top-k experts, SwiGLU experts with separate up and down
 *    projections (agenticcommons.xyz, sections on false dependencies and
 *    weight prefetch);
 *  - BF16 weights (all pages).
 * Where the pages are silent the readings are listed in the design notes
 * (RMSNorm with unit gains, rotate-half RoPE, softmax over the selected k
 * logits, lowest index wins ties, fp64 accumulation).
 *
 * Numerics: every stored activation is fp32; every reduction accumulates in
 * fp64 and is rounded to fp32 once, where the value is stored.  The KV cache
 * holds BF16.  Weights are BF16 bit patterns (uint16).
 *
 * Pins: every part is tested against closed forms, special cases and library
 * routines (numpy/torch on the CPU).  A whole decode step of many layers has no
 * external reference: parity unpinned beyond those per-part pins and the
 * layer algebra (the layer equals x + Attn(n) + MoE(n) of the separately
 * called parts).
 *
 * Error convention: functions returning int give 0 on success and a negative
 * value on invalid arguments (null pointer, page index out of range).
 */
#ifndef MK_ORACLE_H
#define MK_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct or_dims {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, d_head, n_experts, top_k, d_ffn, vocab, page_size;
  double rms_eps, rope_base;
} or_dims;

/* Weights of one layer (host memory, BF16 bit patterns, row-major [out][in]). */
typedef struct or_layer_w {
  const uint16_t* attn_norm;     /* [d] */
  const uint16_t* wq;            /* [Hq*dh][d] */
  const uint16_t* wk;            /* [Hkv*dh][d] */
  const uint16_t* wv;            /* [Hkv*dh][d] */
  const uint16_t* wo;            /* [d][Hq*dh] */
  const uint16_t* w_router;      /* [E][d] */
  const float* router_bias;      /* [E], may be NULL (no bias) */
  const uint16_t* const* w_gate; /* [E] pointers to [F][d]; entries of unselected experts may be NULL */
  const uint16_t* const* w_up;   /* [E] pointers to [F][d] */
  const uint16_t* const* w_down; /* [E] pointers to [d][F] */
} or_layer_w;

/* y[r] = sum_c W[r][c] x[c], fp64 accumulation, rounded to fp32. */
void or_matvec(const uint16_t* W, int64_t rows, int64_t cols, const float* x, float* y);

/* out = x * gamma / sqrt(mean(x^2) + eps). */
void or_rmsnorm(const float* x, const uint16_t* gamma, int d, double eps, float* out);

/* Rotate-half RoPE in place on n_heads vectors of d_head at position pos:
 * (a_i, a_{i+dh/2}) <- (a_i cos t - a_{i+dh/2} sin t, a_i sin t + a_{i+dh/2} cos t), t = pos * base^(-2i/dh). */
void or_rope(float* v, int n_heads, int d_head, int64_t pos, double base);

/* Decode attention for one token: q [Hq][dh] (RoPE applied) over positions 0..n_ctx-1 of one layer's
 * paged cache kv_layer [n_pages][2][Hkv][page_size][dh] via page_table (n_table entries).
 * out [Hq][dh] = softmax(q K^T / sqrt(dh)) V per head, head h reading KV head h / (Hq/Hkv). */
int or_attention(const or_dims* D, const float* q, const uint16_t* kv_layer, int64_t n_pages, const int32_t* page_table,
                 int64_t n_table, int64_t n_ctx, float* out);

/* Router: logits[e] = fp32(sum_i n_i W[e][i]) + bias[e]; sel = top-k by (logit desc, index asc);
 * gate = softmax of the selected logits.  logits_out may be NULL. */
void or_router(const float* n, const uint16_t* w_router, const float* bias, int n_experts, int d, int k, int32_t* sel, float* gate,
               float* logits_out);

/* One SwiGLU expert: y = Wd (silu(Wg n) * (Wu n)), silu(z) = z / (1 + e^-z). */
void or_expert(const float* n, const uint16_t* wg, const uint16_t* wu, const uint16_t* wd, int d, int F, float* y);

/* One parallel layer for B tokens.  For token b at position pos[b] (number of prior positions):
 * n = RMSNorm(x_b); q,k,v = Wq n, Wk n, Wv n; RoPE(q, k, pos[b]); k, v rounded to BF16 and written to
 * slot pos[b] of the cache; attention over positions 0..pos[b]; a = Wo o; router on n (or the forced
 * selection sel_force[b][*] when sel_force != NULL and sel_force[b][0] >= 0); m = sum_j gate_j y_j;
 * x_b <- x_b + a + m.  page_tables: [B][n_table].  Outputs (nullable): sel/gate [B][k], n/attn/moe [B][d],
 * router logits [B][E]. */
int or_layer(const or_dims* D, const or_layer_w* W, int B, const int64_t* pos, const int32_t* page_tables, int64_t n_table,
             uint16_t* kv_layer, int64_t n_pages, float* x, const int32_t* sel_force, int32_t* sel_out, float* gate_out, float* n_out,
             float* attn_out, float* moe_out, float* logits_out);

/* x [B][d] = fp32(embed[token]). */
int or_embed(const or_dims* D, const uint16_t* embed, const int32_t* tokens, int B, float* x);

/* Final RMSNorm, LM head, greedy argmax (lowest index on ties).  logits [B][V], next [B]. */
void or_head(const or_dims* D, const float* x, int B, const uint16_t* final_norm, const uint16_t* lm_head, float* logits, int32_t* next);

/* Whole decode step with every weight in memory.  layers: [n_layers]; kv: [n_layers][n_pages][2][Hkv][ps][dh].
 * sel_out/gate_out: [n_layers][B][k] (nullable); n_out: [n_layers][B][d] (nullable). */
int or_decode_step(const or_dims* D, const or_layer_w* layers, const uint16_t* embed, const uint16_t* final_norm, const uint16_t* lm_head,
                   int B, const int32_t* tokens, const int64_t* pos, const int32_t* page_tables, int64_t n_table, uint16_t* kv,
                   int64_t n_pages, float* logits, int32_t* next, int32_t* sel_out, float* gate_out, float* n_out);

/* BF16 helpers (round to nearest even; NaN kept quiet). */
/* Threads the OpenMP loops of this library run on (omp_get_max_threads), for reporting. */
int or_num_threads(void);

uint16_t or_f32_to_bf16(float f);
float or_bf16_to_f32(uint16_t b);

#ifdef __cplusplus
}
#endif

#endif
