// Kernel argument block of the persistent decode kernel (passed by value at launch).
#pragma once
#include <stdint.h>

namespace mk {

// Device-side per-layer weight table (BF16 bit patterns, row-major [out][in]).
struct LayerW {
  const uint16_t* attn_norm;
  const uint16_t* wq;
  const uint16_t* wk;
  const uint16_t* wv;
  const uint16_t* wo;
  const uint16_t* w_router;
  const uint16_t* w_gate;
  const uint16_t* w_up;
  const uint16_t* w_down;
};

// Fault word layout (uint32[8]) and codes.
enum { ERR_CODE = 0, ERR_TASK = 1, ERR_ABORT = 2 };
enum { ERRC_TIMEOUT = 1, ERRC_TOKEN = 2, ERRC_PAGE = 3, ERRC_SEQLEN = 4, ERRC_OPCODE = 5 };

struct KArgs {
  // shape of the model and of this step
  int32_t L, d, Hq, Hkv, dh, E, k, F, V;
  int32_t B, n_slots, max_pages, n_rt;
  int64_t n_pages;
  float eps;
  int32_t n_tasks, n_counters, c_ticket, c_done;
  int32_t c_lm_pool, c_lm_arrive, c_xfinal;  // LM head: chunk pool, arrivals, readiness of the final residual stream
  // phase table (when ph_on): the list is the embedding tiles (ph_n[0]), then per layer ph_npl runs of one
  // operation, of ph_n[1] .. ph_n[ph_npl] tasks, the same in every layer; it classifies a take (expert tiles
  // of unused slots).  Every workgroup takes the list in order through the ticket counter c_ticket.
  int32_t ph_on, ph_npl, ph_n[8];
  int32_t ph_op[8];      // operation of each per-layer phase
  // expert slots: counter of each layer's used-slot count, first residual arrival counter
  int32_t c_slots_used, c_resid_arrive;
  // model (device)
  const LayerW* layers;
  const uint16_t* embed;
  const uint16_t* lm_head;
  const uint16_t* final_norm;
  const float* router_bias;  // [E] (zeros when the model has none)
  const double* inv_freq;    // [dh/2] RoPE inverse frequencies base^(-2i/dh)
  // this step's inputs and outputs (caller-owned device memory)
  const int32_t* tokens;
  const int32_t* seq_lens;
  // [B] or null: first batch entry of each entry's sequence in this step (a chunk of consecutive positions of
  // one sequence, prefill); null = every entry is its own sequence (decode)
  const int32_t* first_of;
  const int32_t* page_tables;
  uint16_t* kv;
  float* logits;
  // handle-owned scratch
  const int32_t* tasks;
  uint32_t* ctr;
  uint32_t* err;
  float* x;          // [B][d] residual stream
  float* ssq;        // [B][n_rt] partial sums of squares of x per row tile
  float* rope_cs;    // [B][dh/2][2] cos, sin of the new position
  float* qkv;        // [B][Hkv][(grp+2)*dh] projections (q heads of the group, then k, then v)
  float* apart;      // [B][Hkv][apart_stride][grp][dh+2] attention split partials (o, m, l)
  int32_t apart_stride;  // most attention splits of any sequence in the task list (at most ATTN_MAX_SPLITS)
  float* attn_o;     // [B][Hq*dh] merged attention output
  float* opart;      // [Hkv][B][d] O-projection partial per KV group
  float* rlogits;    // [L][B][E] router logits
  double* rpart;     // [n_rt][B][E] router partials of the row tiles (the layer being routed)
  int32_t* route_sel;
  int32_t* slots;    // [L][n_slots][SLOT_WORDS] routing table: expert, token count, (token, rank, gate bits) x 8
  float* route_gate; // [L][B][k]
  float* h;          // [n_slots][B][F] SwiGLU hidden state per expert slot and token of the slot
  float* ypart;      // [B][k][d] gated expert outputs
  float* lmbest_v;   // [B][LM_MAX_WG] best logit per token found by each workgroup
  int32_t* lmbest_i; // [B][LM_MAX_WG] its index
  int32_t* next_tok; // [max_batch]
  float* dump_n;     // [L][B][d] or null
  uint32_t* task_done;     // [n_tasks] or null
  uint64_t* ts;            // [n_tasks][8] (claim, dependencies met, end, hardware id, 4 sub-phase marks) or null
  uint32_t* ctr_snapshot;  // [n_counters] or null
  uint32_t* pagewalk;      // [L][B][Hkv][4] or null: cache pages read, sum of (logical page + 1) * physical page
                           // (mod 2^32), positions attended, written slot (physical page * 16 + slot)
  uint32_t spin_limit;     // polls a dependency wait makes before it reports a time-out
};

}  // namespace mk
