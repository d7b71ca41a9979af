// C ABI of the decode megakernel: handle management, task-list upload and the per-step launch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/mk.h"
#include "mk_desc.h"
#include "mk_kargs.h"
#include "mk_internal.h"
#include "mk_plan.h"

extern "C" hipError_t mk_launch_persistent(const mk::KArgs* a, int kclass, int grid, int mode, hipStream_t stream);
extern "C" int mk_kernel_class(int d_head, int group, int d_model, int d_ffn);

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

#define HIPCHK(expr)                                                                                  \
  do {                                                                                                \
    hipError_t e_ = (expr);                                                                           \
    if (e_ != hipSuccess) return fail(MK_E_HIP, std::string(#expr " failed: ") + hipGetErrorString(e_)); \
  } while (0)

struct DevBuf {
  void* p = nullptr;
  size_t bytes = 0;
};

}  // namespace

struct mk_model {
  mk_model_desc desc{};
  std::vector<float> bias;
  int device = 0;
  int n_cu = 0;
  int grid = 0;
  int kclass = 0;
  uint32_t dbg = 0;
  mk::Tiling tiling{};
  int max_slots = 0;
  int64_t max_tasks = 0;
  int32_t max_counters = 0;
  // device memory owned by the handle
  std::vector<DevBuf> owned;
  mk::LayerW* layers = nullptr;
  const uint16_t *embed = nullptr, *lm_head = nullptr, *final_norm = nullptr;
  float* router_bias = nullptr;
  double* inv_freq = nullptr;
  int32_t* tasks = nullptr;
  uint32_t* ctr = nullptr;
  uint32_t* err = nullptr;
  float *x = nullptr, *ssq = nullptr, *rope_cs = nullptr, *qkv = nullptr, *apart = nullptr, *attn_o = nullptr, *opart = nullptr;
  double* rpart = nullptr;
  float *rlogits = nullptr, *route_gate = nullptr, *h = nullptr, *ypart = nullptr, *lmbest_v = nullptr, *dump_n = nullptr;
  int32_t *route_sel = nullptr, *lmbest_i = nullptr, *next_tok = nullptr, *slots = nullptr;
  uint32_t *task_done = nullptr, *ctr_snapshot = nullptr, *pagewalk = nullptr;
  uint64_t* ts = nullptr;
  // task list
  mk::Plan plan;
  bool have_plan = false, dirty = false;
  int uploaded_grid = -1;    // grid the device task array was laid out for
  int32_t ph_on = 0;         // the list is regular: its phase table is valid
  int32_t ph_npl = 0;        // phases per layer
  int32_t ph_n[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int32_t ph_op[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int32_t* staging = nullptr;  // pinned host copy of the task list
  hipEvent_t upload_done = nullptr;
  bool upload_pending = false;
  bool stepped = false;

  template <class T>
  int alloc(T** out, size_t count) {
    void* p = nullptr;
    const size_t bytes = std::max<size_t>(count * sizeof(T), 256);
    if (hipMalloc(&p, bytes) != hipSuccess) return fail(MK_E_NOMEM, "hipMalloc of " + std::to_string(bytes) + " bytes failed");
    if (hipMemset(p, 0, bytes) != hipSuccess) return fail(MK_E_HIP, "hipMemset failed");
    owned.push_back({p, bytes});
    *out = static_cast<T*>(p);
    return MK_OK;
  }
  void release() {
    for (auto& b : owned) (void)hipFree(b.p);
    owned.clear();
    if (staging) (void)hipHostFree(staging);
    staging = nullptr;
    if (upload_done) (void)hipEventDestroy(upload_done);
    upload_done = nullptr;
  }
};

extern "C" {

const char* mk_last_error(void) { return g_err.c_str(); }

int mk_plan_tasks(const mk_model_desc* desc, const mk_batch* batch, int32_t* tasks_out, int64_t cap, int64_t* n_tasks,
                  int32_t* n_counters) {
  if (!n_tasks) return fail(MK_E_INVAL, "null n_tasks");
  mk::Plan P;
  std::string msg;
  int rc = mk::plan_step(desc, batch, &P, &msg);
  if (rc) return fail(rc, msg);
  *n_tasks = P.n_tasks();
  if (n_counters) *n_counters = P.cl.total;
  if (tasks_out) {
    if (cap < P.n_tasks()) return fail(MK_E_RANGE, "tasks_out holds fewer descriptors than the plan");
    std::memcpy(tasks_out, P.desc.data(), P.desc.size() * sizeof(int32_t));
  }
  return MK_OK;
}

int mk_load_model(const mk_model_desc* desc, const mk_weights* w, mk_model** out) {
  if (!out) return fail(MK_E_INVAL, "null output handle");
  *out = nullptr;
  std::string msg;
  int rc = mk::validate_desc(desc, &msg);
  if (rc) return fail(rc, msg);
  if (!w || !w->embed || !w->lm_head || !w->final_norm || !w->attn_norm || !w->wq || !w->wk || !w->wv || !w->wo || !w->w_router ||
      !w->w_gate || !w->w_up || !w->w_down)
    return fail(MK_E_INVAL, "null weight pointer");
  const int L = desc->n_layers;
  for (int l = 0; l < L; ++l)
    if (!w->attn_norm[l] || !w->wq[l] || !w->wk[l] || !w->wv[l] || !w->wo[l] || !w->w_router[l] || !w->w_gate[l] || !w->w_up[l] ||
        !w->w_down[l])
      return fail(MK_E_INVAL, "null per-layer weight pointer at layer " + std::to_string(l));

  const int kclass = mk_kernel_class(desc->d_head, desc->n_q_heads / desc->n_kv_heads, desc->d_model, desc->d_ffn);
  if (!kclass)
    return fail(MK_E_UNSUPPORTED, "no compiled kernel for this shape (d_head 128 with group 8, d_model <= 2048, d_ffn <= 1024; or "
                                  "d_head 64 with group 2, d_model <= 512, d_ffn <= 512)");
  mk_model* m = new mk_model();
  m->kclass = kclass;
  m->desc = *desc;
  m->desc.router_bias = nullptr;
  HIPCHK(hipGetDevice(&m->device));
  HIPCHK(hipDeviceGetAttribute(&m->n_cu, hipDeviceAttributeMultiprocessorCount, m->device));
  m->grid = std::min(m->n_cu, mk::LM_MAX_WG);
  m->tiling = mk::choose_tiling(desc, desc->max_batch);
  const mk::Tiling& t = m->tiling;
  const int n_up_max = std::max(t.n_up, mk::choose_tiling(desc, 1).n_up);  // small batches cut finer
  const int d = desc->d_model, Hq = desc->n_q_heads, Hkv = desc->n_kv_heads, dh = desc->d_head, E = desc->n_experts;
  const int k = desc->top_k, F = desc->d_ffn, maxB = desc->max_batch, grp = Hq / Hkv;
  m->max_slots = std::min(E, maxB * k);
  mk::CounterLayout cl;
  cl.build(L, Hkv, maxB, m->max_slots, t.n_rt);
  m->max_counters = cl.total;
  m->max_tasks = (int64_t)t.n_rt + (int64_t)L * (t.n_router + Hkv * t.n_qkv_per_group + (int64_t)Hkv * maxB * mk::ATTN_MAX_SPLITS +
                                                 (int64_t)Hkv * maxB * grp +  /* merge tasks: at most one per head */
                                                 (int64_t)m->max_slots * n_up_max + Hkv * t.n_rt + (int64_t)m->max_slots * t.n_rt + t.n_rt) +
                 t.n_lm;

  auto cleanup = [&](int code) {
    m->release();
    delete m;
    return code;
  };
  std::vector<mk::LayerW> lw(L);
  for (int l = 0; l < L; ++l)
    lw[l] = mk::LayerW{(const uint16_t*)w->attn_norm[l], (const uint16_t*)w->wq[l], (const uint16_t*)w->wk[l], (const uint16_t*)w->wv[l],
                       (const uint16_t*)w->wo[l],        (const uint16_t*)w->w_router[l], (const uint16_t*)w->w_gate[l],
                       (const uint16_t*)w->w_up[l],      (const uint16_t*)w->w_down[l]};
  m->bias.assign(E, 0.0f);
  if (desc->router_bias) std::copy(desc->router_bias, desc->router_bias + E, m->bias.begin());
  std::vector<double> invf(dh / 2);
  for (int i = 0; i < dh / 2; ++i) invf[i] = std::pow((double)desc->rope_base, -2.0 * i / dh);

  if ((rc = m->alloc(&m->layers, L)) || (rc = m->alloc(&m->router_bias, E)) || (rc = m->alloc(&m->inv_freq, dh / 2)) ||
      (rc = m->alloc(&m->tasks, (size_t)m->max_tasks * mk::DESC_WORDS)) || (rc = m->alloc(&m->ctr, (size_t)m->max_counters * mk::CTR_STRIDE)) ||
      (rc = m->alloc(&m->err, 8)) || (rc = m->alloc(&m->x, (size_t)maxB * d)) || (rc = m->alloc(&m->ssq, (size_t)maxB * t.n_rt)) ||
      (rc = m->alloc(&m->rope_cs, (size_t)maxB * dh)) || (rc = m->alloc(&m->qkv, (size_t)maxB * Hkv * (grp + 2) * dh)) ||
      (rc = m->alloc(&m->apart, (size_t)maxB * Hkv * mk::ATTN_MAX_SPLITS * grp * (dh + 2))) ||
      (rc = m->alloc(&m->attn_o, (size_t)maxB * Hq * dh)) || (rc = m->alloc(&m->opart, (size_t)Hkv * maxB * d)) ||
      (rc = m->alloc(&m->rlogits, (size_t)L * maxB * E)) || (rc = m->alloc(&m->rpart, (size_t)t.n_rt * maxB * E)) || (rc = m->alloc(&m->route_sel, (size_t)L * maxB * k)) ||
      (rc = m->alloc(&m->route_gate, (size_t)L * maxB * k)) || (rc = m->alloc(&m->h, (size_t)m->max_slots * maxB * F)) ||
      (rc = m->alloc(&m->ypart, (size_t)maxB * k * d)) || (rc = m->alloc(&m->lmbest_v, (size_t)maxB * mk::LM_MAX_WG)) ||
      (rc = m->alloc(&m->lmbest_i, (size_t)maxB * mk::LM_MAX_WG)) || (rc = m->alloc(&m->next_tok, maxB)) ||
      (rc = m->alloc(&m->ctr_snapshot, m->max_counters)) ||
      (rc = m->alloc(&m->slots, (size_t)L * m->max_slots * mk::SLOT_WORDS)))
    return cleanup(rc);
  if (hipHostMalloc((void**)&m->staging, (size_t)m->max_tasks * mk::DESC_WORDS * sizeof(int32_t), hipHostMallocDefault) != hipSuccess) {
    m->staging = nullptr;
    return cleanup(fail(MK_E_NOMEM, "pinned staging allocation failed"));
  }
  if (hipEventCreateWithFlags(&m->upload_done, hipEventDisableTiming) != hipSuccess) return cleanup(fail(MK_E_HIP, "hipEventCreate failed"));
  if (hipMemcpy(m->layers, lw.data(), sizeof(mk::LayerW) * L, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(m->router_bias, m->bias.data(), sizeof(float) * E, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(m->inv_freq, invf.data(), sizeof(double) * invf.size(), hipMemcpyHostToDevice) != hipSuccess)
    return cleanup(fail(MK_E_HIP, "upload of the model tables failed"));
  m->embed = (const uint16_t*)w->embed;
  m->lm_head = (const uint16_t*)w->lm_head;
  m->final_norm = (const uint16_t*)w->final_norm;
  *out = m;
  return MK_OK;
}

int mk_build_tasks(mk_model* m, const mk_batch* batch, int32_t* tasks_out, int64_t cap, int64_t* n_tasks) {
  if (!m || !n_tasks) return fail(MK_E_INVAL, "null handle or n_tasks");
  std::string msg;
  mk::Plan P;
  int rc = mk::plan_step(&m->desc, batch, &P, &msg, (m->dbg & MK_DBG_MERGE_TASKS) != 0);
  if (rc) return fail(rc, msg);
  *n_tasks = P.n_tasks();
  if (P.n_tasks() > m->max_tasks) return fail(MK_E_INVAL, "task list larger than the handle's bound");
  if (tasks_out && cap < P.n_tasks()) return fail(MK_E_RANGE, "tasks_out holds fewer descriptors than the plan");
  if (tasks_out) std::memcpy(tasks_out, P.desc.data(), P.desc.size() * sizeof(int32_t));
  m->plan = std::move(P);
  m->have_plan = true;
  m->dirty = true;
  return MK_OK;
}

// Phases of the list: maximal runs of one operation and layer.  The table is valid when the list is the
// embedding tiles followed, layer by layer, by the same sequence of runs with the same sizes (at most 7 per
// layer); the kernel then passes over the expert tiles of unused slots (otherwise it runs them as empty
// tasks).
static void derive_phases(mk_model* m, const int32_t* q, int64_t n) {
  m->ph_on = 0;
  const int L = m->desc.n_layers;
  std::vector<int32_t> op, layer, len;
  for (int64_t i = 0; i < n; ++i) {
    const int32_t* w = q + i * mk::DESC_WORDS;
    if (op.empty() || op.back() != w[mk::W_OP] || layer.back() != w[mk::W_LAYER]) {
      op.push_back(w[mk::W_OP]);
      layer.push_back(w[mk::W_LAYER]);
      len.push_back(0);
    }
    ++len.back();
  }
  if (op.empty() || op[0] != mk::OP_EMBED || (op.size() - 1) % L) return;
  const int npl = (int)((op.size() - 1) / L);
  if (npl < 1 || npl > 7) return;
  for (int l = 0; l < L; ++l)
    for (int k = 0; k < npl; ++k) {
      const size_t r = 1 + (size_t)l * npl + k;
      if (layer[r] != l || op[r] != op[1 + k] || len[r] != len[1 + k]) return;
    }
  m->ph_npl = npl;
  m->ph_n[0] = len[0];
  for (int k = 0; k < npl; ++k) {
    m->ph_n[1 + k] = len[1 + k];
    m->ph_op[k] = op[1 + k];
  }
  m->ph_on = 1;
}

// Copy the task list to the pinned staging buffer (list order) and derive its phase table.
// MK_DBG_DROP_SIGNAL removes the completion signal of the first QKV task (watchdog test).
static void lay_out_queues(mk_model* m) {
  const mk::Plan& P = m->plan;
  std::memcpy(m->staging, P.desc.data(), P.desc.size() * sizeof(int32_t));
  if (m->dbg & MK_DBG_DROP_SIGNAL)
    for (int64_t i = 0; i < P.n_tasks(); ++i)
      if (m->staging[i * mk::DESC_WORDS + mk::W_OP] == mk::OP_QKV) {
        m->staging[i * mk::DESC_WORDS + mk::W_SIG] = -1;
        break;
      }
  derive_phases(m, m->staging, P.n_tasks());
  m->uploaded_grid = m->grid;
}

// The kernel's working scratch for the step planned in P, carved in one block from `base` (256-byte aligned
// pieces) into the argument block; returns the bytes it needs.  Used by the allocation-free step, whose block
// is the library's static scratch; the counters come first.
static size_t carve_scratch(const mk_model* m, const mk::Plan& P, uint8_t* base, mk::KArgs* a) {
  const mk_model_desc& D = m->desc;
  const size_t B = P.B, d = D.d_model, dh = D.d_head, Hq = D.n_q_heads, Hkv = D.n_kv_heads, grp = Hq / Hkv;
  const size_t stride = *std::max_element(P.splits.begin(), P.splits.end());
  size_t off = 0;
  auto take = [&](size_t bytes) {
    uint8_t* p = base ? base + off : nullptr;
    off += (bytes + 255) & ~(size_t)255;
    return p;
  };
  uint8_t* ctr = take((size_t)P.cl.total * mk::CTR_STRIDE * 4);
  uint8_t* x = take(B * d * 4);
  uint8_t* ssq = take(B * P.t.n_rt * 4);
  uint8_t* rope = take(B * dh * 4);
  uint8_t* qkv = take(B * Hkv * (grp + 2) * dh * 4);
  uint8_t* apart = take(B * Hkv * stride * grp * (dh + 2) * 4);
  uint8_t* attn_o = take(B * Hq * dh * 4);
  uint8_t* opart = take(Hkv * B * d * 4);
  uint8_t* rpart = take((size_t)P.t.n_rt * B * D.n_experts * 8);
  uint8_t* slots = take((size_t)D.n_layers * P.n_slots * mk::SLOT_WORDS * 4);
  uint8_t* h = take((size_t)P.n_slots * B * D.d_ffn * 4);
  uint8_t* ypart = take(B * D.top_k * d * 4);
  uint8_t* lmv = take(B * mk::LM_MAX_WG * 4);
  uint8_t* lmi = take(B * mk::LM_MAX_WG * 4);
  if (a) {
    a->ctr = (uint32_t*)ctr;
    a->x = (float*)x;
    a->ssq = (float*)ssq;
    a->rope_cs = (float*)rope;
    a->qkv = (float*)qkv;
    a->apart = (float*)apart;
    a->attn_o = (float*)attn_o;
    a->opart = (float*)opart;
    a->rpart = (double*)rpart;
    a->slots = (int32_t*)slots;
    a->h = (float*)h;
    a->ypart = (float*)ypart;
    a->lmbest_v = (float*)lmv;
    a->lmbest_i = (int32_t*)lmi;
  }
  return off;
}

static int launch_step(mk_model* m, const int32_t* tokens, const int32_t* seq_lens, const int32_t* first_of, const int32_t* page_tables,
                       void* kv_pages, float* logits_out, void* stream, const mk::ScratchOverride* so = nullptr) {
  if (!m) return fail(MK_E_INVAL, "null handle");
  if (!m->have_plan) return fail(MK_E_STATE, "mk_build_tasks has not been called");
  if (!tokens || !seq_lens || !page_tables || !kv_pages || !logits_out) return fail(MK_E_INVAL, "null step pointer");
  hipStream_t s = (hipStream_t)stream;
  const mk::Plan& P = m->plan;
  if (so) {  // the step must fit the given scratch before anything is enqueued
    const size_t need = carve_scratch(m, P, nullptr, nullptr);
    if (need > so->cap)
      return fail(MK_E_RANGE, "the step needs " + std::to_string(need) + " bytes of scratch; the static scratch holds " +
                                  std::to_string(so->cap));
  }
  if (m->dirty || m->uploaded_grid != m->grid) {
    if (m->upload_pending) HIPCHK(hipEventSynchronize(m->upload_done));  // staging may still feed the previous copy
    lay_out_queues(m);
    HIPCHK(hipMemcpyAsync(m->tasks, m->staging, P.desc.size() * sizeof(int32_t), hipMemcpyHostToDevice, s));
    HIPCHK(hipEventRecord(m->upload_done, s));
    m->upload_pending = true;
    m->dirty = false;
  }
  if (m->task_done && (m->dbg & MK_DBG_COUNT_TASKS)) HIPCHK(hipMemsetAsync(m->task_done, 0, sizeof(uint32_t) * P.n_tasks(), s));
  if (m->ts && (m->dbg & MK_DBG_TIMESTAMPS)) HIPCHK(hipMemsetAsync(m->ts, 0, sizeof(uint64_t) * 8 * P.n_tasks(), s));
  if (m->pagewalk && (m->dbg & MK_DBG_PAGE_WALK))
    HIPCHK(hipMemsetAsync(m->pagewalk, 0, sizeof(uint32_t) * 4 * m->desc.n_layers * P.B * m->desc.n_kv_heads, s));
  const mk_model_desc& D = m->desc;
  mk::KArgs a{};
  a.L = D.n_layers;
  a.d = D.d_model;
  a.Hq = D.n_q_heads;
  a.Hkv = D.n_kv_heads;
  a.dh = D.d_head;
  a.E = D.n_experts;
  a.k = D.top_k;
  a.F = D.d_ffn;
  a.V = D.vocab;
  a.B = P.B;
  a.n_slots = P.n_slots;
  a.max_pages = D.max_pages_per_seq;
  a.n_rt = P.t.n_rt;
  a.c_lm_pool = P.cl.lm_pool;
  a.c_lm_arrive = P.cl.lm_arrive;
  a.c_xfinal = P.cl.xready + D.n_layers;
  a.n_pages = D.n_pages;
  a.eps = D.rms_eps;
  a.n_tasks = (int32_t)P.n_tasks();
  a.n_counters = P.cl.total;
  a.c_ticket = P.cl.ticket;
  a.ph_on = m->ph_on;
  a.ph_npl = m->ph_npl;
  for (int i = 0; i < 8; ++i) {
    a.ph_n[i] = m->ph_n[i];
    a.ph_op[i] = m->ph_op[i];
  }
  a.c_slots_used = P.cl.slots_used;
  a.c_resid_arrive = P.cl.resid_arrive;
  a.c_done = P.cl.done;
  a.layers = m->layers;
  a.embed = m->embed;
  a.lm_head = m->lm_head;
  a.final_norm = m->final_norm;
  a.router_bias = m->router_bias;
  a.inv_freq = m->inv_freq;
  a.tokens = tokens;
  a.seq_lens = seq_lens;
  a.first_of = first_of;
  a.page_tables = page_tables;
  a.kv = (uint16_t*)kv_pages;
  a.logits = logits_out;
  a.tasks = m->tasks;
  a.ctr = m->ctr;
  a.err = m->err;
  a.x = m->x;
  a.ssq = m->ssq;
  a.rope_cs = m->rope_cs;
  a.qkv = m->qkv;
  a.apart = m->apart;
  a.apart_stride = *std::max_element(P.splits.begin(), P.splits.end());
  a.attn_o = m->attn_o;
  a.opart = m->opart;
  a.rlogits = m->rlogits;
  a.rpart = m->rpart;
  a.route_sel = m->route_sel;
  a.slots = m->slots;
  a.route_gate = m->route_gate;
  a.h = m->h;
  a.ypart = m->ypart;
  a.lmbest_v = m->lmbest_v;
  a.lmbest_i = m->lmbest_i;
  a.next_tok = m->next_tok;
  a.dump_n = (m->dbg & MK_DBG_DUMP_N) ? m->dump_n : nullptr;
  a.task_done = (m->dbg & MK_DBG_COUNT_TASKS) ? m->task_done : nullptr;
  a.ts = (m->dbg & MK_DBG_TIMESTAMPS) ? m->ts : nullptr;
  a.ctr_snapshot = m->ctr_snapshot;
  a.pagewalk = (m->dbg & MK_DBG_PAGE_WALK) ? m->pagewalk : nullptr;
  if (so) {  // working scratch from the given block; its counters start at zero
    carve_scratch(m, P, so->base, &a);
    so->zero(a.ctr, (int64_t)P.cl.total * mk::CTR_STRIDE, s);
    HIPCHK(hipGetLastError());
  }
  a.spin_limit = (m->dbg & MK_DBG_DROP_SIGNAL) ? (1u << 12) : (1u << 21);
  HIPCHK(mk_launch_persistent(&a, m->kclass, m->grid, (m->dbg & MK_DBG_WIDE_GEMV) ? 1 : (m->dbg & MK_DBG_VALU_GEMV) ? 2 : 0, s));
  m->stepped = true;
  return MK_OK;
}

int mk_decode_step(mk_model* m, const int32_t* tokens, const int32_t* seq_lens, const int32_t* page_tables, void* kv_pages,
                   float* logits_out, void* stream) {
  return launch_step(m, tokens, seq_lens, nullptr, page_tables, kv_pages, logits_out, stream);
}

}  // extern "C"

namespace mk {
int launch_step_scratch(mk_model* m, const int32_t* tokens, const int32_t* seq_lens, const int32_t* page_tables, void* kv_pages,
                        float* logits_out, void* stream, const ScratchOverride* so) {
  return launch_step(m, tokens, seq_lens, nullptr, page_tables, kv_pages, logits_out, stream, so);
}
int handle_device(const mk_model* m) { return m ? m->device : -1; }
int set_error(int code, const char* msg) { return fail(code, msg); }
}  // namespace mk

extern "C" {

int mk_mixed_step(mk_model* m, const int32_t* tokens, const int32_t* seq_lens, const int32_t* first_of, const int32_t* page_tables,
                  void* kv_pages, float* logits_out, void* stream) {
  if (!first_of) return fail(MK_E_INVAL, "null first_of");
  return launch_step(m, tokens, seq_lens, first_of, page_tables, kv_pages, logits_out, stream);
}

int mk_next_tokens(mk_model* m, int32_t** dev_ptr) {
  if (!m || !dev_ptr) return fail(MK_E_INVAL, "null argument");
  *dev_ptr = m->next_tok;
  return MK_OK;
}

int mk_status(mk_model* m, void* stream) {
  if (!m) return fail(MK_E_INVAL, "null handle");
  HIPCHK(hipStreamSynchronize((hipStream_t)stream));
  uint32_t e[8];
  HIPCHK(hipMemcpy(e, m->err, sizeof(e), hipMemcpyDeviceToHost));
  if (e[mk::ERR_CODE] == 0 && e[mk::ERR_ABORT] == 0) return MK_OK;
  static const char* names[] = {"none", "dependency wait timed out", "token out of range", "page index out of range",
                                "sequence length out of range", "unknown opcode"};
  const uint32_t c = e[mk::ERR_CODE];
  std::string msg = std::string("device fault: ") + (c < 6 ? names[c] : "unknown") + " (task " + std::to_string(e[mk::ERR_TASK]) + ")";
  HIPCHK(hipMemset(m->err, 0, sizeof(e)));
  HIPCHK(hipMemset(m->ctr, 0, sizeof(uint32_t) * m->max_counters * mk::CTR_STRIDE));
  return fail(MK_E_DEVICE, msg);
}

int mk_debug_set(mk_model* m, uint32_t flags) {
  if (!m) return fail(MK_E_INVAL, "null handle");
  if ((flags & MK_DBG_DUMP_N) && !m->dump_n) {
    int rc = m->alloc(&m->dump_n, (size_t)m->desc.n_layers * m->desc.max_batch * m->desc.d_model);
    if (rc) return rc;
  }
  if ((flags & MK_DBG_COUNT_TASKS) && !m->task_done) {
    int rc = m->alloc(&m->task_done, (size_t)m->max_tasks);
    if (rc) return rc;
  }
  if ((flags & MK_DBG_TIMESTAMPS) && !m->ts) {
    int rc = m->alloc(&m->ts, (size_t)m->max_tasks * 8);
    if (rc) return rc;
  }
  if ((flags & MK_DBG_PAGE_WALK) && !m->pagewalk) {
    int rc = m->alloc(&m->pagewalk, (size_t)4 * m->desc.n_layers * m->desc.max_batch * m->desc.n_kv_heads);
    if (rc) return rc;
  }
  if ((flags ^ m->dbg) & MK_DBG_DROP_SIGNAL) m->dirty = true;  // the uploaded task list changes
  m->dbg = flags;
  return MK_OK;
}

int mk_debug_read(mk_model* m, int kind, void* host_dst, int64_t bytes) {
  if (!m || !host_dst || bytes < 0) return fail(MK_E_INVAL, "null argument");
  if (!m->have_plan) return fail(MK_E_STATE, "no step has been planned");
  HIPCHK(hipDeviceSynchronize());
  const mk_model_desc& D = m->desc;
  const int64_t L = D.n_layers, B = m->plan.B;
  const void* src = nullptr;
  int64_t avail = 0;
  switch (kind) {
    case MK_DBGK_ROUTE_SEL: src = m->route_sel; avail = L * B * D.top_k * 4; break;
    case MK_DBGK_ROUTE_GATE: src = m->route_gate; avail = L * B * D.top_k * 4; break;
    case MK_DBGK_ROUTER_LOGITS: src = m->rlogits; avail = L * B * D.n_experts * 4; break;
    case MK_DBGK_NORM_IN:
      if (!(m->dbg & MK_DBG_DUMP_N)) return fail(MK_E_STATE, "MK_DBG_DUMP_N is not enabled");
      src = m->dump_n;
      avail = L * B * D.d_model * 4;
      break;
    case MK_DBGK_COUNTERS: src = m->ctr_snapshot; avail = (int64_t)m->plan.cl.total * 4; break;
    case MK_DBGK_TASK_DONE:
      if (!(m->dbg & MK_DBG_COUNT_TASKS)) return fail(MK_E_STATE, "MK_DBG_COUNT_TASKS is not enabled");
      src = m->task_done;
      avail = m->plan.n_tasks() * 4;
      break;
    case MK_DBGK_TIMESTAMPS:
      if (!(m->dbg & MK_DBG_TIMESTAMPS)) return fail(MK_E_STATE, "MK_DBG_TIMESTAMPS is not enabled");
      src = m->ts;
      avail = m->plan.n_tasks() * 64;
      break;
    case MK_DBGK_PAGE_WALK:
      if (!(m->dbg & MK_DBG_PAGE_WALK)) return fail(MK_E_STATE, "MK_DBG_PAGE_WALK is not enabled");
      src = m->pagewalk;
      avail = L * B * D.n_kv_heads * 16;
      break;
    case MK_DBGK_SLOTS: src = m->slots; avail = L * m->plan.n_slots * mk::SLOT_WORDS * 4; break;
    default: return fail(MK_E_INVAL, "unknown debug kind");
  }
  if (bytes > avail) return fail(MK_E_RANGE, "request larger than the debug buffer");
  HIPCHK(hipMemcpy(host_dst, src, (size_t)bytes, hipMemcpyDeviceToHost));
  return MK_OK;
}

int mk_set_grid(mk_model* m, int32_t n_workgroups) {
  if (!m || n_workgroups < 0 || n_workgroups > mk::LM_MAX_WG) return fail(MK_E_INVAL, "n_workgroups outside 0..1024");
  m->grid = n_workgroups == 0 ? std::min(m->n_cu, mk::LM_MAX_WG) : n_workgroups;
  return MK_OK;
}

int mk_free_model(mk_model* m) {
  if (!m) return fail(MK_E_INVAL, "null handle");
  m->release();
  delete m;
  return MK_OK;
}

}  // extern "C"
