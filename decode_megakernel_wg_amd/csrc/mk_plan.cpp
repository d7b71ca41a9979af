// Host-side task planning for one decode step (no device code, no HIP calls).
//
// The step's graph is expressed as per-tile tasks in topological order, the way the pages describe the
// task list: each task is one operation on one tile, and dependencies are counters, not kernel
// boundaries (agenticcommons.xyz "Cohere North Mini Code megakernel serving engine", section
// Megakernel 的運作方式).  The list is the embedding row tiles, then per layer
//   QKV tiles, ATTN splits, expert UP tiles, [MERGE tasks,] OPROJ tiles, expert DOWN tiles
// (MERGE tasks only for long contexts, whose split-KV partials are merged in parallel; the router is the residual epilogue's last row tile, the residual add the epilogue of the last O-proj or
// down-projection task of a row tile, and the LM head the kernel's closing phase: none of them is a task).
// Workgroups take the next layer's QKV, attention and up-projection tiles and start their weight (and old
// K/V) loads while the current layer's tail still runs (same page, section 三個實際的加速來源, item 3), the
// attention and MoE tasks of one layer share all compute units (item 1, parallel layer), and each KV group's
// O-proj waits only on that group's attention and each expert's down projection only on its own up
// projection (item 2, false dependencies).
#include "mk_plan.h"

#include <algorithm>
#include <cstring>

namespace mk {

static bool is_pow2_in(int v, int lo, int hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }

int validate_desc(const mk_model_desc* d, std::string* msg) {
  if (!d) {
    *msg = "null model descriptor";
    return MK_E_INVAL;
  }
  if (d->abi_version != MK_ABI_VERSION) {
    *msg = "abi_version mismatch";
    return MK_E_INVAL;
  }
  if (d->n_layers < 1 || d->d_model < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->d_head < 1 || d->n_experts < 1 ||
      d->top_k < 1 || d->d_ffn < 1 || d->vocab < 1 || d->max_batch < 1 || d->max_pages_per_seq < 1 || d->n_pages < 1) {
    *msg = "non-positive dimension";
    return MK_E_INVAL;
  }
  if (d->page_size != MK_PAGE_SIZE) {
    *msg = "page_size must be 16";
    return MK_E_UNSUPPORTED;
  }
  if (d->max_batch > MK_MAX_BATCH) {
    *msg = "max_batch above 8";
    return MK_E_UNSUPPORTED;
  }
  if (d->d_head != 64 && d->d_head != 128) {
    *msg = "d_head must be 64 or 128";
    return MK_E_UNSUPPORTED;
  }
  if (d->n_q_heads % d->n_kv_heads || !is_pow2_in(d->n_q_heads / d->n_kv_heads, 2, 8)) {
    *msg = "n_q_heads / n_kv_heads must be 2, 4 or 8";
    return MK_E_UNSUPPORTED;
  }
  if (d->d_model % 256 || d->d_model > 4096) {
    *msg = "d_model must be a multiple of 256, at most 4096";
    return MK_E_UNSUPPORTED;
  }
  if (d->d_ffn % 128 || d->d_ffn > 2048) {
    *msg = "d_ffn must be a multiple of 128, at most 2048";
    return MK_E_UNSUPPORTED;
  }
  if (d->n_q_heads * d->d_head > 8192) {
    *msg = "n_q_heads * d_head above 8192";
    return MK_E_UNSUPPORTED;
  }
  if (d->n_experts > 256 || d->n_experts % 8 || d->top_k > 8 || d->top_k > d->n_experts) {
    *msg = "n_experts a multiple of 8, at most 256, and top_k <= min(8, n_experts) required";
    return MK_E_UNSUPPORTED;
  }
  if (d->vocab % 64) {
    *msg = "vocab must be a multiple of 64";
    return MK_E_UNSUPPORTED;
  }
  if (!(d->rms_eps >= 0.0f) || !(d->rope_base > 0.0f)) {
    *msg = "bad rms_eps or rope_base";
    return MK_E_INVAL;
  }
  return MK_OK;
}

Tiling choose_tiling(const mk_model_desc* d, int batch) {
  Tiling t{};
  t.rt = d->d_model >= 1024 ? 128 : 32;
  t.n_rt = d->d_model / t.rt;
  t.qkv_rows = 64;
  t.n_qkv_per_group = (d->n_q_heads / d->n_kv_heads + 2) * d->d_head / t.qkv_rows;
  t.router_rows = std::min(d->n_experts, 16);
  t.n_router = (d->n_experts + t.router_rows - 1) / t.router_rows;
  // 64 gate + 64 up rows (a 512 KB tile at d_model 2048, four passes, two in flight); at batches of 1-2, 48 + 48
  // rows where d_ffn allows (more, shorter tiles spread the few experts' 50 MB over more compute units:
  // measured +1.5 % at batch 1, -3 to -5 % at batch 8, where many experts already fill the machine)
  t.up_rows = batch <= 2 && d->d_ffn % 48 == 0 ? 48 : 64;
  t.n_up = d->d_ffn / t.up_rows;
  t.lm_rows = 128;  // vocabulary chunk of the LM head's closing phase
  t.n_lm = (d->vocab + t.lm_rows - 1) / t.lm_rows;
  return t;
}

namespace {
struct Emitter {
  std::vector<int32_t>* out;
  int32_t* add(int op, int layer) {
    size_t o = out->size();
    out->resize(o + DESC_WORDS, 0);
    int32_t* w = out->data() + o;
    w[W_OP] = op;
    w[W_LAYER] = layer;
    for (int i = 0; i < N_WAITS; ++i) {
      w[W_WAIT0 + 2 * i] = -1;
      w[W_WAIT0 + 2 * i + 1] = 0;
    }
    w[W_SIG] = -1;
    w[W_SIGR] = 1;
    w[W_ARR] = -1;
    w[W_ARR2] = -1;
    w[W_RSIG] = -1;
    w[W_SEQ] = (int32_t)(o / DESC_WORDS);
    return w;
  }
};
// A task that completes a row tile of layer l's input also adds that tile's router partial for layer l
// (none after the last layer); the last of the n_rt tiles routes layer l and releases its expert slots.
void router_epilogue(int32_t* w, const CounterLayout& cl, const Tiling& t, int l) {
  if (l >= cl.n_layers) return;
  w[W_ARR2] = cl.router_arrive + l;
  w[W_ARRN2] = t.n_rt;
  w[W_RSIG] = cl.slot_ready + l * cl.n_slots;
  w[W_RSIGR] = cl.n_slots;
}
void set_wait(int32_t* w, int i, int32_t c, int32_t target) {
  w[W_WAIT0 + 2 * i] = c;
  w[W_WAIT0 + 2 * i + 1] = target;
}
void set_sig(int32_t* w, int32_t c, int32_t n = 1) {
  w[W_SIG] = c;
  w[W_SIGN] = n;
}
// O-proj and expert-down tasks of row tile r of layer l: the last of the tile's producers adds the branch
// partials into the residual stream (fixed order) and counts the row tile into XREADY[l+1]; the next
// layer's consumers wait for all row tiles and normalise the residual stream themselves.
void resid_epilogue(int32_t* w, const CounterLayout& cl, const Tiling& t, int l, int r, int producers) {
  w[W_RT] = r;
  w[W_ARR] = cl.resid_arrive + l * t.n_rt + r;
  w[W_ARRN] = producers;
  set_sig(w, cl.xready + l + 1);
  router_epilogue(w, cl, t, l + 1);
}
}  // namespace

int plan_step(const mk_model_desc* d, const mk_batch* batch, Plan* P, std::string* msg, bool force_merge) {
  int rc = validate_desc(d, msg);
  if (rc) return rc;
  if (!batch || !batch->seq_lens) {
    *msg = "null batch";
    return MK_E_INVAL;
  }
  const int B = batch->batch;
  if (B < 1 || B > d->max_batch) {
    *msg = "batch outside 1..max_batch";
    return MK_E_INVAL;
  }
  P->B = B;
  P->t = choose_tiling(d, B);
  const Tiling& t = P->t;
  const int L = d->n_layers, Hkv = d->n_kv_heads, E = d->n_experts;
  P->n_slots = std::min(E, B * d->top_k);
  P->cl.build(L, Hkv, B, P->n_slots, t.n_rt);
  const CounterLayout& cl = P->cl;
  P->splits.assign(B, 1);
  // positions per attention split: ATTN_SPLIT_POS, more when the batch's contexts are long, so that a layer
  // has about ATTN_TARGET_TASKS splits over all sequences and KV groups (each split then streams several
  // blocks, and the merge reads fewer partials); beyond ATTN_LONG_MIN_POS positions per split, about
  // ATTN_LONG_TASKS splits, up to ATTN_MAX_SPLIT_POS positions each (more splits beyond that)
  // (splits cover the cached positions in whole 128-position chunks; the last one also takes the new token)
  // cached positions each entry's attention reads: its own length, or for an entry of a chunk (first_of) the
  // position of the chunk's first token (the chunk's own positions come from the step's projections)
  std::vector<int64_t> cached(B);
  int64_t total = 0;
  for (int b = 0; b < B; ++b) {
    const int32_t len = batch->seq_lens[b];
    if (len < 0 || (int64_t)len / MK_PAGE_SIZE >= d->max_pages_per_seq) {
      *msg = "sequence length negative or beyond max_pages_per_seq";
      return MK_E_INVAL;
    }
    const int32_t f = batch->first_of ? batch->first_of[b] : b;
    if (f < 0 || f > b || (f != b && (batch->first_of[f] != f || batch->first_of[b - 1] != f)) ||
        (int64_t)len != (int64_t)batch->seq_lens[f] + (b - f)) {
      *msg = "first_of: entry " + std::to_string(b) + " is not part of a run of consecutive positions of one sequence";
      return MK_E_INVAL;
    }
    cached[b] = batch->seq_lens[f];
    total += std::max<int64_t>(cached[b], 1);
  }
  auto round128 = [](int64_t v) { return (v + 64) / 128 * 128; };
  int64_t split_pos = std::max<int64_t>(ATTN_SPLIT_POS, round128((total * Hkv + ATTN_TARGET_TASKS / 2) / ATTN_TARGET_TASKS));
  // long contexts: about ATTN_LONG_TASKS splits (three quarters of the compute units), each of thousands
  // of positions, which keeps the merges short and every wave streaming many blocks; from
  // ATTN_LONGER_MIN_POS positions per split on, about ATTN_LONGER_TASKS splits (the splits that start after
  // the QKV tiles then cost less than the shorter splits save)
  if (split_pos > ATTN_LONG_MIN_POS) {
    int64_t sp = round128((total * Hkv + ATTN_LONG_TASKS / 2) / ATTN_LONG_TASKS);
    if (sp >= ATTN_LONGER_MIN_POS) sp = round128((total * Hkv + ATTN_LONGER_TASKS / 2) / ATTN_LONGER_TASKS);
    split_pos = std::max<int64_t>(ATTN_LONG_MIN_POS, std::min<int64_t>(sp, ATTN_MAX_SPLIT_POS));
  }
  for (int b = 0; b < B; ++b) {
    const int64_t s = (std::max<int64_t>(cached[b], 1) + split_pos - 1) / split_pos;
    P->splits[b] = (int32_t)std::max<int64_t>(1, std::min<int64_t>(s, ATTN_MAX_SPLITS));
  }
  // merge tasks: when a sequence has many splits (long contexts), or when asked for (tests); each stages its
  // heads' rows of every split of its sequence in LDS, so a slice takes fewer heads as the splits grow
  const int grp = d->n_q_heads / Hkv;
  const int max_splits = *std::max_element(P->splits.begin(), P->splits.end());
  int n_merge = std::min(ATTN_MERGE_TASKS, grp);  // merge tasks per (sequence, KV group): grp is a power of two
  while (n_merge < grp && (int64_t)max_splits * (grp / n_merge) * (d->d_head + 2) > ATTN_MERGE_STAGE_FLOATS) n_merge *= 2;
  P->merge = (force_merge || max_splits >= ATTN_MERGE_MIN_SPLITS) &&
             (int64_t)max_splits * (grp / n_merge) * (d->d_head + 2) <= ATTN_MERGE_STAGE_FLOATS;
  P->desc.clear();
  Emitter em{&P->desc};

  for (int r = 0; r < t.n_rt; ++r) {
    int32_t* w = em.add(OP_EMBED, 0);
    w[W_A] = r;
    w[W_R0] = r * t.rt;
    w[W_R1] = (r + 1) * t.rt;
    w[W_RT] = r;
    set_sig(w, cl.xready + 0);
    router_epilogue(w, cl, t, 0);
  }
  for (int l = 0; l < L; ++l) {
    auto emit_qkv = [&] {
      for (int g = 0; g < Hkv; ++g)
        for (int i = 0; i < t.n_qkv_per_group; ++i) {
          int32_t* w = em.add(OP_QKV, l);
          w[W_A] = g;
          w[W_R0] = i * t.qkv_rows;
          w[W_R1] = (i + 1) * t.qkv_rows;
          set_wait(w, 0, cl.xready + l, t.n_rt);
          set_sig(w, cl.qkv_done + l * Hkv + g);
        }
    };
    auto emit_attn = [&] {
      for (int g = 0; g < Hkv; ++g)
        for (int b = 0; b < B; ++b)
          for (int s = 0; s < P->splits[b]; ++s) {
            int32_t* w = em.add(OP_ATTN, l);
            w[W_A] = b;
            w[W_B] = g;
            w[W_C] = s;
            w[W_D] = P->splits[b];
            w[W_R0] = (int32_t)split_pos;  // cached positions per split (the last one takes the rest)
            set_wait(w, 0, cl.qkv_done + l * Hkv + g, t.n_qkv_per_group);
            if (P->merge) {
              set_sig(w, cl.attn_arrive + (l * B + b) * Hkv + g);  // counted; merged by the MERGE tasks
            } else {
              set_sig(w, cl.attn_done + l * Hkv + g);  // issued only by the split that arrives last
              w[W_ARR] = cl.attn_arrive + (l * B + b) * Hkv + g;
              w[W_ARRN] = P->splits[b];
            }
          }
    };
    auto emit_merge = [&] {
      for (int g = 0; g < Hkv; ++g)
        for (int b = 0; b < B; ++b)
          for (int m = 0; m < n_merge; ++m) {
            int32_t* w = em.add(OP_MERGE, l);
            w[W_A] = b;
            w[W_B] = g;
            w[W_C] = m * (grp / n_merge);  // first head of the slice
            w[W_D] = P->splits[b];
            w[W_R0] = grp / n_merge;       // heads of the slice
            set_wait(w, 0, cl.attn_arrive + (l * B + b) * Hkv + g, P->splits[b]);
            set_sig(w, cl.attn_done + l * Hkv + g);
          }
    };
    auto emit_up = [&] {
      for (int s = 0; s < P->n_slots; ++s)
        for (int i = 0; i < t.n_up; ++i) {
          int32_t* w = em.add(OP_UP, l);
          w[W_A] = s;
          w[W_R0] = i * t.up_rows;
          w[W_R1] = (i + 1) * t.up_rows;
          set_wait(w, 0, cl.slot_ready + l * P->n_slots + s, 1);  // the slot's routing (expert, tokens)
          set_wait(w, 1, cl.xready + l, t.n_rt);                   // the layer's input, staged before routing
          set_wait(w, 2, cl.router_arrive + l, t.n_rt);            // small batches route from the partials themselves
          set_sig(w, cl.up_done + l * P->n_slots + s);
        }
    };
    auto emit_oproj = [&] {
      for (int g = 0; g < Hkv; ++g)
        for (int r = 0; r < t.n_rt; ++r) {
          int32_t* w = em.add(OP_OPROJ, l);
          w[W_A] = g;
          w[W_R0] = r * t.rt;
          w[W_R1] = (r + 1) * t.rt;
          set_wait(w, 0, cl.attn_done + l * Hkv + g, P->merge ? B * n_merge : B);
          resid_epilogue(w, cl, t, l, r, Hkv + P->n_slots);
        }
    };
    auto emit_down = [&] {
      for (int s = 0; s < P->n_slots; ++s)
        for (int r = 0; r < t.n_rt; ++r) {
          int32_t* w = em.add(OP_DOWN, l);
          w[W_A] = s;
          w[W_R0] = r * t.rt;
          w[W_R1] = (r + 1) * t.rt;
          set_wait(w, 0, cl.slot_ready + l * P->n_slots + s, 1);     // routing known: expert weights can stream
          set_wait(w, 1, cl.up_done + l * P->n_slots + s, t.n_up);    // this expert's hidden state is complete
          resid_epilogue(w, cl, t, l, r, Hkv + P->n_slots);
        }
    };
    // per layer: QKV tiles, attention splits, expert up-projection tiles, (merge tasks,) O-projection tiles,
    // expert down-projection tiles (topological; as phases, the attention splits are taken first so that
    // their old K/V stream while the QKV tiles run, and measured faster than the up-projections first; the
    // merge tasks follow the up-projection tiles, which are taken about when the splits' partials land)
    emit_qkv();
    emit_attn();
    emit_up();
    if (P->merge) emit_merge();
    emit_oproj();
    emit_down();
  }
  return MK_OK;
}

}  // namespace mk
