/* C ABI of the MI355X decode megakernel (gfx950).
 *
 * One call of mk_decode_step runs one autoregressive decode step of a
 * parallel-transformer MoE decoder as ONE persistent HIP kernel: one workgroup
 * per compute unit pulls per-tile tasks from a task list in global memory and
 * producers and consumers synchronise through global atomic counters, not
 * kernel boundaries.
 *
 * Passages this interface follows (page title, section):
 *  - agenticcommons.xyz "Cohere North Mini Code megakernel serving engine",
 *    section Megakernel 的運作方式: a single resident block per SM reads a task
 *    list (one operation on one tile per task) from global memory; completed
 *    tasks increment counters that consumers spin on.
 *  - aimodeling.com "Cohere megakernel engine: one CUDA file, 1.58x vLLM on
 *    H100", section "Caveats and takeaways": fixed-size task descriptors of 32
 *    int32 words; batch size at most 8; BF16.  Section "From demo to a full
 *    serving system": paged attention, ragged sequence lengths, continuous
 *    batching.
 *  - agenticcommons.xyz, section 對產品開發者的意義: one calling convention over
 *    tiled GEMM and paged attention.
 *
 * Conventions.  Every call returns int: MK_OK (0) or a negative MK_E_* code;
 * mk_last_error() gives the text of the calling thread's last error.  No C++
 * exception crosses this boundary.  A handle serves one stream at a time and
 * is not re-entrant.  All pointers named "device" are HIP device memory owned
 * by the caller unless stated otherwise.
 */
#ifndef MK_H
#define MK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MK_ABI_VERSION 2
#define MK_DESC_WORDS 32   /* int32 words per task descriptor (128 bytes) */
#define MK_MAX_BATCH 8
#define MK_PAGE_SIZE 16

enum {
  MK_OK = 0,
  MK_E_INVAL = -1,       /* bad argument: null pointer, bad shape, out-of-range value */
  MK_E_UNSUPPORTED = -2, /* shape outside the compiled kernel variants */
  MK_E_NOMEM = -3,       /* device or pinned-host allocation failed */
  MK_E_HIP = -4,         /* a HIP runtime call failed */
  MK_E_STATE = -5,       /* call out of order (e.g. decode before a task list is built) */
  MK_E_RANGE = -6,       /* output buffer too small; the needed size is still reported */
  MK_E_DEVICE = -7       /* the kernel reported a fault (bad token/page, wait timeout) */
};

/* Model shape.  Supported: d_head in {64, 128}; n_q_heads / n_kv_heads in {2, 4, 8};
 * d_model a multiple of 256, at most 4096; d_ffn a multiple of 128, at most 2048;
 * n_experts <= 256, top_k <= 8 and <= n_experts; vocab a multiple of 64; page_size 16;
 * 1 <= max_batch <= 8. */
typedef struct mk_model_desc {
  int32_t abi_version; /* MK_ABI_VERSION */
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, d_head, n_experts, top_k, d_ffn, vocab;
  int32_t page_size;         /* tokens per KV page; must be 16 */
  int32_t max_batch;         /* largest batch any step will use */
  int32_t max_pages_per_seq; /* row length of page_tables */
  int64_t n_pages;           /* pages per layer in the KV pool */
  float rms_eps;             /* RMSNorm epsilon */
  float rope_base;           /* RoPE base (rotate-half pairing (i, i + d_head/2)) */
  const float* router_bias;  /* host [n_experts] added to router logits, or NULL; copied */
} mk_model_desc;

/* Weights: device pointers to BF16, row-major [out][in].  Per-layer entries are host arrays of
 * n_layers device pointers.  Read-only; they must stay valid until mk_free_model. */
typedef struct mk_weights {
  const void* embed;            /* [vocab][d_model] */
  const void* lm_head;          /* [vocab][d_model] (untied) */
  const void* final_norm;       /* [d_model] */
  const void* const* attn_norm; /* [L] -> [d_model] (the layer's RMSNorm gain) */
  const void* const* wq;        /* [L] -> [n_q_heads*d_head][d_model] */
  const void* const* wk;        /* [L] -> [n_kv_heads*d_head][d_model] */
  const void* const* wv;        /* [L] -> [n_kv_heads*d_head][d_model] */
  const void* const* wo;        /* [L] -> [d_model][n_q_heads*d_head] */
  const void* const* w_router;  /* [L] -> [n_experts][d_model] */
  const void* const* w_gate;    /* [L] -> [n_experts][d_ffn][d_model] */
  const void* const* w_up;      /* [L] -> [n_experts][d_ffn][d_model] */
  const void* const* w_down;    /* [L] -> [n_experts][d_model][d_ffn] */
} mk_weights;

/* A step's batch as seen by the task builder.  An entry is one token: a decode token of its own sequence,
 * or one token of a chunk of consecutive positions of one sequence (chunked prefill, mixed prefill +
 * decode steps): first_of[b] names the chunk's first entry; the chunk's entries are consecutive, in
 * position order (seq_lens[b] = seq_lens[first_of[b]] + b - first_of[b]), and read the cache only below the
 * chunk's first position (each entry writes its own K/V slot).  first_of NULL = every entry is a decode
 * token of its own sequence. */
typedef struct mk_batch {
  int32_t batch;            /* 1..max_batch */
  const int32_t* seq_lens;  /* host [batch]: prior positions of each sequence (its new token's position) */
  const int32_t* first_of;  /* host [batch] or NULL: first entry of each entry's chunk */
} mk_batch;

typedef struct mk_model mk_model;

/* Create a handle: validates the shape, records the weight pointers, allocates the handle's own
 * device scratch (counters, fp32 activations, partials, routing and debug buffers) and sizes the
 * grid to one workgroup per compute unit of the current device.
 * Errors: MK_E_INVAL, MK_E_UNSUPPORTED, MK_E_NOMEM, MK_E_HIP.
 * Passage: agenticcommons.xyz "Cohere North Mini Code megakernel serving engine", section 三個實際的加速來源, item 1
 * (the parallel transformer layer: attention and the MoE feed-forward both read one RMSNorm of the residual
 * stream, joined by a fused residual add) and section 為什麼 decode 慢 (a sparse MoE model whose active weights
 * stream from HBM once per step, in BF16); aimodeling.com "Cohere megakernel engine: one CUDA file, 1.58x vLLM
 * on H100", section "Caveats and takeaways" (BF16, batches of at most 8).
 */
int mk_load_model(const mk_model_desc* desc, const mk_weights* w, mk_model** out);

/* Build the step's task list on the host (deterministic, no device work): fixed-size descriptors of
 * MK_DESC_WORDS int32 in topological order (every wait refers to an earlier task).  The list is kept
 * in the handle and uploaded by the next mk_decode_step.  Attention split counts follow the host
 * lengths; split bounds are recomputed on the device from the step's seq_lens, so a list stays valid
 * while lengths grow.  tasks_out (nullable, host) receives a copy when cap >= the task count;
 * *n_tasks always receives the count.
 * Errors: MK_E_INVAL (batch outside 1..max_batch, negative length, null batch), MK_E_RANGE (cap too small).
 * Passage: agenticcommons.xyz "Cohere North Mini Code megakernel serving engine", section Megakernel 的運作方式
 * (the step as a list of tasks in global memory, one operation on one tile each); aimodeling.com "Cohere
 * megakernel engine: one CUDA file, 1.58x vLLM on H100", section "One persistent kernel for the whole decode
 * step" (a task waits only for its own producers, e.g. an O-projection tile for its KV group's attention) and
 * section "Caveats and takeaways" (fixed descriptors of 32 int32 words).
 */
int mk_build_tasks(mk_model* m, const mk_batch* batch, int32_t* tasks_out, int64_t cap, int64_t* n_tasks);

/* Enqueue one decode step on `stream` (a hipStream_t; NULL = default stream); asynchronous.
 *  tokens      device int32 [B]                      input token of each sequence
 *  seq_lens    device int32 [B]                      prior positions (= position of the new token); not modified
 *  page_tables device int32 [B][max_pages_per_seq]   logical page -> physical page; page_tables[b][seq_lens[b]/16] must be valid
 *  kv_pages    device BF16  [n_layers][n_pages][2 (K,V)][n_kv_heads][16][d_head]; positions [0, seq_lens[b]) are read and
 *              position seq_lens[b] is written (post-RoPE K and V) in every layer
 *  logits_out  device fp32  [B][vocab]
 * B is the batch of the last mk_build_tasks.  The greedy next tokens go to the buffer of mk_next_tokens.
 * Errors before launch: MK_E_STATE (no task list), MK_E_INVAL (null pointer), MK_E_HIP.  Faults found by the
 * kernel (token or page out of range, a dependency wait that timed out) are reported by mk_status.
 * Passage: agenticcommons.xyz "Cohere North Mini Code megakernel serving engine", section Megakernel 的運作方式
 * (one resident workgroup per compute unit takes tasks from the list; completions increment counters that
 * consumers spin on) and section 三個實際的加速來源 (tile tasks in place of kernel waves, per-producer dependencies,
 * weights loaded before the activations they meet); aimodeling.com "Cohere megakernel engine: one CUDA file,
 * 1.58x vLLM on H100", section "From demo to a full serving system" (paged attention over ragged sequence
 * lengths).
 */
int mk_decode_step(mk_model* m, const int32_t* tokens, const int32_t* seq_lens, const int32_t* page_tables, void* kv_pages,
                   float* logits_out, void* stream);

/* One step whose batch holds chunks of consecutive positions of one sequence (chunked prefill, or prefill
 * chunks mixed with decode tokens); the same tasks and kernel as mk_decode_step (each entry is a token of
 * the batch), except that the attention of a chunk's entry b reads the cache below the chunk's first
 * position and takes positions first_of..b from this step's own projections (causal within the chunk).
 * Arguments as mk_decode_step, plus
 *  first_of    device int32 [B]   the host first_of of the last mk_build_tasks (its batch's chunk map)
 * Entries of one chunk pass the same page table row.  A first_of that contradicts seq_lens (not a run of
 * consecutive positions) is reported by mk_status as a sequence-length fault.
 * Passage: aimodeling.com "Cohere megakernel engine: one CUDA file, 1.58x vLLM on H100", section "Caveats and
 * takeaways" and debriefse.vercel.app "Cohere släpper inferensmotor som minskar väntan på GPU:n", section
 * "Fortfarande en smal motor": on the pages prefill runs outside the megakernel and is never mixed with
 * decode; this call runs both inside it.
 * Errors before launch: as mk_decode_step, and MK_E_INVAL for a null first_of. */
int mk_mixed_step(mk_model* m, const int32_t* tokens, const int32_t* seq_lens, const int32_t* first_of, const int32_t* page_tables,
                  void* kv_pages, float* logits_out, void* stream);

/* Allocation-free decode step, for callers that cannot allocate device memory while they step (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).  The same step as mk_decode_step on
 * the same handle and arguments, with the same results, but the kernel's working scratch (counters,
 * activations, attention partials, router partials, expert slot table and states, LM-head bests) comes from
 * the library's static device scratch of MK_STATIC_SCRATCH_BYTES instead of the handle's buffers.  Each
 * device holds its own copy of that scratch from the library's load until the process ends.  The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine): it enqueues a zero fill of the
 * scratch's counters (a kernel, not a memset), the task list's upload when mk_build_tasks ran since the last
 * step (into the handle's buffer), and the step.  The current device must be the handle's.  Every call on one
 * device uses that device's one scratch, which keeps the last call's contents: calls that overlap on one device
 * (several streams or handles) race.  The handle's routing records, final counter values and greedy tokens are
 * written as by mk_decode_step; its expert slot table (MK_DBGK_SLOTS) is not.
 * Errors: as mk_decode_step; MK_E_RANGE (nothing enqueued) if the planned step needs more than
 * MK_STATIC_SCRATCH_BYTES (the message gives both sizes); MK_E_STATE if the current device is not the
 * handle's; MK_E_HIP if the scratch's device address cannot be obtained. */
#define MK_STATIC_SCRATCH_BYTES (16u << 20)
int mk_decode_step_static(mk_model* m, const int32_t* tokens, const int32_t* seq_lens, const int32_t* page_tables, void* kv_pages,
                          float* logits_out, void* stream);

/* Device buffer int32 [max_batch] holding the last step's greedy tokens (argmax, lowest index on ties);
 * it may be passed straight back as the next step's `tokens`.  Owned by the handle.
 * Passage: aimodeling.com "Cohere megakernel engine: one CUDA file, 1.58x vLLM on H100", section "From demo to
 * a full serving system" (continuous batching: each step's output tokens are the next step's inputs).  The
 * pages do not name the sampling rule; greedy decoding is the plainest reading of a decode-only throughput
 * test.
 */
int mk_next_tokens(mk_model* m, int32_t** dev_ptr);

/* Synchronise `stream`, then return MK_OK or MK_E_DEVICE if the kernel raised a fault since the last
 * call (the fault word is cleared and the handle's counters are reset).
 * Passage: none on the pages, which do not say what happens when a dependency is never met; every wait here is
 * bounded, and a fault ends the step with every workgroup exiting normally.
 */
int mk_status(mk_model* m, void* stream);

/* Debug switches (bit flags, MK_DBG_*) and read-back of the handle's debug buffers.  MK_DBG_WIDE_GEMV runs
 * batches of 1-2 sequences with the matrix-core arithmetic of batches of 3-8 (hi and lo activation parts in
 * separate instructions accumulating into one sum), so that a sequence's results then equal, bit for bit,
 * its results inside a larger batch; without it the two batch classes agree to rounding only. */
enum { MK_DBG_DUMP_N = 1, MK_DBG_TIMESTAMPS = 2, MK_DBG_WIDE_GEMV = 4, MK_DBG_PAGE_WALK = 8, MK_DBG_DROP_SIGNAL = 16,
       MK_DBG_VALU_GEMV = 32, MK_DBG_COUNT_TASKS = 64, MK_DBG_MERGE_TASKS = 128 };
/* MK_DBG_MERGE_TASKS makes the following mk_build_tasks plan merge tasks whatever the split counts.  By default
 * the split-KV partials of a (sequence, KV group) are merged by the split that arrives last, and only a plan
 * with a sequence of 33 splits or more (long contexts) merges them in separate tasks, one per head of each
 * (sequence, KV group) (none when a sequence has more than 128 splits at d_head 128).  Both give the same
 * results, bit for bit. */
/* MK_DBG_COUNT_TASKS counts every task's completions (MK_DBGK_TASK_DONE). */
/* MK_DBG_VALU_GEMV runs the GEMV tiles of a batch of one sequence on the VALU (fp32 FMAs on the same loads and
 * the same hi + lo activations) instead of the matrix cores, to compare the two engines; results agree to
 * rounding.  MK_DBG_WIDE_GEMV takes precedence. */
/* MK_DBG_PAGE_WALK records every attention page walk (MK_DBGK_PAGE_WALK).  MK_DBG_DROP_SIGNAL exercises the
 * device watchdog from the host: the uploaded task list loses the completion signal of its first QKV task
 * and dependency waits give up after 4096 polls (about 2 ms instead of about 1 s), so the step ends with
 * every workgroup exiting normally and mk_status reporting MK_E_DEVICE (a wait that timed out). */
enum {
  MK_DBGK_ROUTE_SEL = 1,     /* int32 [n_layers][batch][top_k]: last step's expert selection (always recorded) */
  MK_DBGK_ROUTE_GATE = 2,    /* fp32  [n_layers][batch][top_k]: its gates (always recorded) */
  MK_DBGK_ROUTER_LOGITS = 3, /* fp32  [n_layers][batch][n_experts] (always recorded) */
  MK_DBGK_NORM_IN = 4,       /* fp32  [n_layers][batch][d_model]: each layer's RMSNorm output (MK_DBG_DUMP_N) */
  MK_DBGK_COUNTERS = 5,      /* uint32 [n_counters]: final values of the last step, copied just before the kernel
                                resets them to zero for the next step (always recorded) */
  MK_DBGK_TASK_DONE = 6,     /* uint32 [n_tasks]: completions per task in the last step (MK_DBG_COUNT_TASKS) */
  MK_DBGK_TIMESTAMPS = 7,    /* uint64 [n_tasks][8]: claim, dependencies met, end (100 MHz wall clock), hardware id
                                (XCC id << 32 | HW_ID register), then up to 4 task-specific sub-phase marks (0 = unset);
                                MK_DBG_TIMESTAMPS */
  MK_DBGK_PAGE_WALK = 8,     /* uint32 [n_layers][batch][n_kv_heads][4]: per attention walk, the cache pages read, the sum
                                over them of (logical page + 1) * physical page (mod 2^32), the positions attended
                                (cached + new) and 1 + physical page * 16 + slot of the entry's K/V write (0 = none);
                                MK_DBG_PAGE_WALK */
  MK_DBGK_SLOTS = 9          /* int32 [n_layers][n_slots][32]: expert slot table (n_slots = min(n_experts, batch *
                                top_k)): expert (-1 = unused), token count, then (token, rank, gate bits) per token of the
                                slot in ascending token order (always recorded) */
};
/*
 * Passage: none on the pages; the debug records make the step's integer work checkable: the task graph's
 * counters (agenticcommons.xyz "Cohere North Mini Code megakernel serving engine", section Megakernel 的運作方式),
 * the routing and expert slot table (section 三個實際的加速來源, item 1) and the page walks (aimodeling.com "Cohere
 * megakernel engine: one CUDA file, 1.58x vLLM on H100", section "From demo to a full serving system").
 */
int mk_debug_set(mk_model* m, uint32_t flags);
/* Copies `bytes` of debug buffer `kind` to host memory; synchronises the device first.
 * Errors: MK_E_INVAL (unknown kind), MK_E_STATE (kind not enabled), MK_E_RANGE (bytes larger than the buffer). */
int mk_debug_read(mk_model* m, int kind, void* host_dst, int64_t bytes);

/* Override the grid: n_workgroups persistent workgroups (0 = one per compute unit, at most 1024).  Results
 * do not depend on it (every reduction has a fixed order); it exists for testing and tuning.  Takes effect at
 * the next mk_decode_step (every grid takes the same list in order through one counter).
 * Errors: MK_E_INVAL (null handle, n_workgroups outside 0..1024).
 * Passage: agenticcommons.xyz "Cohere North Mini Code megakernel serving engine", section 三個實際的加速來源, item 1
 * (tile tasks spread over whichever compute units are free, so no work is tied to a wave of the grid).
 */
int mk_set_grid(mk_model* m, int32_t n_workgroups);

/* Release the handle and its device memory (after the stream's work has finished). */
int mk_free_model(mk_model* m);

/* Text of the calling thread's last error ("" if none). */
const char* mk_last_error(void);

/* Pure host planning, for tools and tests (no device needed): the task list mk_build_tasks would emit
 * for `desc` and `batch` (without MK_DBG_MERGE_TASKS), in topological order (the order the workgroups take it in).  n_tasks receives the
 * task count, n_counters (nullable) the counter count; tasks_out may be null to query the sizes.
 * Errors: MK_E_INVAL (bad shape or batch), MK_E_RANGE (cap smaller than the task count).
 * Passage: as mk_build_tasks.
 */
int mk_plan_tasks(const mk_model_desc* desc, const mk_batch* batch, int32_t* tasks_out, int64_t cap, int64_t* n_tasks,
                  int32_t* n_counters);

#ifdef __cplusplus
}
#endif

#endif
