// Task descriptors and counter layout shared by the host planner and the persistent kernel.
//
// A descriptor is 32 int32 words (aimodeling.com "Cohere megakernel engine: one CUDA file, 1.58x vLLM
// on H100", section "Caveats and takeaways": one uniform ABI of 32-int32 task descriptors).  The word
// meanings below and the opcode set are this library's own.
#pragma once
#include <stdint.h>

namespace mk {

enum Op : int32_t {
  OP_EMBED = 1,   // x[b][rows] = embed[token_b][rows]; partial sum of squares of the rows  -> XREADY[0]
  OP_ROUTER = 2,  // (reserved: router logits are partials of the residual row tiles; the last tile routes)
  OP_QKV = 3,     // rows [r0, r1) of KV group g's fused [q heads; k; v] projection     -> QKV_DONE[l][g]
  OP_ATTN = 4,    // split s of (sequence b, KV group g): partial softmax(qK^T)V; last arriver combines -> ATTN_DONE[l][g]
  OP_UP = 5,      // gate+up rows [r0, r1) of expert slot s, SwiGLU (waits SLOT_READY)     -> UP_DONE[l][s]
  OP_OPROJ = 6,   // rows [r0, r1) of Wo restricted to group g's columns; residual epilogue (see below)
  OP_DOWN = 7,    // rows [r0, r1) of expert slot s's down projection, times the gate; residual epilogue
  OP_RESID = 8,   // (reserved: the residual add is the epilogue of the last O-proj / down task of a row tile)
  OP_LMHEAD = 9,  // (reserved: the LM head runs as the kernel's closing phase over a shared chunk pool)
  OP_COUNT = 10
};

// Descriptor words.
enum Word : int {
  W_OP = 0,
  W_LAYER = 1,
  W_A = 2,  // EMBED/RESID: row tile; QKV/OPROJ: KV group; UP/DOWN: slot; ATTN: sequence; LMHEAD: tile
  W_B = 3,  // ATTN: KV group
  W_C = 4,  // ATTN: split index
  W_D = 5,  // ATTN: split count
  W_R0 = 6,
  W_R1 = 7,
  W_WAIT0 = 8,  // 4 waits of (counter, target): words 8..15; counter -1 = none
  W_SIG = 16,   // counter to increment on completion (-1 = none)
  W_SIGN = 17,  // increment
  W_ARR = 18,   // arrival counter for the last-arriver epilogue (-1 = none)
  W_ARRN = 19,  // arrivals expected
  W_SIGR = 20,  // counters signalled: [W_SIG, W_SIG + W_SIGR) (router: one per expert slot, the value
                // written there is the slot's routing, at least 1)
  W_RT = 22,    // residual row tile of OPROJ / DOWN / EMBED tasks
  W_ARR2 = 24,  // row-tile tasks: arrival counter of the next layer's router partials (-1 = none: last layer)
  W_ARRN2 = 25, // arrivals expected there (row tiles)
  W_RSIG = 26,  // first expert-slot counter of the next layer, signalled by the tile that routes it
  W_RSIGR = 27, // expert slots
  W_SEQ = 31    // task index (debug)
};
constexpr int N_WAITS = 4;
// Scheduling.  With two or more workgroups the list runs as phases: the embedding tiles, then per layer
// each maximal run of one operation (QKV tiles, attention splits, expert up-projection tiles,
// O-projection tiles, expert down-projection tiles).  Each phase is a pool that every workgroup takes
// tasks from one at a time (an atomic counter; nothing is claimed ahead), moving on to the next phase
// once a take finds the pool empty.  A phase's tasks thus go to whichever workgroups are free, one each,
// instead of queueing behind busy workgroups that hold tickets, and the attention and expert branches
// of a layer share all compute units.  Phases follow the list's topological order and a workgroup enters
// a phase only once every task of the previous one has been taken by a workgroup that runs it at once,
// so the earliest unfinished task can always run.  One workgroup claims the list in order.
constexpr int DESC_WORDS = 32;

// Tile sizes chosen by the planner (rows per task); the kernel reads r0/r1 from the descriptor.
constexpr int ATTN_SPLIT_POS = 256;  // fewest positions per attention split
constexpr int ATTN_TARGET_TASKS = 96;  // attention splits per layer the planner aims for (all sequences, KV groups)
constexpr int ATTN_LONG_MIN_POS = 1024;  // positions per split from which long contexts aim at ATTN_LONG_TASKS
constexpr int ATTN_LONG_TASKS = 192;     // attention splits per layer for long contexts (measured best of 160-320)
constexpr int ATTN_MAX_SPLIT_POS = 4096;  // most positions per split the planner chooses (before the split cap)
constexpr int ATTN_MAX_SPLIT_PAGES = 512;  // pages one split may cover (its page list is staged in LDS; the
                                           // last split of a sequence also takes the growth since planning)
constexpr int ATTN_MAX_SPLITS = 256;
constexpr int SLOT_WORDS = 32;
constexpr int LM_MAX_WG = 1024;  // most workgroups a launch may have (stride of the LM head's per-workgroup bests)  // routing table entry per expert slot: expert, token count, (token, rank, gate) x 8

// Counter index layout for a model/batch; computed identically by planner and host launcher.
struct CounterLayout {
  int32_t ticket, done, xready, phase, qkv_done, router_arrive, slot_ready, attn_arrive, attn_done, up_done,
      resid_arrive, lm_arrive, lm_pool, total;
  int32_t n_layers, n_kv, n_slots, n_row_tiles, batch;
  void build(int L, int Hkv, int B, int slots, int nrt) {
    n_layers = L;
    n_kv = Hkv;
    n_slots = slots;
    n_row_tiles = nrt;
    batch = B;
    int32_t o = 0;
    ticket = o; o += 32;     // own cache line (claim order with one workgroup)
    done = o; o += 32;
    xready = o; o += L + 1;
    phase = o; o += 1 + 5 * L;  // next untaken task of each phase
    qkv_done = o; o += L * Hkv;
    router_arrive = o; o += L;
    slot_ready = o; o += L * slots;
    attn_arrive = o; o += L * B * Hkv;
    attn_done = o; o += L * Hkv;
    up_done = o; o += L * slots;
    resid_arrive = o; o += L * nrt;
    lm_arrive = o; o += 1;
    lm_pool = o; o += 1;     // next unclaimed 128-row vocabulary chunk of the LM head
    total = (o + 31) & ~31;
  }
};

}  // namespace mk
