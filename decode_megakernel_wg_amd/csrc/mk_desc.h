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
  OP_QKV = 3,     // rows [r0, r1) of KV group g's fused [q heads; k; v] projection     -> QKV_DONE[l][g]
  OP_ATTN = 4,    // split s of (sequence b, KV group g): partial softmax(qK^T)V; last arriver combines -> ATTN_DONE[l][g]
                  // (with merge tasks: every split counts itself into ATTN_ARRIVE[l][b][g] instead)
  OP_UP = 5,      // gate+up rows [r0, r1) of expert slot s, SwiGLU (waits SLOT_READY)     -> UP_DONE[l][s]
  OP_OPROJ = 6,   // rows [r0, r1) of Wo restricted to group g's columns; residual epilogue (see below)
  OP_DOWN = 7,    // rows [r0, r1) of expert slot s's down projection, times the gate; residual epilogue
  OP_MERGE = 8    // heads [h0, h0 + nh) of (sequence b, KV group g): log-sum-exp merge of the splits -> ATTN_DONE[l][g]
};
// The router is not a task (the last residual row tile of a layer routes the next), nor is the residual add
// (the epilogue of a row tile's last O-proj or down-projection task), nor the LM head (the kernel's closing
// phase over a shared chunk pool).

// Descriptor words.
enum Word : int {
  W_OP = 0,
  W_LAYER = 1,
  W_A = 2,  // EMBED: row tile; QKV/OPROJ: KV group; UP/DOWN: slot; ATTN, MERGE: sequence
  W_B = 3,  // ATTN, MERGE: KV group
  W_C = 4,  // ATTN: split index; MERGE: first head of the group it merges
  W_D = 5,  // ATTN, MERGE: split count
  W_R0 = 6,
  W_R1 = 7,
  W_WAIT0 = 8,  // 4 waits of (counter, target): words 8..15; counter -1 = none
  W_SIG = 16,   // counter to increment on completion (-1 = none)
  W_SIGN = 17,  // increment
  W_ARR = 18,   // arrival counter for the last-arriver epilogue (-1 = none)
  W_ARRN = 19,  // arrivals expected
  W_SIGR = 20,  // counters signalled: [W_SIG, W_SIG + W_SIGR) (1 for every task of this planner)
  W_RT = 22,    // residual row tile of OPROJ / DOWN / EMBED tasks
  W_ARR2 = 24,  // row-tile tasks: arrival counter of the next layer's router partials (-1 = none: last layer)
  W_ARRN2 = 25, // arrivals expected there (row tiles)
  W_RSIG = 26,  // first expert-slot counter of the next layer, signalled by the tile that routes it
  W_RSIGR = 27, // expert slots
  W_SEQ = 31    // task index (debug)
};
constexpr int N_WAITS = 4;
// Scheduling.  The list is one pool: every workgroup takes the next untaken task in list order through one
// atomic counter (the ticket), runs it, and takes again; nothing is claimed ahead, so a task goes to
// whichever workgroup is free first and the attention and expert branches of a layer share all compute
// units.  Every take but each workgroup's last returns a task (no take comes back from an exhausted pool
// part-way through the list).  The list is topological and a task is taken only by a workgroup that runs it
// at once, so the earliest unfinished task can always run.
// Phases (maximal runs of one operation within a layer: the embedding tiles, then per layer QKV tiles,
// attention splits, expert up-projection tiles, O-projection tiles, expert down-projection tiles) classify
// a take.  Expert phases list their tiles slot by slot, the same number per slot; slots are numbered in
// ascending expert order, so once a layer is routed (its used-slot count published) the tiles of its unused
// slots are the tail of each expert phase, and the workgroup that meets that tail first moves the ticket past
// it.
constexpr int DESC_WORDS = 32;

// Tile sizes chosen by the planner (rows per task); the kernel reads r0/r1 from the descriptor.
constexpr int ATTN_SPLIT_POS = 256;  // fewest positions per attention split
constexpr int ATTN_TARGET_TASKS = 96;  // attention splits per layer the planner aims for (all sequences, KV groups)
constexpr int ATTN_LONG_MIN_POS = 1024;  // positions per split from which long contexts aim at ATTN_LONG_TASKS
constexpr int ATTN_LONG_TASKS = 192;     // attention splits per layer for long contexts (measured best of 160-320)
constexpr int ATTN_LONGER_MIN_POS = 2048;  // positions per split from which ATTN_LONGER_TASKS is aimed at instead
constexpr int ATTN_LONGER_TASKS = 224;     // (measured: 128K 4.55 -> 4.48 ms/step; 64K, with 1408-position splits, is
                                           // fastest at 192: 3.21 against 3.36 ms at 224)
constexpr int ATTN_MAX_SPLIT_POS = 4096;  // most positions per split the planner chooses (before the split cap)
constexpr int ATTN_MAX_SPLIT_PAGES = 512;  // pages one split may cover (its page list is staged in LDS; the
                                           // last split of a sequence also takes the growth since planning)
constexpr int ATTN_MAX_SPLITS = 256;
// Long contexts merge their splits in separate tasks: from ATTN_MERGE_MIN_SPLITS splits of one sequence on,
// the partials of every (sequence, KV group) are merged by up to ATTN_MERGE_TASKS tasks, one per head of the
// group (at most), instead of by the split that arrives last.  One workgroup reads other workgroups' fresh
// partials at only about 10 GB/s (measured), so a last-arriver merge of about 48 splits (200 KB) takes about
// 10 us; one head per task reads an eighth of it, at the cost of one more hop.
constexpr int ATTN_MERGE_MIN_SPLITS = 33;
constexpr int ATTN_MERGE_TASKS = 8;
// A merge task stages its heads' rows of every split ((d_head + 2) floats each) in LDS; a plan whose rows
// exceed the area uses the last-arriver merge.
constexpr int ATTN_MERGE_STAGE_FLOATS = 16640;  // 128 splits x 1 head x (128 + 2) floats
constexpr int SLOT_WORDS = 32;
constexpr int LM_MAX_WG = 1024;  // most workgroups a launch may have (stride of the LM head's per-workgroup bests)  // routing table entry per expert slot: expert, token count, (token, rank, gate) x 8

// Counter index layout for a model/batch; computed identically by planner and host launcher.  Counter c lives
// at word c * CTR_STRIDE of the counter array (one 128-byte line per counter).
constexpr int CTR_STRIDE = 32;
struct CounterLayout {
  int32_t ticket, done, xready, qkv_done, router_arrive, slot_ready, slots_used, attn_arrive, attn_done, up_done,
      resid_arrive, lm_arrive, lm_pool, total;
  int32_t n_layers, n_kv, n_slots, n_row_tiles, batch;
  void build(int L, int Hkv, int B, int slots, int nrt) {
    n_layers = L;
    n_kv = Hkv;
    n_slots = slots;
    n_row_tiles = nrt;
    batch = B;
    int32_t o = 0;
    ticket = o; o += 32;     // next untaken task of the list
    done = o; o += 32;
    xready = o; o += L + 1;
    qkv_done = o; o += L * Hkv;
    router_arrive = o; o += L;
    slot_ready = o; o += L * slots;
    slots_used = o; o += L;  // distinct experts of each layer's routing (0 until the layer is routed)
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
