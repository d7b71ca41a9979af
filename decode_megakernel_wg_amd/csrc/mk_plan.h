// Host-side task planning: shape validation, tiling and the task list of one decode step.
#pragma once
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/mk.h"
#include "mk_desc.h"

namespace mk {

struct Tiling {
  int rt;           // residual row tile: rows of OPROJ / DOWN / RESID / EMBED tasks
  int n_rt;         // d_model / rt
  int qkv_rows;     // rows per QKV task (divides d_head)
  int router_rows;  // experts per ROUTER task
  int up_rows;      // d_ffn rows (of gate and of up) per UP task
  int lm_rows;      // vocabulary rows per chunk of the LM head's closing phase
  int n_qkv_per_group, n_router, n_up, n_lm;
};

struct Plan {
  int B = 0, n_slots = 0;
  Tiling t{};
  CounterLayout cl{};
  std::vector<int32_t> splits;  // attention splits per sequence
  bool merge = false;           // split-KV partials merged by MERGE tasks (else by each group's last split)
  std::vector<int32_t> desc;    // n_tasks * DESC_WORDS
  int64_t n_tasks() const { return (int64_t)desc.size() / DESC_WORDS; }
};

// Returns MK_OK or an error code with a message.
int validate_desc(const mk_model_desc* d, std::string* msg);
// Tile sizes for a batch of `batch` sequences (only the expert up-projection tiles depend on it).
Tiling choose_tiling(const mk_model_desc* d, int batch);
// force_merge: merge tasks whatever the split counts (otherwise only from ATTN_MERGE_MIN_SPLITS splits on).
int plan_step(const mk_model_desc* d, const mk_batch* batch, Plan* out, std::string* msg, bool force_merge = false);

}  // namespace mk
