// Library-internal interface between the host launcher (mk_host.cpp) and the allocation-free step (mk_static.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mk.h"

namespace mk {

// Scratch the step's kernel takes its working buffers from instead of the handle's: `base` (device memory of
// `cap` bytes); `zero(p, n, stream)` enqueues a fill of n 32-bit words at p with zeros (a kernel, so that the
// step contains no memset).
struct ScratchOverride {
  uint8_t* base;
  size_t cap;
  void (*zero)(uint32_t* p, int64_t n, hipStream_t stream);
};

// mk_decode_step with the working scratch carved from `so`; MK_E_RANGE (nothing enqueued) if it does not fit.
int launch_step_scratch(mk_model* m, const int32_t* tokens, const int32_t* seq_lens, const int32_t* page_tables, void* kv_pages,
                        float* logits_out, void* stream, const ScratchOverride* so);
// Device the handle was created on.
int handle_device(const mk_model* m);
// Record an error message for mk_last_error and return code.
int set_error(int code, const char* msg);

}  // namespace mk
