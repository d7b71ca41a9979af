// The allocation-free decode step: the persistent kernel's working scratch in a file-scope device array.
//
// For callers that cannot allocate device memory while they step (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).  The array `scratch` is a host-side stand-in in host code: its
// device address is obtained per device with hipGetSymbolAddress (once, with that device current) and only
// that address is passed to kernels and fills.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "../../include/mk.h"
#include "mk_internal.h"

namespace {

// One copy per device, held from the module's load until the process ends.
__device__ __align__(256) uint8_t scratch[MK_STATIC_SCRATCH_BYTES];

__global__ void zero_words(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0u;
}

void zero_fill(uint32_t* p, int64_t n, hipStream_t stream) {
  const int threads = 256;
  const int64_t blocks = std::min<int64_t>((n + threads - 1) / threads, 1024);
  hipLaunchKernelGGL(zero_words, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(threads), 0, stream, p, n);
}

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
uint8_t* g_ptr[MAX_DEVICES] = {};

// Device address of this device's scratch (the current device's), looked up on its first use.
int scratch_address(int dev, uint8_t** out) {
  if (dev < 0 || dev >= MAX_DEVICES) return mk::set_error(MK_E_STATE, "device index beyond the static scratch table");
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return mk::set_error(MK_E_HIP, (std::string("hipGetSymbolAddress of the static scratch failed: ") + hipGetErrorString(e)).c_str());
    g_ptr[dev] = static_cast<uint8_t*>(p);
  }
  *out = g_ptr[dev];
  return MK_OK;
}

}  // namespace

extern "C" int mk_decode_step_static(mk_model* m, const int32_t* tokens, const int32_t* seq_lens, const int32_t* page_tables,
                                     void* kv_pages, float* logits_out, void* stream) {
  if (!m) return mk::set_error(MK_E_INVAL, "null handle");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return mk::set_error(MK_E_HIP, "hipGetDevice failed");
  if (dev != mk::handle_device(m)) return mk::set_error(MK_E_STATE, "the handle's device is not the current device");
  uint8_t* base = nullptr;
  const int rc = scratch_address(dev, &base);
  if (rc) return rc;
  const mk::ScratchOverride so{base, (size_t)MK_STATIC_SCRATCH_BYTES, zero_fill};
  return mk::launch_step_scratch(m, tokens, seq_lens, page_tables, kv_pages, logits_out, stream, &so);
}
