// Seeded synthetic inputs, device side: fill kernels producing the same bytes as synth.c.
// Used by the GPU harness to materialise large synthetic weights and KV prefixes in HBM
// without a host round trip.  No arithmetic of the decode method lives here.
#include <hip/hip_runtime.h>

#define SYNTH_FN __host__ __device__ static inline
#include "synth_core.h"
#include "../include/synth.h"

namespace {

__global__ __launch_bounds__(256) void fill_bf16_kernel(uint16_t* __restrict__ dst, int64_t n, uint64_t key, uint64_t index0,
                                                        const uint64_t* __restrict__ thr, const uint16_t* __restrict__ guide) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 8;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8; i < n; i += stride) {
    if (i + 8 <= n && ((reinterpret_cast<uintptr_t>(dst + i) & 15) == 0)) {
      uint16_t v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = synth_bf16_from_bits(synth_u64(key, index0 + (uint64_t)(i + j)), thr, guide);
      uint4 w;
      w.x = v[0] | ((uint32_t)v[1] << 16);
      w.y = v[2] | ((uint32_t)v[3] << 16);
      w.z = v[4] | ((uint32_t)v[5] << 16);
      w.w = v[6] | ((uint32_t)v[7] << 16);
      *reinterpret_cast<uint4*>(dst + i) = w;
    } else {
      for (int64_t j = i; j < n && j < i + 8; ++j) dst[j] = synth_bf16_from_bits(synth_u64(key, index0 + (uint64_t)j), thr, guide);
    }
  }
}

// One thread per (layer, position, K/V, head) row of d_head values.
__global__ __launch_bounds__(256) void fill_kv_kernel(uint16_t* __restrict__ kv, int n_layers_buf, int layer0, int64_t n_pages,
                                                      int n_kv_heads, int d_head, int page_size, const int32_t* __restrict__ page_table,
                                                      int64_t pos0, int64_t npos, uint64_t key, const uint64_t* __restrict__ thr,
                                                      const uint16_t* __restrict__ guide, uint32_t* bad) {
  const int64_t rows = (int64_t)n_layers_buf * npos * 2 * n_kv_heads;
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < rows; r += (int64_t)gridDim.x * blockDim.x) {
    int64_t t = r;
    const int head = (int)(t % n_kv_heads);
    t /= n_kv_heads;
    const int kvs = (int)(t % 2);
    t /= 2;
    const int64_t pos = pos0 + t % npos;
    const int lb = (int)(t / npos);
    const int64_t ph = page_table[pos / page_size];
    if (ph < 0 || ph >= n_pages) {
      if (bad) atomicAdd(bad, 1u);
      continue;
    }
    uint16_t* row = kv + ((((int64_t)lb * n_pages + ph) * 2 + kvs) * n_kv_heads + head) * (int64_t)page_size * d_head +
                    (pos % page_size) * (int64_t)d_head;
    const uint64_t i0 = synth_kv_index(layer0 + lb, pos, kvs, head, 0, n_kv_heads, d_head);
    for (int d = 0; d < d_head; ++d) row[d] = synth_bf16_from_bits(synth_u64(key, i0 + (uint64_t)d), thr, guide);
  }
}

int grid_for(int64_t work, int per_block) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

extern "C" int synth_dev_fill_bf16(void* dst, int64_t n, uint64_t seed, uint64_t stream, uint64_t index0, const uint64_t* thr,
                                   const uint16_t* guide, void* hip_stream) {
  if (n < 0 || (n > 0 && (!dst || !thr || !guide))) return -1;
  if (n == 0) return 0;
  const uint64_t key = synth_key(seed, stream);
  fill_bf16_kernel<<<grid_for(n, 256 * 8), 256, 0, (hipStream_t)hip_stream>>>((uint16_t*)dst, n, key, index0, thr, guide);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

extern "C" int synth_dev_fill_kv_paged(void* kv, int n_layers_buf, int layer0, int64_t n_pages, int n_kv_heads, int d_head,
                                       int page_size, const int32_t* page_table, int seq_id, int64_t pos0, int64_t pos1, uint64_t seed,
                                       const uint64_t* thr, const uint16_t* guide, uint32_t* bad_dev, void* hip_stream) {
  if (pos0 < 0 || pos1 < pos0 || page_size <= 0 || n_kv_heads <= 0 || d_head <= 0 || n_layers_buf <= 0) return -1;
  if (pos1 == pos0) return 0;
  if (!kv || !page_table || !thr || !guide) return -1;
  const uint64_t key = synth_key(seed, (uint64_t)seq_id);
  const int64_t rows = (int64_t)n_layers_buf * (pos1 - pos0) * 2 * n_kv_heads;
  fill_kv_kernel<<<grid_for(rows, 256), 256, 0, (hipStream_t)hip_stream>>>((uint16_t*)kv, n_layers_buf, layer0, n_pages, n_kv_heads,
                                                                          d_head, page_size, page_table, pos0, pos1 - pos0, key, thr,
                                                                          guide, bad_dev);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
