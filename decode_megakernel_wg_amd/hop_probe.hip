// Measurement program (not part of the decode path): the costs that decide how the persistent kernel
// synchronises and what it keeps in flight, measured on the part itself.
//
//  1. One dependency hop between two workgroups on different XCDs (workgroups 0 and 1), with the payload
//     published either as (a) plain agent-coherent stores, a vmcnt drain and a relaxed counter increment that
//     the consumer polls before an acquire and the payload loads (the kernel's convention), or (b) 8-byte
//     (value, tag) pairs that the consumer polls directly (flag in the data, no counter).  Round trips of
//     two hops, idle and while every other compute unit streams HBM.
//  2. Agent-scope int64 atomic additions (no return) from many workgroups into a small array, against plain
//     stores of the same count: the cost of summing partial results with order-independent integer atomics.
//  3. Re-read bandwidth of a buffer that fits the 256 MB last-level cache, right after a full read of it,
//     against a 4 GB read: whether a second read of recently streamed data comes back faster.
//  4. How fast one workgroup reads a 4-64 KB payload that a workgroup on another XCD has just published (the
//     kernel's convention: agent-coherent stores, drain, counter; the consumer polls, acquires, reads), by
//     direct 16-byte global->LDS loads, 16-byte loads into registers and 4-byte loads into registers.
//
// Every wait is bounded (a spin limit, then an error flag and an exit), and every background reader stops at
// a flag or after a fixed number of passes, so each kernel ends.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#define CK(x)                                                                                  \
  do {                                                                                         \
    hipError_t e_ = (x);                                                                       \
    if (e_ != hipSuccess) {                                                                    \
      printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);                    \
      exit(1);                                                                                 \
    }                                                                                          \
  } while (0)

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) u4 gu4;

constexpr int HOP_THREADS = 256;
constexpr int HOP_MAXV = 4;          // payload words per thread (payload <= 1024 words)
constexpr uint32_t SPIN_LIMIT = 20000000u;

struct HopArgs {
  float* dA;
  float* dB;        // counter-mode payloads
  uint64_t* lA;
  uint64_t* lB;     // flag-in-data payloads
  uint32_t* ctr;    // [0] A->B, [32] B->A, [64] stop, [96] error
  const u4* bg;
  int64_t bg_n16;   // background buffer in 16-byte units
  uint64_t* out;    // [0] wall-clock ticks for R round trips
  int N, R, mode, bg_on;
};

__device__ bool wait_ctr(HopArgs& p, uint32_t* c, uint32_t target) {
  uint32_t n = 0;
  while (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    if (++n > SPIN_LIMIT) {
      atomicExch(p.ctr + 96, 1u);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  return true;
}

// (a) counter protocol
__device__ void send_ctr(HopArgs& p, float* d, uint32_t* c, int i) {
#pragma unroll
  for (int v = 0; v < HOP_MAXV; ++v) {
    const int j = threadIdx.x + v * HOP_THREADS;
    if (j < p.N) __hip_atomic_store(d + j, (float)i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the payload is stored before the counter moves
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ bool recv_ctr(HopArgs& p, const float* d, uint32_t* c, int i) {
  __shared__ int ok;
  if (threadIdx.x == 0) {
    ok = wait_ctr(p, c, (uint32_t)(i + 1));
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  float v[HOP_MAXV];
#pragma unroll
  for (int k = 0; k < HOP_MAXV; ++k) {
    const int j = threadIdx.x + k * HOP_THREADS;
    v[k] = j < p.N ? d[j] : (float)i;
  }
  bool bad = false;
#pragma unroll
  for (int k = 0; k < HOP_MAXV; ++k) bad |= v[k] != (float)i;
  if (bad) atomicExch(p.ctr + 96, 2u);
  __syncthreads();
  return ok;
}
// (b) flag in the data: (tag = round + 1) << 32 | value
__device__ void send_ll(HopArgs& p, uint64_t* d, int i) {
  const uint64_t tag = (uint64_t)(i + 1) << 32;
#pragma unroll
  for (int v = 0; v < HOP_MAXV; ++v) {
    const int j = threadIdx.x + v * HOP_THREADS;
    if (j < p.N) __hip_atomic_store(d + j, tag | __float_as_uint((float)i), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}
__device__ bool recv_ll(HopArgs& p, uint64_t* d, int i) {
  const uint32_t tag = (uint32_t)(i + 1);
  for (uint32_t n = 0;; ++n) {
    uint64_t v[HOP_MAXV];
#pragma unroll
    for (int k = 0; k < HOP_MAXV; ++k) {
      const int j = threadIdx.x + k * HOP_THREADS;
      v[k] = j < p.N ? __hip_atomic_load(d + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                     : ((uint64_t)tag << 32) | __float_as_uint((float)i);
    }
    int mine = 1;
    bool bad = false;
#pragma unroll
    for (int k = 0; k < HOP_MAXV; ++k) {
      mine &= (uint32_t)(v[k] >> 32) == tag;
      bad |= __uint_as_float((uint32_t)v[k]) != (float)i;
    }
    if (__syncthreads_and(mine)) {
      if (bad) atomicExch(p.ctr + 96, 2u);
      return true;
    }
    if (n > SPIN_LIMIT) {
      atomicExch(p.ctr + 96, 1u);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

__global__ __launch_bounds__(HOP_THREADS, 1) void hop_kernel(HopArgs p) {
  const int wg = blockIdx.x;
  if (wg == 0 || wg == 1) {
    const uint64_t t0 = wall_clock64();
    for (int i = 0; i < p.R; ++i) {
      bool ok;
      if (wg == 0) {
        if (p.mode == 0) {
          send_ctr(p, p.dA, p.ctr, i);
          ok = recv_ctr(p, p.dB, p.ctr + 32, i);
        } else {
          send_ll(p, p.lA, i);
          ok = recv_ll(p, p.lB, i);
        }
      } else {
        if (p.mode == 0) {
          ok = recv_ctr(p, p.dA, p.ctr, i);
          if (ok) send_ctr(p, p.dB, p.ctr + 32, i);
        } else {
          ok = recv_ll(p, p.lA, i);
          if (ok) send_ll(p, p.lB, i);
        }
      }
      if (!ok) break;
    }
    if (wg == 0 && threadIdx.x == 0) {
      p.out[0] = wall_clock64() - t0;
      __hip_atomic_store(p.ctr + 64, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  if (!p.bg_on) return;
  // background: every other workgroup streams its own stripe of the buffer (16 loads of 16 bytes per
  // thread in flight) until workgroup 0 is done, at most 1000 passes
  const int nbg = gridDim.x - 2, me = wg - 2;
  const int64_t stripe = p.bg_n16 / nbg;
  const u4* base = p.bg + (int64_t)me * stripe;
  uint32_t acc = 0;
  __shared__ int stop;
  for (int pass = 0; pass < 1000; ++pass) {
    for (int64_t o = 0; o + 16 * HOP_THREADS <= stripe; o += 16 * HOP_THREADS) {
      u4 v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = __builtin_nontemporal_load((gu4*)(base + o + u * HOP_THREADS + threadIdx.x));
#pragma unroll
      for (int u = 0; u < 16; ++u) acc += v[u].x ^ v[u].w;
      if ((o & (16 * HOP_THREADS * 16 - 1)) == 0) {
        if (threadIdx.x == 0) stop = (int)__hip_atomic_load(p.ctr + 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (stop) {
          if (acc == 0x12345u) p.out[1] = acc;
          return;
        }
      }
    }
  }
  if (acc == 0x12345u) p.out[1] = acc;
}

// Each workgroup adds (its index + 1) to acc[0, n) (mode 0, int64 atomics), or stores it to its own row of
// n values (mode 1), reps times.
__global__ __launch_bounds__(256) void atom_kernel(long long* acc, int n, int reps, int mode) {
  const long long v = blockIdx.x + 1;
  for (int r = 0; r < reps; ++r)
    for (int i = threadIdx.x; i < n; i += 256) {
      if (mode == 0) __hip_atomic_fetch_add(acc + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else __hip_atomic_store(acc + i + (long long)blockIdx.x * n, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

__global__ __launch_bounds__(256) void read_kernel(const u4* buf, int64_t n16, uint64_t* out) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * 256 * 8;
  for (int64_t o = (int64_t)blockIdx.x * 256 * 8; o + 256 * 8 <= n16; o += stride) {
    u4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *(gu4*)(buf + o + u * 256 + threadIdx.x);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u].x ^ v[u].w;
  }
  if (acc == 0x12345u) out[1] = acc;
}

// 4. fresh payloads: round r publishes NW words at pay + r * NW (never read before); workgroup 1 produces,
// workgroup 0 consumes; out[r] = consumer ticks from the acquire to every word read, out[64 + r] = wrong words.
constexpr int FR_NT = 512;
constexpr int FR_MAXW = 16384;  // words per payload (64 KB)
struct FreshArgs {
  float* pay;
  uint32_t* ctr;  // [0] produced rounds, [32] consumed rounds, [64] stop, [96] error
  const u4* bg;
  int64_t bg_n16;
  uint64_t* out;
  int NW, R, path, bg_on;
};
__device__ bool fresh_wait(FreshArgs& p, uint32_t* c, uint32_t target) {
  uint32_t n = 0;
  while (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    if (++n > SPIN_LIMIT) {
      atomicExch(p.ctr + 96, 1u);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  return true;
}
__global__ __launch_bounds__(FR_NT, 1) void fresh_kernel(FreshArgs p) {
  const int wg = blockIdx.x, tid = threadIdx.x;
  __shared__ float lds[FR_MAXW];
  __shared__ int ok;
  __shared__ uint64_t t0;
  if (wg == 1) {
    for (int r = 0; r < p.R; ++r) {
      if (tid == 0) ok = fresh_wait(p, p.ctr + 32, (uint32_t)r);
      __syncthreads();
      if (!ok) return;
      float* d = p.pay + (int64_t)r * p.NW;
      for (int j = tid; j < p.NW; j += FR_NT) __hip_atomic_store(d + j, (float)(r + j), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      if (tid == 0) __hip_atomic_fetch_add(p.ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  if (wg == 0) {
    for (int r = 0; r < p.R; ++r) {
      if (tid == 0) {
        ok = fresh_wait(p, p.ctr, (uint32_t)(r + 1));
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        t0 = wall_clock64();
      }
      __syncthreads();
      if (!ok) return;
      const float* d = p.pay + (int64_t)r * p.NW;
      int bad = 0;
      if (p.path == 0) {  // direct 16-byte global->LDS loads, every one in flight at once
        const int n16 = p.NW / 4, wave = tid >> 6, lane = tid & 63;
        for (int c0 = wave * 64; c0 < n16; c0 += FR_NT)
          if (c0 + lane < n16)
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(d + (int64_t)(c0 + lane) * 4),
                                             (__attribute__((address_space(3))) void*)(lds + (int64_t)c0 * 4), 16, 0, 0);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        for (int j = tid; j < p.NW; j += FR_NT) bad += lds[j] != (float)(r + j);
      } else if (p.path == 1) {  // 16-byte loads into registers
        for (int j = 4 * tid; j < p.NW; j += 4 * FR_NT) {
          const u4 v = *(gu4*)(d + j);
          bad += (__uint_as_float(v.x) != (float)(r + j)) + (__uint_as_float(v.w) != (float)(r + j + 3));
        }
      } else {  // 4-byte loads into registers
        for (int j = tid; j < p.NW; j += FR_NT) bad += d[j] != (float)(r + j);
      }
      const int tb = __syncthreads_count(bad);
      if (tid == 0) {
        p.out[r] = wall_clock64() - t0;
        p.out[64 + r] = (uint64_t)tb;
        __hip_atomic_fetch_add(p.ctr + 32, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (tid == 0) __hip_atomic_store(p.ctr + 64, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  if (!p.bg_on) return;
  const int nbg = gridDim.x - 2, me = wg - 2;
  const int64_t stripe = p.bg_n16 / nbg;
  const u4* base = p.bg + (int64_t)me * stripe;
  uint32_t acc = 0;
  __shared__ int stop;
  for (int pass = 0; pass < 1000; ++pass) {
    for (int64_t o = 0; o + 16 * FR_NT <= stripe; o += 16 * FR_NT) {
      u4 v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = __builtin_nontemporal_load((gu4*)(base + o + u * FR_NT + tid));
#pragma unroll
      for (int u = 0; u < 16; ++u) acc += v[u].x ^ v[u].w;
      if ((o & (16 * FR_NT * 16 - 1)) == 0) {
        if (tid == 0) stop = (int)__hip_atomic_load(p.ctr + 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (stop) {
          if (acc == 0x12345u) p.out[200] = acc;
          return;
        }
      }
    }
  }
  if (acc == 0x12345u) p.out[200] = acc;
}

int main() {
  CK(hipSetDevice(0));
  const int64_t bg_bytes = 4ll << 30;
  void* bg;
  CK(hipMalloc(&bg, bg_bytes));
  CK(hipMemset(bg, 1, bg_bytes));
  float *dA, *dB;
  uint64_t *lA, *lB, *out;
  uint32_t* ctr;
  CK(hipMalloc(&dA, 1 << 16));
  CK(hipMalloc(&dB, 1 << 16));
  CK(hipMalloc(&lA, 1 << 16));
  CK(hipMalloc(&lB, 1 << 16));
  CK(hipMalloc(&ctr, 4096));
  CK(hipMalloc(&out, 64));
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));

  printf("## 1. One dependency hop between workgroups on different XCDs\n\n");
  printf("| background HBM stream | protocol | payload (4-byte words) | us per round trip (two hops) | errors |\n|---|---|---|---|---|\n");
  const int Ns[2] = {64, 1024};
  for (int bgon = 0; bgon < 2; ++bgon)
    for (int mode = 0; mode < 2; ++mode)
      for (int ni = 0; ni < 2; ++ni) {
        HopArgs p{};
        p.dA = dA; p.dB = dB; p.lA = lA; p.lB = lB; p.ctr = ctr; p.out = out;
        p.bg = (const u4*)bg; p.bg_n16 = bg_bytes / 16;
        p.N = Ns[ni]; p.R = 2000; p.mode = mode; p.bg_on = bgon;
        CK(hipMemset(ctr, 0, 4096));
        CK(hipMemset(lA, 0, 1 << 16));
        CK(hipMemset(lB, 0, 1 << 16));
        CK(hipMemset(out, 0, 64));
        hipLaunchKernelGGL(hop_kernel, dim3(256), dim3(HOP_THREADS), 0, 0, p);
        CK(hipDeviceSynchronize());
        uint64_t ticks;
        uint32_t err;
        CK(hipMemcpy(&ticks, out, 8, hipMemcpyDeviceToHost));
        CK(hipMemcpy(&err, ctr + 96, 4, hipMemcpyDeviceToHost));
        printf("| %s | %s | %d | %.3f | %u |\n", bgon ? "254 workgroups" : "none",
               mode ? "flag in the data (8-byte pairs)" : "stores, drain, counter", p.N, ticks * 10.0 / 1000.0 / p.R, err);
        fflush(stdout);
      }

  printf("\n## 2. int64 atomic additions (agent scope, no return) against plain stores\n\n");
  printf("| workgroups | words per workgroup | repetitions | atomics: us, G ops/s, wrong sums | stores: us, G ops/s |\n|---|---|---|---|---|\n");
  long long* acc;
  const size_t acc_bytes = (size_t)16384 * 2048 * 8;
  CK(hipMalloc(&acc, acc_bytes));
  struct Case { int wgs, n, reps; } cases[] = {{192, 2048, 1}, {192, 2048, 16}, {1536, 2048, 8}, {256, 16384, 4}};
  for (auto c : cases) {
    float ms[2];
    int wrong = 0;
    for (int mode = 0; mode < 2; ++mode) {
      CK(hipMemset(acc, 0, acc_bytes));
      hipLaunchKernelGGL(atom_kernel, dim3(c.wgs), dim3(256), 0, 0, acc, c.n, c.reps, mode);
      CK(hipDeviceSynchronize());
      CK(hipMemset(acc, 0, acc_bytes));
      CK(hipEventRecord(e0));
      hipLaunchKernelGGL(atom_kernel, dim3(c.wgs), dim3(256), 0, 0, acc, c.n, c.reps, mode);
      CK(hipEventRecord(e1));
      CK(hipEventSynchronize(e1));
      CK(hipEventElapsedTime(&ms[mode], e0, e1));
      if (mode == 0) {
        long long* h = (long long*)malloc((size_t)c.n * 8);
        CK(hipMemcpy(h, acc, (size_t)c.n * 8, hipMemcpyDeviceToHost));
        const long long want = (long long)c.reps * c.wgs * (c.wgs + 1) / 2;
        for (int i = 0; i < c.n; ++i) wrong += h[i] != want;
        free(h);
      }
    }
    const double ops = (double)c.wgs * c.n * c.reps;
    printf("| %d | %d | %d | %.1f, %.1f, %d | %.1f, %.1f |\n", c.wgs, c.n, c.reps, ms[0] * 1e3, ops / (ms[0] * 1e-3) / 1e9, wrong,
           ms[1] * 1e3, ops / (ms[1] * 1e-3) / 1e9);
    fflush(stdout);
  }

  printf("\n## 3. Re-reading a buffer right after reading it (first read after a 4 GB read)\n\n");
  printf("| buffer | first read GB/s | second | third |\n|---|---|---|---|\n");
  const int64_t sizes[3] = {64ll << 20, 128ll << 20, 192ll << 20};
  for (int si = 0; si < 3; ++si) {
    hipLaunchKernelGGL(read_kernel, dim3(2048), dim3(256), 0, 0, (const u4*)bg, bg_bytes / 16, out);
    const u4* b = (const u4*)((char*)bg + (1ll << 30));
    float ms[3];
    for (int k = 0; k < 3; ++k) {
      CK(hipEventRecord(e0));
      hipLaunchKernelGGL(read_kernel, dim3(2048), dim3(256), 0, 0, b, sizes[si] / 16, out);
      CK(hipEventRecord(e1));
      CK(hipEventSynchronize(e1));
      CK(hipEventElapsedTime(&ms[k], e0, e1));
    }
    printf("| %lld MB | %.0f | %.0f | %.0f |\n", (long long)(sizes[si] >> 20), sizes[si] / ms[0] / 1e6, sizes[si] / ms[1] / 1e6,
           sizes[si] / ms[2] / 1e6);
  }
  CK(hipEventRecord(e0));
  hipLaunchKernelGGL(read_kernel, dim3(2048), dim3(256), 0, 0, (const u4*)bg, bg_bytes / 16, out);
  CK(hipEventRecord(e1));
  CK(hipEventSynchronize(e1));
  float ms;
  CK(hipEventElapsedTime(&ms, e0, e1));
  printf("| 4096 MB (one read) | %.0f | | |\n", bg_bytes / ms / 1e6);

  printf("\n## 4. Reading a payload another workgroup has just published (agent-coherent stores, drain, counter; poll, acquire)\n\n");
  printf("| background HBM stream | consumer loads | payload | us from the acquire to the last word (median of 30 rounds) | GB/s | wrong words |\n|---|---|---|---|---|---|\n");
  const int FR_R = 32;
  float* pay;
  uint64_t* fout;
  CK(hipMalloc(&pay, (size_t)FR_R * FR_MAXW * 4));
  CK(hipMalloc(&fout, 256 * 8));
  int ncu;
  CK(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, 0));
  const char* paths[3] = {"16-byte direct to LDS", "16-byte to registers", "4-byte to registers"};
  for (int bgon = 0; bgon < 2; ++bgon)
    for (int nw : {1024, 4096, 16384})
      for (int path = 0; path < 3; ++path) {
        FreshArgs f{pay, ctr, (const u4*)bg, bg_bytes / 16, fout, nw, FR_R, path, bgon};
        CK(hipMemset(ctr, 0, 4096));
        CK(hipMemset(fout, 0, 256 * 8));
        CK(hipMemset(pay, 0, (size_t)FR_R * FR_MAXW * 4));
        hipLaunchKernelGGL(fresh_kernel, dim3(bgon ? ncu : 2), dim3(FR_NT), 0, 0, f);
        CK(hipDeviceSynchronize());
        uint64_t h[256];
        uint32_t err;
        CK(hipMemcpy(h, fout, sizeof(h), hipMemcpyDeviceToHost));
        CK(hipMemcpy(&err, ctr + 96, 4, hipMemcpyDeviceToHost));
        uint64_t t[FR_R - 2], wrong = 0;
        for (int r = 2; r < FR_R; ++r) {
          t[r - 2] = h[r];
          wrong += h[64 + r];
        }
        for (int i = 0; i < FR_R - 2; ++i)  // median
          for (int j = i + 1; j < FR_R - 2; ++j)
            if (t[j] < t[i]) { uint64_t x = t[i]; t[i] = t[j]; t[j] = x; }
        const double us = t[(FR_R - 2) / 2] * 0.01;
        printf("| %s | %s | %d KB | %.2f | %.1f | %llu%s |\n", bgon ? "254 workgroups" : "none", paths[path], nw / 256, us,
               nw * 4.0 / (us * 1e3), (unsigned long long)wrong, err ? " (wait timed out)" : "");
        fflush(stdout);
      }
  printf("\ndone\n");
  return 0;
}
