// The decode megakernel for MI355X (gfx950): one persistent kernel per decode step.
//
// Design (pages: agenticcommons.xyz "Cohere North Mini Code megakernel serving engine", sections
// Megakernel 的運作方式 and 三個實際的加速來源; aimodeling.com "Cohere megakernel engine: one CUDA file,
// 1.58x vLLM on H100", section "One persistent kernel for the whole decode step"):
//  * one 512-thread workgroup per compute unit stays resident for the whole step and claims tasks
//    (one operation on one tile) from a task list in global memory, in list order, through an atomic
//    ticket; the next ticket is claimed while the current task runs;
//  * dependencies are global counters: a finished task increments its counter, a task that needs an
//    input spins on the producer's counter (no grid barrier, no kernel boundary);
//  * weight tiles (immutable) and old KV pages are loaded into registers BEFORE the task waits for its
//    activations, so HBM streams while dependencies resolve (weight prefetch, item 3);
//  * tile-granular claiming removes wave quantization and interleaves the attention and MoE branches of
//    the parallel layer (item 1); per-KV-group and per-expert counters remove false dependencies (item 2).
// MI355X specifics: wave64; cross-XCD visibility of task outputs uses write-through (sc1) stores plus a
// vmcnt drain before the relaxed counter increment, and an agent-scope acquire (L1/L2 invalidate) after
// the wait; an agent-scope release (L2 writeback) per task costs ~17 us under load on this part and is
// avoided.  Reductions have a fixed order everywhere (no floating-point atomics), so results do not depend
// on the grid size or on which workgroup ran which task.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "mk_desc.h"
#include "mk_kargs.h"

namespace mk {

constexpr int NT = 512;          // threads per workgroup
constexpr int NW = NT / 64;      // waves per workgroup
constexpr int XS_FLOATS = 32768; // 128 KB LDS staging area
constexpr uint32_t SPIN_LIMIT = 1u << 21;

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
template <int N, int R>
struct NVR {
  static constexpr int nv = N, rpw = R;
};
// Rows per wave per GEMV pass for NV 16-byte vectors per row and lane (passes hold 4-8 vectors per lane).
template <int NV>
struct RpwOf {
  static constexpr int value = NV == 1 ? 4 : NV == 2 ? 4 : NV == 4 ? 2 : 1;
};
// A compiled shape class of the kernel: head dim, GQA group, and the 16-byte-vector counts per lane of
// the three GEMV reduction lengths (d_model, d_ffn, group * d_head).  One kernel is instantiated per
// class so that each task type has a single code path (the register allocator handles one variant per
// task far better than a switch over many).
template <int DH_, int GRP_, int NVD_, int NVF_, int NVO_>
struct Cfg {
  static constexpr int DH = DH_, GRP = GRP_, NVD = NVD_, NVF = NVF_, NVO = NVO_;
};
// Global-address-space views: loads through them are global_load (vmcnt only), never flat loads,
// which would also count against lgkmcnt and make every LDS wait wait for in-flight weight loads.
typedef const __attribute__((address_space(1))) u4 gu4;
typedef const __attribute__((address_space(1))) u2 gu2;
__device__ __forceinline__ gu4* as_global(const void* p) { return (gu4*)(p); }
__device__ __forceinline__ gu2* as_global2(const void* p) { return (gu2*)(p); }

// The kernel's argument block, read in place from the kernarg segment (constant address space) so
// that task functions take it by reference without a private-memory copy.
typedef const __attribute__((address_space(4))) KArgs KA;

struct Lds {
  float xs[XS_FLOATS];   // activation staging (GEMV inputs), attention reduction scratch
  float q[8 * 128];      // attention: RoPE'd, scaled queries of one KV group
  float sc[8 * 256];     // attention: scores of one chunk [head][position]
  float pt[256 * 8];     // attention: probabilities of one chunk [position][head]
  int pages[ATTN_MAX_SPLIT_PAGES];  // attention: physical pages of the split
  float kn[128], vn[128];// attention: the new token's K and V (BF16-rounded)
  float hm[8], hl[8], hscale[8], pnew[8];
  float inv[8];          // per-token RMSNorm scale
  float ssqv[8 * 32];    // per-token partial sums of squares (row tiles)
  float gu[2 * 32 * 8];  // UP: gate/up values [row][token]
  float bestv[8 * NW];
  int besti[8 * NW];
  // routing of the current layer
  int sel[8 * 8];
  float gate[8 * 8];
  uint32_t used[8];      // bitmask of selected experts (256 bits)
  int slot_e, slot_n, slot_b[8], slot_j[8];
  float slot_g[8];
  int slotw[SLOT_WORDS];
  int task, next, flag;
};

// ------------------------------------------------------------------------------------------ helpers

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f2bf(float f) {  // round to nearest even
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// agent-coherent (write-through) stores for values other workgroups read in the same step
__device__ __forceinline__ void pub(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void pubi(int32_t* p, int32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void drain_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
// sum over each 16-lane row (every lane of the row gets it)
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  return v;
}
// sum over each 8-lane half row
__device__ __forceinline__ float row8_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  return v;
}
// value of lane (i ^ 16) within each 32-lane half (ds_swizzle, bit mode: and 0x1f, xor 0x10)
__device__ __forceinline__ float swz_xor16(float v) { return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F)); }
__device__ __forceinline__ float rdl(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }
// full-wave sum, uniform result, fixed order
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return ((rdl(v, 0) + rdl(v, 16)) + rdl(v, 32)) + rdl(v, 48);
}
__device__ __forceinline__ double wave_sum_d(double v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return __shfl(v, 0);
}
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ void raise_error(KA& a, uint32_t code, int task) {
  if (atomicCAS(&a.err[ERR_CODE], 0u, code) == 0u) atomicExch(&a.err[ERR_TASK], (uint32_t)task);
  __hip_atomic_store(&a.err[ERR_ABORT], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0 spins until counter c reaches target (or the step is aborted).
__device__ __forceinline__ void spin_ge(KA& a, int32_t c, int32_t target, int task) {
  if (c < 0) return;
  uint32_t n = 0;
  while (__hip_atomic_load(&a.ctr[c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (uint32_t)target) {
    if ((++n & 63) == 0) {
      if (__hip_atomic_load(&a.err[ERR_ABORT], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return;
      if (n > SPIN_LIMIT) {
        raise_error(a, ERRC_TIMEOUT, task);
        return;
      }
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Debug trace: sub-phase mark k (0..3) of task t.
__device__ __forceinline__ void mark(KA& a, int t, int k) {
  if (a.ts && threadIdx.x == 0) a.ts[(int64_t)t * 8 + 4 + k] = wall_clock64();
}

// Wait for descriptor waits [i0, i1), then make the producers' data visible to the whole workgroup.
__device__ __forceinline__ void wait_deps(KA& a, const int32_t* w, int i0, int i1, int task) {
  if (threadIdx.x == 0) {
    for (int i = i0; i < i1; ++i) spin_ge(a, w[W_WAIT0 + 2 * i], w[W_WAIT0 + 2 * i + 1], task);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (a.ts) a.ts[(int64_t)task * 8 + 1] = wall_clock64();
  }
  __syncthreads();
}

// Every thread has issued its published stores: drain them, then count the task as complete.
__device__ __forceinline__ void signal(KA& a, int32_t c, int32_t n) {
  drain_stores();
  __syncthreads();
  if (threadIdx.x == 0 && c >= 0) __hip_atomic_fetch_add(&a.ctr[c], (uint32_t)n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Arrive on a last-arriver counter; returns true (to every thread) in the workgroup that arrives last.
__device__ __forceinline__ bool arrive_last(KA& a, int32_t c, int32_t n, Lds& S) {
  drain_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t old = __hip_atomic_fetch_add(&a.ctr[c], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    S.flag = (old == (uint32_t)(n - 1));
    if (S.flag) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  return S.flag != 0;
}

// RMSNorm of the residual stream into LDS: xs[b][i] = x[b][i] * gamma[i] * inv_rms[b], for b < nb
// (token list tok[] maps staging row -> batch row; null = identity).
__device__ __forceinline__ void stage_norm(KA& a, const uint16_t* gamma, int nb, const int* tok, Lds& S) {
  const int d = a.d, nrt = a.n_rt;
  // one round trip: raw x rows, the partial sums of squares and the gain are loaded together
  constexpr int MAXE = 4096 / NT;  // gain elements per thread (d_model <= 4096)
  float gv[MAXE];
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
    const int c = threadIdx.x + e * NT;
    gv[e] = c < d ? bf2f(gamma[c]) : 0.f;
  }
  for (int i = threadIdx.x; i < nb * d; i += NT) {
    const int j = i / d, c = i - j * d;
    const int b = tok ? tok[j] : j;
    S.xs[i] = a.x[b * d + c];
  }
  if (threadIdx.x < nb * nrt) {
    const int j = threadIdx.x / nrt, r = threadIdx.x - j * nrt;
    const int b = tok ? tok[j] : j;
    S.ssqv[threadIdx.x] = a.ssq[b * nrt + r];
  }
  __syncthreads();
  if (threadIdx.x < nb) {
    float ss = 0.f;
    for (int r = 0; r < nrt; ++r) ss += S.ssqv[threadIdx.x * nrt + r];
    S.inv[threadIdx.x] = 1.0f / sqrtf(ss / (float)d + a.eps);
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
    const int c = threadIdx.x + e * NT;
    if (c < d)
      for (int j = 0; j < nb; ++j) S.xs[j * d + c] *= gv[e] * S.inv[j];
  }
  __syncthreads();
}

// ------------------------------------------------------------------------------------------ GEMV core
// A row tile W[0..nrows) x [0..K) (row stride ld) times NB staged vectors xs[b][0..K) (pitch xp).
// Wave w handles rows [p*NW*RPW + w*RPW, +RPW) of pass p; lane l reads 16-byte vectors l, l+64, ...
// of each row (NV per row).  Loads of pass p+1 are issued before pass p is computed; the caller
// issues pass 0 before its dependency wait.

template <int NV, int RPW>
struct WBuf {
  u4 v[RPW][NV];
};

// Row addressing of a tile: row r lives at base + r * ld (one segment), or rows [split, ...) at a second base.
struct Rows1 {
  const uint16_t* base;
  int64_t ld;
  __device__ __forceinline__ const uint16_t* operator()(int r) const { return base + (int64_t)r * ld; }
};
struct Rows2 {
  const uint16_t* base0;
  const uint16_t* base1;
  int64_t ld;
  int split;
  __device__ __forceinline__ const uint16_t* operator()(int r) const {
    return r < split ? base0 + (int64_t)r * ld : base1 + (int64_t)(r - split) * ld;
  }
};

template <int NV, int RPW, class RowPtr>
__device__ __forceinline__ void gemv_load(WBuf<NV, RPW>& buf, const RowPtr& W, int nrows, int K8, int pass) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row0 = pass * NW * RPW + wave * RPW;
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int row = row0 + r;
    gu4* rp = as_global(row < nrows ? W(row) : nullptr);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c8 = lane + 64 * i;
      if (row < nrows && c8 < K8)
        buf.v[r][i] = __builtin_nontemporal_load(rp + c8);
      else
        buf.v[r][i] = u4{0, 0, 0, 0};
    }
  }
}

__device__ __forceinline__ float dot8(u4 w, const f4& x0, const f4& x1, float acc) {
  acc = fmaf(bf_lo(w.x), x0.x, acc);
  acc = fmaf(bf_hi(w.x), x0.y, acc);
  acc = fmaf(bf_lo(w.y), x0.z, acc);
  acc = fmaf(bf_hi(w.y), x0.w, acc);
  acc = fmaf(bf_lo(w.z), x1.x, acc);
  acc = fmaf(bf_hi(w.z), x1.y, acc);
  acc = fmaf(bf_lo(w.w), x1.z, acc);
  acc = fmaf(bf_hi(w.w), x1.w, acc);
  return acc;
}
__device__ __forceinline__ double dot8d(u4 w, const f4& x0, const f4& x1, double acc) {
  acc = fma((double)bf_lo(w.x), (double)x0.x, acc);
  acc = fma((double)bf_hi(w.x), (double)x0.y, acc);
  acc = fma((double)bf_lo(w.y), (double)x0.z, acc);
  acc = fma((double)bf_hi(w.y), (double)x0.w, acc);
  acc = fma((double)bf_lo(w.z), (double)x1.x, acc);
  acc = fma((double)bf_hi(w.z), (double)x1.y, acc);
  acc = fma((double)bf_lo(w.w), (double)x1.z, acc);
  acc = fma((double)bf_hi(w.w), (double)x1.w, acc);
  return acc;
}

// Computes one pass and hands every (row, b) sum to out(row, b, value) on lane 0 of the owning wave.
template <int NV, int RPW, int NB, class Out>
__device__ __forceinline__ void gemv_compute(const WBuf<NV, RPW>& buf, const float* xs, int xp, int nb, int nrows, int K8, int pass,
                                             Out& out, int b0) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row0 = pass * NW * RPW + wave * RPW;
  float acc[RPW][NB];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[r][b] = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c8 = lane + 64 * i;
    if (c8 < K8) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const f4 x0 = *reinterpret_cast<const f4*>(xs + (b0 + b) * xp + c8 * 8);
        const f4 x1 = *reinterpret_cast<const f4*>(xs + (b0 + b) * xp + c8 * 8 + 4);
#pragma unroll
        for (int r = 0; r < RPW; ++r) acc[r][b] = dot8(buf.v[r][i], x0, x1, acc[r][b]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int row = row0 + r;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float s = wave_sum(acc[r][b]);
      if (row < nrows && b0 + b < nb && lane == 0) out(row, b0 + b, s);
    }
  }
}

// Drive a whole tile: pass 0 is in buf0 and, when the tile has more passes, pass 1 is in buf1.
template <int NV, int RPW, int NB, class RowPtr, class Out>
__device__ __forceinline__ void gemv_run2(WBuf<NV, RPW>& buf0, WBuf<NV, RPW>& buf1, const RowPtr& W, int nrows, int K, const float* xs,
                                          int xp, int nb, Out& out) {
  const int K8 = K >> 3;
  const int np = (nrows + NW * RPW - 1) / (NW * RPW);
  for (int p = 0; p < np; p += 2) {
    for (int b0 = 0; b0 < nb; b0 += NB) gemv_compute<NV, RPW, NB>(buf0, xs, xp, nb, nrows, K8, p, out, b0);
    if (p + 2 < np) gemv_load(buf0, W, nrows, K8, p + 2);
    if (p + 1 >= np) break;
    for (int b0 = 0; b0 < nb; b0 += NB) gemv_compute<NV, RPW, NB>(buf1, xs, xp, nb, nrows, K8, p + 1, out, b0);
    if (p + 3 < np) gemv_load(buf1, W, nrows, K8, p + 3);
  }
}
template <int NV, int RPW, int NB, class RowPtr, class Out>
__device__ __forceinline__ void gemv_run(WBuf<NV, RPW>& buf0, const RowPtr& W, int nrows, int K, const float* xs, int xp, int nb, Out& out) {
  WBuf<NV, RPW> buf1;
  if (nrows > NW * RPW) gemv_load(buf1, W, nrows, K >> 3, 1);
  gemv_run2<NV, RPW, NB>(buf0, buf1, W, nrows, K, xs, xp, nb, out);
}

// fp64-accumulating variant for the router (products of BF16 and fp32 are exact in fp64).
template <int NV, int RPW, int NB, class Out>
__device__ __forceinline__ void gemv_run_f64(WBuf<NV, RPW>& buf0, int nrows, int K, const float* xs, int xp, int nb, Out& out) {
  const int K8 = K >> 3;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // router tiles hold at most NW*RPW rows: one pass
  double acc[RPW][NB];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[r][b] = 0.0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c8 = lane + 64 * i;
    if (c8 < K8) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const f4 x0 = *reinterpret_cast<const f4*>(xs + b * xp + c8 * 8);
        const f4 x1 = *reinterpret_cast<const f4*>(xs + b * xp + c8 * 8 + 4);
#pragma unroll
        for (int r = 0; r < RPW; ++r) acc[r][b] = dot8d(buf0.v[r][i], x0, x1, acc[r][b]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int row = wave * RPW + r;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const double s = wave_sum_d(acc[r][b]);
      if (row < nrows && b < nb && lane == 0) out(row, b, s);
    }
  }
}

// ------------------------------------------------------------------------------------------ routing
// Done once per layer by the router tile that finishes last: top-k of each token's router logits (logit
// descending, lower index first on ties; a NaN ranks lowest), gates = softmax of the selected logits,
// and the table of expert slots (slot s = the s-th distinct selected expert in ascending id, with the
// tokens that chose it, their selection rank and gate).  Expert tasks read their slot's entry.
__device__ __forceinline__ void route_layer(KA& a, int l, Lds& S) {
  const int E = a.E, k = a.k, B = a.B, tid = threadIdx.x;
  const float* lg = a.rlogits + (int64_t)l * B * E;
  float* key = S.xs;  // [B][E] logits with NaN replaced by -inf
  for (int i = tid; i < B * E; i += NT) {
    const float v = lg[i];
    key[i] = v == v ? v : -INFINITY;
  }
  if (tid < 8) S.used[tid] = 0u;
  __syncthreads();
  // rank of (b, e) among the token's logits
  for (int i = tid; i < B * E; i += NT) {
    const int b = i / E, e = i - b * E;
    const float v = key[i];
    const float* kb = key + b * E;
    int rank = 0;
    for (int q = 0; q < E; ++q) {
      const float u = kb[q];
      rank += (u > v) || (u == v && q < e);
    }
    if (rank < k) {
      S.sel[b * 8 + rank] = e;
      atomicOr(&S.used[e >> 5], 1u << (e & 31));
    }
  }
  __syncthreads();
  if (tid < B) {
    const int b = tid;
    const float mx = key[b * E + S.sel[b * 8]];
    float z = 0.f;
    for (int j = 0; j < k; ++j) z += expf(key[b * E + S.sel[b * 8 + j]] - mx);
    for (int j = 0; j < k; ++j) {
      const float gt = expf(key[b * E + S.sel[b * 8 + j]] - mx) / z;
      S.gate[b * 8 + j] = gt;
      pubi(&a.route_sel[((int64_t)l * B + b) * k + j], S.sel[b * 8 + j]);
      pub(&a.route_gate[((int64_t)l * B + b) * k + j], gt);
    }
  }
  __syncthreads();
  // slot table
  for (int s = tid; s < a.n_slots; s += NT) {
    int e = -1, cnt = 0;
    for (int wd = 0; wd < 8 && e < 0; ++wd) {
      const uint32_t m = S.used[wd];
      const int pc = __popc(m);
      if (cnt + pc > s) {
        uint32_t mm = m;
        for (int q = 0; q < s - cnt; ++q) mm &= mm - 1;
        e = wd * 32 + __ffs(mm) - 1;
      }
      cnt += pc;
    }
    int32_t* ent = a.slots + ((int64_t)l * a.n_slots + s) * SLOT_WORDS;
    int n = 0;
    if (e >= 0)
      for (int b = 0; b < B; ++b)
        for (int j = 0; j < k; ++j)
          if (S.sel[b * 8 + j] == e && n < 8) {
            pubi(ent + 2 + 3 * n, b);
            pubi(ent + 3 + 3 * n, j);
            pubi(ent + 4 + 3 * n, __float_as_int(S.gate[b * 8 + j]));
            ++n;
          }
    pubi(ent + 0, e);
    pubi(ent + 1, n);
  }
}

// Load slot s's routing entry into LDS (valid after the layer's routing was published); false if unused.
__device__ __forceinline__ bool load_slot(KA& a, int l, int s, Lds& S) {
  if (threadIdx.x < SLOT_WORDS) S.slotw[threadIdx.x] = a.slots[((int64_t)l * a.n_slots + s) * SLOT_WORDS + threadIdx.x];
  __syncthreads();
  if (threadIdx.x == 0) {
    S.slot_e = S.slotw[0];
    S.slot_n = S.slot_e >= 0 ? min(S.slotw[1], 8) : 0;
    for (int i = 0; i < S.slot_n; ++i) {
      S.slot_b[i] = S.slotw[2 + 3 * i];
      S.slot_j[i] = S.slotw[3 + 3 * i];
      S.slot_g[i] = __int_as_float(S.slotw[4 + 3 * i]);
    }
  }
  __syncthreads();
  return S.slot_e >= 0 && S.slot_e < a.E;
}

// ------------------------------------------------------------------------------------------ task bodies

__device__ __forceinline__ void task_embed(KA& a, const int32_t* w, int t, Lds& S) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r0 = w[W_R0], r1 = w[W_R1], rt = w[W_A];
  if (wave < a.B) {
    const int b = wave;
    int tok = a.tokens[b];
    if (tok < 0 || tok >= a.V) {
      if (lane == 0) raise_error(a, ERRC_TOKEN, t);
      tok = 0;
    }
    float acc = 0.f;
    for (int r = r0 + lane; r < r1; r += 64) {
      const float v = bf2f(a.embed[(int64_t)tok * a.d + r]);
      pub(&a.x[b * a.d + r], v);
      acc = fmaf(v, v, acc);
    }
    const float s = wave_sum(acc);
    if (lane == 0) pub(&a.ssq[b * a.n_rt + rt], s);
  }
  // RoPE angles of each sequence's new position (fp64 angle, then cos/sin), once per step
  if (rt == 0) {
    const int half = a.dh / 2;
    for (int i = threadIdx.x; i < a.B * half; i += NT) {
      const int b = i / half, j = i - b * half;
      const double th = (double)a.seq_lens[b] * a.inv_freq[j];
      double sn, cs;
      sincos(th, &sn, &cs);
      pub(&a.rope_cs[(b * half + j) * 2 + 0], (float)cs);
      pub(&a.rope_cs[(b * half + j) * 2 + 1], (float)sn);
    }
  }
  signal(a, w[W_SIG], w[W_SIGN]);
}

__device__ __forceinline__ void task_resid(KA& a, const int32_t* w, int t, Lds& S) {
  wait_deps(a, w, 0, N_WAITS, t);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r0 = w[W_R0], r1 = w[W_R1], rt = w[W_A];
  const int d = a.d, B = a.B;
  if (wave < B) {
    const int b = wave;
    float acc = 0.f;
    for (int r = r0 + lane; r < r1; r += 64) {
      float v = a.x[b * d + r];
      for (int g = 0; g < a.Hkv; ++g) v += a.opart[((int64_t)g * B + b) * d + r];
      for (int j = 0; j < a.k; ++j) v += a.ypart[((int64_t)b * a.k + j) * d + r];
      pub(&a.x[b * d + r], v);
      acc = fmaf(v, v, acc);
    }
    const float s = wave_sum(acc);
    if (lane == 0) pub(&a.ssq[b * a.n_rt + rt], s);
  }
  signal(a, w[W_SIG], w[W_SIGN]);
}


// Generic "prefetch, wait, stage, stream" GEMV task.  Stage(): fills S.xs after the wait.  The first two
// passes of the tile are loaded before the dependency wait (a one-token tile uses 16-vector passes, so up
// to 256 KB per workgroup is in flight while its inputs are being produced).
template <int NV>
struct RpwBig {
  static constexpr int value = NV == 1 ? 8 : NV == 2 ? 8 : NV == 4 ? 4 : 2;
};
template <int NV, int RPW, int NB, class RowPtr, class Stage, class Out>
__device__ __forceinline__ void gemv_task_nb(KA& a, const int32_t* w, int t, const RowPtr& W, int nrows, int K, int nb, int wait0,
                                             int wait1, Stage& stage, Out& out, Lds& S) {
  WBuf<NV, RPW> buf0, buf1;
  gemv_load(buf0, W, nrows, K >> 3, 0);
  if (nrows > NW * RPW) gemv_load(buf1, W, nrows, K >> 3, 1);
  wait_deps(a, w, wait0, wait1, t);
  stage();
  gemv_run2<NV, RPW, NB>(buf0, buf1, W, nrows, K, S.xs, K, nb, out);
}
template <int NV, class RowPtr, class Stage, class Out>
__device__ __forceinline__ void gemv_task(KA& a, const int32_t* w, int t, const RowPtr& W, int nrows, int K, int nb, int wait0, int wait1,
                                          Stage&& stage, Out&& out, Lds& S) {
  if (nb <= 1) gemv_task_nb<NV, RpwBig<NV>::value, 1>(a, w, t, W, nrows, K, nb, wait0, wait1, stage, out, S);
  else if (nb <= 2) gemv_task_nb<NV, RpwOf<NV>::value, 2>(a, w, t, W, nrows, K, nb, wait0, wait1, stage, out, S);
  else gemv_task_nb<NV, RpwOf<NV>::value, 4>(a, w, t, W, nrows, K, nb, wait0, wait1, stage, out, S);  // 5..8 tokens: two groups
}

template <class C>
__device__ __forceinline__ void task_qkv(KA& a, const int32_t* w, int t, Lds& S) {
  const int l = w[W_LAYER], g = w[W_A], r0 = w[W_R0], r1 = w[W_R1];
  const int grp = a.Hq / a.Hkv, dh = a.dh, d = a.d;
  const LayerW& L = a.layers[l];
  const uint16_t* W;
  if (r0 < grp * dh) W = L.wq + ((int64_t)g * grp * dh + r0) * d;
  else if (r0 < (grp + 1) * dh) W = L.wk + ((int64_t)g * dh + (r0 - grp * dh)) * d;
  else W = L.wv + ((int64_t)g * dh + (r0 - (grp + 1) * dh)) * d;
  const int rows = (grp + 2) * dh;
  float* out = a.qkv + (int64_t)g * rows + r0;
  const int64_t bstride = (int64_t)a.Hkv * rows;
  gemv_task<C::NVD>(
      a, w, t, Rows1{W, d}, r1 - r0, d, a.B, 0, N_WAITS, [&] { stage_norm(a, L.attn_norm, a.B, nullptr, S); },
      [&](int r, int b, float v) { pub(out + b * bstride + r, v); }, S);
  signal(a, w[W_SIG], w[W_SIGN]);
}

template <class C>
__device__ __forceinline__ void task_router(KA& a, const int32_t* w, int t, Lds& S) {
  const int l = w[W_LAYER], r0 = w[W_R0], r1 = w[W_R1];
  const LayerW& L = a.layers[l];
  const int d = a.d, nrows = r1 - r0, K8 = d >> 3;
  const uint16_t* W = L.w_router + (int64_t)r0 * d;
  float* lg = a.rlogits + (int64_t)l * a.B * a.E;
  auto out = [&](int r, int b, double v) { pub(lg + b * a.E + r0 + r, (float)v + a.router_bias[r0 + r]); };
  auto go = [&](auto nvr) {
    constexpr int NV = decltype(nvr)::nv, RPW = decltype(nvr)::rpw;
    WBuf<NV, RPW> buf0;
    gemv_load(buf0, Rows1{W, d}, nrows, K8, 0);
    wait_deps(a, w, 0, N_WAITS, t);
    stage_norm(a, L.attn_norm, a.B, nullptr, S);
    if (a.dump_n && r0 == 0)
      for (int i = threadIdx.x; i < a.B * d; i += NT) a.dump_n[(int64_t)l * a.B * d + i] = S.xs[i];
    const int nb = a.B;
    if (nb <= 1) gemv_run_f64<NV, RPW, 1>(buf0, nrows, d, S.xs, d, nb, out);
    else if (nb <= 2) gemv_run_f64<NV, RPW, 2>(buf0, nrows, d, S.xs, d, nb, out);
    else if (nb <= 4) gemv_run_f64<NV, RPW, 4>(buf0, nrows, d, S.xs, d, nb, out);
    else gemv_run_f64<NV, RPW, 8>(buf0, nrows, d, S.xs, d, nb, out);
  };
  (void)K8;
  go(NVR<C::NVD, 2>{});
  if (arrive_last(a, w[W_ARR], w[W_ARRN], S)) {
    route_layer(a, l, S);
    signal(a, w[W_SIG], w[W_SIGN]);
  }
}

template <class C>
__device__ __forceinline__ void task_oproj(KA& a, const int32_t* w, int t, Lds& S) {
  const int l = w[W_LAYER], g = w[W_A], r0 = w[W_R0], r1 = w[W_R1];
  const int grp = a.Hq / a.Hkv, K = grp * a.dh, ldo = a.Hq * a.dh, B = a.B, d = a.d;
  const uint16_t* W = a.layers[l].wo + (int64_t)r0 * ldo + (int64_t)g * K;
  float* out = a.opart + (int64_t)g * B * d + r0;
  gemv_task<C::NVO>(
      a, w, t, Rows1{W, ldo}, r1 - r0, K, B, 0, N_WAITS,
      [&] {
        for (int i = threadIdx.x; i < B * K; i += NT) {
          const int b = i / K, c = i - b * K;
          S.xs[i] = a.attn_o[(int64_t)b * ldo + (int64_t)g * K + c];
        }
        __syncthreads();
      },
      [&](int r, int b, float v) { pub(out + (int64_t)b * d + r, v); }, S);
  signal(a, w[W_SIG], w[W_SIGN]);
}

template <class C>
__device__ __forceinline__ void task_up(KA& a, const int32_t* w, int t, Lds& S) {
  const int l = w[W_LAYER], s = w[W_A], r0 = w[W_R0], r1 = w[W_R1];
  const int d = a.d, F = a.F, nr = r1 - r0;
  wait_deps(a, w, 0, N_WAITS, t);
  if (load_slot(a, l, s, S)) {
    const int e = S.slot_e, n = S.slot_n;
    const LayerW& L = a.layers[l];
    // gate rows then up rows of this tile, as one 2*nr-row tile (two bases)
    const uint16_t* Wg = L.w_gate + ((int64_t)e * F + r0) * d;
    const uint16_t* Wu = L.w_up + ((int64_t)e * F + r0) * d;
    const Rows2 rows{Wg, Wu, d, nr};
    auto out = [&](int r, int b, float v) { S.gu[r * 8 + b] = v; };
    auto run = [&](auto nvr, auto nbc) {
      constexpr int NV = decltype(nvr)::nv, RPW = decltype(nvr)::rpw, NB = decltype(nbc)::value;
      WBuf<NV, RPW> b0, b1;
      gemv_load(b0, rows, 2 * nr, d >> 3, 0);  // the expert's weights stream while its inputs are staged
      if (2 * nr > NW * RPW) gemv_load(b1, rows, 2 * nr, d >> 3, 1);
      stage_norm(a, L.attn_norm, n, S.slot_b, S);
      gemv_run2<NV, RPW, NB>(b0, b1, rows, 2 * nr, d, S.xs, d, n, out);
    };
    if (n <= 1) run(NVR<C::NVD, RpwBig<C::NVD>::value>{}, std::integral_constant<int, 1>{});
    else if (n <= 2) run(NVR<C::NVD, RpwOf<C::NVD>::value>{}, std::integral_constant<int, 2>{});
    else run(NVR<C::NVD, RpwOf<C::NVD>::value>{}, std::integral_constant<int, 4>{});
    __syncthreads();
    for (int i = threadIdx.x; i < nr * n; i += NT) {
      const int r = i / n, j = i - r * n;
      const float gv = S.gu[r * 8 + j], uv = S.gu[(nr + r) * 8 + j];
      const float h = gv / (1.0f + expf(-gv)) * uv;
      pub(a.h + ((int64_t)s * a.B + j) * F + r0 + r, h);
    }
  }
  signal(a, w[W_SIG], w[W_SIGN]);
}

template <class C>
__device__ __forceinline__ void task_down(KA& a, const int32_t* w, int t, Lds& S) {
  const int l = w[W_LAYER], s = w[W_A], r0 = w[W_R0], r1 = w[W_R1];
  const int d = a.d, F = a.F, nr = r1 - r0;
  wait_deps(a, w, 0, 1, t);  // routing is known: this expert's weights can stream before its hidden state exists
  if (load_slot(a, l, s, S)) {
    const int e = S.slot_e, n = S.slot_n;
    const uint16_t* W = a.layers[l].w_down + ((int64_t)e * d + r0) * F;
    gemv_task<C::NVF>(
        a, w, t, Rows1{W, F}, nr, F, n, 1, N_WAITS,
        [&] {
          for (int i = threadIdx.x; i < n * F; i += NT) S.xs[i] = a.h[(int64_t)s * a.B * F + i];
          __syncthreads();
        },
        [&](int r, int j, float v) { pub(a.ypart + ((int64_t)S.slot_b[j] * a.k + S.slot_j[j]) * d + r0 + r, S.slot_g[j] * v); }, S);
  } else {
    wait_deps(a, w, 1, N_WAITS, t);
  }
  signal(a, w[W_SIG], w[W_SIGN]);
}

template <class C>
__device__ __forceinline__ void task_lmhead(KA& a, const int32_t* w, int t, Lds& S) {
  const int r0 = w[W_R0], r1 = w[W_R1], tile = w[W_A];
  const int d = a.d, B = a.B, nr = r1 - r0;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint16_t* W = a.lm_head + (int64_t)r0 * d;
  if (threadIdx.x < 8 * NW) {
    S.bestv[threadIdx.x] = -INFINITY;
    S.besti[threadIdx.x] = 0x7fffffff;
  }
  // each wave keeps its own running best per token (rows are visited in increasing order per wave)
  gemv_task<C::NVD>(
      a, w, t, Rows1{W, d}, nr, d, B, 0, N_WAITS, [&] { stage_norm(a, a.final_norm, B, nullptr, S); },
      [&](int r, int b, float v) {
        a.logits[(int64_t)b * a.V + r0 + r] = v;
        float& bv = S.bestv[b * NW + wave];
        int& bi = S.besti[b * NW + wave];
        if (v > bv || (v == bv && r0 + r < bi)) {
          bv = v;
          bi = r0 + r;
        }
      },
      S);
  __syncthreads();
  if (threadIdx.x < B) {
    const int b = threadIdx.x;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int q = 0; q < NW; ++q) {
      const float v = S.bestv[b * NW + q];
      const int i = S.besti[b * NW + q];
      if (v > bv || (v == bv && i < bi)) {
        bv = v;
        bi = i;
      }
    }
    pub(&a.lmbest_v[b * a.n_lm + tile], bv);
    pubi(&a.lmbest_i[b * a.n_lm + tile], bi);
  }
  if (arrive_last(a, w[W_ARR], w[W_ARRN], S)) {
    if (wave < B) {
      const int b = wave;
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int q = lane; q < a.n_lm; q += 64) {
        const float v = a.lmbest_v[b * a.n_lm + q];
        const int i = a.lmbest_i[b * a.n_lm + q];
        if (v > bv || (v == bv && i < bi)) {
          bv = v;
          bi = i;
        }
      }
      for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if (lane == 0) a.next_tok[b] = bi;
    }
  }
}

// ------------------------------------------------------------------------------------------ attention
// Split s of (sequence b, KV group g) covers positions [j0, j1) of the sequence's 0..len window (len =
// its prior length; position len is the new token, taken from this step's projections, RoPE'd, rounded
// to BF16 and written to the cache by the split that holds it).  The split's page list and its first
// chunk of K and V (256 positions) are loaded BEFORE the task waits for this step's queries.  Each thread
// owns one 8-dim slice of NP positions of a chunk: it forms the scores of every head of the group for
// its positions (queries in registers, slice sums by DPP), and after the chunk's softmax it accumulates
// p * V for its slice and positions.  The per-thread partial outputs are reduced once per split.
template <int DH, int GRP>
__device__ __forceinline__ void attn_split(KA& a, const int32_t* w, int t, Lds& S) {
  constexpr int DPT = 4;            // dims per thread slice
  constexpr int SL = DH / DPT;      // slices per position (32 or 16)
  constexpr int PPP = NT / SL;      // positions per pass (16 or 32)
  constexpr int CH = 128;           // positions per chunk
  constexpr int NP = CH / PPP;      // positions per thread per chunk (8 or 4)
  const int l = w[W_LAYER], b = w[W_A], g = w[W_B], s = w[W_C], nsplit = w[W_D];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int sl = tid % SL, pp = tid / SL;
  const int Hkv = a.Hkv;
  int len = a.seq_lens[b];
  if (len < 0 || len / 16 >= a.max_pages) {
    if (tid == 0) raise_error(a, ERRC_SEQLEN, t);
    len = 0;
  }
  const int npos = len + 1;
  int chunk = (npos + nsplit - 1) / nsplit;
  chunk = (chunk + CH - 1) / CH * CH;
  if (chunk > ATTN_MAX_SPLIT_PAGES * 16) {  // lengths grew far beyond the planned split count
    if (tid == 0) raise_error(a, ERRC_SEQLEN, t);
    chunk = ATTN_MAX_SPLIT_PAGES * 16;
  }
  const int j0 = min(s * chunk, npos), j1 = min(j0 + chunk, npos);
  const int jc1 = min(j1, len);  // cached positions end
  const bool has_new = (j0 <= len && len < j1);
  const int32_t* ptab = a.page_tables + (int64_t)b * a.max_pages;
  uint16_t* kvl = a.kv + (int64_t)l * a.n_pages * 2 * Hkv * 16 * DH;
  const int64_t vstride = (int64_t)Hkv * 16 * DH;

  // page list of the split
  const int np0 = j0 >> 4, npg = jc1 > j0 ? ((jc1 - 1) >> 4) - np0 + 1 : 0;
  for (int i = tid; i < npg; i += NT) {
    int ph = ptab[np0 + i];
    if (ph < 0 || ph >= a.n_pages) {
      raise_error(a, ERRC_PAGE, t);
      ph = -1;
    }
    S.pages[i] = ph;
  }
  __syncthreads();
  auto load_chunk = [&](int c0, u2 (&kk)[NP], u2 (&vv)[NP]) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int pos = c0 + pp + PPP * i;
      kk[i] = vv[i] = u2{0, 0};
      if (pos < jc1) {
        const int ph = S.pages[(pos >> 4) - np0];
        if (ph >= 0) {
          const int64_t base = (((int64_t)ph * 2) * Hkv + g) * 16 * DH + (pos & 15) * DH + sl * DPT;
          kk[i] = __builtin_nontemporal_load(as_global2(kvl + base));
          vv[i] = __builtin_nontemporal_load(as_global2(kvl + base + vstride));
        }
      }
    }
  };
  u2 kc[NP], vc[NP];
  load_chunk(j0, kc, vc);  // old K/V stream while this step's projections are produced

  wait_deps(a, w, 0, N_WAITS, t);

  // queries of the group: RoPE at position len, times 1/sqrt(dh)
  const float* qsrc = a.qkv + ((int64_t)b * Hkv + g) * (GRP + 2) * DH;
  const float* cs = a.rope_cs + (int64_t)b * (DH / 2) * 2;
  const float qscale = 1.0f / sqrtf((float)DH);
  for (int i = tid; i < GRP * DH / 2; i += NT) {
    const int h = i / (DH / 2), j = i - h * (DH / 2);
    const float c = cs[2 * j], sn = cs[2 * j + 1];
    const float x0 = qsrc[h * DH + j], x1 = qsrc[h * DH + j + DH / 2];
    S.q[h * DH + j] = (x0 * c - x1 * sn) * qscale;
    S.q[h * DH + j + DH / 2] = (x0 * sn + x1 * c) * qscale;
  }
  if (has_new) {
    for (int j = tid; j < DH / 2; j += NT) {
      const float c = cs[2 * j], sn = cs[2 * j + 1];
      const float x0 = qsrc[GRP * DH + j], x1 = qsrc[GRP * DH + j + DH / 2];
      S.kn[j] = bf2f(f2bf(x0 * c - x1 * sn));
      S.kn[j + DH / 2] = bf2f(f2bf(x0 * sn + x1 * c));
    }
    for (int j = tid; j < DH; j += NT) S.vn[j] = bf2f(f2bf(qsrc[(GRP + 1) * DH + j]));
  }
  if (tid < GRP) {
    S.hm[tid] = -INFINITY;
    S.hl[tid] = 0.f;
  }
  __syncthreads();
  if (has_new) {  // the new token's K/V go to the cache slot of position len (layer l)
    const int ph = ptab[len >> 4];
    if (ph >= 0 && ph < a.n_pages) {
      const int64_t base = (((int64_t)ph * 2) * Hkv + g) * 16 * DH + (len & 15) * DH;
      for (int j = tid; j < DH; j += NT) {
        kvl[base + j] = f2bf(S.kn[j]);
        kvl[base + vstride + j] = f2bf(S.vn[j]);
      }
    } else if (tid == 0) {
      raise_error(a, ERRC_PAGE, t);
    }
  }
  mark(a, t, 0);
  float qr[GRP][DPT];
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    const f4 q0 = *reinterpret_cast<const f4*>(S.q + h * DH + sl * DPT);
    qr[h][0] = q0.x; qr[h][1] = q0.y; qr[h][2] = q0.z; qr[h][3] = q0.w;
  }
  float o[GRP][DPT];
#pragma unroll
  for (int h = 0; h < GRP; ++h)
#pragma unroll
    for (int i = 0; i < DPT; ++i) o[h][i] = 0.f;

  for (int c0 = j0; c0 < jc1; c0 += CH) {
    // scores of this thread's positions, summed over the SL lanes of each position
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int pl = pp + PPP * i;
      const int pos = c0 + pl;
      const u2 k2 = kc[i];
      const float kf[DPT] = {bf_lo(k2.x), bf_hi(k2.x), bf_lo(k2.y), bf_hi(k2.y)};
#pragma unroll
      for (int h = 0; h < GRP; ++h) {
        float sc = 0.f;
#pragma unroll
        for (int e = 0; e < DPT; ++e) sc = fmaf(qr[h][e], kf[e], sc);
        sc = row16_sum(sc);
        if (SL == 32) sc += swz_xor16(sc);
        if (sl == h) S.sc[h * CH + pl] = pos < jc1 ? sc : -INFINITY;
      }
    }
    __syncthreads();
    // online softmax update, one wave per head
    if (wave < GRP) {
      const int h = wave;
      constexpr int R = CH / 64;
      float v[R];
      float vm = -INFINITY;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        v[r] = S.sc[h * CH + lane + 64 * r];
        vm = fmaxf(vm, v[r]);
      }
      const float mold = S.hm[h];
      const float mnew = fmaxf(mold, wave_max(vm));
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float pr = v[r] == -INFINITY ? 0.f : expf(v[r] - mnew);
        S.pt[(lane + 64 * r) * 8 + h] = pr;
        ps += pr;
      }
      const float psum = wave_sum(ps);
      if (lane == 0) {
        const float sc = mold == -INFINITY ? 0.f : expf(mold - mnew);
        S.hscale[h] = sc;
        S.hl[h] = S.hl[h] * sc + psum;
        S.hm[h] = mnew;
      }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      const float sc = S.hscale[h];
#pragma unroll
      for (int e = 0; e < DPT; ++e) o[h][e] *= sc;
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int pl = pp + PPP * i;
      const u2 v2 = vc[i];
      const float vf[DPT] = {bf_lo(v2.x), bf_hi(v2.x), bf_lo(v2.y), bf_hi(v2.y)};
      float pr[8];
      const f4 p0 = *reinterpret_cast<const f4*>(S.pt + pl * 8);
      const f4 p1 = *reinterpret_cast<const f4*>(S.pt + pl * 8 + 4);
      pr[0] = p0.x; pr[1] = p0.y; pr[2] = p0.z; pr[3] = p0.w; pr[4] = p1.x; pr[5] = p1.y; pr[6] = p1.z; pr[7] = p1.w;
#pragma unroll
      for (int h = 0; h < GRP; ++h)
#pragma unroll
        for (int e = 0; e < DPT; ++e) o[h][e] = fmaf(pr[h], vf[e], o[h][e]);
    }
    __syncthreads();
    if (c0 + CH < jc1) load_chunk(c0 + CH, kc, vc);
  }
  mark(a, t, 1);
  // the new token
  if (has_new) {
    if (wave < GRP) {
      const int h = wave;
      float sc = 0.f;
      for (int i = lane; i < DH; i += 64) sc = fmaf(S.q[h * DH + i], S.kn[i], sc);
      sc = wave_sum(sc);
      if (lane == 0) {
        const float mold = S.hm[h], mnew = fmaxf(mold, sc);
        const float scl = mold == -INFINITY ? 0.f : expf(mold - mnew);
        const float pn = expf(sc - mnew);
        S.hscale[h] = scl;
        S.pnew[h] = pn;
        S.hl[h] = S.hl[h] * scl + pn;
        S.hm[h] = mnew;
      }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      const float sc = S.hscale[h];
#pragma unroll
      for (int e = 0; e < DPT; ++e) o[h][e] *= sc;
      if (pp == 0) {
        const float pn = S.pnew[h];
#pragma unroll
        for (int e = 0; e < DPT; ++e) o[h][e] = fmaf(pn, S.vn[sl * DPT + e], o[h][e]);
      }
    }
  }
  // reduce the per-thread partial outputs over positions: lanes of one slice within the wave, then the
  // waves in order through LDS
#pragma unroll
  for (int h = 0; h < GRP; ++h)
#pragma unroll
    for (int e = 0; e < DPT; ++e) {
      float v = o[h][e];
      if (SL == 16) v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      o[h][e] = v;
    }
  float* red = S.xs;  // [NW][GRP][DH]
  if (lane < SL) {
#pragma unroll
    for (int h = 0; h < GRP; ++h)
#pragma unroll
      for (int e = 0; e < DPT; ++e) red[(wave * GRP + h) * DH + sl * DPT + e] = o[h][e];
  }
  __syncthreads();
  float* part = a.apart + ((((int64_t)b * Hkv + g) * ATTN_MAX_SPLITS + s) * GRP) * (DH + 2);
  for (int i = tid; i < GRP * DH; i += NT) {
    const int h = i / DH, dd = i - h * DH;
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < NW; ++q) v += red[(q * GRP + h) * DH + dd];
    pub(part + h * (DH + 2) + dd, v);
  }
  if (tid < GRP) {
    pub(part + tid * (DH + 2) + DH, S.hm[tid]);
    pub(part + tid * (DH + 2) + DH + 1, S.hl[tid]);
  }
  mark(a, t, 2);
  // the last split of (b, g) to finish merges all splits (log-sum-exp) and publishes the group's output
  if (arrive_last(a, w[W_ARR], w[W_ARRN], S)) {
    mark(a, t, 3);
    const float* p0 = a.apart + (((int64_t)b * Hkv + g) * ATTN_MAX_SPLITS) * GRP * (DH + 2);
    float* wsc = S.xs;                        // [GRP][nsplit] weights exp(m_s - M)
    float* lsum = S.xs + GRP * ATTN_MAX_SPLITS;  // [GRP]
    for (int i = tid; i < GRP * nsplit; i += NT) {
      const int h = i / nsplit, q = i - h * nsplit;
      wsc[i] = p0[((int64_t)q * GRP + h) * (DH + 2) + DH];
    }
    __syncthreads();
    if (wave < GRP) {
      const int h = wave;
      float M = -INFINITY;
      for (int q = lane; q < nsplit; q += 64) M = fmaxf(M, wsc[h * nsplit + q]);
      M = wave_max(M);
      float Ls = 0.f;
      for (int q = lane; q < nsplit; q += 64) {
        const float mq = wsc[h * nsplit + q];
        const float wq = mq == -INFINITY ? 0.f : expf(mq - M);
        wsc[h * nsplit + q] = wq;
        Ls = fmaf(p0[((int64_t)q * GRP + h) * (DH + 2) + DH + 1], wq, Ls);
      }
      Ls = wave_sum(Ls);
      if (lane == 0) lsum[h] = Ls;
    }
    __syncthreads();
    for (int i = tid; i < GRP * DH; i += NT) {
      const int h = i / DH, dd = i - h * DH;
      float ov = 0.f;
      int q = 0;
      for (; q + 8 <= nsplit; q += 8) {
        float vv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) vv[u] = p0[((int64_t)(q + u) * GRP + h) * (DH + 2) + dd];
#pragma unroll
        for (int u = 0; u < 8; ++u) ov = fmaf(vv[u], wsc[h * nsplit + q + u], ov);
      }
      for (; q < nsplit; ++q) ov = fmaf(p0[((int64_t)q * GRP + h) * (DH + 2) + dd], wsc[h * nsplit + q], ov);
      pub(a.attn_o + (int64_t)b * a.Hq * DH + ((int64_t)g * GRP + h) * DH + dd, ov / lsum[h]);
    }
    signal(a, w[W_SIG], w[W_SIGN]);
  }
}

template <class C>
__device__ __forceinline__ void task_attn(KA& a, const int32_t* w, int t, Lds& S) {
  attn_split<C::DH, C::GRP>(a, w, t, S);
}

// ------------------------------------------------------------------------------------------ the kernel

// One task.  The argument block is re-derived from an opaque copy of its address on every task so
// that no field is hoisted out of the task loop (that would pin dozens of registers for the kernel's
// whole life).
template <class C>
__device__ __forceinline__ void run_task(KA* a0, const int32_t* w, int t, uint32_t& nxt, Lds& S) {
  KA* ap = a0;
  __asm__ volatile("" : "+s"(ap));
  KA& a = *ap;
  const int tid = threadIdx.x;
  if (a.ts && tid == 0) {
    a.ts[(int64_t)t * 8 + 0] = wall_clock64();
    a.ts[(int64_t)t * 8 + 1] = 0;
    // hardware id: XCC id in the high word, the wave's HW_ID register in the low word
    a.ts[(int64_t)t * 8 + 3] = ((uint64_t)__builtin_amdgcn_s_getreg((20) | (0 << 6) | (15 << 11)) << 32) |
                               (uint64_t)__builtin_amdgcn_s_getreg((4) | (0 << 6) | (31 << 11));
  }
  switch (w[W_OP]) {
    case OP_EMBED: task_embed(a, w, t, S); break;
    case OP_ROUTER: task_router<C>(a, w, t, S); break;
    case OP_QKV: task_qkv<C>(a, w, t, S); break;
    case OP_ATTN: task_attn<C>(a, w, t, S); break;
    case OP_UP: task_up<C>(a, w, t, S); break;
    case OP_OPROJ: task_oproj<C>(a, w, t, S); break;
    case OP_DOWN: task_down<C>(a, w, t, S); break;
    case OP_RESID: task_resid(a, w, t, S); break;
    case OP_LMHEAD: task_lmhead<C>(a, w, t, S); break;
    default:
      if (tid == 0) raise_error(a, ERRC_OPCODE, t);
  }
  if (a.task_done && tid == 0) atomicAdd(&a.task_done[t], 1u);
  if (a.ts && tid == 0) a.ts[(int64_t)t * 8 + 2] = wall_clock64();
}

// The last workgroup out resets the counters for the next step (stream order makes it visible).
__device__ __forceinline__ void exit_step(KA& a, Lds& S) {
  const int tid = threadIdx.x;
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(&a.ctr[a.c_done], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    S.flag = (old == gridDim.x - 1);
    if (S.flag) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  if (S.flag) {
    if (a.ctr_snapshot)
      for (int i = tid; i < a.n_counters; i += NT) a.ctr_snapshot[i] = a.ctr[i];
    for (int i = tid; i < a.n_counters; i += NT) __hip_atomic_store(&a.ctr[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <class C>
__global__ __launch_bounds__(NT, 1) void mk_persistent(KArgs args) {
  KA* const a0 = (KA*)(__builtin_amdgcn_kernarg_segment_ptr());
  (void)args;
  __shared__ Lds S;
  const int tid = threadIdx.x;
  KA& a = *a0;
  if (tid == 0) S.next = (int)__hip_atomic_fetch_add(&a.ctr[a.c_ticket], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  for (;;) {
    const int t = S.next;
    __syncthreads();
    if (t >= a.n_tasks) break;
    // claim the next task now; its ticket returns while this one runs
    uint32_t nxt = 0;
    if (tid == 0) nxt = __hip_atomic_fetch_add(&a.ctr[a.c_ticket], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int32_t* w = a.tasks + (int64_t)t * DESC_WORDS;
    run_task<C>(a0, w, t, nxt, S);
    if (tid == 0) S.next = (int)nxt;
    __syncthreads();
  }
  exit_step(a, S);
}

}  // namespace mk
// Compiled shape classes: (d_head, group, d_model bound, d_ffn bound, group*d_head bound).
using CfgFull = mk::Cfg<128, 8, 4, 2, 2>;  // d_head 128, group 8, d_model <= 2048, d_ffn <= 1024, group*d_head = 1024
using CfgTiny = mk::Cfg<64, 2, 1, 1, 1>;   // d_head 64, group 2, d_model <= 512, d_ffn <= 512, group*d_head = 128

extern "C" int mk_kernel_class(int d_head, int group, int d_model, int d_ffn) {
  if (d_head == 128 && group == 8 && d_model <= 64 * 8 * CfgFull::NVD && d_ffn <= 64 * 8 * CfgFull::NVF) return 1;
  if (d_head == 64 && group == 2 && d_model <= 64 * 8 * CfgTiny::NVD && d_ffn <= 64 * 8 * CfgTiny::NVF) return 2;
  return 0;
}

extern "C" hipError_t mk_launch_persistent(const mk::KArgs* a, int kclass, int grid, hipStream_t stream) {
  if (kclass == 1) hipLaunchKernelGGL(mk::mk_persistent<CfgFull>, dim3(grid), dim3(mk::NT), 0, stream, *a);
  else if (kclass == 2) hipLaunchKernelGGL(mk::mk_persistent<CfgTiny>, dim3(grid), dim3(mk::NT), 0, stream, *a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}
