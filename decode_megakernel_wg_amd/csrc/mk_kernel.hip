// The decode megakernel for MI355X (gfx950): one persistent kernel per decode step.
//
// Design (pages: agenticcommons.xyz "Cohere North Mini Code megakernel serving engine", sections
// Megakernel 的運作方式 and 三個實際的加速來源; aimodeling.com "Cohere megakernel engine: one CUDA file,
// 1.58x vLLM on H100", section "One persistent kernel for the whole decode step"):
//  * one 512-thread workgroup per compute unit stays resident for the whole step and takes tasks (one
//    operation on one tile) from a task list in global memory, one at a time, in list order, through one
//    atomic counter, so each task goes to whichever compute unit is free first;
//  * dependencies are global counters: a finished task increments its counter, a task that needs an
//    input spins on the producer's counter (no grid barrier, no kernel boundary);
//  * weight tiles (immutable) and old KV pages are loaded into registers BEFORE the task waits for its
//    activations, so HBM streams while dependencies resolve (weight prefetch, item 3);
//  * tile-granular tasks remove wave quantization, and the attention and MoE branches of the parallel
//    layer share every compute unit (item 1); per-KV-group and per-expert counters remove false
//    dependencies (item 2).
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
constexpr int XS_FLOATS = 16384; // 64 KB LDS staging area (fp32 activations, attention scratch)
constexpr int XBP = 2048 + 32;    // bf16 row pitch of the split activations (rows 64 bytes apart modulo the bank window)
constexpr int NKP = 16;           // GEMV loads (16 bytes per lane) per pass and wave

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
// A compiled shape class of the kernel: head dim, GQA group, bounds of the three GEMV reduction lengths
// (d_model <= 512 NVD, d_ffn <= 512 NVF, group * d_head <= 512 NVO) and the batch class NB.  One kernel is instantiated per
// class so that each task type has a single code path (the register allocator handles one variant per
// task far better than a switch over many).
template <int DH_, int GRP_, int NVD_, int NVF_, int NVO_, int NB_>
struct Cfg {
  static constexpr int DH = DH_, GRP = GRP_, NVD = NVD_, NVF = NVF_, NVO = NVO_;
  // batch class of the GEMV tiles: at most 2 tokens (2) or at most 8 (8) on the matrix cores, or one token with the
  // VALU dot-product engine in the GEMV tiles (1; everything else as class 2)
  static constexpr int NB = NB_;
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
  uint16_t xb[16 * XBP + 64]; // GEMV inputs split into BF16 hi and lo parts (xb_off)
  float q[8 * 128];      // attention: RoPE'd, scaled queries of one KV group
  float sc[8 * 128];     // attention: scores of one chunk [head][position]; LM head: tile logits [row][token]
  float pt[256 * 8];     // attention: probabilities of one chunk [position][head]
  int pages[ATTN_MAX_SPLIT_PAGES];  // attention: physical pages of the split
  float kn[128], vn[128];// attention: the new token's K and V (BF16-rounded)
  float hm[8], hl[8], hscale[8], pnew[8];
  float inv[8];          // per-token RMSNorm scale
  float ssqv[8 * 32];    // per-token partial sums of squares (row tiles)
  float gu[2 * 64 * 8];  // UP: gate/up values [row][token] (up to 64 rows each)
  // routing of the current layer
  int sel[8 * 8];
  float gate[8 * 8];
  uint32_t used[8];      // bitmask of selected experts (256 bits)
  int slot_e, slot_n, slot_b[8], slot_j[8];
  float slot_g[8];
  int slotw[SLOT_WORDS];
  int32_t desc[DESC_WORDS];     // the task's descriptor
  int pool_tile;                // the index a take returned (the ticket's value before a maximum)
  int pool_used;                // a layer's used-slot count read with a take (0 = not yet routed)
  int lmq[4];                   // LM head: ring of claimed vocabulary chunks
  uint32_t wval;                // value a wait observed (expert slot words)
  int flag;
  int xb_layer;  // l + 1 while xb holds layer l's normalised input of every token (split); 0 otherwise
  int route_layer;  // l + 1 while sel / used hold layer l's routing; 0 otherwise
};

// A task descriptor staged in LDS; every word is read as a wave-uniform (scalar) value.
struct Desc {
  const int32_t* p;
  __device__ __forceinline__ int32_t operator[](int i) const { return __builtin_amdgcn_readfirstlane(p[i]); }
};

// Offset (bf16 elements) of token t's part p (0 = hi, 1 = lo) in S.xb.  Rows are XBP apart (64 bytes
// modulo the 256-byte bank window) and the lo rows start 128 bytes further, so the four slots read
// together (tokens 0..3 of one part, or tokens 0..1 of both) fall in distinct bank windows.
__device__ __forceinline__ int xb_off(int t, int p) { return p * (8 * XBP + 64) + t * XBP; }

// ------------------------------------------------------------------------------------------ helpers

// The thread index as an opaque value: each use goes through an empty volatile asm, so the compiler cannot
// hoist values derived from it out of the persistent task loop (where they would stay live, and be spilled,
// across every task body).
__device__ __forceinline__ int tidx() {
  int t = (int)__builtin_amdgcn_workitem_id_x();
  __asm__ volatile("" : "+v"(t));
  return t;
}

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
// Workgroup barrier for data exchanged through LDS only: LDS operations complete (lgkmcnt(0)), then
// s_barrier.  Unlike __syncthreads it does not wait for outstanding global loads (weights in flight).
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

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
__device__ __forceinline__ float rdl(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }
// full-wave sum, uniform result, fixed order
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return ((rdl(v, 0) + rdl(v, 16)) + rdl(v, 32)) + rdl(v, 48);
}
// full-wave maximum, uniform result: within each 16-lane row by DPP, then the four rows
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  return fmaxf(fmaxf(rdl(v, 0), rdl(v, 16)), fmaxf(rdl(v, 32), rdl(v, 48)));
}

// Counter c.  Counters lie one 128-byte line apart: every workgroup polls and adds to them, and counters that
// share a line (the phase pools, a layer's readiness counters) would serialize each other's atomics.
__device__ __forceinline__ uint32_t* ctr_at(KA& a, int64_t c) { return a.ctr + c * CTR_STRIDE; }

__device__ __forceinline__ void raise_error(KA& a, uint32_t code, int task) {
  if (atomicCAS(&a.err[ERR_CODE], 0u, code) == 0u) atomicExch(&a.err[ERR_TASK], (uint32_t)task);
  __hip_atomic_store(&a.err[ERR_ABORT], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0 spins until counter c reaches target (or the step is aborted); returns the value it saw.  After
// a.spin_limit polls (about 0.4 us each) the wait reports a time-out and aborts the step: every other wait
// then returns at its next abort check, so every workgroup still runs out its task list and exits.
__device__ __forceinline__ uint32_t spin_ge(KA& a, int32_t c, int32_t target, int task) {
  if (c < 0) return 0u;
  uint32_t n = 0, v;
  while ((v = __hip_atomic_load(ctr_at(a, c), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) < (uint32_t)target) {
    if ((++n & 63) == 0) {
      if (__hip_atomic_load(&a.err[ERR_ABORT], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return 0u;
      if (n > a.spin_limit) {
        raise_error(a, ERRC_TIMEOUT, task);
        return 0u;
      }
    }
    __builtin_amdgcn_s_sleep(16);  // ~0.4 us between polls: fewer requests to the counters' memory channels
  }
  return v;
}

// Debug trace: sub-phase mark k (0..3) of task t.
__device__ __forceinline__ void mark(KA& a, int t, int k) {
  if (a.ts && tidx() == 0) a.ts[(int64_t)t * 8 + 4 + k] = wall_clock64();
}

// Wait for descriptor waits [i0, i1), then make the producers' data visible to the whole workgroup.
__device__ __forceinline__ void wait_deps(KA& a, Desc w, int i0, int i1, int task) {
  if (i0 >= i1) return;
  if (tidx() == 0) {
    for (int i = i0; i < i1; ++i) spin_ge(a, w[W_WAIT0 + 2 * i], w[W_WAIT0 + 2 * i + 1], task);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (a.ts) a.ts[(int64_t)task * 8 + 1] = wall_clock64();
  }
  __syncthreads();
}

// Wait i of the descriptor, returning the counter value it observed (to every thread).  Expert-slot
// counters carry the routing of their slot in that value.
__device__ __forceinline__ uint32_t wait_value(KA& a, Desc w, int i, int task, Lds& S) {
  if (tidx() == 0) {
    S.wval = spin_ge(a, w[W_WAIT0 + 2 * i], w[W_WAIT0 + 2 * i + 1], task);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (a.ts) a.ts[(int64_t)task * 8 + 1] = wall_clock64();
  }
  __syncthreads();
  return S.wval;
}

// Every thread has issued its published stores: drain them, then count the task as complete.
__device__ __forceinline__ void signal(KA& a, int32_t c, int32_t n) {
  drain_stores();
  __syncthreads();
  if (tidx() == 0 && c >= 0) __hip_atomic_fetch_add(ctr_at(a, c), (uint32_t)n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Arrive on a last-arriver counter; returns true (to every thread) in the workgroup that arrives last.
__device__ __forceinline__ bool arrive_last(KA& a, int32_t c, int32_t n, Lds& S) {
  drain_stores();
  __syncthreads();
  if (tidx() == 0) {
    uint32_t old = __hip_atomic_fetch_add(ctr_at(a, c), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    S.flag = (old == (uint32_t)(n - 1));
    if (S.flag) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  return S.flag != 0;
}

// Copy n16 16-byte chunks from global memory (contiguous) to LDS (contiguous) with direct global->LDS
// loads, spread over the workgroup's waves: no registers are held, and every chunk is in flight at once.
// Completion is tracked by vmcnt: the caller drains (vmcnt(0)) and synchronises before reading dst.
__device__ __forceinline__ void lds_copy(const void* src, void* dst, int n16) {
  const int wave = tidx() >> 6, lane = tidx() & 63;
  for (int c0 = wave * 64; c0 < n16; c0 += NT) {
    if (c0 + lane < n16)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)((const char*)src + (int64_t)(c0 + lane) * 16),
                                       (__attribute__((address_space(3))) void*)((char*)dst + (int64_t)c0 * 16), 16, 0, 0);
  }
}

// The RMSNorm gain of one consumer, loaded (two elements per word) before the consumer waits for its
// input: gains are weights, immutable during the step.
constexpr int NORM_PAIRS = 4096 / 2 / NT;  // gain pairs per thread (d_model <= 4096)
struct NormGain {
  uint32_t g[NORM_PAIRS];
};
__device__ __forceinline__ NormGain norm_gain(const uint16_t* gamma, int d) {
  NormGain n;
  const uint32_t* g2 = reinterpret_cast<const uint32_t*>(gamma);
#pragma unroll
  for (int e = 0; e < NORM_PAIRS; ++e) {
    const int p = tidx() + e * NT;
    n.g[e] = 2 * p < d ? g2[p] : 0u;
  }
  return n;
}

// Request the residual-stream rows of staging rows j < nb (token tok[j], null = identity) into S.xs and
// their row tiles' partial sums of squares into S.ssqv, straight into LDS, in one round trip.
__device__ __forceinline__ void stage_norm_issue(KA& a, int nb, const int* tok, Lds& S) {
  const int d = a.d, nrt = a.n_rt;
  for (int j = 0; j < nb; ++j) lds_copy(a.x + (tok ? tok[j] : j) * d, S.xs + j * d, d / 4);
  // partial sums of squares: one 4-byte lane per row tile, issued by the last wave
  if ((tidx() >> 6) == NW - 1) {
    const int lane = tidx() & 63;
    for (int j = 0; j < nb; ++j)
      if (lane < nrt)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(a.ssq + (tok ? tok[j] : j) * nrt + lane),
                                         (__attribute__((address_space(3))) void*)(S.ssqv + j * nrt), 4, 0, 0);
  }
}

// RMSNorm of the residual stream straight into the BF16 hi/lo matrix-core operand (xb_off(j, 0) and
// xb_off(j, 1) for staging row j < nb, token tok[j]): n = x[b][i] * (gamma[i] * inv_rms[b]) with
// inv_rms[b] = 1 / sqrt(sum of the row tiles' partial sums of squares, added in tile order, / d + eps);
// one read of the staged rows, no normalised fp32 copy.
__device__ __forceinline__ void stage_split(KA& a, const NormGain& gn, int nb, const int* tok, Lds& S) {
  const int d = a.d, nrt = a.n_rt;
  stage_norm_issue(a, nb, tok, S);
  drain_stores();
  __syncthreads();
  if (tidx() == 0) S.xb_layer = 0;
  {
    const int wave = tidx() >> 6, lane = tidx() & 63;
    for (int j = wave; j < nb; j += NW) {
      // lane 0 adds the partials in tile order (every consumer forms inv_rms with the same additions),
      // with every partial read first
      if (lane == 0) {
        float v[32];
#pragma unroll
        for (int r = 0; r < 32; ++r) v[r] = r < nrt ? S.ssqv[j * nrt + r] : 0.f;
        float ss = 0.f;
#pragma unroll
        for (int r = 0; r < 32; ++r)
          if (r < nrt) ss += v[r];
        S.inv[j] = 1.0f / sqrtf(ss / (float)d + a.eps);
      }
    }
  }
  lds_sync();
#pragma unroll
  for (int e = 0; e < NORM_PAIRS; ++e) {
    const int p = tidx() + e * NT;
    if (2 * p < d) {
      const float g0 = bf_lo(gn.g[e]), g1 = bf_hi(gn.g[e]);
      for (int j = 0; j < nb; ++j) {
        const float inv = S.inv[j];
        const float2 xv = *reinterpret_cast<const float2*>(S.xs + j * d + 2 * p);
        const float x0 = xv.x * (g0 * inv), x1 = xv.y * (g1 * inv);
        const uint16_t h0 = f2bf(x0), h1 = f2bf(x1);
        const uint16_t l0 = f2bf(x0 - bf2f(h0)), l1 = f2bf(x1 - bf2f(h1));
        *reinterpret_cast<uint32_t*>(S.xb + xb_off(j, 0) + 2 * p) = (uint32_t)h0 | ((uint32_t)h1 << 16);
        *reinterpret_cast<uint32_t*>(S.xb + xb_off(j, 1) + 2 * p) = (uint32_t)l0 | ((uint32_t)l1 << 16);
      }
    }
  }
  lds_sync();
}

// ------------------------------------------------------------------------------------------ weight rows
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

// ------------------------------------------------------------------------------------------ routing
// Done once per layer by the workgroup that completes the layer's router logits: top-k of each token's
// router logits (logit descending, lower index first on ties; a NaN ranks lowest), gates = softmax of the
// selected logits,
// and the table of expert slots (slot s = the s-th distinct selected expert in ascending id, with the
// tokens that chose it, their selection rank and gate).  Each slot's readiness counter (ctr[slot0 + s])
// then receives the slot's expert and token mask (see slot_routing), so expert tasks learn their expert
// from the wait itself.
// Top-k of every token's key (S.xs [B][E]) into S.sel [b][rank] and the bitmask of selected experts S.used.
__device__ __forceinline__ void route_rank(KA& a, Lds& S) {
  const int E = a.E, k = a.k, B = a.B, tid = tidx();
  float* key = S.xs;  // [B][E] router logits with NaN replaced by -inf (filled by the caller)
  if (tid < 8) S.used[tid] = 0u;
  __syncthreads();
  // rank of (b, e) among the token's logits: rq adjacent threads (an aligned group of lanes) share one
  // (b, e), each counting over its part of the keys (4-wide LDS reads), and their counts are added across
  // the lanes (E a multiple of 8; four parts when E is a multiple of 16)
  {
    const int rq = E % 16 == 0 ? 4 : 1;
    for (int i0 = tid; i0 < B * E * rq; i0 += NT) {
      const int i = i0 / rq, qq = i0 - i * rq;
      const int b = i / E, e = i - b * E;
      const float v = key[i];
      const float* kb = key + b * E;
      const int span = E / rq, q0 = qq * span;
      int rank = 0;
#pragma unroll 4
      for (int q = q0; q < q0 + span; q += 4) {
        const f4 u = *reinterpret_cast<const f4*>(kb + q);
        rank += (u.x > v) || (u.x == v && q < e);
        rank += (u.y > v) || (u.y == v && q + 1 < e);
        rank += (u.z > v) || (u.z == v && q + 2 < e);
        rank += (u.w > v) || (u.w == v && q + 3 < e);
      }
      if (rq == 4) {
        rank += __shfl_xor(rank, 1);
        rank += __shfl_xor(rank, 2);
      }
      if (qq == 0 && rank < k) {
        S.sel[b * 8 + rank] = e;
        atomicOr(&S.used[e >> 5], 1u << (e & 31));
      }
    }
  }
  __syncthreads();
}
__device__ __forceinline__ void route_select(KA& a, int l, int32_t slot0, Lds& S) {
  const int E = a.E, k = a.k, B = a.B, tid = tidx();
  float* key = S.xs;
  route_rank(a, S);
  if (tid == 0) S.route_layer = l + 1;  // S.sel / S.used hold layer l's routing
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
  // slot table (n_slots <= 64 < NT: thread s builds slot s and keeps its counter value)
  uint32_t sv = 0;
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
    uint32_t mask = 0;
    if (e >= 0)
      for (int b = 0; b < B; ++b)
        for (int j = 0; j < k; ++j)
          if (S.sel[b * 8 + j] == e && n < 8) {
            pubi(ent + 2 + 3 * n, b);
            pubi(ent + 3 + 3 * n, j);
            pubi(ent + 4 + 3 * n, __float_as_int(S.gate[b * 8 + j]));
            mask |= 1u << b;
            ++n;
          }
    pubi(ent + 0, e);
    pubi(ent + 1, n);
    sv = e >= 0 ? (mask << 16) | (uint32_t)(e + 1) : 0x80000000u;
  }
  // Unused slots: their tasks will neither run nor arrive, so their arrivals on each row tile's residual
  // counter are made here, and the layer's used-slot count is published for the phase takes, all before any
  // slot is released.  Until a slot is released only O-projection tiles (at most Hkv per row tile) can have
  // arrived, so the last arrival of a row tile is still a down-projection tile's and runs the epilogue.
  int nu = 0;
#pragma unroll
  for (int wd = 0; wd < 8; ++wd) nu += __popc(S.used[wd]);
  const int n_empty = a.n_slots - nu;
  if (slot0 >= 0) {
    if (n_empty > 0)
      for (int r = tid; r < a.n_rt; r += NT)
        __hip_atomic_fetch_add(ctr_at(a, a.c_resid_arrive + l * a.n_rt + r), (uint32_t)n_empty, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) __hip_atomic_store(ctr_at(a, a.c_slots_used + l), (uint32_t)nu, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // publish the entries, then release the slots (one counter each, value = routing)
  drain_stores();
  __syncthreads();
  if (tid < a.n_slots && slot0 >= 0) __hip_atomic_store(ctr_at(a, slot0 + tid), sv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Residual rows [r0, r1): x += sum over KV groups of the O-projection partials + sum over the k selections
// of the gated expert outputs (fixed order: groups ascending, then selections ascending); the partial sum
// of squares of each token's new rows goes to ssq[b][rt].  Every partial of a row is loaded before any is
// added, so the whole update costs one round trip to memory.  The new rows stay in LDS at xs[B*n ...] for
// the next layer's router partial.
__device__ __forceinline__ void resid_rows(KA& a, int r0, int r1, int rt, Lds& S) {
  const int wave = tidx() >> 6, lane = tidx() & 63;
  const int d = a.d, B = a.B, n = r1 - r0, Hkv = a.Hkv, k = a.k;
  float* sq = S.xs;           // [B][n] squares of the new rows
  float* xr = S.xs + B * n;   // [B][n] the new rows
  for (int i = tidx(); i < B * n; i += NT) {
    const int b = i / n, r = r0 + (i - b * n);
    const float xv = a.x[b * d + r];
    float op[8], yp[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) op[g] = g < Hkv ? a.opart[((int64_t)g * B + b) * d + r] : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) yp[j] = j < k ? a.ypart[((int64_t)b * k + j) * d + r] : 0.f;
    float v = xv;
#pragma unroll
    for (int g = 0; g < 8; ++g)
      if (g < Hkv) v += op[g];
    for (int g = 8; g < Hkv; ++g) v += a.opart[((int64_t)g * B + b) * d + r];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < k) v += yp[j];
    pub(&a.x[b * d + r], v);
    sq[i] = v * v;
    xr[i] = v;
  }
  __syncthreads();
  if (wave < B) {
    const int b = wave;
    float acc = 0.f;
    for (int r = lane; r < n; r += 64) acc += sq[b * n + r];
    const float s = wave_sum(acc);
    if (lane == 0) pub(&a.ssq[b * a.n_rt + rt], s);
  }
}

// Router partial of one residual row tile for layer l: u[b][e] = sum over the tile's rows i of
// W_router[l][e][i] * x[b][i] * gamma_l[i], accumulated in fp64 (each product is exact in fp64), in column
// order per thread and then in a fixed tree over the threads of an expert.  The layer's router logit is
// then inv_rms[b] * (sum of the row tiles' partials in tile order) + bias[e]: the RMSNorm scale is the one
// factor that needs the whole residual stream, so the router runs as soon as the last row tile is done.
// The router and gain slices are requested (router_pre) before the tile's residual update, so their
// round trip overlaps that of the residual partials.
constexpr int RP_MAXV = 8;  // 16-byte vectors of router weights per thread (64 columns)
struct RouterPre {
  u4 wv[RP_MAXV], gv[RP_MAXV];
  int tpe, cols;
};
__device__ __forceinline__ void router_pre(KA& a, int l, int r0, int r1, RouterPre& rp) {
  const int E = a.E, n = r1 - r0, d = a.d, tid = tidx();
  int tpe = NT / E;  // threads per expert: a power of two, at least 8 columns each
  while (tpe > 1 && n / tpe < 8) tpe >>= 1;
  while (n / tpe > 8 * RP_MAXV) tpe <<= 1;
  rp.tpe = tpe;
  rp.cols = n / tpe;
  const LayerW& L = a.layers[l];
  if (tid < E * tpe) {
    const int e = tid / tpe, q = tid - e * tpe, c0 = q * rp.cols;
    const uint16_t* wr = L.w_router + (int64_t)e * d + r0 + c0;
    const uint16_t* gm = L.attn_norm + r0 + c0;
#pragma unroll
    for (int v = 0; v < RP_MAXV; ++v) {
      if (8 * v < rp.cols) {
        rp.wv[v] = *reinterpret_cast<const u4*>(wr + 8 * v);
        rp.gv[v] = *reinterpret_cast<const u4*>(gm + 8 * v);
      }
    }
  }
}
__device__ __forceinline__ void router_partial(KA& a, const RouterPre& rp, int r0, int r1, int rt, const float* xr) {
  const int B = a.B, E = a.E, n = r1 - r0, tid = tidx(), tpe = rp.tpe, cols = rp.cols;
  if (tid < E * tpe) {
    const int e = tid / tpe, q = tid - e * tpe, c0 = q * cols;
    double acc[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[b] = 0.0;
#pragma unroll
    for (int v = 0; v < RP_MAXV; ++v) {
      if (8 * v < cols) {
        const u4 wv = rp.wv[v], gv = rp.gv[v];
        const float wf[8] = {bf_lo(wv.x), bf_hi(wv.x), bf_lo(wv.y), bf_hi(wv.y), bf_lo(wv.z), bf_hi(wv.z), bf_lo(wv.w), bf_hi(wv.w)};
        const float gf[8] = {bf_lo(gv.x), bf_hi(gv.x), bf_lo(gv.y), bf_hi(gv.y), bf_lo(gv.z), bf_hi(gv.z), bf_lo(gv.w), bf_hi(gv.w)};
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          if (b < B) {
            const float* xb = xr + b * n + c0 + 8 * v;
#pragma unroll
            for (int u = 0; u < 8; ++u) acc[b] = fma((double)wf[u], (double)xb[u] * (double)gf[u], acc[b]);
          }
        }
      }
    }
    // fixed tree over the tpe threads of the expert (adjacent lanes)
    for (int o = 1; o < tpe; o <<= 1)
#pragma unroll
      for (int b = 0; b < 8; ++b) acc[b] += __shfl_xor(acc[b], o);
    if (q == 0)
      for (int b = 0; b < B; ++b)
        __hip_atomic_store(reinterpret_cast<unsigned long long*>(a.rpart) + ((int64_t)rt * B + b) * E + e,
                           (unsigned long long)__double_as_longlong(acc[b]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Router logits of layer l into S.xs [B][E] (NaN as -inf) from the row tiles' fp64 partials: inv_rms[b] is
// formed from the row tiles' partial sums of squares exactly as every consumer's RMSNorm forms it, and the
// partials are added in tile order.  The partial sums of squares and the router partials are requested
// together (one round trip).  publish: also record the logits (and the debug RMSNorm dump).
__device__ __forceinline__ void route_logits(KA& a, int l, Lds& S, bool publish) {
  const int B = a.B, E = a.E, nrt = a.n_rt, d = a.d, tid = tidx();
  const float ssq = tid < B * nrt ? a.ssq[tid] : 0.f;
  const double* rp = a.rpart;
  double* sums = reinterpret_cast<double*>(S.xs + B * E);  // [B][E], after the keys
  for (int i = tid; i < B * E; i += NT) {
    const int b = i / E, e = i - b * E;
    double sum = 0.0;
    int r = 0;
    for (; r + 16 <= nrt; r += 16) {  // 16 partials requested together, then added in tile order
      double v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = rp[((int64_t)(r + u) * B + b) * E + e];
#pragma unroll
      for (int u = 0; u < 16; ++u) sum += v[u];
    }
    for (; r < nrt; ++r) sum += rp[((int64_t)r * B + b) * E + e];
    sums[i] = sum;
  }
  if (tid < B * nrt) S.ssqv[tid] = ssq;
  __syncthreads();
  if (tid < B) {
    float ss = 0.f;
    for (int r = 0; r < nrt; ++r) ss += S.ssqv[tid * nrt + r];
    S.inv[tid] = 1.0f / sqrtf(ss / (float)d + a.eps);
  }
  __syncthreads();
  float* key = S.xs;
  for (int i = tid; i < B * E; i += NT) {
    const int b = i / E, e = i - b * E;
    const float lg = (float)(sums[i] * (double)S.inv[b]) + a.router_bias[e];
    if (publish) pub(a.rlogits + ((int64_t)l * B + b) * E + e, lg);
    key[i] = lg == lg ? lg : -INFINITY;
  }
  if (publish && a.dump_n) {  // debug: the RMSNorm output this layer's consumers stage
    const uint16_t* gm = a.layers[l].attn_norm;
    for (int i = tid; i < B * d; i += NT) {
      const int b = i / d, c = i - b * d;
      a.dump_n[(int64_t)l * B * d + i] = a.x[i] * (bf2f(gm[c]) * S.inv[b]);
    }
  }
  __syncthreads();
}

// The workgroup that completes a layer's router partials: logits, routing, slot table, slot release.
__device__ __forceinline__ void route_from_partials(KA& a, int l, int32_t slot0, Lds& S) {
  route_logits(a, l, S, true);
  route_select(a, l, slot0, S);
}

// A row tile of layer lnext's input is complete (rows and sum of squares published): count it into the
// layer's readiness counter, then add its router partial; the last row tile routes the layer.
__device__ __forceinline__ void row_tile_done(KA& a, Desc w, int lnext, int r0, int r1, int rt, const float* xr,
                                              const RouterPre& rp, Lds& S) {
  signal(a, w[W_SIG], w[W_SIGN]);
  if (w[W_ARR2] >= 0) {
    router_partial(a, rp, r0, r1, rt, xr);
    if (arrive_last(a, w[W_ARR2], w[W_ARRN2], S)) route_from_partials(a, lnext, w[W_RSIG], S);
  }
}

// End of an O-proj / expert-down task: the last producer of the row tile adds the partials into x.
__device__ __forceinline__ void resid_chain(KA& a, Desc w, Lds& S) {
  if (arrive_last(a, w[W_ARR], w[W_ARRN], S)) {
    const int r0 = w[W_R0], r1 = w[W_R1], lnext = w[W_LAYER] + 1;
    RouterPre rp;
    if (w[W_ARR2] >= 0) router_pre(a, lnext, r0, r1, rp);
    resid_rows(a, r0, r1, w[W_RT], S);
    row_tile_done(a, w, lnext, r0, r1, w[W_RT], S.xs + a.B * (r1 - r0), rp, S);
  }
}

// ------------------------------------------------------------------------------------------ MFMA GEMV core
// A tile of nrows x K BF16 weights times nb <= 8 activation vectors on v_mfma_f32_16x16x32_bf16, fp32
// accumulation.  Operand layout of the instruction (checked on gfx950): lane l holds A[l%16][8(l/16)+v],
// B[8(l/16)+v][l%16] and D[4(l/16)+i][l%16].
//
// Row quads.  A row m = 4r + h of the A operand holds weight row r of a quad of four rows at K-part h,
// where part h of a 128-wide K block is its 16-byte chunks h, h+4, h+8 and h+12.  Lane l therefore loads
// chunk 4(l/16) + l%4 of quad row (l%16)/4: every four consecutive lanes read 64 contiguous bytes of one
// row, a pattern the per-CU load path serves about twice as fast as the plain A layout's sixteen rows of
// 16 bytes (measured on this part).  The activations take the same K order: B column n = 4s + h holds
// activation slot s at K-part h, so D[4r + h][4s + h] is row r times slot s over part h, and the four
// parts are added across the four lanes of a quad.  The activations are split into BF16 hi + lo parts
// (~16 mantissa bits): for nb <= 2 the four slots are (hi, token 0), (hi, token 1), (lo, token 0),
// (lo, token 1) and one MFMA covers a quad and K block; for larger nb a slot is a token, one MFMA takes
// the hi parts and one the lo parts of four tokens, both accumulating into the same D.
//
// Wave w owns a 16-row block (four quads) and a K slice (w / ks, w % ks); a pass is four K blocks of its
// four quads, 16 loads of 16 bytes per lane; the K-slice partials of a row block are added in a fixed
// order through LDS.
struct MGeo {
  int nrows, K, rbn, ks, kw, nkb, np;
};
__device__ __forceinline__ MGeo mgeo(int nrows, int K) {
  MGeo g;
  g.nrows = nrows;
  g.K = K;
  g.rbn = (nrows + 15) >> 4;  // row blocks (at most NW)
  int ks = 1;
  while (g.rbn * ks * 2 <= NW && K % (256 * ks) == 0) ks *= 2;
  g.ks = ks;
  g.kw = K / ks;       // a multiple of 128
  g.nkb = g.kw >> 7;   // 128-wide K blocks per slice
  g.np = (g.nkb + 3) >> 2;
  return g;
}
struct MBuf {
  u4 v[NKP];  // unit t = 4 * (K block) + quad
};
// per-quad accumulators: slots of tokens 0..3 (or of nb <= 2), and of tokens 4..7
struct MAcc {
  f4 a[4], b[4];
};
__device__ __forceinline__ void macc_zero(MAcc& m) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    m.a[q] = f4{0.f, 0.f, 0.f, 0.f};
    m.b[q] = f4{0.f, 0.f, 0.f, 0.f};
  }
}

// Column offset (bf16 elements) of this lane's 16-byte chunk within pass `pass` of its K slice.
__device__ __forceinline__ int mg_col(const MGeo& g, int kp, int pass, int lane) {
  return kp * g.kw + 512 * pass + 32 * (lane >> 4) + 8 * (lane & 3);
}

template <class RowPtr>
__device__ __forceinline__ void mg_load(MBuf& buf, const RowPtr& W, const MGeo& g, int pass) {
  const int wave = tidx() >> 6, lane = tidx() & 63;
  const int rb = wave / g.ks, kp = wave - rb * g.ks;
  const int c = mg_col(g, kp, pass, lane);
  gu4* rp[4];
  bool ok[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = rb * 16 + 4 * q + ((lane & 15) >> 2);
    ok[q] = rb < g.rbn && row < g.nrows;
    rp[q] = as_global((ok[q] ? W(row) : W(0)) + c);
  }
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const bool kok = 4 * pass + kb < g.nkb;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      buf.v[4 * kb + q] = (ok[q] && kok) ? __builtin_nontemporal_load(rp[q] + 16 * kb) : u4{0, 0, 0, 0};
  }
}

__device__ __forceinline__ u4 lds16(const uint16_t* p) { return *reinterpret_cast<const u4*>(p); }
__device__ __forceinline__ f4 mfma(u4 av, u4 bv, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv), c, 0, 0, 0);
}

// K blocks KB0 .. KB0 + KB - 1 of the pass (units 4 * KB0 ...), all present.
template <int NB, int KB, int KB0 = 0>
__device__ __forceinline__ void mg_compute_kb(const MBuf& buf, MAcc& acc, const MGeo& g, int pass, int nb, Lds& S) {
  constexpr int kb0 = KB0;
  const int wave = tidx() >> 6, lane = tidx() & 63;
  const int rb = wave / g.ks, kp = wave - rb * g.ks;
  if (rb >= g.rbn) return;
  const int s = (lane & 15) >> 2;  // this lane's B slot
  const int c = mg_col(g, kp, pass, lane) + 128 * kb0;
  if (NB <= 2) {
    // slot s = (part s / 2, token s % 2); absent tokens read token 0 (their D columns are never used)
    const int tk = s & 1;
    const uint16_t* xp = S.xb + xb_off(tk < nb ? tk : 0, s >> 1) + c;
    u4 x0 = lds16(xp), x1 = KB > 1 ? lds16(xp + 128) : x0;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const u4 cx = x0;
      x0 = x1;
      if (kb + 2 < KB) x1 = lds16(xp + 128 * (kb + 2));
#pragma unroll
      for (int q = 0; q < 4; ++q) acc.a[q] = mfma(buf.v[4 * (kb0 + kb) + q], cx, acc.a[q]);
    }
    // two activation reads ahead of the MFMAs (the scheduler would otherwise put each read right before its
    // first use)
    __builtin_amdgcn_sched_group_barrier(0x100, KB > 1 ? 2 : 1, 0);
#pragma unroll
    for (int i = 0; i < KB - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, KB > 1 ? 8 : 4, 0);
  } else {
    // group 0: tokens 0..3 into acc.a; group 1: tokens 4..7 into acc.b
    const int t0 = s < nb ? s : 0, t1 = 4 + s < nb ? 4 + s : 0;
    const uint16_t* xh0 = S.xb + xb_off(t0, 0) + c;
    const uint16_t* xl0 = S.xb + xb_off(t0, 1) + c;
    const uint16_t* xh1 = S.xb + xb_off(t1, 0) + c;
    const uint16_t* xl1 = S.xb + xb_off(t1, 1) + c;
    const bool g1 = NB > 4 && nb > 4;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const u4 h0 = lds16(xh0 + 128 * kb), l0 = lds16(xl0 + 128 * kb);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc.a[q] = mfma(buf.v[4 * (kb0 + kb) + q], h0, acc.a[q]);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc.a[q] = mfma(buf.v[4 * (kb0 + kb) + q], l0, acc.a[q]);
      if (g1) {
        const u4 h1 = lds16(xh1 + 128 * kb), l1 = lds16(xl1 + 128 * kb);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc.b[q] = mfma(buf.v[4 * (kb0 + kb) + q], h1, acc.b[q]);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc.b[q] = mfma(buf.v[4 * (kb0 + kb) + q], l1, acc.b[q]);
      }
    }
  }
}
// A pass of the tile: all four K blocks, or the K tail's one to three (768 = 6 blocks: a pass of 4, then 2).
template <int NB>
__device__ __forceinline__ void mg_compute_any(const MBuf& buf, MAcc& acc, const MGeo& g, int pass, int nb, Lds& S) {
  const int left = g.nkb - 4 * pass;
  if (left >= 4) {
    mg_compute_kb<NB, 4>(buf, acc, g, pass, nb, S);
  } else if (left >= 2) {
    mg_compute_kb<NB, 2>(buf, acc, g, pass, nb, S);
    if (left == 3) mg_compute_kb<NB, 1, 2>(buf, acc, g, pass, nb, S);
  } else {
    mg_compute_kb<NB, 1>(buf, acc, g, pass, nb, S);
  }
}

// Per lane and quad q: the four K parts added across the quad's lanes (lanes 4i..4i+3 all get the sum), and
// for nb <= 2 the lo slots added to the hi slots.  Lane l with l % 4 == 0 then holds row 4q + l / 16 of the
// row block for slot (l / 4) % 4: token s in va (nb <= 2: s < 2 only), token 4 + s in vb.
__device__ __forceinline__ float pick4(f4 v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }
template <int NB>
__device__ __forceinline__ void mg_lane_values(const MAcc& acc, int nb, float (&va)[4], float (&vb)[4]) {
  const int i = tidx() & 3;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float x = pick4(acc.a[q], i);
    x += dpp<0xB1>(x);  // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);  // quad_perm [2,3,0,1]
    if (NB <= 2) x += dpp<0x128>(x);  // row_ror:8: slot s + 2 (lo) onto slot s (hi)
    va[q] = x;
    float y = 0.f;
    if (NB > 4 && nb > 4) {
      y = pick4(acc.b[q], i);
      y += dpp<0xB1>(y);
      y += dpp<0x4E>(y);
    }
    vb[q] = y;
  }
}
// Hand (row within the 16-row block, token, value) of this lane's results to f.
template <int NB, class F>
__device__ __forceinline__ void mg_emit(const float (&va)[4], const float (&vb)[4], int nb, F&& f) {
  const int lane = tidx() & 63;
  if (lane & 3) return;
  const int s = (lane >> 2) & 3;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 4 * q + (lane >> 4);
    if (NB <= 2) {
      if (s < nb) f(r, s, va[q]);
    } else {
      if (s < nb) f(r, s, va[q]);
      if (4 + s < nb) f(r, 4 + s, vb[q]);
    }
  }
}

// Sum the K-slice partials of each row block (fixed order) and hand (row, token, value) to out().
template <int NB, class Out>
__device__ __forceinline__ void mg_finish(const MAcc& acc, const MGeo& g, int nb, Out& out, Lds& S) {
  const int wave = tidx() >> 6, lane = tidx() & 63;
  const int rb = wave / g.ks, kp = wave - rb * g.ks;
  float va[4], vb[4];
  mg_lane_values<NB>(acc, nb, va, vb);
  if (g.ks > 1) {
    float* red = S.pt;  // [NW][4 quads][16 quad leaders][2]
    if (rb < g.rbn && (lane & 3) == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        red[((wave * 4 + q) * 16 + (lane >> 2)) * 2 + 0] = va[q];
        red[((wave * 4 + q) * 16 + (lane >> 2)) * 2 + 1] = vb[q];
      }
    }
    __syncthreads();
    if (kp == 0 && rb < g.rbn && (lane & 3) == 0) {
      for (int p = 1; p < g.ks; ++p) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          va[q] += red[(((wave + p) * 4 + q) * 16 + (lane >> 2)) * 2 + 0];
          vb[q] += red[(((wave + p) * 4 + q) * 16 + (lane >> 2)) * 2 + 1];
        }
      }
    }
  }
  if (kp == 0 && rb < g.rbn)
    mg_emit<NB>(va, vb, nb, [&](int r, int j, float v) {
      const int row = rb * 16 + r;
      if (row < g.nrows) out(row, j, v);
    });
}

// Split the staged fp32 inputs S.xs[nb][K] into BF16 hi and lo parts.
__device__ __forceinline__ void split_x(int nb, int K, Lds& S) {
  if (tidx() == 0) S.xb_layer = 0;
  for (int i = tidx(); i < nb * K; i += NT) {
    const int j = i / K, c = i - j * K;
    const float x = S.xs[i];
    const uint16_t h = f2bf(x);
    S.xb[xb_off(j, 0) + c] = h;
    S.xb[xb_off(j, 1) + c] = f2bf(x - bf2f(h));
  }
  lds_sync();
}

// VALU engine of the GEMV tiles (batch class 1: one token; selected by MK_DBG_VALU_GEMV to compare the two
// engines on the same loads): lane l's 16-byte weight chunk of quad q and K block kb (the row-quad layout
// above) times the 8 activations of the same chunk, as fp32 FMAs into one partial per quad; the activations
// are the BF16 hi + lo parts added back in fp32 (exact: the same operand the matrix cores see).
struct VAcc {
  float v[4];  // [quad]
};
template <int KB, int KB0 = 0>
__device__ __forceinline__ void mgv_compute_kb(const MBuf& buf, VAcc& acc, const MGeo& g, int pass, Lds& S) {
  const int wave = tidx() >> 6, lane = tidx() & 63;
  const int rb = wave / g.ks, kp = wave - rb * g.ks;
  if (rb >= g.rbn) return;
  const int c = mg_col(g, kp, pass, lane) + 128 * KB0;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    __builtin_amdgcn_sched_barrier(0);  // one K block's operands live at a time (no hoisting across blocks)
    const u4 hv = lds16(S.xb + xb_off(0, 0) + c + 128 * kb), lv = lds16(S.xb + xb_off(0, 1) + c + 128 * kb);
    const uint32_t hw[4] = {hv.x, hv.y, hv.z, hv.w}, lw[4] = {lv.x, lv.y, lv.z, lv.w};
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf_lo(hw[i]) + bf_lo(lw[i]);
      x[2 * i + 1] = bf_hi(hw[i]) + bf_hi(lw[i]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u4 wv = buf.v[4 * (KB0 + kb) + q];
      const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc.v[q] = fmaf(bf_lo(ww[i]), x[2 * i], acc.v[q]);
        acc.v[q] = fmaf(bf_hi(ww[i]), x[2 * i + 1], acc.v[q]);
      }
    }
  }
}
__device__ __forceinline__ void mgv_compute_any(const MBuf& buf, VAcc& acc, const MGeo& g, int pass, Lds& S) {
  const int left = g.nkb - 4 * pass;
  if (left >= 4) {
    mgv_compute_kb<4>(buf, acc, g, pass, S);
  } else if (left >= 2) {
    mgv_compute_kb<2>(buf, acc, g, pass, S);
    if (left == 3) mgv_compute_kb<1, 2>(buf, acc, g, pass, S);
  } else {
    mgv_compute_kb<1>(buf, acc, g, pass, S);
  }
}
// Row 4q + rr of the row block (rr = (lane % 16) / 4) is spread over the 16 lanes with that rr (lane % 4 and
// lane / 16 free): added across them (two DPP steps, two lane swaps), then the K-slice partials of the block
// in a fixed order through LDS; lanes 0, 4, 8, 12 hand (row, token 0, value) to out().
template <class Out>
__device__ __forceinline__ void mgv_finish(const VAcc& acc, const MGeo& g, Out& out, Lds& S) {
  const int wave = tidx() >> 6, lane = tidx() & 63;
  const int rb = wave / g.ks, kp = wave - rb * g.ks;
  float r[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float v = acc.v[q];
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    r[q] = v;
  }
  const bool lead = rb < g.rbn && lane < 16 && (lane & 3) == 0;
  if (g.ks > 1) {
    float* red = S.pt;  // [NW][4 quads][4 rows]
    if (lead)
#pragma unroll
      for (int q = 0; q < 4; ++q) red[(wave * 4 + q) * 4 + (lane >> 2)] = r[q];
    __syncthreads();
    if (kp == 0 && lead)
      for (int p = 1; p < g.ks; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) r[q] += red[((wave + p) * 4 + q) * 4 + (lane >> 2)];
  }
  if (kp == 0 && lead)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = rb * 16 + 4 * q + (lane >> 2);
      if (row < g.nrows) out(row, 0, r[q]);
    }
}

// Prefetch, wait, stage, stream.  The first `ahead` passes of the tile (16 KB per wave each) are requested
// before the dependency wait [wait0, wait1), so weights stream while the inputs are still being produced;
// afterwards pass p+1 is requested before pass p is computed.  A tile that stages its inputs only after
// its weights are known (expert up-projection at larger batches) requests one pass ahead, so that its
// inputs do not queue behind two passes.
template <int NB, bool SPLIT, class RowPtr, class Stage, class Out>
__device__ __forceinline__ void mgemv_task(KA& a, Desc w, int t, const RowPtr& W, int nrows, int K, int nb, int wait0,
                                           int wait1, Stage&& stage, Out&& out, Lds& S, int ahead = 2) {
  const MGeo g = mgeo(nrows, K);
  MBuf b0, b1;
  mg_load(b0, W, g, 0);
  if (ahead > 1 && g.np > 1) mg_load(b1, W, g, 1);
  wait_deps(a, w, wait0, wait1, t);
  stage();
  if (SPLIT) split_x(nb, K, S);
  if (ahead == 1 && g.np > 1) mg_load(b1, W, g, 1);
  mark(a, t, 0);
  if constexpr (NB == 1) {  // one token (the class is launched for batches of 1 only)
    VAcc acc;
#pragma unroll
    for (int q = 0; q < 4; ++q) acc.v[q] = 0.f;
    for (int p = 0; p < g.np; p += 2) {
      mgv_compute_any(b0, acc, g, p, S);
      if (p + 2 < g.np) mg_load(b0, W, g, p + 2);
      if (p + 1 >= g.np) break;
      mgv_compute_any(b1, acc, g, p + 1, S);
      if (p + 3 < g.np) mg_load(b1, W, g, p + 3);
    }
    mgv_finish(acc, g, out, S);
  } else {
    MAcc acc;
    macc_zero(acc);
    for (int p = 0; p < g.np; p += 2) {
      mg_compute_any<NB>(b0, acc, g, p, nb, S);
      if (p + 2 < g.np) mg_load(b0, W, g, p + 2);
      if (p + 1 >= g.np) break;
      mg_compute_any<NB>(b1, acc, g, p + 1, nb, S);
      if (p + 3 < g.np) mg_load(b1, W, g, p + 3);
    }
    mg_finish<NB>(acc, g, nb, out, S);
  }
  mark(a, t, 1);
}

// ------------------------------------------------------------------------------------------ task bodies

__device__ __forceinline__ void task_embed(KA& a, Desc w, int t, Lds& S) {
  const int wave = tidx() >> 6, lane = tidx() & 63;
  const int r0 = w[W_R0], r1 = w[W_R1], rt = w[W_A];
  RouterPre rp;
  if (w[W_ARR2] >= 0) router_pre(a, 0, r0, r1, rp);
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
      S.xs[b * (r1 - r0) + r - r0] = v;
      acc = fmaf(v, v, acc);
    }
    const float s = wave_sum(acc);
    if (lane == 0) pub(&a.ssq[b * a.n_rt + rt], s);
  }
  // RoPE angles of each sequence's new position (fp64 angle, then cos/sin), once per step
  if (rt == 0) {
    const int half = a.dh / 2;
    for (int i = tidx(); i < a.B * half; i += NT) {
      const int b = i / half, j = i - b * half;
      const double th = (double)a.seq_lens[b] * a.inv_freq[j];
      double sn, cs;
      sincos(th, &sn, &cs);
      pub(&a.rope_cs[(b * half + j) * 2 + 0], (float)cs);
      pub(&a.rope_cs[(b * half + j) * 2 + 1], (float)sn);
    }
  }
  __syncthreads();
  row_tile_done(a, w, 0, r0, r1, rt, S.xs, rp, S);
}



template <class C>
__device__ __forceinline__ void task_qkv(KA& a, Desc w, int t, Lds& S) {
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
  const NormGain gn = norm_gain(L.attn_norm, d);
  // a workgroup that staged this layer's input for its previous task keeps it
  const bool staged = __builtin_amdgcn_readfirstlane(S.xb_layer) == l + 1;
  mgemv_task<C::NB, false>(
      a, w, t, Rows1{W, d}, r1 - r0, d, a.B, 0, N_WAITS,
      [&] {
        if (!staged) {
          stage_split(a, gn, a.B, nullptr, S);
        }
      },
      [&](int r, int b, float v) { pub(out + b * bstride + r, v); }, S);
  if (tidx() == 0) S.xb_layer = l + 1;  // xb keeps this layer's split input (read after later barriers)
  signal(a, w[W_SIG], w[W_SIGN]);
}

template <class C>
__device__ __forceinline__ void task_oproj(KA& a, Desc w, int t, Lds& S) {
  const int l = w[W_LAYER], g = w[W_A], r0 = w[W_R0], r1 = w[W_R1];
  const int grp = a.Hq / a.Hkv, K = grp * a.dh, ldo = a.Hq * a.dh, B = a.B, d = a.d;
  const uint16_t* W = a.layers[l].wo + (int64_t)r0 * ldo + (int64_t)g * K;
  float* out = a.opart + (int64_t)g * B * d + r0;
  mgemv_task<C::NB, true>(
      a, w, t, Rows1{W, ldo}, r1 - r0, K, B, 0, N_WAITS,
      [&] {
        for (int b = 0; b < B; ++b) lds_copy(a.attn_o + (int64_t)b * ldo + (int64_t)g * K, S.xs + b * K, K / 4);
        drain_stores();
        __syncthreads();
      },
      [&](int r, int b, float v) { pub(out + (int64_t)b * d + r, v); }, S);
  resid_chain(a, w, S);
}

// Routing of an expert slot as its readiness counter carries it: bits 0..15 = expert + 1, bits 16..23 =
// mask of the tokens that selected it; bit 31 alone = slot unused this step.  Tokens of the slot in
// ascending order go to S.slot_b; returns the expert, or -1 for an unused slot.
__device__ __forceinline__ int slot_routing(KA& a, uint32_t v, Lds& S) {
  const int e = (int)(v & 0xffffu) - 1;
  if ((v >> 31) || e < 0 || e >= a.E) return -1;
  if (tidx() == 0) {
    uint32_t m = (v >> 16) & 0xffu;
    int n = 0;
    for (int b = 0; b < a.B; ++b)
      if (m & (1u << b)) S.slot_b[n++] = b;
    S.slot_n = n;
  }
  __syncthreads();
  return S.slot_n > 0 ? e : -1;
}

// Expert slot s of the routing held in S.sel / S.used (slot s = the s-th selected expert in ascending id)
// and its tokens, as slot_routing gives them; -1 for an unused slot.
__device__ __forceinline__ int slot_local(KA& a, int s, Lds& S) {
  if (tidx() == 0) {
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
    int n = 0;
    if (e >= 0)
      for (int b = 0; b < a.B; ++b)
        for (int j = 0; j < a.k; ++j)
          if (S.sel[b * 8 + j] == e) {
            S.slot_b[n++] = b;
            break;
          }
    S.slot_n = n;
    S.slot_e = e;
  }
  __syncthreads();
  const int e = __builtin_amdgcn_readfirstlane(S.slot_e);
  return S.slot_n > 0 ? e : -1;
}

template <class C>
__device__ __forceinline__ void task_up(KA& a, Desc w, int t, Lds& S) {
  const int l = w[W_LAYER], s = w[W_A], r0 = w[W_R0], r1 = w[W_R1];
  const int d = a.d, F = a.F, B = a.B, nr = r1 - r0;
  const LayerW& L = a.layers[l];
  const NormGain gn = norm_gain(L.attn_norm, d);
  const uint16_t* wg0 = L.w_gate;
  const uint16_t* wu0 = L.w_up;
  __asm__ volatile("" ::"s"(wg0), "s"(wu0));
  // Small batches: the layer's input exists before its routing does, so every token's normalised input is
  // staged (and split into BF16 hi/lo) while the router is still being completed, once per workgroup and
  // layer (consecutive tiles of the layer reuse it); once the slot is released only the expert's weights
  // are in flight.  Larger batches stage only the slot's tokens, after routing (staging all of them costs
  // more than it saves there, measured).
  const bool early = B <= 2;
  int e;
  if (early) {
    if (__builtin_amdgcn_readfirstlane(S.xb_layer) != l + 1) {  // not staged by this workgroup's last task
      wait_deps(a, w, 1, 2, t);
      stage_split(a, gn, B, nullptr, S);
      if (tidx() == 0) S.xb_layer = l + 1;
    }
    // the routing itself, from the router partials, as soon as the last row tile has added its own (no
    // wait for the routing workgroup to publish it); kept for this workgroup's later tiles of the layer
    if (__builtin_amdgcn_readfirstlane(S.route_layer) != l + 1) {
      wait_deps(a, w, 2, 3, t);
      route_logits(a, l, S, false);
      route_rank(a, S);
      if (tidx() == 0) S.route_layer = l + 1;
    }
    e = slot_local(a, s, S);
  } else {
    e = slot_routing(a, wait_value(a, w, 0, t, S), S);
  }
  if (e >= 0) {
    const int n = S.slot_n;
    // gate rows then up rows of this tile, as one 2*nr-row tile over two bases
    const uint16_t* Wg = wg0 + ((int64_t)e * F + r0) * d;
    const uint16_t* Wu = wu0 + ((int64_t)e * F + r0) * d;
    auto out = [&](int r, int j, float v) { S.gu[r * 8 + (early ? j : S.slot_b[j])] = v; };
    // small batches: inputs already staged, two passes requested ahead; larger batches stage the slot's
    // tokens once the first pass is in flight
    mgemv_task<C::NB, false>(
        a, w, t, Rows2{Wg, Wu, d, nr}, 2 * nr, d, early ? B : n, 0, 0,
        [&] {
          mark(a, t, 2);  // weights requested
          if (!early) {
            stage_split(a, gn, n, S.slot_b, S);
          }
        },
        out, S, early ? 2 : 1);
    __syncthreads();
    for (int i = tidx(); i < nr * n; i += NT) {
      const int r = i / n, j = i - r * n, b = S.slot_b[j];
      const float gv = S.gu[r * 8 + b], uv = S.gu[(nr + r) * 8 + b];
      const float h = gv / (1.0f + expf(-gv)) * uv;
      pub(a.h + ((int64_t)s * B + j) * F + r0 + r, h);
    }
    signal(a, w[W_SIG], w[W_SIGN]);
  }
  // an unused slot's tiles signal nothing: only the same slot's down-projection tiles wait on them
}

template <class C>
__device__ __forceinline__ void task_down(KA& a, Desc w, int t, Lds& S) {
  const int l = w[W_LAYER], s = w[W_A], r0 = w[W_R0], r1 = w[W_R1];
  const int d = a.d, F = a.F, nr = r1 - r0;
  const uint16_t* wd0 = a.layers[l].w_down;
  __asm__ volatile("" ::"s"(wd0));
  // the slot's routing is known: this expert's weights stream before its hidden state exists
  const int e = slot_routing(a, wait_value(a, w, 0, t, S), S);
  if (e >= 0) {
    const int n = S.slot_n;
    const uint16_t* W = wd0 + ((int64_t)e * d + r0) * F;
    const int32_t* ent = a.slots + ((int64_t)l * a.n_slots + s) * SLOT_WORDS;
    mgemv_task<C::NB, true>(
        a, w, t, Rows1{W, F}, nr, F, n, 1, N_WAITS,
        [&] {
          // hidden state of the slot's tokens, and their selection ranks and gates
          if (tidx() < SLOT_WORDS) S.slotw[tidx()] = ent[tidx()];
          lds_copy(a.h + (int64_t)s * a.B * F, S.xs, n * F / 4);
          drain_stores();
          __syncthreads();
          if (tidx() < n) {
            S.slot_j[tidx()] = S.slotw[3 + 3 * tidx()];
            S.slot_g[tidx()] = __int_as_float(S.slotw[4 + 3 * tidx()]);
          }
          __syncthreads();
        },
        [&](int r, int j, float v) { pub(a.ypart + ((int64_t)S.slot_b[j] * a.k + S.slot_j[j]) * d + r0 + r, S.slot_g[j] * v); }, S);
    resid_chain(a, w, S);
  }
  // an unused slot's arrival on the row tile was made by the routing workgroup
}

// LM head, the kernel's closing phase (not a task): once a workgroup's task phases are exhausted it takes
// 128-row vocabulary chunks from a shared pool (one atomic per chunk, claimed ahead of use) and streams
// them as 16 KB-per-wave passes, each requested two passes before its use, so every compute unit keeps
// reading until the vocabulary is done, whatever its share of the layers was.  Its first chunk is
// requested before it waits for the final residual stream.  Each workgroup publishes its best logit per
// token (maximum, lowest index on ties: an order-independent choice); the last one to finish reduces them
// to the next tokens.
template <class C>
__device__ __forceinline__ void lm_phase(KA& a, Lds& S) {
  constexpr int CHR = 128;  // rows per chunk: one 16-row block per wave, no K split
  constexpr int LMQ = 4;    // ring of claimed chunk ids
  const int d = a.d, B = a.B, V = a.V;
  const int wave = tidx() >> 6, lane = tidx() & 63;
  const MGeo g = mgeo(CHR, d);
  const int np = g.np, nch = (V + CHR - 1) / CHR;
  const int ahead = np >= 2 ? 2 : 3;  // chunks claimed ahead, so pass q + 2 always has its chunk id
  const NormGain gn = norm_gain(a.final_norm, d);
  if (tidx() == 0)
    for (int k = 0; k < ahead; ++k)
      S.lmq[k] = (int)__hip_atomic_fetch_add(ctr_at(a, a.c_lm_pool), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  auto load = [&](MBuf& buf, int q) {
    const int k = q / np, p = q - k * np;
    const int id = S.lmq[k % LMQ];
    if (id >= nch) return;
    MGeo gc = g;
    gc.nrows = min(CHR, V - id * CHR);
    mg_load(buf, Rows1{a.lm_head + (int64_t)id * CHR * d, d}, gc, p);
  };
  MBuf b0, b1;
  const bool any = S.lmq[0] < nch;
  if (any) {
    load(b0, 0);
    load(b1, 1);
  }
  if (tidx() == 0) {
    spin_ge(a, a.c_xfinal, a.n_rt, -1);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  // best (value, row) of this lane's tokens so far: token (lane / 4) % 4 and, for batches above 4, 4 + that
  float bv[2] = {-INFINITY, -INFINITY};
  int bi[2] = {0x7fffffff, 0x7fffffff};
  if (any) {
    stage_split(a, gn, B, nullptr, S);
    MAcc acc;
    macc_zero(acc);
    uint32_t pend = 0;
    bool done = false;
    // pass q: compute, then request pass q + 2 into the same buffer
    auto comp = [&](MBuf& buf, int q) {
      const int k = q / np, p = q - k * np;
      if (p == 0) {
        // chunk k starts: publish the claim made at the start of chunk k - 1, claim chunk k + ahead
        if (k > 0) {
          if (tidx() == 0) S.lmq[(k - 1 + ahead) % LMQ] = (int)pend;
          __syncthreads();
        }
        if (tidx() == 0) pend = __hip_atomic_fetch_add(ctr_at(a, a.c_lm_pool), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        macc_zero(acc);
      }
      const int id = S.lmq[k % LMQ];
      if (id >= nch) {
        done = true;
        return;
      }
      mg_compute_any<C::NB>(buf, acc, g, p, B, S);
      if (p == np - 1) {
        float va[4], vb[4];
        mg_lane_values<C::NB>(acc, B, va, vb);
        mg_emit<C::NB>(va, vb, B, [&](int r, int j, float v) {
          const int row = id * CHR + wave * 16 + r;
          if (row < V) {
            a.logits[(int64_t)j * V + row] = v;
            if (j < 4) {
              if (v > bv[0] || (v == bv[0] && row < bi[0])) {
                bv[0] = v;
                bi[0] = row;
              }
            } else if (v > bv[1] || (v == bv[1] && row < bi[1])) {
              bv[1] = v;
              bi[1] = row;
            }
          }
        });
      }
      load(buf, q + 2);
    };
    for (int q = 0; !done; q += 2) {
      comp(b0, q);
      if (done) break;
      comp(b1, q + 1);
    }
  }
  // this workgroup's best per token: the 4 lanes of a token in each wave (lanes 4s + 16i), then the waves in
  // order
#pragma unroll
  for (int u = 0; u < 2; ++u) {
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const float ov = __shfl_xor(bv[u], o);
      const int oi = __shfl_xor(bi[u], o);
      if (ov > bv[u] || (ov == bv[u] && oi < bi[u])) {
        bv[u] = ov;
        bi[u] = oi;
      }
    }
  }
  float* wbv = S.sc;                                  // [NW][16]
  int* wbi = reinterpret_cast<int*>(S.sc + NW * 16);  // [NW][16]
  if (lane < 16 && (lane & 3) == 0) {
    const int sl = lane >> 2;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      wbv[wave * 16 + 4 * u + sl] = bv[u];
      wbi[wave * 16 + 4 * u + sl] = bi[u];
    }
  }
  __syncthreads();
  if (tidx() < B) {
    const int b = tidx();
    float v = -INFINITY;
    int ix = 0x7fffffff;
    for (int q = 0; q < NW; ++q) {
      const float ov = wbv[q * 16 + b];
      const int oi = wbi[q * 16 + b];
      if (ov > v || (ov == v && oi < ix)) {
        v = ov;
        ix = oi;
      }
    }
    pub(&a.lmbest_v[b * LM_MAX_WG + blockIdx.x], v);
    pubi(&a.lmbest_i[b * LM_MAX_WG + blockIdx.x], ix);
  }
  if (arrive_last(a, a.c_lm_arrive, gridDim.x, S)) {
    if (wave < B) {
      const int b = wave;
      float v = -INFINITY;
      int ix = 0x7fffffff;
      for (int q = lane; q < (int)gridDim.x; q += 64) {
        const float ov = a.lmbest_v[b * LM_MAX_WG + q];
        const int oi = a.lmbest_i[b * LM_MAX_WG + q];
        if (ov > v || (ov == v && oi < ix)) {
          v = ov;
          ix = oi;
        }
      }
      for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(v, o);
        const int oi = __shfl_xor(ix, o);
        if (ov > v || (ov == v && oi < ix)) {
          v = ov;
          ix = oi;
        }
      }
      if (lane == 0) a.next_tok[b] = ix;
    }
  }
}

// ------------------------------------------------------------------------------------------ attention
// Batch entry j's new key (RoPE at its position, from the angles task_embed computed) and value of KV group
// g, both rounded to BF16 as the cache stores them, into S.kn / S.vn.
template <int DH, int GRP>
__device__ __forceinline__ void stage_new_kv(KA& a, int j, int g, Lds& S) {
  const float* src = a.qkv + ((int64_t)j * a.Hkv + g) * (GRP + 2) * DH;
  const float* cs = a.rope_cs + (int64_t)j * (DH / 2) * 2;
  for (int i = tidx(); i < DH / 2; i += NT) {
    const float c = cs[2 * i], sn = cs[2 * i + 1];
    const float x0 = src[GRP * DH + i], x1 = src[GRP * DH + i + DH / 2];
    S.kn[i] = bf2f(f2bf(x0 * c - x1 * sn));
    S.kn[i + DH / 2] = bf2f(f2bf(x0 * sn + x1 * c));
  }
  for (int i = tidx(); i < DH; i += NT) S.vn[i] = bf2f(f2bf(src[(GRP + 1) * DH + i]));
}

// Where the step's entry b reads the cache.  Entries b0..b of a chunk (consecutive positions of one sequence
// in one step, prefill: first_of[b] = b0) all read the cached positions [0, len0), len0 being the position of
// the chunk's first token, and take the keys and values of positions len0..len from this step's projections
// (the cache slots of those positions are written in this same step).  A decode entry is a chunk of one.
struct SeqView {
  int len;   // the entry's own position (its query's RoPE position, the slot its K/V are written to)
  int b0;    // first entry of its chunk
  int len0;  // cached positions read: [0, len0)
};
__device__ __forceinline__ SeqView seq_view(KA& a, int b, int t) {
  SeqView v;
  v.len = a.seq_lens[b];
  if (v.len < 0 || v.len / 16 >= a.max_pages) {
    if (tidx() == 0) raise_error(a, ERRC_SEQLEN, t);
    v.len = 0;
  }
  v.b0 = a.first_of ? a.first_of[b] : b;
  v.len0 = v.len - (b - v.b0);
  if (v.b0 < 0 || v.b0 > b || v.len0 < 0 || a.seq_lens[v.b0] != v.len0) {  // not a chunk of consecutive positions
    if (tidx() == 0) raise_error(a, ERRC_SEQLEN, t);
    v.b0 = b;
    v.len0 = v.len;
  }
  return v;
}

// Debug page-walk record of (layer, entry, KV group): pages read (npg from logical page np0), positions
// attended; all additions are modulo 2^32 and commutative, so the splits' order does not matter.
__device__ __forceinline__ uint32_t* walk_rec(KA& a, int l, int b, int g) {
  return a.pagewalk ? a.pagewalk + (((int64_t)l * a.B + b) * a.Hkv + g) * 4 : nullptr;
}

// The last split of (b, g) to finish merges all splits (log-sum-exp) and publishes the group's output.  In
// a plan with merge tasks (no arrival counter) the split only counts its published partial.
template <int DH, int GRP>
__device__ __forceinline__ void attn_merge(KA& a, Desc w, int t, int b, int g, int nsplit, Lds& S) {
  const int tid = tidx(), wave = tid >> 6, lane = tid & 63;
  const int Hkv = a.Hkv;
  if (w[W_ARR] < 0) {
    signal(a, w[W_SIG], w[W_SIGN]);
    return;
  }
  if (arrive_last(a, w[W_ARR], w[W_ARRN], S)) {
    mark(a, t, 3);
    const float* p0 = a.apart + (((int64_t)b * Hkv + g) * a.apart_stride) * GRP * (DH + 2);
    nsplit = min(nsplit, a.apart_stride);
    float* wsc = S.xs;                               // [GRP][nsplit] running max, then weights exp(m_s - M)
    float* lsc = S.xs + GRP * ATTN_MAX_SPLITS;       // [GRP][nsplit] running sums
    float* lsum = S.xs + 2 * GRP * ATTN_MAX_SPLITS;  // [GRP]
    // One round trip: each thread requests its two outputs' values of the first 32 splits, then the splits'
    // (max, sum) pairs go to LDS; later 32-split chunks (long contexts) are requested as they are merged.
    static_assert(GRP * DH <= 2 * NT, "two outputs per thread");
    const bool has0 = tid < GRP * DH, has1 = tid + NT < GRP * DH;
    const int h0 = has0 ? tid / DH : 0, d0 = has0 ? tid - h0 * DH : 0;
    const int h1 = has1 ? (tid + NT) / DH : h0, d1 = has1 ? (tid + NT) - h1 * DH : d0;
    constexpr int MQ = 32;
    float v0[MQ], v1[MQ];
    auto load_chunk = [&](int q) {
#pragma unroll
      for (int u = 0; u < MQ; ++u) {
        const bool ok = has0 && q + u < nsplit;
        v0[u] = ok ? p0[((int64_t)(q + u) * GRP + h0) * (DH + 2) + d0] : 0.f;
        v1[u] = ok ? p0[((int64_t)(q + u) * GRP + h1) * (DH + 2) + d1] : 0.f;
      }
    };
    load_chunk(0);
    for (int i = tid; i < GRP * nsplit; i += NT) {
      const int h = i / nsplit, q = i - h * nsplit;
      const float* r = p0 + ((int64_t)q * GRP + h) * (DH + 2) + DH;
      wsc[i] = r[0];
      lsc[i] = r[1];
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
        Ls = fmaf(lsc[h * nsplit + q], wq, Ls);
      }
      Ls = wave_sum(Ls);
      if (lane == 0) lsum[h] = Ls;
    }
    __syncthreads();
    float o0 = 0.f, o1 = 0.f;
    for (int q = 0; q < nsplit; q += MQ) {
      if (q > 0) load_chunk(q);
#pragma unroll
      for (int u = 0; u < MQ; ++u) {
        if (q + u < nsplit) {
          o0 = fmaf(v0[u], wsc[h0 * nsplit + q + u], o0);
          o1 = fmaf(v1[u], wsc[h1 * nsplit + q + u], o1);
        }
      }
    }
    if (has0) pub(a.attn_o + (int64_t)b * a.Hq * DH + ((int64_t)g * GRP + h0) * DH + d0, o0 / lsum[h0]);
    if (has1) pub(a.attn_o + (int64_t)b * a.Hq * DH + ((int64_t)g * GRP + h1) * DH + d1, o1 / lsum[h1]);
    signal(a, w[W_SIG], w[W_SIGN]);
  }
}

// MERGE task: heads [h0, h0 + nh) of (sequence b, KV group g), once every split of (b, g) has published its
// partial.  The arithmetic is the last-arriver merge's, operation for operation (per head: the maximum, the
// weights and their sum on one wave; per output: the splits added in order, then one division), so both
// give the same bits; a long context's partials (about 200 KB per group) are then read by several
// workgroups instead of one.  The slice of every split (nh rows of o, maximum and sum) is copied straight
// into LDS in one round trip, 16 bytes per lane (4 where a slice is not a whole number of 16-byte chunks).
// Not inlined: inlined, it changed the register allocation of the 8-token class elsewhere (more spills;
// batch 8 about 8 % slower, measured), and it runs a few times per layer at most.
template <int DH, int GRP>
__device__ __attribute__((noinline)) void task_merge(KA& a, Desc w, int t, Lds& S) {
  const int tid = tidx(), wave = tid >> 6, lane = tid & 63;
  const int b = w[W_A], g = w[W_B], h0 = w[W_C], nh = w[W_R0];
  const int nsplit = min((int)w[W_D], a.apart_stride);
  constexpr int ROWF = DH + 2;            // floats per head row of a partial: o, running max, running sum
  constexpr int CHB = ROWF % 4 == 0 ? 16 : 4;  // bytes per direct load
  const int row = nh * ROWF;              // floats of one split's slice (contiguous in the partials)
  static_assert(sizeof(S.xb) / 4 >= ATTN_MERGE_STAGE_FLOATS, "the merge staging area holds what the planner allows");
  if (nh < 1 || h0 < 0 || h0 + nh > GRP || nh * DH > NT || nsplit * row > ATTN_MERGE_STAGE_FLOATS) {
    if (tid == 0) raise_error(a, ERRC_OPCODE, t);
    return;
  }
  wait_deps(a, w, 0, N_WAITS, t);
  mark(a, t, 0);
  const float* p0 = a.apart + (((int64_t)b * a.Hkv + g) * a.apart_stride) * GRP * ROWF;
  float* st = reinterpret_cast<float*>(S.xb);  // [nsplit][nh][ROWF]
  if (tid == 0) S.xb_layer = 0;                 // the staged GEMV input is overwritten
  {
    constexpr int CF = CHB / 4;                 // floats per chunk
    const int per = row / CF, n = nsplit * per;
    for (int c0 = wave * 64; c0 < n; c0 += NT) {
      const int c = c0 + lane;
      if (c < n) {
        const int q = c / per, k = c - q * per;
        const auto src = (const __attribute__((address_space(1))) void*)(p0 + ((int64_t)q * GRP + h0) * ROWF + k * CF);
        const auto dst = (__attribute__((address_space(3))) void*)(st + (int64_t)c0 * CF);
        if constexpr (CHB == 16) __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
        else __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
      }
    }
  }
  drain_stores();
  __syncthreads();
  float* wsc = S.xs;                               // [nh][nsplit] weights exp(m_s - M)
  float* lsum = S.xs + GRP * ATTN_MAX_SPLITS;      // [nh]
  if (wave < nh) {
    const int h = wave;
    float M = -INFINITY;
    for (int q = lane; q < nsplit; q += 64) M = fmaxf(M, st[q * row + h * ROWF + DH]);
    M = wave_max(M);
    float Ls = 0.f;
    for (int q = lane; q < nsplit; q += 64) {
      const float mq = st[q * row + h * ROWF + DH];
      const float wq = mq == -INFINITY ? 0.f : expf(mq - M);
      wsc[h * nsplit + q] = wq;
      Ls = fmaf(st[q * row + h * ROWF + DH + 1], wq, Ls);
    }
    Ls = wave_sum(Ls);
    if (lane == 0) lsum[h] = Ls;
  }
  __syncthreads();
  mark(a, t, 1);
  if (tid < nh * DH) {
    const int hl = tid / DH, d = tid - hl * DH;
    float o = 0.f;
    for (int q = 0; q < nsplit; ++q) o = fmaf(st[q * row + hl * ROWF + d], wsc[hl * nsplit + q], o);
    pub(a.attn_o + (int64_t)b * a.Hq * DH + ((int64_t)g * GRP + h0 + hl) * DH + d, o / lsum[hl]);
  }
  signal(a, w[W_SIG], w[W_SIGN]);
}

// d_head 64 (the tiny shape; d_head 128 runs attn_split_w below): split s of (sequence b, KV group g)
// covers positions [j0, j1) of the sequence's 0..len window (len = its prior length; position len is the
// new token, taken from this step's projections, RoPE'd, rounded to BF16 and written to the cache by the
// split that holds it).  The split's page list and its first two chunks of K and V (128 positions each)
// are loaded BEFORE the task waits for this step's queries.  Scores run
// on MFMA: each wave takes 16 positions of a chunk with K as the A operand (as stored) and the group's
// RoPE'd, scaled queries as BF16 hi + lo B operands held in registers for the whole split.  After the
// chunk's online softmax (one wave per head), each thread accumulates p * V for a 4-dim slice of its
// positions; the next chunk's K/V loads are in flight meanwhile.  The per-thread partial outputs are
// reduced once per split, and the last split of (b, g) to finish merges all splits.
template <int DH, int GRP>
__device__ __forceinline__ void attn_split(KA& a, Desc w, int t, Lds& S) {
  constexpr int DPT = 4;            // V / output dims per thread slice
  constexpr int SL = DH / DPT;      // slices per position (32 or 16)
  constexpr int PPP = NT / SL;      // positions per V pass (16 or 32)
  constexpr int CH = 128;           // positions per chunk: 8 waves x 16-position MFMA blocks
  constexpr int NP = CH / PPP;      // V positions per thread per chunk (8 or 4)
  constexpr int NKK = DH / 32;      // MFMA k-steps over the head dim
  static_assert(CH == NW * 16, "one 16-position score block per wave");
  const int l = w[W_LAYER], b = w[W_A], g = w[W_B], s = w[W_C], nsplit = w[W_D];
  const int tid = tidx(), wave = tid >> 6, lane = tid & 63;
  const int sl = tid % SL, pp = tid / SL;
  const int Hkv = a.Hkv;
  const SeqView sv = seq_view(a, b, t);
  const int len = sv.len, len0 = sv.len0, b0 = sv.b0;
  // the planner cuts the cached positions [0, len0) into splits of w[W_R0] positions (whole 128-position
  // chunks, fixed for the task list's life); the last split takes the rest of the cached positions (a
  // context that grew since planning adds to it) and the new positions len0..len
  const int chunk = w[W_R0];
  const bool last = s == nsplit - 1;
  const int j0 = chunk > 0 ? (int)min<int64_t>((int64_t)s * chunk, len0) : 0;
  int jc1 = last ? len0 : min(j0 + chunk, len0);  // cached positions end
  if (chunk <= 0 || chunk % CH != 0 || jc1 - j0 > ATTN_MAX_SPLIT_PAGES * 16) {  // bad descriptor, or lengths
    if (tid == 0) raise_error(a, ERRC_SEQLEN, t);                                  // far beyond the plan
    jc1 = j0;
  }
  const bool has_new = last;
  const int32_t* ptab = a.page_tables + (int64_t)b * a.max_pages;
  uint16_t* kvl = a.kv + (int64_t)l * a.n_pages * 2 * Hkv * 16 * DH;
  const int64_t vstride = (int64_t)Hkv * 16 * DH;
  uint32_t* const pw = walk_rec(a, l, b, g);

  // page list of the split
  const int np0 = j0 >> 4, npg = jc1 > j0 ? ((jc1 - 1) >> 4) - np0 + 1 : 0;
  for (int i = tid; i < npg; i += NT) {
    int ph = ptab[np0 + i];
    if (ph < 0 || ph >= a.n_pages) {
      raise_error(a, ERRC_PAGE, t);
      ph = -1;
    }
    S.pages[i] = ph;
    if (pw) atomicAdd(pw + 1, (uint32_t)(np0 + i + 1) * (uint32_t)ph);
  }
  if (pw && tid == 0) {
    atomicAdd(pw + 0, (uint32_t)npg);
    atomicAdd(pw + 2, (uint32_t)(jc1 - j0 + (has_new ? b - b0 + 1 : 0)));
  }
  __syncthreads();
  auto kv_base = [&](int pos) -> int64_t {
    const int ph = S.pages[(pos >> 4) - np0];
    return ph < 0 ? -1 : (((int64_t)ph * 2) * Hkv + g) * 16 * DH + (pos & 15) * DH;
  };
  // K of the wave's 16 positions in the plain A-operand layout (16 positions x 32 dims per load); V in
  // 4-dim slices
  auto load_chunk = [&](int c0, u4 (&kk)[NKK], u2 (&vv)[NP]) {
    const int pos = c0 + 16 * wave + (lane & 15);
    const int64_t kb = pos < jc1 ? kv_base(pos) : -1;
#pragma unroll
    for (int q = 0; q < NKK; ++q)
      kk[q] = kb >= 0 ? __builtin_nontemporal_load(as_global(kvl + kb + 8 * (lane >> 4) + 32 * q)) : u4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int pos = c0 + pp + PPP * i;
      const int64_t base = pos < jc1 ? kv_base(pos) : -1;
      vv[i] = base >= 0 ? __builtin_nontemporal_load(as_global2(kvl + base + vstride + sl * DPT)) : u2{0, 0};
    }
  };
  u4 kc[NKK], kx[NKK];
  u2 vc[NP], vx[NP];
  // the split's first two chunks of old K/V stream while this step's projections are produced
  load_chunk(j0, kc, vc);
  load_chunk(j0 + CH, kx, vx);

  wait_deps(a, w, 0, N_WAITS, t);

  // queries of the group: RoPE at position len, times 1/sqrt(dh); fp32 copy for the new token's score and
  // BF16 hi/lo copies (heads as MFMA columns, zero columns beyond the group) for the cached positions
  const float* qsrc = a.qkv + ((int64_t)b * Hkv + g) * (GRP + 2) * DH;
  const float* cs = a.rope_cs + (int64_t)b * (DH / 2) * 2;
  const float qscale = 1.0f / sqrtf((float)DH);
  uint16_t* qb = S.xb;  // [2][16][DH]: hi then lo
  if (tid == 0) S.xb_layer = 0;
  for (int i = tid; i < 16 * DH; i += NT) {
    if (i >= GRP * DH) {
      qb[i] = 0;
      qb[16 * DH + i] = 0;
    }
  }
  for (int i = tid; i < GRP * DH / 2; i += NT) {
    const int h = i / (DH / 2), j = i - h * (DH / 2);
    const float c = cs[2 * j], sn = cs[2 * j + 1];
    const float x0 = qsrc[h * DH + j], x1 = qsrc[h * DH + j + DH / 2];
    const float y0 = (x0 * c - x1 * sn) * qscale, y1 = (x0 * sn + x1 * c) * qscale;
    S.q[h * DH + j] = y0;
    S.q[h * DH + j + DH / 2] = y1;
    const uint16_t h0 = f2bf(y0), h1 = f2bf(y1);
    qb[h * DH + j] = h0;
    qb[h * DH + j + DH / 2] = h1;
    qb[16 * DH + h * DH + j] = f2bf(y0 - bf2f(h0));
    qb[16 * DH + h * DH + j + DH / 2] = f2bf(y1 - bf2f(h1));
  }
  if (has_new) stage_new_kv<DH, GRP>(a, b, g, S);
  if (tid < GRP) {
    S.hm[tid] = -INFINITY;
    S.hl[tid] = 0.f;
  }
  __syncthreads();
  if (has_new) {  // this entry's K/V go to the cache slot of position len (layer l)
    const int ph = ptab[len >> 4];
    if (ph >= 0 && ph < a.n_pages) {
      const int64_t base = (((int64_t)ph * 2) * Hkv + g) * 16 * DH + (len & 15) * DH;
      for (int j = tid; j < DH; j += NT) {
        kvl[base + j] = f2bf(S.kn[j]);
        kvl[base + vstride + j] = f2bf(S.vn[j]);
      }
      if (pw && tid == 0) pw[3] = 1u + (uint32_t)ph * 16u + (uint32_t)(len & 15);
    } else if (tid == 0) {
      raise_error(a, ERRC_PAGE, t);
    }
  }
  mark(a, t, 0);
  // query operands: head j in column j, 32 dims per k-step
  u4 qh[NKK], ql[NKK];
#pragma unroll
  for (int q = 0; q < NKK; ++q) {
    qh[q] = *reinterpret_cast<const u4*>(qb + (lane & 15) * DH + 8 * (lane >> 4) + 32 * q);
    ql[q] = *reinterpret_cast<const u4*>(qb + 16 * DH + (lane & 15) * DH + 8 * (lane >> 4) + 32 * q);
  }
  float o[GRP][DPT];
#pragma unroll
  for (int h = 0; h < GRP; ++h)
#pragma unroll
    for (int i = 0; i < DPT; ++i) o[h][i] = 0.f;

  for (int c0 = j0; c0 < jc1; c0 += CH) {
    // scores on MFMA: D[position][head] = K (16 positions x 32 dims) times q^T (32 dims x heads), hi + lo
    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < NKK; ++q) {
      const bf16x8 av = __builtin_bit_cast(bf16x8, kc[q]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, qh[q]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, ql[q]), acc, 0, 0, 0);
    }
    if ((lane & 15) < GRP) {
      const int h = lane & 15;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pl = 16 * wave + 4 * (lane >> 4) + r;
        S.sc[h * CH + pl] = c0 + pl < jc1 ? acc[r] : -INFINITY;
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
    // rotate: the next chunk is in flight or has landed; request the one after it
#pragma unroll
    for (int q = 0; q < NKK; ++q) kc[q] = kx[q];
#pragma unroll
    for (int i = 0; i < NP; ++i) vc[i] = vx[i];
    if (c0 + 2 * CH < jc1) load_chunk(c0 + 2 * CH, kx, vx);
  }
  mark(a, t, 1);
  // the new positions len0..len, one at a time (entries b0..b; a decode entry has only its own)
  if (has_new) {
    for (int j = b0; j <= b; ++j) {
      if (b0 != b) {  // a chunk: entry j's key and value (S.kn / S.vn held the previous one)
        __syncthreads();
        stage_new_kv<DH, GRP>(a, j, g, S);
        __syncthreads();
      }
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
  }
  if (nsplit > a.apart_stride && tid == 0) raise_error(a, ERRC_SEQLEN, t);  // a list planned for another stride
  float* part = a.apart + ((((int64_t)b * Hkv + g) * a.apart_stride + min(s, a.apart_stride - 1)) * GRP) * (DH + 2);
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
  attn_merge<DH, GRP>(a, w, t, b, g, nsplit, S);
}

// d_head 128: split s of (sequence b, KV group g) with every wave independent.  The split's cached
// positions are cut into blocks of 32; wave w takes blocks w, w + 8, w + 16, ... and runs them start to
// finish on its own (no workgroup barrier inside the loop): K of the block in registers (row quads, see
// the GEMV core), V straight into the wave's own 8 KB LDS area by direct loads (swizzled 16-byte slots),
// the next block of both requested before the current one is computed.  Scores on MFMA (K rows as A,
// the group's RoPE'd, scaled queries as BF16 hi + lo B operands), online softmax per head over the
// block (eight lanes per head), then P.V on MFMA: O^T[d][h] += V^T[d][pos] P^T[pos][h] with V^T gathered
// from the wave's LDS area and P as BF16 hi + lo parts.  Each wave keeps its own running (max, sum, O);
// the waves are combined once at the end, then the new token (position len, last split only) is added.
constexpr int WAVE_SHIFT_DIV = 16;
template <int DH, int GRP>
__device__ __forceinline__ void attn_split_w(KA& a, Desc w, int t, Lds& S) {
  static_assert(DH == 128 && GRP == 8, "wave-independent attention: d_head 128, eight heads per KV group");
  constexpr int WB = 32;                 // positions per wave block
  constexpr int NKQ = WB / 4;            // K loads (position quads) per block and lane
  constexpr int VLD = WB * DH * 2 / 16 / 64;  // 16-byte direct V loads per block and lane (8)
  constexpr int VW = WB * DH;            // bf16 elements of a wave's V area (8 KB)
  static_assert(NKQ + VLD < 64, "vmcnt field");
  const int l = w[W_LAYER], b = w[W_A], g = w[W_B], s = w[W_C], nsplit = w[W_D];
  const int tid = tidx(), wave = tid >> 6, lane = tid & 63;
  const int Hkv = a.Hkv;
  const SeqView sv = seq_view(a, b, t);
  const int len = sv.len, len0 = sv.len0, b0 = sv.b0;
  // the planner cuts the cached positions [0, len0) into splits of w[W_R0] positions (whole 128-position
  // chunks, fixed for the task list's life); the last split takes the rest of the cached positions (a
  // context that grew since planning adds to it) and the new positions len0..len
  const int chunk = w[W_R0];
  const bool last = s == nsplit - 1;
  const int j0 = chunk > 0 ? (int)min<int64_t>((int64_t)s * chunk, len0) : 0;
  int jc1 = last ? len0 : min(j0 + chunk, len0);  // cached positions end
  if (chunk <= 0 || chunk % 128 != 0 || jc1 - j0 > ATTN_MAX_SPLIT_PAGES * 16) {
    if (tid == 0) raise_error(a, ERRC_SEQLEN, t);
    jc1 = j0;
  }
  const bool has_new = last;
  const int32_t* ptab = a.page_tables + (int64_t)b * a.max_pages;
  uint16_t* kvl = a.kv + (int64_t)l * a.n_pages * 2 * Hkv * 16 * DH;
  const int64_t vstride = (int64_t)Hkv * 16 * DH;
  uint32_t* const pw = walk_rec(a, l, b, g);

  // page list of the split
  const int np0 = j0 >> 4, npg = jc1 > j0 ? ((jc1 - 1) >> 4) - np0 + 1 : 0;
  for (int i = tid; i < npg; i += NT) {
    int ph = ptab[np0 + i];
    if (ph < 0 || ph >= a.n_pages) {
      raise_error(a, ERRC_PAGE, t);
      ph = -1;
    }
    S.pages[i] = ph;
    if (pw) atomicAdd(pw + 1, (uint32_t)(np0 + i + 1) * (uint32_t)ph);
  }
  if (pw && tid == 0) {
    atomicAdd(pw + 0, (uint32_t)npg);
    atomicAdd(pw + 2, (uint32_t)(jc1 - j0 + (has_new ? b - b0 + 1 : 0)));
  }
  if (tid == 0) S.xb_layer = 0;  // the V areas overwrite the staged GEMV input
  __syncthreads();
  // cache offset of a position's K row (the layer's first row for positions beyond the split or on a bad
  // page: every load instruction is issued, so each block is exactly NKQ + VLD loads and the V waits
  // below can count them; those rows' scores become -inf and their V rows are zeroed where read)
  auto kv_off = [&](int pos) -> int64_t {
    if (pos >= jc1) return 0;
    const int ph = S.pages[(pos >> 4) - np0];
    return ph < 0 ? 0 : (((int64_t)ph * 2) * Hkv + g) * 16 * DH + (pos & 15) * DH;
  };
  const int nblk = (jc1 - j0 + WB - 1) / WB;
  // blocks of this wave: round-robin over the waves for R rounds, then the tail round-robin over the first
  // half of the waves only (they share a SIMD with the second half and, older, are issued first: at many
  // blocks per wave, the second half finishes last otherwise)
  const int nb_base = nblk / NW;
  const int wshift = nb_base / WAVE_SHIFT_DIV;
  const int R = nb_base - wshift;
  const int T = nblk - R * NW;
  const int wcnt = wshift == 0 ? nb_base + (wave < nblk - nb_base * NW ? 1 : 0)
                               : R + (wave < NW / 2 ? (T - wave + NW / 2 - 1) / (NW / 2) : 0);
  auto blk = [&](int i) { return (wshift == 0 || i < R) ? i * NW + wave : R * NW + (i - R) * (NW / 2) + wave; };
  uint16_t* const va0 = reinterpret_cast<uint16_t*>(S.xs) + wave * VW;  // the wave's two V areas
  uint16_t* const va1 = S.xb + wave * VW;
  static_assert(NW * VW * 2 <= XS_FLOATS * 4 && NW * VW <= 16 * XBP + 64, "V areas fit the staging areas");
  auto load_k = [&](int i, u4 (&kk)[NKQ]) {  // block i of this wave
    const int c0 = j0 + blk(i) * WB;
#pragma unroll
    for (int u = 0; u < NKQ; ++u) {
      const int pos = c0 + 4 * u + ((lane & 15) >> 2);
      kk[u] = __builtin_nontemporal_load(as_global(kvl + kv_off(pos) + 32 * (lane >> 4) + 8 * (lane & 3)));
    }
  };
  // V row r of the block keeps its 16-byte chunk c in slot c ^ 2((r >> 3) & 3) of the row
  auto load_v = [&](int i, uint16_t* va) {
    const int c0 = j0 + blk(i) * WB;
#pragma unroll
    for (int j = 0; j < VLD; ++j) {
      const int n = j * 64 + lane;
      const int r = n >> 4, cg = (n & 15) ^ (2 * ((r >> 3) & 3));
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(kvl + kv_off(c0 + r) + vstride + cg * 8),
                                       (__attribute__((address_space(3))) void*)(va + j * 512), 16, 0, 0);
    }
  };
  u4 kc[NKQ], kx[NKQ];
  // the wave's first two blocks of old K/V stream while this step's projections are produced
  load_k(0, kc);
  load_v(0, va0);
  load_k(1, kx);
  load_v(1, va1);

  wait_deps(a, w, 0, N_WAITS, t);

  // queries of the group: RoPE at position len, times 1/sqrt(dh); fp32 copy for the new token's score and
  // BF16 hi/lo copies (heads as MFMA columns, zero columns beyond the group) for the cached positions,
  // staged in the probability area (free until the loop)
  const float* qsrc = a.qkv + ((int64_t)b * Hkv + g) * (GRP + 2) * DH;
  const float* cs = a.rope_cs + (int64_t)b * (DH / 2) * 2;
  const float qscale = 1.0f / sqrtf((float)DH);
  uint16_t* qb = reinterpret_cast<uint16_t*>(S.pt);  // [2][16][DH]: hi then lo
  static_assert(2 * 16 * DH * 2 <= (int)sizeof(S.pt), "query staging fits the probability area");
  for (int i = tid; i < 16 * DH; i += NT) {
    if (i >= GRP * DH) {
      qb[i] = 0;
      qb[16 * DH + i] = 0;
    }
  }
  for (int i = tid; i < GRP * DH / 2; i += NT) {
    const int h = i / (DH / 2), j = i - h * (DH / 2);
    const float c = cs[2 * j], sn = cs[2 * j + 1];
    const float x0 = qsrc[h * DH + j], x1 = qsrc[h * DH + j + DH / 2];
    const float y0 = (x0 * c - x1 * sn) * qscale, y1 = (x0 * sn + x1 * c) * qscale;
    S.q[h * DH + j] = y0;
    S.q[h * DH + j + DH / 2] = y1;
    const uint16_t h0 = f2bf(y0), h1 = f2bf(y1);
    qb[h * DH + j] = h0;
    qb[h * DH + j + DH / 2] = h1;
    qb[16 * DH + h * DH + j] = f2bf(y0 - bf2f(h0));
    qb[16 * DH + h * DH + j + DH / 2] = f2bf(y1 - bf2f(h1));
  }
  if (has_new) stage_new_kv<DH, GRP>(a, b, g, S);
  for (int i = tid; i < 32; i += NT) S.sc[i] = 0.f;  // zero B rows for the heads beyond the group
  __syncthreads();
  if (has_new) {  // this entry's K/V go to the cache slot of position len (layer l)
    const int ph = ptab[len >> 4];
    if (ph >= 0 && ph < a.n_pages) {
      const int64_t base = (((int64_t)ph * 2) * Hkv + g) * 16 * DH + (len & 15) * DH;
      for (int j = tid; j < DH; j += NT) {
        kvl[base + j] = f2bf(S.kn[j]);
        kvl[base + vstride + j] = f2bf(S.vn[j]);
      }
      if (pw && tid == 0) pw[3] = 1u + (uint32_t)ph * 16u + (uint32_t)(len & 15);
    } else if (tid == 0) {
      raise_error(a, ERRC_PAGE, t);
    }
  }
  // query operands: B column 4s + h holds head 4hg + s at K-part h (chunk 4(l/16) + h of the head's vector)
  constexpr int NHG = GRP / 4;
  u4 qh[NHG], ql[NHG];
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg) {
    const int hd = 4 * hg + ((lane & 15) >> 2);
    qh[hg] = *reinterpret_cast<const u4*>(qb + hd * DH + 32 * (lane >> 4) + 8 * (lane & 3));
    ql[hg] = *reinterpret_cast<const u4*>(qb + 16 * DH + hd * DH + 32 * (lane >> 4) + 8 * (lane & 3));
  }
  __syncthreads();  // the probability area becomes the waves' score / probability scratch
  mark(a, t, 0);

  float* const scw = S.pt + wave * (GRP * WB);                       // [head][32] scores (fp32)
  uint16_t* const pbw = reinterpret_cast<uint16_t*>(scw);           // then [hi: 8 rows][lo: 8 rows] x 32 BF16
  float* const alw = S.gu + wave * 8;                               // per-head rescale of the block
  const uint16_t* const zrow = reinterpret_cast<const uint16_t*>(S.sc);
  const int q4 = lane >> 4, hc = lane & 15;                         // P.V: lane's position group and column
  const int sh = lane >> 3, sp = (lane & 7) * 4;                    // softmax: lane's head and positions
  float m_run = -INFINITY, l_run = 0.f;                             // of head sh (lanes 8sh..8sh+7)
  f4 oacc[DH / 16];
#pragma unroll
  for (int db = 0; db < DH / 16; ++db) oacc[db] = f4{0.f, 0.f, 0.f, 0.f};

  for (int i = 0; i < wcnt; ++i) {
    const int c0 = j0 + blk(i) * WB;
    // scores: for position quad u and head group hg, D[4r + h][4s + h] is position 4u + r times head
    // 4hg + s over K-part h (hi, then lo); the parts are added across each lane quad
#pragma unroll
    for (int u = 0; u < NKQ; ++u) {
#pragma unroll
      for (int hg = 0; hg < NHG; ++hg) {
        f4 acc = mfma(kc[u], qh[hg], f4{0.f, 0.f, 0.f, 0.f});
        acc = mfma(kc[u], ql[hg], acc);
        float v = pick4(acc, lane & 3);
        v += dpp<0xB1>(v);
        v += dpp<0x4E>(v);
        const int hd = 4 * hg + ((lane >> 2) & 3), pl = 4 * u + (lane >> 4);
        if ((lane & 3) == 0) scw[hd * WB + pl] = c0 + pl < jc1 ? v : -INFINITY;
      }
    }
    // online softmax of head sh over the block: lanes 8sh..8sh+7 hold four positions each
    const f4 s4 = *reinterpret_cast<const f4*>(scw + sh * WB + sp);
    float bm = fmaxf(fmaxf(s4.x, s4.y), fmaxf(s4.z, s4.w));
    bm = fmaxf(bm, dpp<0xB1>(bm));
    bm = fmaxf(bm, dpp<0x4E>(bm));
    bm = fmaxf(bm, dpp<0x141>(bm));
    const float mnew = fmaxf(m_run, bm);
    const float alpha = m_run == -INFINITY ? 0.f : expf(m_run - mnew);
    float pr[4] = {s4.x, s4.y, s4.z, s4.w};
    float ps = 0.f;
    uint32_t hw[2], lw[2];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pr[e] = pr[e] == -INFINITY ? 0.f : expf(pr[e] - mnew);
      ps += pr[e];
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint16_t a0 = f2bf(pr[2 * e]), a1 = f2bf(pr[2 * e + 1]);
      hw[e] = (uint32_t)a0 | ((uint32_t)a1 << 16);
      lw[e] = (uint32_t)f2bf(pr[2 * e] - bf2f(a0)) | ((uint32_t)f2bf(pr[2 * e + 1] - bf2f(a1)) << 16);
    }
    ps += dpp<0xB1>(ps);
    ps += dpp<0x4E>(ps);
    ps += dpp<0x141>(ps);
    l_run = l_run * alpha + ps;
    m_run = mnew;
    // the block's probabilities overwrite its scores (this wave's reads above are complete: LDS operations
    // of one wave run in order)
    *reinterpret_cast<u2*>(pbw + sh * WB + sp) = u2{hw[0], hw[1]};
    *reinterpret_cast<u2*>(pbw + (GRP + sh) * WB + sp) = u2{lw[0], lw[1]};
    if ((lane & 7) == 0) alw[sh] = alpha;
    // this block's V has landed (the loads issued after it are the next block's NKQ + VLD, when that block
    // exists)
    if (i + 1 < wcnt) __builtin_amdgcn_s_waitcnt((0x0F70 | ((NKQ + VLD) & 15)) | (((NKQ + VLD) >> 4) << 14));
    else drain_stores();
    const uint16_t* va = i & 1 ? va1 : va0;
    const u4 ph = lds16(hc < GRP ? pbw + hc * WB + 8 * q4 : zrow + 8 * q4);
    const u4 pl = lds16(hc < GRP ? pbw + (GRP + hc) * WB + 8 * q4 : zrow + 8 * q4);
    const float sc = alw[hc & (GRP - 1)];
    const int nvalid = jc1 - c0 - 8 * q4;  // this lane's rows 8(l/16) + v are valid while v < nvalid
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint32_t ve[4][8];
#pragma unroll
      for (int dq = 0; dq < 4; ++dq) {
        const int dcol = 16 * (4 * half + dq) + hc;
        const uint16_t* vcol = va + (((dcol >> 3) ^ (2 * q4)) << 3) + (dcol & 7);
#pragma unroll
        for (int v = 0; v < 8; ++v) ve[dq][v] = vcol[(8 * q4 + v) * DH];
      }
#pragma unroll
      for (int dq = 0; dq < 4; ++dq) {
        uint32_t wv[4];
#pragma unroll
        for (int v2 = 0; v2 < 4; ++v2) {
          const uint32_t e0 = 2 * v2 < nvalid ? ve[dq][2 * v2] : 0u;
          const uint32_t e1 = 2 * v2 + 1 < nvalid ? ve[dq][2 * v2 + 1] : 0u;
          wv[v2] = e0 | (e1 << 16);
        }
        const u4 av = {wv[0], wv[1], wv[2], wv[3]};
        f4& o = oacc[4 * half + dq];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] *= sc;
        o = mfma(av, ph, o);
        o = mfma(av, pl, o);
      }
    }
    // the block's LDS reads are complete before its areas are reused
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __asm__ volatile("" ::: "memory");
#pragma unroll
    for (int u = 0; u < NKQ; ++u) kc[u] = kx[u];
    if (i + 2 < wcnt) {
      load_k(i + 2, kx);
      load_v(i + 2, i & 1 ? va1 : va0);
    }
  }
  drain_stores();  // no direct V load is left in flight (the areas are reused below)
  mark(a, t, 1);
  // combine the waves: O[h][d] = sum_w exp(m_w - M) O_w[h][d], l = sum_w exp(m_w - M) l_w, M = max_w m_w
  __syncthreads();
  float* const ow = S.xs;                     // [NW][GRP][DH]
  float* const mlw = S.xs + NW * GRP * DH;    // [NW][GRP] maxima, then [NW][GRP] sums
  if (hc < GRP) {
#pragma unroll
    for (int db = 0; db < DH / 16; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) ow[(wave * GRP + hc) * DH + 16 * db + 4 * q4 + e] = oacc[db][e];
  }
  if ((lane & 7) == 0) {
    mlw[wave * GRP + sh] = m_run;
    mlw[NW * GRP + wave * GRP + sh] = l_run;
  }
  __syncthreads();
  static_assert(GRP * DH == 2 * NT, "two outputs per thread");
  float o2[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = tid + k * NT, h = i / DH, dd = i - h * DH;
    float M = -INFINITY;
#pragma unroll
    for (int q = 0; q < NW; ++q) M = fmaxf(M, mlw[q * GRP + h]);
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int q = 0; q < NW; ++q) {
      const float mq = mlw[q * GRP + h];
      const float wq = mq == -INFINITY ? 0.f : expf(mq - M);
      o = fmaf(wq, ow[(q * GRP + h) * DH + dd], o);
      L = fmaf(wq, mlw[NW * GRP + q * GRP + h], L);
    }
    o2[k] = o;
    if (dd == 0) {
      S.hm[h] = M;
      S.hl[h] = L;
    }
  }
  __syncthreads();
  // the new positions len0..len, one at a time (entries b0..b; a decode entry has only its own)
  if (has_new) {
    for (int j = b0; j <= b; ++j) {
      if (b0 != b) {  // a chunk: entry j's key and value (S.kn / S.vn held the previous one)
        __syncthreads();
        stage_new_kv<DH, GRP>(a, j, g, S);
        __syncthreads();
      }
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
      for (int k = 0; k < 2; ++k) {
        const int i = tid + k * NT, h = i / DH, dd = i - h * DH;
        o2[k] = fmaf(S.pnew[h], S.vn[dd], o2[k] * S.hscale[h]);
      }
    }
  }
  if (nsplit > a.apart_stride && tid == 0) raise_error(a, ERRC_SEQLEN, t);  // a list planned for another stride
  float* part = a.apart + ((((int64_t)b * Hkv + g) * a.apart_stride + min(s, a.apart_stride - 1)) * GRP) * (DH + 2);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = tid + k * NT, h = i / DH, dd = i - h * DH;
    pub(part + h * (DH + 2) + dd, o2[k]);
  }
  if (tid < GRP) {
    pub(part + tid * (DH + 2) + DH, S.hm[tid]);
    pub(part + tid * (DH + 2) + DH + 1, S.hl[tid]);
  }
  mark(a, t, 2);
  attn_merge<DH, GRP>(a, w, t, b, g, nsplit, S);
}

template <class C>
__device__ __forceinline__ void task_attn(KA& a, Desc w, int t, Lds& S) {
  if constexpr (C::DH == 128 && C::GRP == 8) attn_split_w<C::DH, C::GRP>(a, w, t, S);
  else attn_split<C::DH, C::GRP>(a, w, t, S);
}

// ------------------------------------------------------------------------------------------ the kernel

// One task.  The argument block is re-derived from an opaque copy of its address on every task so
// that no field is hoisted out of the task loop (that would pin dozens of registers for the kernel's
// whole life).
template <class C>
__device__ __forceinline__ void run_task(KA* a0, Desc w, int t, Lds& S) {
  KA* ap = a0;
  __asm__ volatile("" : "+s"(ap));
  KA& a = *ap;
  const int tid = tidx();
  if (a.ts && tid == 0) {
    a.ts[(int64_t)t * 8 + 0] = wall_clock64();
    a.ts[(int64_t)t * 8 + 1] = 0;
    // hardware id: XCC id in the high word, the wave's HW_ID register in the low word
    a.ts[(int64_t)t * 8 + 3] = ((uint64_t)__builtin_amdgcn_s_getreg((20) | (0 << 6) | (15 << 11)) << 32) |
                               (uint64_t)__builtin_amdgcn_s_getreg((4) | (0 << 6) | (31 << 11));
  }
  switch (w[W_OP]) {
    case OP_EMBED: task_embed(a, w, t, S); break;
    case OP_QKV: task_qkv<C>(a, w, t, S); break;
    case OP_ATTN: task_attn<C>(a, w, t, S); break;
    case OP_UP: task_up<C>(a, w, t, S); break;
    case OP_OPROJ: task_oproj<C>(a, w, t, S); break;
    case OP_DOWN: task_down<C>(a, w, t, S); break;
    case OP_MERGE: task_merge<C::DH, C::GRP>(a, w, t, S); break;
    default:
      if (tid == 0) raise_error(a, ERRC_OPCODE, t);
  }
  if (a.task_done && tid == 0) atomicAdd(&a.task_done[t], 1u);
  if (a.ts && tid == 0) a.ts[(int64_t)t * 8 + 2] = wall_clock64();
}

// The last workgroup out resets the counters for the next step (stream order makes it visible).
__device__ __forceinline__ void exit_step(KA& a, Lds& S) {
  const int tid = tidx();
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(ctr_at(a, a.c_done), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    S.flag = (old == gridDim.x - 1);
    if (S.flag) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  if (S.flag) {
    if (a.ctr_snapshot)
      for (int i = tid; i < a.n_counters; i += NT) a.ctr_snapshot[i] = *ctr_at(a, i);
    for (int i = tid; i < a.n_counters; i += NT) __hip_atomic_store(ctr_at(a, i), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Copy the descriptor at position pos of the task array into LDS: wave 0, lanes 0..7, 16 bytes each,
// straight from global memory to LDS (no registers held while the copy is in flight; it completes under
// vmcnt).
__device__ __forceinline__ void fetch_desc(KA& a, int pos, int32_t* dst) {
  const int lane = tidx() & 63;
  if (tidx() < 64 && lane < DESC_WORDS / 4)
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(a.tasks + (int64_t)pos * DESC_WORDS + 4 * lane),
                                     (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}

template <class C>
__global__ __launch_bounds__(NT, 1) void mk_persistent(KArgs args) {
  KA* const a0 = (KA*)(__builtin_amdgcn_kernarg_segment_ptr());
  (void)args;
  __shared__ Lds S;
  const int tid = tidx();
  KA& a = *a0;
  const int count = a.n_tasks;
  if (tid == 0) {
    S.xb_layer = 0;
    S.route_layer = 0;
  }
  __syncthreads();
  // The list is one pool: every take (an atomic on the ticket counter) returns the next untaken task in
  // list order, so a task goes to whichever workgroup is free first and no take comes back empty before the
  // list's end.  Expert tiles of a batch above one are classified with the list's phase table: a tile found
  // (with its descriptor, once its layer is routed) to belong to an unused slot starts the unused tail of its
  // phase, and the ticket is moved past the phase in one step (an atomic maximum).  No task of that tail is
  // handed out any more; the phase's next task is this workgroup's if the maximum found the ticket at or
  // below it.
  const bool skip_unused = a.ph_on && a.B > 1;
  const int n0 = a.ph_n[0], npl = a.ph_npl;
  int per_layer = 0;
  for (int k = 0; k < npl; ++k) per_layer += a.ph_n[1 + k];
  int nu_l = 0, nu_v = 0;  // used-slot count nu_v of layer nu_l - 1, once seen (it never changes after)
  for (;;) {
    int pos = -1;
    for (;;) {
      if (tid == 0) S.pool_tile = (int)__hip_atomic_fetch_add(ctr_at(a, a.c_ticket), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      int tk = __builtin_amdgcn_readfirstlane(S.pool_tile);
      __syncthreads();  // read by every wave before the next take overwrites it
      while (tk < count) {
        fetch_desc(a, tk, S.desc);
        if (!skip_unused || tk < n0) {
          pos = tk;
          break;
        }
        // phase k of layer l, offset off within it, first task after it pend
        const int l = (tk - n0) / per_layer;
        int off = tk - n0 - l * per_layer, k = 0, pend = n0 + l * per_layer;
        while (k < npl - 1 && off >= a.ph_n[1 + k]) {
          off -= a.ph_n[1 + k];
          pend += a.ph_n[1 + k++];
        }
        const int cnt = a.ph_n[1 + k];
        pend += cnt;
        const bool moe = a.ph_op[k] == OP_UP || a.ph_op[k] == OP_DOWN;
        const bool known = nu_l == l + 1;
        if (moe && !known && tid == 1)
          S.pool_used = (int)__hip_atomic_load(ctr_at(a, a.c_slots_used + l), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        drain_stores();
        __syncthreads();
        int nu = 0;
        if (moe) {
          nu = known ? nu_v : __builtin_amdgcn_readfirstlane(S.pool_used);
          if (nu > 0) {
            nu_l = l + 1;
            nu_v = nu;
          }
        }
        __syncthreads();
        // expert phases list their tiles slot by slot, cnt / n_slots per slot, slots in ascending expert
        // order: once the layer is routed, the tiles of its unused slots are the phase's tail
        if (!moe || nu == 0 || off < nu * (cnt / a.n_slots)) {
          pos = tk;
          break;
        }
        const int target = pend < count ? pend + 1 : count;
        if (tid == 0) S.pool_tile = (int)__hip_atomic_fetch_max(ctr_at(a, a.c_ticket), (uint32_t)target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const int old = __builtin_amdgcn_readfirstlane(S.pool_tile);
        __syncthreads();
        if (pend >= count || old > pend) break;  // the next task was taken by another workgroup: take again
        tk = pend;
      }
      if (pos >= 0 || tk >= count) break;
    }
    if (pos < 0) break;
    drain_stores();  // the descriptor has landed in LDS
    __syncthreads();
    const Desc w{S.desc};
    run_task<C>(a0, w, w[W_SEQ], S);
    drain_stores();
    __syncthreads();  // every wave is done with the descriptor
  }
  lm_phase<C>(*(KA*)a0, S);
  exit_step(a, S);
}

}  // namespace mk
// Compiled shape classes: (d_head, group, d_model bound, d_ffn bound, group*d_head bound), each in two batch
// classes (at most 2 tokens: one MFMA per weight block; at most 8: hi and lo MFMAs for each group of 4).
using CfgFull2 = mk::Cfg<128, 8, 4, 2, 2, 2>;  // d_head 128, group 8, d_model <= 2048, d_ffn <= 1024, group*d_head = 1024
using CfgFull8 = mk::Cfg<128, 8, 4, 2, 2, 8>;
using CfgFull1 = mk::Cfg<128, 8, 4, 2, 2, 1>;  // one token, VALU GEMV tiles
using CfgTiny2 = mk::Cfg<64, 2, 1, 1, 1, 2>;   // d_head 64, group 2, d_model <= 512, d_ffn <= 512, group*d_head = 128
using CfgTiny8 = mk::Cfg<64, 2, 1, 1, 1, 8>;
using CfgTiny1 = mk::Cfg<64, 2, 1, 1, 1, 1>;

extern "C" int mk_kernel_class(int d_head, int group, int d_model, int d_ffn) {
  if (d_head == 128 && group == 8 && d_model <= 64 * 8 * CfgFull2::NVD && d_ffn <= 64 * 8 * CfgFull2::NVF) return 1;
  if (d_head == 64 && group == 2 && d_model <= 64 * 8 * CfgTiny2::NVD && d_ffn <= 64 * 8 * CfgTiny2::NVF) return 2;
  return 0;
}

// mode 0: batch class by batch size; 1: the 8-token class at every batch size; 2: the VALU GEMV class at batch 1
// (larger batches as mode 0).
extern "C" hipError_t mk_launch_persistent(const mk::KArgs* a, int kclass, int grid, int mode, hipStream_t stream) {
  const bool small = a->B <= 2 && mode != 1, valu = a->B == 1 && mode == 2;
  if (kclass == 1 && valu) hipLaunchKernelGGL(mk::mk_persistent<CfgFull1>, dim3(grid), dim3(mk::NT), 0, stream, *a);
  else if (kclass == 1 && small) hipLaunchKernelGGL(mk::mk_persistent<CfgFull2>, dim3(grid), dim3(mk::NT), 0, stream, *a);
  else if (kclass == 1) hipLaunchKernelGGL(mk::mk_persistent<CfgFull8>, dim3(grid), dim3(mk::NT), 0, stream, *a);
  else if (kclass == 2 && valu) hipLaunchKernelGGL(mk::mk_persistent<CfgTiny1>, dim3(grid), dim3(mk::NT), 0, stream, *a);
  else if (kclass == 2 && small) hipLaunchKernelGGL(mk::mk_persistent<CfgTiny2>, dim3(grid), dim3(mk::NT), 0, stream, *a);
  else if (kclass == 2) hipLaunchKernelGGL(mk::mk_persistent<CfgTiny8>, dim3(grid), dim3(mk::NT), 0, stream, *a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}
