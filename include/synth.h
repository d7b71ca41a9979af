/* Seeded synthetic inputs: C interface.
 *
 * The generator is shared by the CPU oracle's tests and by the GPU harness;
 * it holds none of the decode method's arithmetic.  Host functions live in
 * libsynth_host.so (gcc), device fills in libsynth_dev.so (hipcc).  Every value
 * is a pure function of (seed, stream, logical index), see synth/synth_core.h.
 *
 * Error convention: 0 on success, negative on invalid arguments.  No function
 * allocates memory that it hands back; all buffers belong to the caller.
 */
#ifndef SYNTH_H
#define SYNTH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Tables for N(0, sigma) rounded to BF16.  thr: caller buffer of at least
 * 0x7F81 uint64; guide: caller buffer of 65536 uint16.  *n_out receives the
 * number of threshold entries used.  Returns 0, or -1 (bad argument), -2. */
int synth_table_build(double sigma, uint64_t* thr, uint16_t* guide, int32_t* n_out);

/* dst[i] = BF16 sample for element (index0 + i) of (seed, stream); host memory. */
void synth_fill_bf16(uint16_t* dst, int64_t n, uint64_t seed, uint64_t stream, uint64_t index0, const uint64_t* thr,
                     const uint16_t* guide);

/* Fill positions [pos0, pos1) of sequence seq_id, layers [layer0, layer0 + n_layers_buf), into a paged
 * host KV buffer laid out [n_layers_buf][n_pages][2 (K,V)][n_kv_heads][page_size][d_head] BF16.
 * page_table (host, n_table entries) maps logical page -> physical page.
 * Returns 0, -1 (bad range), -2 (page index out of [0, n_pages)). */
int synth_fill_kv_paged(uint16_t* kv, int n_layers_buf, int layer0, int64_t n_pages, int n_kv_heads, int d_head, int page_size,
                        const int32_t* page_table, int64_t n_table, int seq_id, int64_t pos0, int64_t pos1, uint64_t seed,
                        const uint64_t* thr, const uint16_t* guide);

/* The plain SplitMix64 sequence from `state` (its first n outputs); the stream generator's core. */
void synth_splitmix64(uint64_t state, int64_t n, uint64_t* out);

/* Raw 64-bit draws of (seed, stream), elements index0 .. index0+n-1. */
void synth_u64_fill(uint64_t seed, uint64_t stream, uint64_t index0, int64_t n, uint64_t* out);

/* Start token of sequence `seq`: uniform over [0, vocab). */
int32_t synth_token(uint64_t seed, int seq, int vocab);

/* n integers clamp(floor(exp(U(ln lo, ln hi))), lo, hi). */
void synth_loguniform_ints(uint64_t seed, uint64_t stream, int n, int64_t lo, int64_t hi, int64_t* out);

/* Uniform random permutation of 0..n-1 (Fisher-Yates). */
void synth_permutation(uint64_t seed, uint64_t stream, int n, int32_t* out);

/* out[perm[r-1]] = (float)(-scale * ln r), r = 1..n_experts, perm = synth_permutation(seed, 0). */
void synth_skew_bias(uint64_t seed, int n_experts, double scale, float* out);

/* ---- device fills (libsynth_dev.so); pointers are device memory, `stream` a hipStream_t ---- */

/* Same values as synth_fill_bf16, written to device memory. thr/guide: device copies of the tables. */
int synth_dev_fill_bf16(void* dst, int64_t n, uint64_t seed, uint64_t stream, uint64_t index0, const uint64_t* thr,
                        const uint16_t* guide, void* hip_stream);

/* Same values as synth_fill_kv_paged into a device KV buffer; page_table is device memory.
 * Pages outside [0, n_pages) are skipped and counted in *bad_dev (device uint32, nullable). */
int synth_dev_fill_kv_paged(void* kv, int n_layers_buf, int layer0, int64_t n_pages, int n_kv_heads, int d_head, int page_size,
                            const int32_t* page_table, int seq_id, int64_t pos0, int64_t pos1, uint64_t seed, const uint64_t* thr,
                            const uint16_t* guide, uint32_t* bad_dev, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif
