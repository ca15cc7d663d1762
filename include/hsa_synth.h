/*
 * hsa_synth.h - seeded synthetic inputs on the GPU, and the benchmark's read roof
 * (test and benchmark harness; not part of the cache). The same counter generator as the Python module
 * `synth`, so either side can regenerate any token at random access:
 *
 *   ctr = stream << 56 | key << 32 | (i >> 1)
 *   h   = mix64(seed + (ctr + 1) * 0x9E3779B97F4A7C15)     (SplitMix64 output
 *         function; Steele, Lea and Flood, OOPSLA 2014)
 *   w   = low 32 bits of h for even i, high 32 bits for odd i
 *   z   = (2 * (byte0(w) + byte1(w) + byte2(w)) - 765) / 256
 *
 * Element e of the row of token position p has counter index i = p * row_len + e.
 */
#ifndef HSA_SYNTH_H
#define HSA_SYNTH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Fill out[n_rows][row_len] (row_len even): row r uses key keys[r] (or `key` when
 * keys is NULL) and position pos[r] (or pos0 + r when pos is NULL). as_bf16 != 0
 * stores z rounded to bf16 (nearest even) as uint16 bits, else float32 z.
 * keys, pos, out: device pointers. Returns 0, or -1 on a bad argument, -5 on a HIP
 * error. */
int32_t hsa_synth_rows(uint64_t seed, uint32_t stream_id, const uint32_t* keys, uint32_t key,
                       const int64_t* pos, int64_t pos0, int64_t n_rows, int32_t row_len,
                       int32_t as_bf16, void* out, void* stream);

/* Benchmark roof: read `bytes` (a multiple of 16) at device pointer buf with a
 * streaming read kernel of `blocks` workgroups of 256 threads, each reading one
 * contiguous chunk and folding it (out: device, `blocks` uint32, written only for a
 * marker fold value). Enqueued on `stream`. Returns 0, -1 on a bad argument, -5 on
 * a HIP error. */
int32_t hsa_roof_read(const void* buf, int64_t bytes, uint32_t* out, int32_t blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HSA_SYNTH_H */
