/*
 * pa_probe.h: C ABI of libpa_probe.so, the measurement probes the benchmark runs beside the decode
 * step. They are not part of the decode path: they measure the numbers that bound it on the GPU at
 * hand, the rate at which HBM streams reads (sequentially, and in the decode's own pattern of blocks
 * through the tables) and the latency of the dependent loads a decode workgroup makes before its
 * first K/V tile arrives. [P3] "Asynchronous KV Cache Prefetching",
 * sections 2.2 and 3.2, names both: decode attention streams the cache at memory speed, and the
 * block-table lookup in front of each block's load is exposed latency. The fourth, the MFMA rate,
 * is the matching ceiling for the prefill, whose roofline is the matrix peak ([P1] "25. Paged
 * attention and prefix caching", stretch exercise 4: a block of queries makes it a dense contraction).
 *
 * Every pointer is device memory owned by the caller; each call enqueues one kernel on `stream` and
 * returns 0, or -1 for an invalid argument, -3 when the launch fails.
 */
#ifndef PA_PROBE_H_
#define PA_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* pa_probe_stream_t;

/* pa_probe_stream_read: read `bytes` bytes at `src` (16-byte aligned, bytes a multiple of 16) once,
 * with 16-byte loads, `unroll` (1, 2, 4 or 8) loads in flight per thread per step, from `workgroups`
 * workgroups of 256 threads striding over the buffer; each workgroup writes the XOR of every 32-bit
 * word it read to out[workgroup] (uint32, `workgroups` entries), so no load can be dropped. */
int pa_probe_stream_read(const void* src, size_t bytes, int32_t workgroups, int32_t unroll, uint32_t* out,
                         pa_probe_stream_t stream);

/* pa_probe_first_tile: the dependent loads in front of a decode workgroup's first K/V tile, with no
 * attention arithmetic. One workgroup of 4 waves per (sequence i, kv head h), i < num_seqs, h <
 * num_kv_heads; wave w reads seq_lens[i] and its tile's block id block_tables[i * max_blocks + j]
 * with j = w clamped to the sequence's last block, then that block's K and V rows of head h:
 * block_size rows of row_bytes bytes each in pools laid out [num_blocks, num_kv_heads, block_size,
 * row_bytes]. With `dependent` = 1 the table index waits for the length (length -> table -> tile,
 * three loads in a chain); with 0 the index is clamped to the table row instead, so the length and
 * the table entry load together (two loads in a chain, as the decode kernels issue them). Each
 * workgroup writes the XOR of what its waves read to out[i * num_kv_heads + h]. row_bytes a
 * multiple of 16, block_size * row_bytes <= 16384. */
int pa_probe_first_tile(const void* k_pool, const void* v_pool, const int32_t* block_tables, const int32_t* seq_lens,
                        int32_t num_seqs, int32_t num_kv_heads, int32_t max_blocks, int32_t num_blocks,
                        int32_t block_size, int32_t row_bytes, int32_t dependent, uint32_t* out,
                        pa_probe_stream_t stream);

/* pa_probe_paged_read: every K and V block a decode call over these tables reads, and nothing else:
 * for each (sequence i, kv head h), blocks 0 .. ceil(seq_lens[i] / block_size) - 1 of row i of
 * block_tables (ids clamped to the pool), each block_size rows of row_bytes bytes of head h in pools
 * laid out [num_blocks, num_kv_heads, block_size, row_bytes]; block_size * row_bytes must be 1, 2, 4
 * or 8 KiB. A workgroup of 4 waves takes 4 * blocks_per_wave consecutive blocks of one (sequence,
 * kv head), blocks_per_wave per wave, with `unroll` (1, 2 or 4) blocks' loads in flight per wave per
 * step; `nontemporal` = 1 issues them as nontemporal loads. Each workgroup writes the XOR of what it
 * read to out[] (one uint32 per workgroup: num_seqs * ceil(max_blocks / (4 * blocks_per_wave)) *
 * num_kv_heads entries). It is the decode's byte stream without the attention, so its rate is the
 * ceiling of that access pattern: 4 KiB pieces at the places the tables name, not one sequential
 * sweep. */
int pa_probe_paged_read(const void* k_pool, const void* v_pool, const int32_t* block_tables, const int32_t* seq_lens,
                        int32_t num_seqs, int32_t num_kv_heads, int32_t max_blocks, int32_t num_blocks,
                        int32_t block_size, int32_t row_bytes, int32_t blocks_per_wave, int32_t unroll,
                        int32_t nontemporal, uint32_t* out, pa_probe_stream_t stream);

/* pa_probe_mfma: the bf16 matrix rate, with no memory traffic. `workgroups` workgroups of 256 threads
 * (4 waves); each wave runs `iters` rounds of 8 independent v_mfma_f32_16x16x32_bf16 (16384 flops
 * each) into 8 accumulators, each MFMA followed by `valu_per_mfma` (0, 2 or 4) independent fp32 FMAs
 * on other registers, in that order. With 256 * w workgroups every SIMD holds w waves. Each thread
 * writes one float of what it computed to out[workgroup * 256 + thread] (workgroups * 256 floats), so
 * no instruction can be dropped. Flops per call: workgroups * 4 * iters * 8 * 16384. */
int pa_probe_mfma(int32_t workgroups, int32_t iters, int32_t valu_per_mfma, float* out, pa_probe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H_ */
