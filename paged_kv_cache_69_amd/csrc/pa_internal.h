// Internal declarations shared by the HIP sources of libpa.so (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

constexpr float kLog2eHost = 1.4426950408889634f;  // log2(e): scores are kept in base-2 units

// Everything a decode launch needs, in one kernel argument.
struct DecodeParams {
  const void* q;             // [B, T, Hq, D]
  const void* k_pool;        // [N, Hkv, b, D]
  const void* v_pool;        // [N, Hkv, b, D]
  const int32_t* block_tables;  // [B, MB]
  const int32_t* seq_lens;   // [B]
  void* out;                 // [B, T, Hq, D] (single-pass launches)
  float* part_ml;            // [B*T*Hq, parts, 2]: (m, l) per partition (partitioned launches)
  float* part_acc;           // [B*T*Hq, parts, D]: unnormalised accumulator per partition
  const float* scales;       // 8-bit pools: [N, Hkv, 2] (K scale, V scale) of each (block, kv head); else null
  const void* k_new;         // fused append: [B, T, Hkv, D] new rows for positions L - T .. L - 1
  const void* v_new;
  float qk_scale_log2;       // scale * log2(e): scores are kept in base-2 exponent units
  int32_t B, T, Hq, Hkv, G, D, MB, block_size;
  int32_t num_blocks;        // N: physical blocks in each pool
  int32_t rows;              // T * G query rows that share one kv head
  int32_t row_groups;        // workgroups along the rows, per (sequence, kv head, partition)
  int32_t parts;             // partitions per sequence in the grid (1 for single pass)
  int32_t part_tokens;       // positions per partition (single pass: >= every length)
  int32_t out_dtype;         // pa_dtype of out
  int32_t partial;           // 1: write (m, l, acc) partials; 0: write normalised out
  int32_t kv_int8;           // 1: the pools hold 8-bit codes scaled by `scales`
  int32_t kv_fp8;            // with kv_int8: the codes are E4M3 values (else int8 integers)
  int32_t append;            // 1: also store k_new / v_new into the pools (MFMA kernel, bf16 pools)
  int32_t prefix_tokens;     // cascade: positions every sequence shares (0: none)
  int32_t prefix_parts;      // cascade: workspace slots 0 .. prefix_parts-1 hold the prefix's partials
                             // (one per group of mfma_waves() chunks)
  int32_t prefix_part_tokens;  // cascade: positions of the prefix per chunk (one wave's share)
  int32_t lpt;               // single pass on the MFMA kernel: sequences dealt longest first
  int32_t wave_parts;        // split launches on the MFMA kernel: consecutive partitions per wave (<= 1: one)
  int32_t* slot_counts;      // balanced ranges: [B] slots each sequence's rows use (the merge reads them);
                             // null otherwise (one slot per partition)
};

hipError_t launch_write_kv(const pa_dims& d, const void* k_new, const void* v_new, void* k_pool,
                           void* v_pool, const int32_t* block_tables, const int32_t* positions,
                           hipStream_t stream);

// 8-bit pools (int8 or, with fp8, E4M3 codes): append with per-(block, kv head) scales.
hipError_t launch_write_kv_int8(const pa_dims& d, const void* k_new, const void* v_new, int8_t* k_pool,
                                int8_t* v_pool, float* scales, const int32_t* block_tables,
                                const int32_t* positions, bool fp8, hipStream_t stream);

// Rows handled by one VALU workgroup for `rows` query rows per kv head.
int valu_rows_per_group(int rows);
bool valu_supported(const pa_dims& d);
hipError_t launch_decode_valu(const DecodeParams& p, int kv_dtype, hipStream_t stream);

// PA_CHECK=1: the preconditions of pa.h checked on host copies (PA_OK when unset or capturing).
// max_seq_len > 0 also bounds every length.
int debug_check(const pa_dims* dims, const int32_t* block_tables, const int32_t* seq_lens,
                const int32_t* positions, int32_t max_seq_len, hipStream_t stream);

// PA_CHECK=1, cascade: every sequence holds at least prefix_tokens + T positions and its first
// prefix_tokens / b table entries are sequence 0's.
int debug_check_prefix(const pa_dims* dims, const int32_t* block_tables, const int32_t* seq_lens,
                       int32_t prefix_tokens, hipStream_t stream);

bool mfma_supported(const pa_dims& d);       // bf16 pools
bool mfma_int8_supported(const pa_dims& d);  // 8-bit pools (int8 or E4M3)
hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t stream);
// Cascade: in one launch, the shared prefix's partitions for all sequences' rows at once (slots
// 0 .. prefix_parts-1) and the sequences' own partitions.
hipError_t launch_cascade(const DecodeParams& p, hipStream_t stream);
int mfma_waves();  // waves per MFMA workgroup (prefix chunks merged into one cascade slot)
int mfma_lpt_max_seqs();  // largest batch the single pass can order longest first

hipError_t launch_merge_partials(const DecodeParams& p, hipStream_t stream);

// Split context with balanced wave ranges (pa_decode_balanced.hip): bf16 or 8-bit pools, head_dim 128,
// b in {16, 32}, T * G <= 16, up to 1024 sequences whose q rows of one kv head fit 48 KiB of LDS.
bool balanced_supported(const pa_dims& d);
hipError_t launch_balanced(const DecodeParams& p, hipStream_t stream);

// Copy-on-write block copies: pairs [n, 2] (source, destination) on the device; for 8-bit pools the
// blocks' [Hkv, 2] scales too (scales non-null).
hipError_t launch_copy_blocks(const pa_dims& d, void* k_pool, void* v_pool, float* scales, const int32_t* pairs,
                              int32_t num_pairs, hipStream_t stream);
// PA_CHECK=1: every pair in [0, num_blocks), destinations distinct and never a source.
int debug_check_copies(const pa_dims* dims, const int32_t* pairs, int32_t num_pairs, hipStream_t stream);

// Paged prefill (packed chunks, q_start offsets): bf16 q/KV, head_dim 128, G <= 128, b in {4, 8, 16, 32}.
bool prefill_supported(const pa_dims& d);
hipError_t launch_prefill(const pa_dims& d, const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_tables, const int32_t* seq_lens, const int32_t* q_start, float scale,
                          void* out, hipStream_t stream);
hipError_t launch_write_kv_varlen(const pa_dims& d, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                  const int32_t* block_tables, const int32_t* seq_lens, const int32_t* q_start,
                                  hipStream_t stream);
// PA_CHECK=1, prefill: q_start starts at 0 and never decreases, every chunk fits its sequence and
// the q_tokens bound, lengths fit the table, used entries lie in the pool, and the chunks' slots
// are distinct.
int debug_check_prefill(const pa_dims* dims, const int32_t* block_tables, const int32_t* seq_lens,
                        const int32_t* q_start, hipStream_t stream);

}  // namespace pa
