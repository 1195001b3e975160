/*
 * pa.h: C ABI of libpa.so, a paged-KV-cache decode step for AMD Instinct
 * MI355X (gfx950).
 *
 * The KV cache of one attention layer is two pools, K and V, each shaped
 * [num_blocks, num_kv_heads, block_size, head_dim] and row-major (head_dim is
 * fastest). A sequence's logical position p lives in physical block
 * block_tables[seq][p / block_size] at offset p % block_size ([P1] "25. Paged
 * attention and prefix caching", section "Paging"; [P5] "Chapter 7 Paged KV
 * Cache and Memory Management", sections 3.1-3.2).
 *
 * Conventions that apply to every entry point:
 *  - Every data pointer is device memory owned by the caller: a tensor that is
 *    contiguous in the stated layout, 16-byte aligned for q, k_new, v_new, the
 *    pools and out.
 *  - The library allocates nothing and keeps no state between calls. It is
 *    re-entrant. All work is enqueued on `stream` (0 is the null stream), and
 *    nothing synchronises with the host.
 *  - Return value: PA_OK, or a negative pa_status. On error nothing is
 *    launched, except for PA_ERR_LAUNCH, which reports a failed launch.
 *  - Preconditions the library does not check (breaking them is undefined
 *    behaviour):
 *      * 1 <= seq_lens[i] <= max_blocks_per_seq * block_size, and
 *        seq_lens[i] >= q_tokens;
 *      * block_tables[i][j] is in [0, num_blocks) for j < ceil(seq_lens[i] /
 *        block_size). Entries past that point are never read, so any padding
 *        value is allowed;
 *      * the slots written by pa_write_kv are distinct, and no other sequence
 *        reads them (copy-on-write is the caller's job: [P1] section
 *        "Sharing blocks: forks and copy-on-write").
 *    With the environment variable PA_CHECK=1, every entry point first copies
 *    block_tables, seq_lens and positions to the host (synchronising the
 *    stream), checks them with pa_check_inputs_host, and returns
 *    PA_ERR_INVALID_ARG without launching anything when a check fails. This
 *    is a debugging aid: it is skipped while the stream is being captured
 *    into a graph.
 *
 * Sources: [P1] "25. Paged attention and prefix caching"
 *          (inference.shantanugoel.com); [P2] "Модуль 09: PagedAttention:
 *          пейджинг KV-кэша" (hermes-agent.ru); [P4] "PagedAttention and the
 *          KV Cache" (kanthi.in); [P5] "Chapter 7 Paged KV Cache and Memory
 *          Management" (zero-to-sglang).
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's hipStream_t; declared here so the header needs no HIP include. */
typedef struct ihipStream_t* pa_stream_t;

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1, /* null pointer, bad dimension, bad dtype code, workspace too small */
  PA_ERR_UNSUPPORTED = -2, /* valid arguments, but no kernel for this (dtype, head_dim, block, rows) */
  PA_ERR_LAUNCH = -3,      /* the HIP runtime reported an error for the launch */
  PA_ERR_NO_BLOCKS = -4,   /* block manager: the pool has too few free blocks (nothing changed) */
  PA_ERR_TOO_LARGE = -5    /* pa_decode_partitioned_noalloc: partials beyond its fixed device scratch */
} pa_status;

/* PA_INT8 and PA_FP8_E4M3 are pool dtypes only: 8-bit codes (int8
 * integers, or OCP E4M3 floats) with one fp32 scale per (block, kv head),
 * used by the *_int8 and *_fp8 entry points. */
typedef enum { PA_F32 = 0, PA_BF16 = 1, PA_INT8 = 2, PA_FP8_E4M3 = 3 } pa_dtype;

/* Kernel choice for the attention entry points. PA_VARIANT_AUTO picks the
 * fastest kernel this library has for the shape. The other values force one
 * kernel family and return PA_ERR_UNSUPPORTED if it cannot serve the shape. */
typedef enum {
  PA_VARIANT_AUTO = 0,
  PA_VARIANT_VALU = 1, /* vector-ALU kernel: up to 8 query rows per kv head in one workgroup */
  PA_VARIANT_MFMA = 2  /* matrix-core kernel: bf16, 16 or 32 query rows per kv head */
} pa_variant;

/* Split-context schedules (pa_dims.split_schedule). Every schedule gives the same partials, each with
 * its own reference maximum, so the merged output agrees to rounding; ONE_PER_WAVE and TWO_PER_WAVE
 * give the same bits.
 *   PA_SPLIT_ONE_PER_WAVE: one wave per partition.
 *   PA_SPLIT_TWO_PER_WAVE: a wave walks two consecutive partitions of one sequence (bf16 pools,
 *     T * G <= 16; elsewhere one per wave).
 *   PA_SPLIT_BALANCED: for each kv head the tiles of all sequences form one list, cut into equal
 *     ranges (each at least one partition long), one per pair of waves, one pair per SIMD of the
 *     GPU; the two waves of a pair share their range from its two ends, so they end together
 *     whatever their relative speed. Each wave leaves one partial per sequence it touched, which the
 *     merge adds like any others (so the last bits of the output may change from call to call).
 *     Needs bf16 or 8-bit pools, D = 128, b in {16, 32}, T * G <= 16,
 *     B <= 1024 and B * T * G * 256 <= 48 KiB (PA_ERR_UNSUPPORTED otherwise); the workspace then
 *     holds 2P + 2 slots per row and B int32 slot counts. */
typedef enum {
  PA_SPLIT_AUTO = 0,
  PA_SPLIT_ONE_PER_WAVE = 1,
  PA_SPLIT_TWO_PER_WAVE = 2,
  PA_SPLIT_BALANCED = 3
} pa_split_schedule;

/* Problem dimensions.
 * B = num_seqs; T = q_tokens, the new tokens per sequence, which are causal
 * among themselves; Hq = num_q_heads; Hkv = num_kv_heads; G = Hq / Hkv is the
 * GQA group (query head h reads kv head h / G: [P1] section "Attention that
 * reads through the table"); D = head_dim; b = block_size; N = num_blocks;
 * MB = max_blocks_per_seq, the width of block_tables. */
typedef struct {
  int32_t num_seqs;
  int32_t q_tokens;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t q_dtype;   /* pa_dtype of q and of k_new/v_new */
  int32_t kv_dtype;  /* pa_dtype of the pools; must equal q_dtype */
  int32_t out_dtype; /* pa_dtype of out */
  int32_t variant;   /* pa_variant */
  int32_t split_schedule; /* pa_split_schedule: how split calls on the matrix-core kernels share
                             out the partitions. PA_SPLIT_AUTO (0) lets the library choose
                             (pa_decode_partitioned_schedule); the others force a schedule and are
                             ignored by the vector-ALU kernel. Any other value: PA_ERR_INVALID_ARG. */
} pa_dims;

/* pa_write_kv: the KV-append scatter.
 * For every sequence i < B and new token t < T, with pos = positions[i*T + t]:
 *   k_pool[block_tables[i*MB + pos / b]][h][pos % b][:] = k_new[i][t][h][:]
 *   v_pool[...same slot...]                               = v_new[i][t][h][:]
 * for every kv head h. This is the scatter half of `update` in [P1] section
 * "The paged cache"; [P2] `Sequence.append`; and the step of the decode-step
 * sketch in [P4] section "Block table and allocator" that stores the new
 * token's K and V in the last block.
 *   k_new, v_new : [B, T, Hkv, D], dtype q_dtype (== kv_dtype)
 *   k_pool, v_pool : [N, Hkv, b, D], written in place, bit-exact copies
 *   block_tables : int32 [B, MB];  positions : int32 [B, T], each in
 *                  [0, MB * b)
 * Requires D * sizeof(dtype) to be a multiple of 16 bytes. Each copied row
 * is bit-for-bit identical to its source. */
int pa_write_kv(const pa_dims* dims, const void* k_new, const void* v_new, void* k_pool,
                void* v_pool, const int32_t* block_tables, const int32_t* positions,
                pa_stream_t stream);

/* pa_decode: single-pass paged decode attention.
 * For every sequence i, query token t < T and query head h, with
 * L = seq_lens[i], kv head g = h / G and visible positions
 * p = 0 .. L - T + t (the T new tokens are the last T positions; causal mask
 * from [P5] section 4.1):
 *   s_p = scale * dot(q[i][t][h][:], K[p])     K[p] = k_pool[table(i,p)][g][p % b][:]
 *   out[i][t][h][:] = sum_p softmax(s)_p * V[p]
 * This is [P1] section "Attention that reads through the table", [P2]
 * section 5 and [P5] sections 4.1-4.2. It is exact softmax attention, computed
 * with a blockwise online softmax and an fp32 running max, sum and
 * accumulator.
 *   q : [B, T, Hq, D], q_dtype;  out : [B, T, Hq, D], out_dtype
 *   k_pool, v_pool : [N, Hkv, b, D], kv_dtype (read only)
 *   block_tables : int32 [B, MB];  seq_lens : int32 [B]
 * One workgroup runs per (sequence, kv head), and loops over the whole
 * sequence. On the MFMA kernel, batches of 128 to 512 sequences (more
 * workgroups than the GPU holds at once) are dealt longest first: the j-th
 * workgroup of each kv head takes the sequence of length rank j, so the last
 * workgroups to start are the shortest. Use pa_decode_partitioned for long
 * contexts.
 * Supported: kv dtype (= q dtype) PA_BF16 or PA_F32, D in {64, 128}, b in
 * {4, 8, 16, 32}, fp32 or bf16 out. The VALU kernel serves all of these and
 * any T * G: groups of up to 8 query rows share one workgroup. The MFMA
 * kernel serves PA_BF16 with D = 128 and T * G <= 32 (query rows padded to
 * 16 or 32), and PA_VARIANT_AUTO picks it there. */
int pa_decode(const pa_dims* dims, const void* q, const void* k_pool, const void* v_pool,
              const int32_t* block_tables, const int32_t* seq_lens, float scale, void* out,
              pa_stream_t stream);

/* Bytes of device workspace pa_decode_partitioned needs for these dims:
 * B * T * Hq * S * (D + 2) * 4 plus alignment, with S = 2P + 2 slots per row
 * and B * 4 more bytes when the call runs balanced ranges (the schedule
 * pa_decode_partitioned_schedule returns for these arguments), else S = P,
 * and P = ceil(max_seq_len / partition_tokens). Returns 0 for invalid
 * arguments. */
size_t pa_decode_partitioned_workspace_bytes(const pa_dims* dims, int32_t max_seq_len,
                                             int32_t partition_tokens);

/* pa_decode_partitioned: split-context decode (flash-decoding) with a merge pass.
 * Each sequence's positions are cut into partitions of partition_tokens.
 * Workgroup (i, kv head, k) writes the fp32 partial (m_k, l_k, acc_k[D]) of
 * partition k for its query rows. A second kernel on the same stream merges
 * them exactly ([P5] section 4.2, block merging in three steps):
 *   M = max_k m_k;  l = sum_k l_k e^(m_k - M);
 *   out = sum_k acc_k e^(m_k - M) / l.
 * Partitions with no visible position (l_k = 0) are skipped. Partitioning
 * long sequences across programs with a final merge is the production
 * technique named in [P1] section "Attention that reads through the table";
 * [P2] section 5 also names it.
 *   max_seq_len : host-known upper bound of seq_lens (the host keeps a copy of
 *                 the tables: [P5] section 3.1). It sizes the grid. Every
 *                 seq_lens[i] must be <= max_seq_len.
 *   partition_tokens : > 0, and a multiple of 16 and of b
 *   workspace : device scratch of >= pa_decode_partitioned_workspace_bytes()
 *               bytes, 256-byte aligned, owned by the caller; its contents on
 *               entry are irrelevant.
 * Other arguments and the supported shapes are as for pa_decode. Two calls
 * that share one workspace must be ordered by the caller, for example by
 * using the same stream: calls that overlap on one workspace race. On the
 * matrix-core kernels the partitions are shared out to waves by a schedule
 * (pa_dims.split_schedule, pa_decode_partitioned_schedule). */
int pa_decode_partitioned(const pa_dims* dims, const void* q, const void* k_pool,
                          const void* v_pool, const int32_t* block_tables,
                          const int32_t* seq_lens, float scale, void* out, int32_t max_seq_len,
                          int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                          pa_stream_t stream);

/* pa_decode_partitioned_schedule: the pa_split_schedule (1, 2 or 3) a split
 * call with these arguments runs on the matrix-core kernels. With
 * PA_SPLIT_AUTO, when one partition per wave would need more than the 2048
 * waves the GPU holds at once (B * Hkv * ceil(max_seq_len /
 * partition_tokens) > 2048), it is BALANCED where the dims allow it, else
 * TWO_PER_WAVE for bf16 pools with T * G <= 16; ONE_PER_WAVE otherwise.
 * Balanced calls may differ from one call to the next in the last bits of
 * the output (each pair of waves splits its range where their timing puts
 * the meeting point); ONE_PER_WAVE and TWO_PER_WAVE give the same bits on
 * every call. A forced schedule is returned as the call would run it
 * (PA_ERR_UNSUPPORTED for a balanced schedule the dims do not allow).
 * Host-only; PA_ERR_INVALID_ARG for invalid dims or sizes. */
int pa_decode_partitioned_schedule(const pa_dims* dims, int32_t max_seq_len, int32_t partition_tokens);

/* pa_decode_partitioned_noalloc: pa_decode_partitioned with no workspace
 * argument and no allocation of any kind, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The partials go to a fixed device
 * scratch array of PA_NOALLOC_SCRATCH_BYTES inside the library: each GPU the
 * call runs on holds one such array from its first use until the process
 * ends. The call runs on the current device (the one `stream` belongs to);
 * its first call there looks up that device's array once.
 *   Result, arguments and supported shapes: those of pa_decode_partitioned
 *   (same kernels, so the output is the same bits).
 *   Limit: pa_decode_partitioned_workspace_bytes(dims, max_seq_len,
 *   partition_tokens) must not exceed PA_NOALLOC_SCRATCH_BYTES, else
 *   PA_ERR_TOO_LARGE and nothing is launched.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (other streams, other threads) race; order them, for example on one
 * stream. The array's contents on entry are irrelevant (each call overwrites
 * what it reads), and nothing in it needs clearing. */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int pa_decode_partitioned_noalloc(const pa_dims* dims, const void* q, const void* k_pool,
                                  const void* v_pool, const int32_t* block_tables,
                                  const int32_t* seq_lens, float scale, void* out,
                                  int32_t max_seq_len, int32_t partition_tokens,
                                  pa_stream_t stream);

/* pa_write_kv_decode: one decode step in one launch: pa_write_kv of the T new
 * tokens at each sequence's last T positions (positions[i][t] = seq_lens[i] -
 * T + t, so no positions argument), then pa_decode. The results (pools and
 * out) are bit for bit those of the two separate calls. The workgroup of each
 * (sequence, kv head) stores that head's new rows itself and, in the tile that
 * holds them, reads them from k_new / v_new rather than from the pool, so no
 * part of the launch waits for its own stores ([P4] section "Block table and
 * allocator": a decode step appends the new token's K and V, then attends).
 *   k_new, v_new : [B, T, Hkv, D], q_dtype;  k_pool, v_pool : written in place
 * Other arguments as pa_decode. Supported: the MFMA shapes of pa_decode
 * (PA_BF16, D = 128, b in {4, 8, 16, 32}, T * G <= 32); otherwise
 * PA_ERR_UNSUPPORTED (use pa_write_kv and pa_decode). The new rows' slots
 * must not be read by another sequence in the same call. */
int pa_write_kv_decode(const pa_dims* dims, const void* q, const void* k_new, const void* v_new,
                       void* k_pool, void* v_pool, const int32_t* block_tables,
                       const int32_t* seq_lens, float scale, void* out, pa_stream_t stream);

/* pa_write_kv_decode_partitioned: the same fused step on the split-context
 * path (pa_decode_partitioned's workspace, rules and merge pass). */
int pa_write_kv_decode_partitioned(const pa_dims* dims, const void* q, const void* k_new,
                                   const void* v_new, void* k_pool, void* v_pool,
                                   const int32_t* block_tables, const int32_t* seq_lens,
                                   float scale, void* out, int32_t max_seq_len,
                                   int32_t partition_tokens, void* workspace,
                                   size_t workspace_bytes, pa_stream_t stream);

/* pa_decode_cascade: decode over sequences that all share their first
 * prefix_tokens positions (the same physical blocks: a forked or
 * prefix-cached prompt, [P1] section "Sharing blocks: forks and
 * copy-on-write"; [P2] section 4). The result is pa_decode's.
 * The shared prefix is attended once per kv head for the query rows of all
 * sequences together, instead of once per sequence: it is cut into chunks
 * (the library picks their size from the dims, a multiple of 16 and of b,
 * so that the prefix work fills the GPU), each processed for all B * T * G
 * rows of a kv head, 32 rows per wave; the four waves of a workgroup merge
 * their chunks into one partial. Each sequence's own positions (prefix_tokens .. L - 1)
 * run in partitions of partition_tokens as in pa_decode_partitioned, and one
 * merge pass combines the prefix's and the sequence's partials exactly
 * ([P5] section 4.2). Two launches on `stream`: the prefix's chunks and the
 * sequences' own partitions run side by side in the first, the merge is
 * the second.
 *   prefix_tokens : a multiple of 16 and of b (0: no shared prefix, same as
 *                   pa_decode_partitioned)
 *   max_seq_len   : host-known bound of seq_lens, >= prefix_tokens
 *   partition_tokens : a multiple of 16 and of b
 *   workspace     : >= pa_decode_cascade_workspace_bytes() bytes, 256-byte
 *                   aligned; contents on entry irrelevant
 * Preconditions (checked under PA_CHECK=1): block_tables[i][j] ==
 * block_tables[0][j] for j < prefix_tokens / b, and seq_lens[i] >=
 * prefix_tokens + q_tokens (the new tokens lie past the prefix). Supported:
 * the MFMA shapes of pa_decode (PA_BF16, D = 128, T * G <= 32). */
size_t pa_decode_cascade_workspace_bytes(const pa_dims* dims, int32_t prefix_tokens,
                                         int32_t max_seq_len, int32_t partition_tokens);
int pa_decode_cascade(const pa_dims* dims, const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_tables, const int32_t* seq_lens, float scale, void* out,
                      int32_t prefix_tokens, int32_t max_seq_len, int32_t partition_tokens,
                      void* workspace, size_t workspace_bytes, pa_stream_t stream);

/* pa_write_kv_decode_cascade: pa_write_kv of the T new tokens at each
 * sequence's last T positions (seq_lens[i] - T .. seq_lens[i] - 1), then
 * pa_decode_cascade, in the same two launches as pa_decode_cascade: the
 * suffix items that hold the new positions store them and read them from
 * k_new / v_new rather than from the pool ([P4] section "Block table and
 * allocator"), so the results (pools and out) are bit for bit those of
 * pa_write_kv followed by pa_decode_cascade.
 *   k_new, v_new : [B, T, Hkv, D], q_dtype, 16-byte aligned
 * Other arguments, shapes and preconditions as pa_decode_cascade; the new
 * positions must lie past the shared prefix (seq_lens[i] - T >=
 * prefix_tokens, checked under PA_CHECK=1), in each sequence's private
 * blocks. Null k_new or v_new: PA_ERR_INVALID_ARG. */
int pa_write_kv_decode_cascade(const pa_dims* dims, const void* q, const void* k_new, const void* v_new,
                               void* k_pool, void* v_pool, const int32_t* block_tables,
                               const int32_t* seq_lens, float scale, void* out, int32_t prefix_tokens,
                               int32_t max_seq_len, int32_t partition_tokens, void* workspace,
                               size_t workspace_bytes, pa_stream_t stream);

/* ---- int8 KV cache ([P2] "Модуль 09: PagedAttention: пейджинг KV-кэша",
 * section 6: block-wise KV quantisation).
 *
 * Pools hold int8 codes, [N, Hkv, b, D] like the float pools, plus one fp32
 * scale per (block, kv head) for K and one for V, interleaved:
 * scales [N, Hkv, 2] holds (K scale, V scale) of each (block, kv head), so
 * a tile's two scales share one 8-byte word. A stored value is code * scale. For each (block, head) the scale is the largest magnitude of
 * that head's values in the block divided by 127, and each code is the value
 * divided by the scale, rounded half to even and clipped to [-127, 127], the
 * division done in fp32. The per-element error is then at most the range
 * over 254. dims->kv_dtype must be PA_INT8; q_dtype (and the dtype of new
 * rows) is PA_BF16 or PA_F32. Each call halves the K/V bytes a bf16 pool
 * would move.
 */

/* pa_write_kv_int8: append the T new tokens of every sequence into int8 pools.
 * positions[i][0..T) must be consecutive (a decode step's newest positions).
 * For each block that receives new rows of sequence i and kv head h, with m =
 * the offset of its first new row:
 *   - m = 0: the block holds no valid rows; its scale becomes
 *     max|new rows| / 127 and the new rows are quantised with it;
 *   - m > 0: the scale becomes max(old scale, max|new rows| / 127). If it
 *     grew, the m old codes are re-quantised: code' = clip(round(code *
 *     old_scale / new_scale)), each product and quotient in fp32. The new rows
 *     are then quantised with the new scale.
 * A scale of 0 (all-zero values) gives codes 0. A block written here must not
 * be read or written by another sequence in the same call.
 *   k_new, v_new : [B, T, Hkv, D], q_dtype;  k_pool, v_pool : int8 [N, Hkv, b, D]
 *   scales : fp32 [N, Hkv, 2] (read and written)
 *   block_tables : int32 [B, MB];  positions : int32 [B, T]
 * Supported: D a multiple of 16. */
int pa_write_kv_int8(const pa_dims* dims, const void* k_new, const void* v_new, int8_t* k_pool,
                     int8_t* v_pool, float* scales, const int32_t* block_tables,
                     const int32_t* positions, pa_stream_t stream);

/* pa_decode_int8: pa_decode over int8 pools, i.e. exact softmax attention
 * over the values code * scale. The MFMA kernel keeps the codes exact on the
 * matrix cores and applies the per-block scales in fp32.
 * For the K products q is converted to fp16, which holds every bf16 value
 * of magnitude 2^-14 .. 2^15 exactly. A query row whose largest |q| reaches
 * 2^15 is first multiplied by a power of two that brings it below 2^15 (exact),
 * and its scores by the inverse, so any finite q works; elements far below
 * the row's largest then round to fp16 subnormals (absolute error under
 * 2^-25 of the row's scale). The FP8 path keeps q in bf16.
 * Supported: q_dtype PA_BF16, D = 128, b in {16, 32}, T * G <= 32. */
int pa_decode_int8(const pa_dims* dims, const void* q, const int8_t* k_pool, const int8_t* v_pool,
                   const float* scales, const int32_t* block_tables,
                   const int32_t* seq_lens, float scale, void* out, pa_stream_t stream);

/* pa_decode_partitioned_int8: pa_decode_partitioned over int8 pools (same
 * workspace size and rules, same supported shapes as pa_decode_int8). */
int pa_decode_partitioned_int8(const pa_dims* dims, const void* q, const int8_t* k_pool,
                               const int8_t* v_pool, const float* scales,
                               const int32_t* block_tables, const int32_t* seq_lens, float scale,
                               void* out, int32_t max_seq_len, int32_t partition_tokens,
                               void* workspace, size_t workspace_bytes, pa_stream_t stream);

/* ---- Paged prefill ([P1] "25. Paged attention and prefix caching", stretch
 * exercise 4; [P4] "PagedAttention and the KV Cache", section "Prefill vs
 * decode under paging"; [P5] section 4.1).
 *
 * A prefill (or chunked-prefill) step gives sequence i a chunk of
 * n_i = q_start[i+1] - q_start[i] new tokens, packed one after another:
 * rows q_start[i] .. q_start[i+1] - 1 of q, k_new and v_new. They are the
 * sequence's newest positions L_i - n_i .. L_i - 1 (L_i = seq_lens[i] counts
 * the history and the chunk), so chunk token j sits at position
 * L_i - n_i + j. In these calls dims->q_tokens is a host-known bound on every
 * n_i (it sizes the grid); q_start is int32 [B + 1] on the device, with
 * q_start[0] = 0 and q_start[i] <= q_start[i+1]. A chunk may be empty
 * (n_i = 0); n_i <= L_i. Under PA_CHECK=1 these and the general preconditions
 * are checked on host copies (pa_check_prefill_host).
 */

/* pa_write_kv_varlen: store each chunk's K and V rows at their positions:
 * row q_start[i] + j of k_new / v_new ([Q, Hkv, D], kv_dtype, Q = q_start[B])
 * goes, bit for bit, to slot (block_tables[i][p / b], p % b) of the pools,
 * p = L_i - n_i + j. Same dtypes and rules as pa_write_kv; the slots written
 * must be distinct. */
int pa_write_kv_varlen(const pa_dims* dims, const void* k_new, const void* v_new, void* k_pool,
                       void* v_pool, const int32_t* block_tables, const int32_t* seq_lens,
                       const int32_t* q_start, pa_stream_t stream);

/* pa_prefill: causal attention of every chunk token over its sequence's
 * paged history and the chunk: row q_start[i] + j, query head h attends to
 * positions 0 .. L_i - n_i + j of kv head h / G, each read through the block
 * table (the chunk's own K/V must already be in the pools, e.g. from
 * pa_write_kv_varlen on the same stream).
 *   q   : [Q, Hq, D], q_dtype        out : [Q, Hq, D], out_dtype (fp32 or bf16)
 *   scale : finite and > 0 (PA_ERR_INVALID_ARG otherwise)
 * One launch on `stream`. Supported: bf16 q and KV, head_dim 128,
 * b in {4, 8, 16, 32}, G <= 128 (PA_ERR_UNSUPPORTED otherwise). */
int pa_prefill(const pa_dims* dims, const void* q, const void* k_pool, const void* v_pool,
               const int32_t* block_tables, const int32_t* seq_lens, const int32_t* q_start,
               float scale, void* out, pa_stream_t stream);

/* pa_check_prefill_host: the prefill preconditions on host arrays
 * (block_tables [B, MB], seq_lens [B], q_start [B + 1]): q_start[0] = 0 and
 * non-decreasing; 0 <= n_i <= min(L_i, q_tokens); L_i <= MB * b; used table
 * entries in [0, num_blocks); the chunks' (block, offset) slots distinct.
 * Returns PA_OK or PA_ERR_INVALID_ARG; launches nothing. */
int pa_check_prefill_host(const pa_dims* dims, const int32_t* block_tables, const int32_t* seq_lens,
                          const int32_t* q_start);

/* ---- Block management ([P1] "25. Paged attention and prefix caching",
 * sections "The allocator", "The paged cache", "Sharing blocks: forks and
 * copy-on-write" and "Prefix caching"; [P2] section 4).
 *
 * pa_copy_blocks: for each pair i, copy physical block block_pairs[2i] onto
 * block block_pairs[2i+1] in both pools (all kv heads; the Hkv * b * D
 * elements of a block are contiguous) and, for 8-bit pools, the block's
 * 2 * Hkv scales with it: a block's scales are part of the block ([P2]
 * section 6), and the copy is the whole block. This is the data half of
 * copy-on-write: pa_bm_reserve returns the pairs.
 *   dims : num_kv_heads, block_size, head_dim, num_blocks and kv_dtype are
 *          used (PA_F32, PA_BF16, PA_INT8 or PA_FP8_E4M3)
 *   scales : 8-bit pools: the pools' fp32 [N, Hkv, 2] scales (required);
 *            float pools: must be NULL
 *   block_pairs : int32 [num_pairs, 2] on the device
 * Preconditions (checked under PA_CHECK=1, pa_check_copies_host): every id in
 * [0, num_blocks); destinations distinct; no destination is also a source.
 * One launch on `stream`; num_pairs = 0 launches nothing. */
int pa_copy_blocks(const pa_dims* dims, void* k_pool, void* v_pool, float* scales,
                   const int32_t* block_pairs, int32_t num_pairs, pa_stream_t stream);

/* pa_check_copies_host: the pa_copy_blocks preconditions on host pairs. */
int pa_check_copies_host(const pa_dims* dims, const int32_t* block_pairs, int32_t num_pairs);

/* Host block manager (host memory only; nothing here touches the GPU). One
 * manager owns the block ids of one pool pair: a first-in first-out free list
 * over 0 .. num_blocks-1, a reference count per block (tables and prefix-cache
 * entries that hold it), and a block table and length per sequence (int64
 * ids chosen by the caller). Not thread-safe: one caller at a time. Calls
 * return PA_OK (or a count, >= 0) or a negative pa_status; a failed call
 * changes nothing. */
typedef struct pa_block_manager pa_block_manager;

/* A manager over num_blocks blocks of block_size positions; NULL on invalid
 * sizes or when memory runs out. */
pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size);
void pa_bm_destroy(pa_block_manager* m);
int32_t pa_bm_num_free(const pa_block_manager* m);
int32_t pa_bm_refcount(const pa_block_manager* m, int32_t block);
int32_t pa_bm_num_seqs(const pa_block_manager* m);
/* A new, empty sequence (error if the id is in use). */
int pa_bm_add_seq(pa_block_manager* m, int64_t seq);
/* Make blocks exist for positions [length, length + new_tokens) of seq, before
 * they are written. A block in that range that other tables or the prefix
 * cache also hold is replaced by a fresh block first (copy-on-write); the
 * (old, fresh) pairs go to copies (int32 [copies_capacity, 2], host) in table
 * order, their count to *num_copies, and the caller must copy those blocks
 * (pa_copy_blocks) before writing. PA_ERR_NO_BLOCKS when the pool cannot
 * supply every block the call needs (the caller may evict cached prefixes or
 * preempt a sequence, then retry). The length is unchanged. */
int pa_bm_reserve(pa_block_manager* m, int64_t seq, int32_t new_tokens, int32_t* copies,
                  int32_t copies_capacity, int32_t* num_copies);
/* Record that seq now holds `length` tokens (after their K/V are written); it
 * never decreases here, and may not pass the reserved blocks. */
int pa_bm_commit(pa_block_manager* m, int64_t seq, int32_t length);
/* child starts as an alias of parent: the same table and length, every block
 * shared (beam search, parallel sampling). */
int pa_bm_fork(pa_block_manager* m, int64_t parent, int64_t child);
/* Drop seq and release its blocks. */
int pa_bm_free_seq(pa_block_manager* m, int64_t seq);
/* Roll seq back to `length` (<= its length) tokens, releasing blocks it no
 * longer needs. */
int pa_bm_truncate(pa_block_manager* m, int64_t seq, int32_t length);
int32_t pa_bm_seq_length(const pa_block_manager* m, int64_t seq);
/* The block count of seq's table; with out != NULL also the table itself
 * (error if capacity is smaller). */
int32_t pa_bm_seq_blocks(const pa_block_manager* m, int64_t seq, int32_t* out, int32_t capacity);
/* Block tables and lengths of a batch, for the attention entry points:
 * tables int32 [num_seqs, width] (rows padded with `pad`), lengths int32
 * [num_seqs], both host memory. */
int pa_bm_build_tables(const pa_block_manager* m, const int64_t* seqs, int32_t num_seqs, int32_t width,
                       int32_t pad, int32_t* tables, int32_t* lengths);
/* Prefix cache: full blocks keyed by the whole token prefix that ends with
 * them, each holding its own reference, in least-recently-used order.
 * attach: create seq with the longest run of cached full blocks of the
 * prompt, always leaving at least one prompt token to prefill; returns the
 * tokens reused (the new length). remember: publish seq's full blocks (its
 * first num_tokens / b) under the prefixes of `tokens`; returns how many were
 * new. evict: drop least-recently-used entries that no table holds, until
 * blocks_wanted blocks are free or no such entry remains; returns the free
 * count. */
int32_t pa_bm_prefix_attach(pa_block_manager* m, int64_t seq, const int32_t* tokens, int32_t num_tokens);
int32_t pa_bm_prefix_remember(pa_block_manager* m, int64_t seq, const int32_t* tokens, int32_t num_tokens);
int32_t pa_bm_prefix_evict(pa_block_manager* m, int32_t blocks_wanted);
int32_t pa_bm_prefix_entries(const pa_block_manager* m);

/* ---- FP8 KV cache: OCP E4M3 codes (1 sign, 4 exponent bits with bias 7, 3
 * mantissa bits, largest finite 448, NaN at S.1111.111) with one fp32 scale
 * per (block, kv head), the format [P2] section 6 names beside int8 (and
 * [P1] "Attention that reads through the table" among what production paged
 * kernels add). Same shapes, rules and supported shapes as the int8 entry
 * points, with kv_dtype PA_FP8_E4M3 and these differences:
 *   scale = max |x| / 448 (float32); code = E4M3(x / scale), the quotient in
 *   float32, rounded to the nearest E4M3 value with ties to the even code,
 *   saturated at +-448 (a value that rounds to zero keeps its sign);
 *   re-encoding on a scale increase uses (value(code) * old_scale) / new_scale;
 *   decode attends over value(code) * scale. */
int pa_write_kv_fp8(const pa_dims* dims, const void* k_new, const void* v_new, uint8_t* k_pool,
                    uint8_t* v_pool, float* scales, const int32_t* block_tables,
                    const int32_t* positions, pa_stream_t stream);
int pa_decode_fp8(const pa_dims* dims, const void* q, const uint8_t* k_pool, const uint8_t* v_pool,
                  const float* scales, const int32_t* block_tables,
                  const int32_t* seq_lens, float scale, void* out, pa_stream_t stream);
int pa_decode_partitioned_fp8(const pa_dims* dims, const void* q, const uint8_t* k_pool,
                              const uint8_t* v_pool, const float* scales,
                              const int32_t* block_tables, const int32_t* seq_lens, float scale,
                              void* out, int32_t max_seq_len, int32_t partition_tokens,
                              void* workspace, size_t workspace_bytes, pa_stream_t stream);

/* pa_check_inputs_host: the preconditions above, checked on host copies.
 *   block_tables : int32 [B, MB] (required)
 *   seq_lens     : int32 [B], or NULL to skip the checks that need lengths
 *   positions    : int32 [B, T], or NULL to skip the write-slot checks
 * Checks, for every sequence i (with L = seq_lens[i] when given):
 *   q_tokens <= L <= MB * b; block_tables[i][j] in [0, num_blocks) for
 *   j < ceil(L / b); every position in [0, MB * b) with its block's table
 *   entry in [0, num_blocks); and no two (i, t) writing the same
 *   (block, offset) slot.
 * Returns PA_OK, or PA_ERR_INVALID_ARG at the first violation (also for
 * invalid dims or a NULL block_tables). Host memory only; launches nothing. */
int pa_check_inputs_host(const pa_dims* dims, const int32_t* block_tables, const int32_t* seq_lens,
                         const int32_t* positions);

/* Static text for a status code. Never NULL. */
const char* pa_status_string(int status);

/* ABI version: bumped when a signature or a struct layout changes. */
int pa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
