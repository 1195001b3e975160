// extern "C" entry points of libpa.so: argument checks, kernel choice, launches.
// The declarations, and their citations of the pages, are in include/pa.h.
#include <math.h>
#include <stdlib.h>

#include <algorithm>
#include <mutex>

#include "pa_internal.h"

namespace {

using pa::DecodeParams;

constexpr int kAbiVersion = 2;
constexpr int32_t kSinglePassTokens = 0x7ffffff0;  // one partition that covers any length
#ifndef PA_LPT_MIN_SEQS
#define PA_LPT_MIN_SEQS 128
#endif
constexpr int32_t kLptMinSeqs = PA_LPT_MIN_SEQS;  // smaller batches fit the GPU in one round
// Split waves the GPU holds at once: 256 CUs x 4 SIMDs x 2 waves (the split kernels' register use).
#ifndef PA_RESIDENT_SPLIT_WAVES
#define PA_RESIDENT_SPLIT_WAVES 2048
#endif
constexpr int64_t kResidentSplitWaves = PA_RESIDENT_SPLIT_WAVES;

bool valid_dtype(int32_t t) { return t == PA_F32 || t == PA_BF16; }
int dtype_size(int32_t t) { return t == PA_F32 ? 4 : 2; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape checks shared by every entry point. Returns PA_OK when the dims describe a valid problem.
int check_shape(const pa_dims* d) {
  if (!d) return PA_ERR_INVALID_ARG;
  if (d->num_seqs < 0 || d->q_tokens < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1 ||
      d->head_dim < 1 || d->block_size < 1 || d->num_blocks < 1 || d->max_blocks_per_seq < 1)
    return PA_ERR_INVALID_ARG;
  if (d->num_q_heads % d->num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (d->variant < PA_VARIANT_AUTO || d->variant > PA_VARIANT_MFMA) return PA_ERR_INVALID_ARG;
  if (d->split_schedule < PA_SPLIT_AUTO || d->split_schedule > PA_SPLIT_BALANCED) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

// Float pools: q, kv and out dtypes are PA_F32 / PA_BF16, with q and kv alike.
int check_dims(const pa_dims* d) {
  const int st = check_shape(d);
  if (st != PA_OK) return st;
  if (!valid_dtype(d->q_dtype) || !valid_dtype(d->kv_dtype) || !valid_dtype(d->out_dtype))
    return PA_ERR_INVALID_ARG;
  if (d->q_dtype != d->kv_dtype) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

// 8-bit pools: kv dtype PA_INT8 or PA_FP8_E4M3 (kv8); q (and new rows) and out PA_F32 / PA_BF16.
int check_dims_int8(const pa_dims* d, int32_t kv8 = PA_INT8) {
  const int st = check_shape(d);
  if (st != PA_OK) return st;
  if (d->kv_dtype != kv8 || !valid_dtype(d->q_dtype) || !valid_dtype(d->out_dtype)) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH; }

// A launch's status is read with hipGetLastError, which also reports an earlier failed runtime call
// of this thread that nobody read (the caller's, say). That error is not the launch's: drop it just
// before launching.
void discard_stale_error() { (void)hipGetLastError(); }

// Which kernel family serves these dims, or PA_ERR_UNSUPPORTED.
int choose_variant(const pa_dims* d, int* variant) {
  const bool mfma = pa::mfma_supported(*d);
  const bool valu = pa::valu_supported(*d);
  switch (d->variant) {
    case PA_VARIANT_MFMA:
      if (!mfma) return PA_ERR_UNSUPPORTED;
      *variant = PA_VARIANT_MFMA;
      return PA_OK;
    case PA_VARIANT_VALU:
      if (!valu) return PA_ERR_UNSUPPORTED;
      *variant = PA_VARIANT_VALU;
      return PA_OK;
    default:
      if (mfma) {
        *variant = PA_VARIANT_MFMA;
        return PA_OK;
      }
      if (valu) {
        *variant = PA_VARIANT_VALU;
        return PA_OK;
      }
      return PA_ERR_UNSUPPORTED;
  }
}

DecodeParams base_params(const pa_dims* d, const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* block_tables, const int32_t* seq_lens, float scale, void* out) {
  DecodeParams p = {};
  p.q = q;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  p.out = out;
  p.qk_scale_log2 = scale * pa::kLog2eHost;
  p.B = d->num_seqs;
  p.T = d->q_tokens;
  p.Hq = d->num_q_heads;
  p.Hkv = d->num_kv_heads;
  p.G = d->num_q_heads / d->num_kv_heads;
  p.D = d->head_dim;
  p.MB = d->max_blocks_per_seq;
  p.block_size = d->block_size;
  p.num_blocks = d->num_blocks;
  p.rows = p.T * p.G;
  p.out_dtype = d->out_dtype;
  p.slot_counts = nullptr;
  return p;
}

int launch_attention(const pa_dims* d, int variant, DecodeParams& p, hipStream_t stream) {
  discard_stale_error();
  if (variant == PA_VARIANT_MFMA) {
    p.row_groups = 1;
    return launch_status(pa::launch_decode_mfma(p, stream));
  }
  p.row_groups = (p.rows + pa::valu_rows_per_group(p.rows) - 1) / pa::valu_rows_per_group(p.rows);
  return launch_status(pa::launch_decode_valu(p, d->kv_dtype, stream));
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace split: (m, l) pairs first, then the accumulators, each 256-byte aligned. `parts` slots per row.
void workspace_layout(const pa_dims* d, int32_t parts, size_t* ml_bytes, size_t* acc_bytes) {
  const size_t rows = (size_t)d->num_seqs * d->q_tokens * d->num_q_heads;
  *ml_bytes = align256(rows * (size_t)parts * 2 * sizeof(float));
  *acc_bytes = align256(rows * (size_t)parts * d->head_dim * sizeof(float));
}

// Positions of the shared prefix per prefix item of a cascade call: chunks small enough that the prefix
// waves (32 query rows x one chunk x one kv head each) number about kCascadePrefixWaves, a multiple of
// 16 and of b, at most the prefix. A function of the dims alone, so the workspace size is too. (1024:
// 80.2 us per prefix call, against 80.9 with 2048, 80.4 with 512 and 89.8 with 4096.)
#ifndef PA_CASCADE_PREFIX_WAVES
#define PA_CASCADE_PREFIX_WAVES 1024
#endif
constexpr int64_t kCascadePrefixWaves = PA_CASCADE_PREFIX_WAVES;
int32_t cascade_chunk(const pa_dims* d, int32_t prefix_tokens) {
  int32_t unit = 16;
  while (unit % d->block_size != 0) unit += 16;
  if (prefix_tokens <= unit) return unit;
  const int64_t rows = (int64_t)d->num_seqs * d->q_tokens * (d->num_q_heads / d->num_kv_heads);
  const int64_t items_per_chunk = (rows + 31) / 32 * d->num_kv_heads;  // 32 query rows per prefix wave
  const int64_t chunks = std::max<int64_t>(1, kCascadePrefixWaves / std::max<int64_t>(1, items_per_chunk));
  const int64_t chunk = ((prefix_tokens + chunks - 1) / chunks + unit - 1) / unit * unit;
  return (int32_t)std::min<int64_t>(std::max<int64_t>(chunk, unit), ((prefix_tokens + unit - 1) / unit) * unit);
}

// Workspace slots of a cascade call: the prefix's (one per workgroup of chunks), then the longest
// suffix's partitions.
int32_t cascade_prefix_slots(const pa_dims* d, int32_t prefix_tokens) {
  const int32_t chunk = cascade_chunk(d, prefix_tokens);
  const int32_t chunks = (prefix_tokens + chunk - 1) / chunk;
  return (chunks + pa::mfma_waves() - 1) / pa::mfma_waves();
}
int32_t cascade_parts(const pa_dims* d, int32_t prefix_tokens, int32_t max_seq_len, int32_t partition_tokens) {
  return cascade_prefix_slots(d, prefix_tokens) + (max_seq_len - prefix_tokens + partition_tokens - 1) / partition_tokens;
}


// The split schedule of the matrix-core kernels (pa_split_schedule), or PA_ERR_UNSUPPORTED for a forced
// balanced schedule the dims do not allow. Automatic choice, once one partition per wave would need more
// waves than the GPU holds at once (B * Hkv * parts bounds the waves from above): balanced ranges where
// the dims allow them (on the long-context workloads they end every SIMD's work together), else two
// consecutive partitions per wave for bf16 pools and 16 query rows per kv head; one partition per wave
// otherwise, and for 8-bit pools (half the bytes per tile: every wave they can get in flight).
int32_t split_schedule(const pa_dims* d, int32_t parts) {
  const bool rows16 = d->q_tokens * (d->num_q_heads / d->num_kv_heads) <= 16;
  const bool two_ok = rows16 && d->kv_dtype == PA_BF16;
  const bool big = (int64_t)d->num_seqs * d->num_kv_heads * parts > kResidentSplitWaves;
  switch (d->split_schedule) {
    case PA_SPLIT_BALANCED: return pa::balanced_supported(*d) ? PA_SPLIT_BALANCED : PA_ERR_UNSUPPORTED;
    case PA_SPLIT_ONE_PER_WAVE: return PA_SPLIT_ONE_PER_WAVE;
    case PA_SPLIT_TWO_PER_WAVE: return two_ok ? PA_SPLIT_TWO_PER_WAVE : PA_SPLIT_ONE_PER_WAVE;
    default:
      if (big && pa::balanced_supported(*d)) return PA_SPLIT_BALANCED;
      return big && two_ok ? PA_SPLIT_TWO_PER_WAVE : PA_SPLIT_ONE_PER_WAVE;
  }
}

// Workspace of a split call with `parts` partitions per row: the slots per row, and the bytes of the
// (m, l) pairs, the accumulators and the per-sequence slot counts, in that order. Balanced ranges are
// at least one partition long, so a sequence meets at most parts + 1 of them, each with a slot per
// wave of its pair: 2 parts + 2 slots, and the counts (one int32 per sequence) the merge reads.
int32_t split_layout(const pa_dims* d, int32_t parts, size_t* ml, size_t* acc, size_t* counts) {
  const bool bal = split_schedule(d, parts) == PA_SPLIT_BALANCED;
  const int32_t slots = bal ? 2 * parts + 2 : parts;
  workspace_layout(d, slots, ml, acc);
  *counts = bal ? align256((size_t)d->num_seqs * sizeof(int32_t)) : 0;
  return slots;
}

// Every decode entry point: argument checks, kernel choice, the attention launch and, for a split
// run, the merge launch. int8 pools carry their scales and run on the MFMA kernel.
int decode_entry(const pa_dims* dims, bool int8, bool split, const void* q, const void* k_pool, const void* v_pool,
                 const float* scales, const int32_t* block_tables, const int32_t* seq_lens,
                 float scale, void* out, int32_t max_seq_len, int32_t partition_tokens, void* workspace,
                 size_t workspace_bytes, pa_stream_t stream, const void* k_new = nullptr,
                 const void* v_new = nullptr, bool fp8 = false) {
  const bool append = k_new != nullptr || v_new != nullptr;
  int st = int8 ? check_dims_int8(dims, fp8 ? PA_FP8_E4M3 : PA_INT8) : check_dims(dims);
  if (st != PA_OK) return st;
  if (dims->num_seqs == 0) return PA_OK;
  if (!q || !k_pool || !v_pool || !block_tables || !seq_lens || !out) return PA_ERR_INVALID_ARG;
  if (int8 && (!scales || (reinterpret_cast<uintptr_t>(scales) & 7u) != 0)) return PA_ERR_INVALID_ARG;
  if (int8 && append) return PA_ERR_UNSUPPORTED;  // 8-bit pools append with pa_write_kv_int8 / _fp8
  if (append && (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new))) return PA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out)) return PA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return PA_ERR_INVALID_ARG;
  int32_t parts = 1;
  if (split) {
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return PA_ERR_INVALID_ARG;
    if (max_seq_len < 1 || partition_tokens < 1) return PA_ERR_INVALID_ARG;
    if (partition_tokens % 16 != 0 || partition_tokens % dims->block_size != 0) return PA_ERR_INVALID_ARG;
    if (workspace_bytes < pa_decode_partitioned_workspace_bytes(dims, max_seq_len, partition_tokens))
      return PA_ERR_INVALID_ARG;
    parts = (max_seq_len + partition_tokens - 1) / partition_tokens;
  }
  int variant = 0;
  if (int8) {
    if (dims->variant == PA_VARIANT_VALU || !pa::mfma_int8_supported(*dims)) return PA_ERR_UNSUPPORTED;
    variant = PA_VARIANT_MFMA;
  } else if (append) {
    if (dims->variant == PA_VARIANT_VALU || !pa::mfma_supported(*dims)) return PA_ERR_UNSUPPORTED;
    variant = PA_VARIANT_MFMA;
  } else {
    st = choose_variant(dims, &variant);
    if (st != PA_OK) return st;
  }
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  st = pa::debug_check(dims, block_tables, seq_lens, nullptr, split ? max_seq_len : 0, s);
  if (st != PA_OK) return st;

  DecodeParams p = base_params(dims, q, k_pool, v_pool, block_tables, seq_lens, scale, out);
  p.scales = scales;
  p.kv_int8 = int8 ? 1 : 0;
  p.kv_fp8 = int8 && fp8 ? 1 : 0;
  p.k_new = k_new;
  p.v_new = v_new;
  p.append = append ? 1 : 0;
  if (!split) {
    p.parts = 1;
    p.part_tokens = kSinglePassTokens;
    p.partial = 0;
    // batches of many sequences run as several rounds of workgroups: deal the longest first
    p.lpt = variant == PA_VARIANT_MFMA && dims->num_seqs >= kLptMinSeqs && dims->num_seqs <= pa::mfma_lpt_max_seqs();
    return launch_attention(dims, variant, p, s);
  }
  size_t ml_bytes = 0, acc_bytes = 0, count_bytes = 0;
  const int32_t slots = split_layout(dims, parts, &ml_bytes, &acc_bytes, &count_bytes);  // slots per row
  const int32_t schedule = variant == PA_VARIANT_MFMA ? split_schedule(dims, parts) : PA_SPLIT_ONE_PER_WAVE;
  if (schedule < 0) return schedule;
  p.part_tokens = partition_tokens;
  p.partial = 1;
  p.part_ml = static_cast<float*>(workspace);
  p.part_acc = reinterpret_cast<float*>(static_cast<char*>(workspace) + ml_bytes);
  if (schedule == PA_SPLIT_BALANCED) {
    p.parts = slots;
    p.slot_counts = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + ml_bytes + acc_bytes);
    discard_stale_error();
    st = launch_status(pa::launch_balanced(p, s));
  } else {
    p.parts = parts;  // one slot per partition (the workspace rows are `parts` slots apart, the rest unused)
    p.wave_parts = schedule == PA_SPLIT_TWO_PER_WAVE ? 2 : 1;
    st = launch_attention(dims, variant, p, s);
  }
  if (st != PA_OK) return st;
  return launch_status(pa::launch_merge_partials(p, s));
}

}  // namespace

// Both cascade entry points: argument checks, then the prefix and suffix items in one launch and the
// merge. With k_new / v_new the suffix items also append the new rows (they follow the shared prefix).
static int cascade_entry(const pa_dims* dims, bool append, const void* q, const void* k_new, const void* v_new,
                         const void* k_pool, const void* v_pool, const int32_t* block_tables,
                         const int32_t* seq_lens, float scale, void* out, int32_t prefix_tokens,
                         int32_t max_seq_len, int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                         pa_stream_t stream) {
  int st = check_dims(dims);
  if (st != PA_OK) return st;
  if (dims->num_seqs == 0) return PA_OK;
  if (!q || !k_pool || !v_pool || !block_tables || !seq_lens || !out || !workspace) return PA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out)) return PA_ERR_INVALID_ARG;
  if (append && (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new))) return PA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return PA_ERR_INVALID_ARG;
  if (!isfinite(scale) || prefix_tokens < 0 || max_seq_len < 1 || partition_tokens < 1) return PA_ERR_INVALID_ARG;
  if (max_seq_len < prefix_tokens) return PA_ERR_INVALID_ARG;
  const int32_t b = dims->block_size;
  if (partition_tokens % 16 != 0 || partition_tokens % b != 0 || prefix_tokens % 16 != 0 || prefix_tokens % b != 0)
    return PA_ERR_INVALID_ARG;
  if (workspace_bytes < pa_decode_cascade_workspace_bytes(dims, prefix_tokens, max_seq_len, partition_tokens))
    return PA_ERR_INVALID_ARG;
  if (dims->variant == PA_VARIANT_VALU || !pa::mfma_supported(*dims)) return PA_ERR_UNSUPPORTED;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  st = pa::debug_check(dims, block_tables, seq_lens, nullptr, max_seq_len, s);
  if (st == PA_OK) st = pa::debug_check_prefix(dims, block_tables, seq_lens, prefix_tokens, s);
  if (st != PA_OK) return st;

  const int32_t parts = cascade_parts(dims, prefix_tokens, max_seq_len, partition_tokens);
  size_t ml_bytes = 0, acc_bytes = 0;
  workspace_layout(dims, parts, &ml_bytes, &acc_bytes);
  DecodeParams p = base_params(dims, q, k_pool, v_pool, block_tables, seq_lens, scale, out);
  p.parts = parts;
  p.part_tokens = partition_tokens;
  p.partial = 1;
  p.prefix_tokens = prefix_tokens;
  p.prefix_part_tokens = cascade_chunk(dims, prefix_tokens);
  p.prefix_parts = cascade_prefix_slots(dims, prefix_tokens);
  p.part_ml = static_cast<float*>(workspace);
  p.part_acc = reinterpret_cast<float*>(static_cast<char*>(workspace) + ml_bytes);
  p.row_groups = 1;
  p.k_new = k_new;
  p.v_new = v_new;
  p.append = append ? 1 : 0;
  // the prefix's items and the sequences' own partitions in one launch, then the merge
  discard_stale_error();
  st = launch_status(p.prefix_parts > 0 ? pa::launch_cascade(p, s) : pa::launch_decode_mfma(p, s));
  if (st != PA_OK) return st;
  return launch_status(pa::launch_merge_partials(p, s));
}


// ---- the fixed device scratch of pa_decode_partitioned_noalloc. In host code `scratch` names a host-side
// stand-in, not device memory: the array's device address on a GPU comes from hipGetSymbolAddress with that
// device current, once per device, and only that address is handed to kernels.
constexpr size_t kNoallocScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's address of `scratch`, looked up on the first call on the device.
int noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return PA_ERR_LAUNCH;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}
}  // namespace

extern "C" {

int pa_abi_version(void) { return kAbiVersion; }

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case PA_ERR_LAUNCH: return "kernel launch failed";
    case PA_ERR_NO_BLOCKS: return "the block pool has too few free blocks";
    case PA_ERR_TOO_LARGE: return "the partials exceed the fixed device scratch of pa_decode_partitioned_noalloc (32 MiB)";
    default: return "unknown status";
  }
}

int pa_write_kv(const pa_dims* dims, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                const int32_t* block_tables, const int32_t* positions, pa_stream_t stream) {
  const int st = check_dims(dims);
  if (st != PA_OK) return st;
  if (dims->num_seqs == 0) return PA_OK;
  if (!k_new || !v_new || !k_pool || !v_pool || !block_tables || !positions) return PA_ERR_INVALID_ARG;
  if ((int64_t)dims->head_dim * dtype_size(dims->kv_dtype) % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
    return PA_ERR_INVALID_ARG;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int chk = pa::debug_check(dims, block_tables, nullptr, positions, 0, s);
  if (chk != PA_OK) return chk;
  discard_stale_error();
  return launch_status(pa::launch_write_kv(*dims, k_new, v_new, k_pool, v_pool, block_tables, positions, s));
}

int pa_decode(const pa_dims* dims, const void* q, const void* k_pool, const void* v_pool,
              const int32_t* block_tables, const int32_t* seq_lens, float scale, void* out,
              pa_stream_t stream) {
  return decode_entry(dims, false, false, q, k_pool, v_pool, nullptr, block_tables, seq_lens, scale, out, 0, 0,
                      nullptr, 0, stream);
}

size_t pa_decode_partitioned_workspace_bytes(const pa_dims* dims, int32_t max_seq_len,
                                             int32_t partition_tokens) {
  if (check_shape(dims) != PA_OK || max_seq_len < 1 || partition_tokens < 1) return 0;
  const int32_t parts = (max_seq_len + partition_tokens - 1) / partition_tokens;
  size_t ml = 0, acc = 0, counts = 0;
  split_layout(dims, parts, &ml, &acc, &counts);
  return ml + acc + counts;
}

int pa_decode_partitioned_schedule(const pa_dims* dims, int32_t max_seq_len, int32_t partition_tokens) {
  if (check_shape(dims) != PA_OK || max_seq_len < 1 || partition_tokens < 1) return PA_ERR_INVALID_ARG;
  return split_schedule(dims, (max_seq_len + partition_tokens - 1) / partition_tokens);
}

int pa_decode_partitioned(const pa_dims* dims, const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_tables, const int32_t* seq_lens, float scale, void* out,
                          int32_t max_seq_len, int32_t partition_tokens, void* workspace,
                          size_t workspace_bytes, pa_stream_t stream) {
  return decode_entry(dims, false, true, q, k_pool, v_pool, nullptr, block_tables, seq_lens, scale, out,
                      max_seq_len, partition_tokens, workspace, workspace_bytes, stream);
}

int pa_decode_partitioned_noalloc(const pa_dims* dims, const void* q, const void* k_pool, const void* v_pool,
                                  const int32_t* block_tables, const int32_t* seq_lens, float scale, void* out,
                                  int32_t max_seq_len, int32_t partition_tokens, pa_stream_t stream) {
  int st = check_dims(dims);
  if (st != PA_OK) return st;
  if (dims->num_seqs == 0) return PA_OK;
  const size_t need = pa_decode_partitioned_workspace_bytes(dims, max_seq_len, partition_tokens);
  if (need == 0) return PA_ERR_INVALID_ARG;
  if (need > kNoallocScratchBytes) return PA_ERR_TOO_LARGE;
  void* ws = nullptr;
  st = noalloc_scratch(&ws);
  if (st != PA_OK) return st;
  return decode_entry(dims, false, true, q, k_pool, v_pool, nullptr, block_tables, seq_lens, scale, out, max_seq_len,
                      partition_tokens, ws, kNoallocScratchBytes, stream);
}

int pa_write_kv_decode(const pa_dims* dims, const void* q, const void* k_new, const void* v_new, void* k_pool,
                       void* v_pool, const int32_t* block_tables, const int32_t* seq_lens, float scale, void* out,
                       pa_stream_t stream) {
  return decode_entry(dims, false, false, q, k_pool, v_pool, nullptr, block_tables, seq_lens, scale, out, 0, 0,
                      nullptr, 0, stream, k_new, v_new);
}

int pa_write_kv_decode_partitioned(const pa_dims* dims, const void* q, const void* k_new, const void* v_new,
                                   void* k_pool, void* v_pool, const int32_t* block_tables, const int32_t* seq_lens,
                                   float scale, void* out, int32_t max_seq_len, int32_t partition_tokens,
                                   void* workspace, size_t workspace_bytes, pa_stream_t stream) {
  return decode_entry(dims, false, true, q, k_pool, v_pool, nullptr, block_tables, seq_lens, scale, out,
                      max_seq_len, partition_tokens, workspace, workspace_bytes, stream, k_new, v_new);
}

size_t pa_decode_cascade_workspace_bytes(const pa_dims* dims, int32_t prefix_tokens, int32_t max_seq_len,
                                         int32_t partition_tokens) {
  if (check_shape(dims) != PA_OK || prefix_tokens < 0 || max_seq_len < 1 || partition_tokens < 1 ||
      max_seq_len < prefix_tokens)
    return 0;
  const int32_t parts = cascade_parts(dims, prefix_tokens, max_seq_len, partition_tokens);
  size_t ml = 0, acc = 0;
  workspace_layout(dims, parts, &ml, &acc);
  return ml + acc;
}

int pa_decode_cascade(const pa_dims* dims, const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_tables, const int32_t* seq_lens, float scale, void* out,
                      int32_t prefix_tokens, int32_t max_seq_len, int32_t partition_tokens, void* workspace,
                      size_t workspace_bytes, pa_stream_t stream) {
  return cascade_entry(dims, false, q, nullptr, nullptr, k_pool, v_pool, block_tables, seq_lens, scale, out,
                       prefix_tokens, max_seq_len, partition_tokens, workspace, workspace_bytes, stream);
}

int pa_write_kv_decode_cascade(const pa_dims* dims, const void* q, const void* k_new, const void* v_new,
                               void* k_pool, void* v_pool, const int32_t* block_tables, const int32_t* seq_lens,
                               float scale, void* out, int32_t prefix_tokens, int32_t max_seq_len,
                               int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                               pa_stream_t stream) {
  return cascade_entry(dims, true, q, k_new, v_new, k_pool, v_pool, block_tables, seq_lens, scale, out,
                       prefix_tokens, max_seq_len, partition_tokens, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {
int write_kv_q8(const pa_dims* dims, const void* k_new, const void* v_new, void* k_pool, void* v_pool, float* scales,
                const int32_t* block_tables, const int32_t* positions, bool fp8, pa_stream_t stream) {
  const int st = check_dims_int8(dims, fp8 ? PA_FP8_E4M3 : PA_INT8);
  if (st != PA_OK) return st;
  if (dims->num_seqs == 0) return PA_OK;
  if (!k_new || !v_new || !k_pool || !v_pool || !scales || !block_tables || !positions) return PA_ERR_INVALID_ARG;
  if (dims->head_dim % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_new) || !aligned16(v_new)) return PA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(scales) & 7u) != 0) return PA_ERR_INVALID_ARG;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int chk = pa::debug_check(dims, block_tables, nullptr, positions, 0, s);
  if (chk != PA_OK) return chk;
  discard_stale_error();
  return launch_status(pa::launch_write_kv_int8(*dims, k_new, v_new, static_cast<int8_t*>(k_pool),
                                                static_cast<int8_t*>(v_pool), scales, block_tables, positions, fp8,
                                                s));
}
}  // namespace

extern "C" {

int pa_write_kv_int8(const pa_dims* dims, const void* k_new, const void* v_new, int8_t* k_pool,
                     int8_t* v_pool, float* scales, const int32_t* block_tables, const int32_t* positions,
                     pa_stream_t stream) {
  return write_kv_q8(dims, k_new, v_new, k_pool, v_pool, scales, block_tables, positions, false, stream);
}

int pa_write_kv_fp8(const pa_dims* dims, const void* k_new, const void* v_new, uint8_t* k_pool,
                    uint8_t* v_pool, float* scales, const int32_t* block_tables, const int32_t* positions,
                    pa_stream_t stream) {
  return write_kv_q8(dims, k_new, v_new, k_pool, v_pool, scales, block_tables, positions, true, stream);
}

int pa_decode_fp8(const pa_dims* dims, const void* q, const uint8_t* k_pool, const uint8_t* v_pool,
                  const float* scales, const int32_t* block_tables, const int32_t* seq_lens, float scale, void* out,
                  pa_stream_t stream) {
  return decode_entry(dims, true, false, q, k_pool, v_pool, scales, block_tables, seq_lens, scale, out, 0, 0, nullptr,
                      0, stream, nullptr, nullptr, true);
}

int pa_decode_partitioned_fp8(const pa_dims* dims, const void* q, const uint8_t* k_pool,
                              const uint8_t* v_pool, const float* scales, const int32_t* block_tables,
                              const int32_t* seq_lens, float scale, void* out, int32_t max_seq_len,
                              int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                              pa_stream_t stream) {
  return decode_entry(dims, true, true, q, k_pool, v_pool, scales, block_tables, seq_lens, scale, out, max_seq_len,
                      partition_tokens, workspace, workspace_bytes, stream, nullptr, nullptr, true);
}

int pa_decode_int8(const pa_dims* dims, const void* q, const int8_t* k_pool, const int8_t* v_pool,
                   const float* scales, const int32_t* block_tables, const int32_t* seq_lens, float scale, void* out,
                   pa_stream_t stream) {
  return decode_entry(dims, true, false, q, k_pool, v_pool, scales, block_tables, seq_lens, scale, out, 0, 0, nullptr,
                      0, stream);
}

int pa_decode_partitioned_int8(const pa_dims* dims, const void* q, const int8_t* k_pool,
                               const int8_t* v_pool, const float* scales, const int32_t* block_tables,
                               const int32_t* seq_lens, float scale, void* out, int32_t max_seq_len,
                               int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                               pa_stream_t stream) {
  return decode_entry(dims, true, true, q, k_pool, v_pool, scales, block_tables, seq_lens, scale, out, max_seq_len,
                      partition_tokens, workspace, workspace_bytes, stream);
}

int pa_copy_blocks(const pa_dims* dims, void* k_pool, void* v_pool, float* scales, const int32_t* block_pairs,
                   int32_t num_pairs, pa_stream_t stream) {
  if (!dims || dims->num_kv_heads < 1 || dims->block_size < 1 || dims->head_dim < 1 || dims->num_blocks < 1)
    return PA_ERR_INVALID_ARG;
  const int32_t t = dims->kv_dtype;
  if (t != PA_F32 && t != PA_BF16 && t != PA_INT8 && t != PA_FP8_E4M3) return PA_ERR_INVALID_ARG;
  const bool q8 = t == PA_INT8 || t == PA_FP8_E4M3;
  if (q8 != (scales != nullptr)) return PA_ERR_INVALID_ARG;  // 8-bit pools bring their scales; float pools none
  if (num_pairs < 0) return PA_ERR_INVALID_ARG;
  if (num_pairs == 0) return PA_OK;
  if (!k_pool || !v_pool || !block_pairs || !aligned16(k_pool) || !aligned16(v_pool)) return PA_ERR_INVALID_ARG;
  if (q8 && (reinterpret_cast<uintptr_t>(scales) & 7u) != 0) return PA_ERR_INVALID_ARG;
  const int64_t row = (int64_t)dims->head_dim * (t == PA_F32 ? 4 : t == PA_BF16 ? 2 : 1);
  if ((row * dims->block_size * dims->num_kv_heads) % 16 != 0) return PA_ERR_UNSUPPORTED;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int chk = pa::debug_check_copies(dims, block_pairs, num_pairs, s);
  if (chk != PA_OK) return chk;
  discard_stale_error();
  return launch_status(pa::launch_copy_blocks(*dims, k_pool, v_pool, scales, block_pairs, num_pairs, s));
}

int pa_write_kv_varlen(const pa_dims* dims, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                       const int32_t* block_tables, const int32_t* seq_lens, const int32_t* q_start,
                       pa_stream_t stream) {
  const int st = check_dims(dims);
  if (st != PA_OK) return st;
  if (dims->num_seqs == 0) return PA_OK;
  if (!k_new || !v_new || !k_pool || !v_pool || !block_tables || !seq_lens || !q_start) return PA_ERR_INVALID_ARG;
  if ((int64_t)dims->head_dim * dtype_size(dims->kv_dtype) % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
    return PA_ERR_INVALID_ARG;
  if (dims->num_seqs > 65535) return PA_ERR_UNSUPPORTED;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int chk = pa::debug_check_prefill(dims, block_tables, seq_lens, q_start, s);
  if (chk != PA_OK) return chk;
  discard_stale_error();
  return launch_status(
      pa::launch_write_kv_varlen(*dims, k_new, v_new, k_pool, v_pool, block_tables, seq_lens, q_start, s));
}

int pa_prefill(const pa_dims* dims, const void* q, const void* k_pool, const void* v_pool,
               const int32_t* block_tables, const int32_t* seq_lens, const int32_t* q_start, float scale, void* out,
               pa_stream_t stream) {
  const int st = check_dims(dims);
  if (st != PA_OK) return st;
  if (dims->num_seqs == 0) return PA_OK;
  if (!q || !k_pool || !v_pool || !block_tables || !seq_lens || !q_start || !out) return PA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out)) return PA_ERR_INVALID_ARG;
  if (!isfinite(scale) || !(scale > 0.f)) return PA_ERR_INVALID_ARG;
  if (dims->variant == PA_VARIANT_VALU || !pa::prefill_supported(*dims)) return PA_ERR_UNSUPPORTED;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int chk = pa::debug_check_prefill(dims, block_tables, seq_lens, q_start, s);
  if (chk != PA_OK) return chk;
  discard_stale_error();
  return launch_status(pa::launch_prefill(*dims, q, k_pool, v_pool, block_tables, seq_lens, q_start, scale, out, s));
}

}  // extern "C"

#if PA_TIMELINE
#include "pa_wave_timeline.h"
#include "pa_timeline.h"

extern "C" int pa_timeline_read(int32_t family, void* host, size_t bytes) {
  if (!host) return -1;
  if (family == PA_TIMELINE_MFMA) return pa::timeline_read_mfma(host, bytes);
  if (family == PA_TIMELINE_BALANCED) return pa::timeline_read_balanced(host, bytes);
  return -1;
}

extern "C" int pa_timeline_clear(void) {
  const int a = pa::timeline_clear_mfma();
  return a != 0 ? a : pa::timeline_clear_balanced();
}
#endif
