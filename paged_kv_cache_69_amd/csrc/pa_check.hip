// Host-side checks of the preconditions the kernels rely on but do not test (see pa.h): the
// entry points run them on host copies of the index arrays when PA_CHECK=1.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "pa_internal.h"

namespace {

bool dims_ok(const pa_dims* d) {
  return d && d->num_seqs >= 0 && d->q_tokens >= 1 && d->num_kv_heads >= 1 && d->block_size >= 1 &&
         d->num_blocks >= 1 && d->max_blocks_per_seq >= 1;
}

// Copy `count` int32 from device memory on `stream` (which is drained first).
bool copy_to_host(std::vector<int32_t>& dst, const int32_t* src, int64_t count, hipStream_t stream) {
  dst.resize((size_t)count);
  if (count == 0) return true;
  if (hipMemcpyAsync(dst.data(), src, (size_t)count * sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return false;
  return hipStreamSynchronize(stream) == hipSuccess;
}

}  // namespace

extern "C" int pa_check_inputs_host(const pa_dims* dims, const int32_t* block_tables, const int32_t* seq_lens,
                                    const int32_t* positions) {
  if (!dims_ok(dims) || !block_tables) return PA_ERR_INVALID_ARG;
  const int64_t B = dims->num_seqs, T = dims->q_tokens, MB = dims->max_blocks_per_seq;
  const int64_t b = dims->block_size, N = dims->num_blocks;
  auto entry_ok = [&](int64_t i, int64_t j) {
    const int32_t e = block_tables[i * MB + j];
    return e >= 0 && e < N;
  };
  if (seq_lens) {
    for (int64_t i = 0; i < B; ++i) {
      const int64_t L = seq_lens[i];
      if (L < T || L > MB * b) return PA_ERR_INVALID_ARG;
      for (int64_t j = 0; j < (L + b - 1) / b; ++j)
        if (!entry_ok(i, j)) return PA_ERR_INVALID_ARG;
    }
  }
  if (positions) {
    std::vector<int64_t> slots;
    slots.reserve((size_t)(B * T));
    for (int64_t i = 0; i < B; ++i) {
      for (int64_t t = 0; t < T; ++t) {
        const int64_t pos = positions[i * T + t];
        if (pos < 0 || pos >= MB * b || !entry_ok(i, pos / b)) return PA_ERR_INVALID_ARG;
        slots.push_back((int64_t)block_tables[i * MB + pos / b] * b + pos % b);
      }
    }
    std::sort(slots.begin(), slots.end());
    if (std::adjacent_find(slots.begin(), slots.end()) != slots.end()) return PA_ERR_INVALID_ARG;
  }
  return PA_OK;
}

extern "C" int pa_check_prefill_host(const pa_dims* dims, const int32_t* block_tables, const int32_t* seq_lens,
                                     const int32_t* q_start) {
  if (!dims_ok(dims) || !block_tables || !seq_lens || !q_start) return PA_ERR_INVALID_ARG;
  const int64_t B = dims->num_seqs, MB = dims->max_blocks_per_seq;
  const int64_t b = dims->block_size, N = dims->num_blocks;
  if (q_start[0] != 0) return PA_ERR_INVALID_ARG;
  std::vector<int64_t> slots;
  for (int64_t i = 0; i < B; ++i) {
    const int64_t n = (int64_t)q_start[i + 1] - q_start[i];
    const int64_t L = seq_lens[i];
    if (n < 0 || n > dims->q_tokens || n > L || L > MB * b) return PA_ERR_INVALID_ARG;
    for (int64_t j = 0; j < (L + b - 1) / b; ++j) {
      const int32_t e = block_tables[i * MB + j];
      if (e < 0 || e >= N) return PA_ERR_INVALID_ARG;
    }
    for (int64_t pos = L - n; pos < L; ++pos) slots.push_back((int64_t)block_tables[i * MB + pos / b] * b + pos % b);
  }
  std::sort(slots.begin(), slots.end());
  if (std::adjacent_find(slots.begin(), slots.end()) != slots.end()) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

extern "C" int pa_check_copies_host(const pa_dims* dims, const int32_t* pairs, int32_t num_pairs) {
  if (!dims_ok(dims) || num_pairs < 0 || (num_pairs > 0 && !pairs)) return PA_ERR_INVALID_ARG;
  std::vector<int32_t> dsts, srcs;
  for (int32_t i = 0; i < num_pairs; ++i) {
    const int32_t s = pairs[2 * i], d = pairs[2 * i + 1];
    if (s < 0 || s >= dims->num_blocks || d < 0 || d >= dims->num_blocks) return PA_ERR_INVALID_ARG;
    srcs.push_back(s);
    dsts.push_back(d);
  }
  std::sort(dsts.begin(), dsts.end());
  if (std::adjacent_find(dsts.begin(), dsts.end()) != dsts.end()) return PA_ERR_INVALID_ARG;
  for (const int32_t s : srcs)
    if (std::binary_search(dsts.begin(), dsts.end(), s)) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

namespace pa {

int debug_check_copies(const pa_dims* dims, const int32_t* pairs, int32_t num_pairs, hipStream_t stream) {
  const char* env = getenv("PA_CHECK");
  if (!env || strcmp(env, "1") != 0) return PA_OK;
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &capture) != hipSuccess || capture != hipStreamCaptureStatusNone) return PA_OK;
  std::vector<int32_t> host;
  if (!copy_to_host(host, pairs, 2 * (int64_t)num_pairs, stream)) return PA_ERR_LAUNCH;
  return pa_check_copies_host(dims, host.data(), num_pairs);
}

int debug_check_prefill(const pa_dims* dims, const int32_t* block_tables, const int32_t* seq_lens,
                        const int32_t* q_start, hipStream_t stream) {
  const char* env = getenv("PA_CHECK");
  if (!env || strcmp(env, "1") != 0) return PA_OK;
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &capture) != hipSuccess || capture != hipStreamCaptureStatusNone) return PA_OK;
  const int64_t B = dims->num_seqs;
  std::vector<int32_t> tables, lens, starts;
  if (!copy_to_host(tables, block_tables, B * dims->max_blocks_per_seq, stream) ||
      !copy_to_host(lens, seq_lens, B, stream) || !copy_to_host(starts, q_start, B + 1, stream))
    return PA_ERR_LAUNCH;
  return pa_check_prefill_host(dims, tables.data(), lens.data(), starts.data());
}

int debug_check(const pa_dims* dims, const int32_t* block_tables, const int32_t* seq_lens,
                const int32_t* positions, int32_t max_seq_len, hipStream_t stream) {
  const char* env = getenv("PA_CHECK");
  if (!env || strcmp(env, "1") != 0) return PA_OK;
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &capture) != hipSuccess || capture != hipStreamCaptureStatusNone) return PA_OK;
  const int64_t B = dims->num_seqs;
  std::vector<int32_t> tables, lens, pos;
  if (!copy_to_host(tables, block_tables, B * dims->max_blocks_per_seq, stream)) return PA_ERR_LAUNCH;
  if (seq_lens && !copy_to_host(lens, seq_lens, B, stream)) return PA_ERR_LAUNCH;
  if (positions && !copy_to_host(pos, positions, B * dims->q_tokens, stream)) return PA_ERR_LAUNCH;
  if (max_seq_len > 0)
    for (const int32_t L : lens)
      if (L > max_seq_len) return PA_ERR_INVALID_ARG;
  return pa_check_inputs_host(dims, tables.data(), seq_lens ? lens.data() : nullptr,
                              positions ? pos.data() : nullptr);
}

int debug_check_prefix(const pa_dims* dims, const int32_t* block_tables, const int32_t* seq_lens,
                       int32_t prefix_tokens, hipStream_t stream) {
  const char* env = getenv("PA_CHECK");
  if (!env || strcmp(env, "1") != 0) return PA_OK;
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &capture) != hipSuccess || capture != hipStreamCaptureStatusNone) return PA_OK;
  const int64_t B = dims->num_seqs, MB = dims->max_blocks_per_seq;
  std::vector<int32_t> tables, lens;
  if (!copy_to_host(tables, block_tables, B * MB, stream) || !copy_to_host(lens, seq_lens, B, stream))
    return PA_ERR_LAUNCH;
  const int64_t nb = prefix_tokens / dims->block_size;
  if (nb > MB) return PA_ERR_INVALID_ARG;
  for (int64_t i = 0; i < B; ++i) {
    if (lens[i] < prefix_tokens + dims->q_tokens) return PA_ERR_INVALID_ARG;
    for (int64_t j = 0; j < nb; ++j)
      if (tables[i * MB + j] != tables[j]) return PA_ERR_INVALID_ARG;
  }
  return PA_OK;
}

}  // namespace pa
