// KV-append scatter: each new token's K and V rows go to their slot in the pool.
//
// Slot of position p: physical block table[p / b], offset p % b ([P1] "25. Paged
// attention and prefix caching", section "Paging"). Each K or V row of one kv
// head is D * sizeof(dtype) contiguous bytes, both in the new-token tensor
// [B, T, Hkv, D] and in the pool [N, Hkv, b, D]. So the scatter is a
// bit-exact copy of 16-byte chunks: one thread per chunk, and consecutive
// threads cover consecutive chunks of a row, so the reads and writes are
// coalesced.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

struct WriteParams {
  const char* k_new;
  const char* v_new;
  char* k_pool;
  char* v_pool;
  const int32_t* block_tables;
  const int32_t* positions;
  int32_t T, Hkv, MB, block_size;
  int32_t chunks_per_row;   // D * sizeof(dtype) / 16
  int32_t row_bytes;        // D * sizeof(dtype)
  int64_t block_bytes;      // Hkv * b * row_bytes
  int32_t total_chunks;     // B * T * 2 * Hkv * chunks_per_row (< 2^31, checked by the launcher)
};

// Thread idx copies chunk `chunk` of the (token, K or V, kv head) row. The new row's chunk is
// loaded first: its address does not depend on the slot, so that load overlaps the position and
// block-table lookups that the store address needs.
__global__ __launch_bounds__(256) void write_kv_kernel(const WriteParams p) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= p.total_chunks) return;
  const int chunk = idx % p.chunks_per_row;
  const int row = idx / p.chunks_per_row;  // (tok * 2 + which) * Hkv + kvh
  const int kvh = row % p.Hkv;
  const int which = (row / p.Hkv) & 1;     // 0: K, 1: V
  const int tok = row / (2 * p.Hkv);       // i * T + t
  const int64_t src = ((int64_t)tok * p.Hkv + kvh) * p.row_bytes + chunk * 16;
  const u32x4 v = load16((which ? p.v_new : p.k_new) + src);
  const int pos = p.positions[tok];
  const int phys = p.block_tables[(int64_t)(tok / p.T) * p.MB + pos / p.block_size];
  const int64_t dst = (int64_t)phys * p.block_bytes +
                      ((int64_t)kvh * p.block_size + pos % p.block_size) * p.row_bytes + chunk * 16;
  *reinterpret_cast<u32x4*>((which ? p.v_pool : p.k_pool) + dst) = v;
}

}  // namespace

hipError_t launch_write_kv(const pa_dims& d, const void* k_new, const void* v_new, void* k_pool,
                           void* v_pool, const int32_t* block_tables, const int32_t* positions,
                           hipStream_t stream) {
  const int elt = d.kv_dtype == PA_F32 ? 4 : 2;
  WriteParams p;
  p.k_new = static_cast<const char*>(k_new);
  p.v_new = static_cast<const char*>(v_new);
  p.k_pool = static_cast<char*>(k_pool);
  p.v_pool = static_cast<char*>(v_pool);
  p.block_tables = block_tables;
  p.positions = positions;
  p.T = d.q_tokens;
  p.Hkv = d.num_kv_heads;
  p.MB = d.max_blocks_per_seq;
  p.block_size = d.block_size;
  p.row_bytes = d.head_dim * elt;
  p.chunks_per_row = p.row_bytes / 16;
  p.block_bytes = (int64_t)d.num_kv_heads * d.block_size * p.row_bytes;
  const int64_t total = (int64_t)d.num_seqs * d.q_tokens * 2 * d.num_kv_heads * p.chunks_per_row;
  if (total == 0) return hipSuccess;
  if (total > 0x7fffff00LL) return hipErrorInvalidValue;
  p.total_chunks = (int32_t)total;
  const int64_t blocks = (total + 255) / 256;
  write_kv_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace pa
