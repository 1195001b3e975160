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

// ---- int8 pools ([P2] "Модуль 09: PagedAttention: пейджинг KV-кэша", section 6): codes with one
// scale per (block, kv head). A workgroup per (sequence, kv head), wave 0 for K and wave 1 for V,
// appends that head's T new rows, block by block: the block's scale grows to cover the new rows (a block first written at offset 0 takes theirs
// alone), the codes already in it are re-quantised when the scale grew, then the new rows are
// quantised. Every code is decided with the same fp32 operations the definition states: the scale
// amax / 127, the quotient x / scale (correctly rounded), round half to even, clip to [-127, 127].

struct WriteInt8Params {
  const void* k_new;
  const void* v_new;
  int8_t* k_pool;
  int8_t* v_pool;
  float* scales;  // [N, Hkv, 2]: K scale, V scale of each (block, kv head)
  const int32_t* block_tables;
  const int32_t* positions;
  int32_t T, Hkv, MB, block_size, D;
  int32_t new_f32;  // new rows are fp32 (else bf16)
};

__device__ __forceinline__ float new_value(const WriteInt8Params& p, const void* base, int64_t idx) {
  if (p.new_f32) return static_cast<const float*>(base)[idx];
  return __uint_as_float((uint32_t)static_cast<const uint16_t*>(base)[idx] << 16);
}


template <bool FP8>
__global__ __launch_bounds__(128) void write_kv_int8_kernel(const WriteInt8Params p) {
  constexpr float kCodeMax = FP8 ? 448.f : 127.f;  // largest code magnitude: scale = max|x| / kCodeMax
  const int lane = threadIdx.x & 63;
  const int which = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // 0: K, 1: V
  const int kvh = blockIdx.x % p.Hkv;
  const int seq = blockIdx.x / p.Hkv;
  const int D = p.D, b = p.block_size;
  {
    const void* src = which ? p.v_new : p.k_new;
    int8_t* pool = which ? p.v_pool : p.k_pool;
    for (int t = 0; t < p.T;) {
      const int pos0 = p.positions[(int64_t)seq * p.T + t];
      const int first = pos0 % b;
      const int n = min(p.T - t, b - first);  // new rows landing in this block (positions are consecutive)
      const int blk = p.block_tables[(int64_t)seq * p.MB + pos0 / b];
      const int64_t row0 = ((int64_t)blk * p.Hkv + kvh) * b;  // row index of offset 0 in the pool
      // largest magnitude among the new rows of this head
      float a = 0.f;
      for (int r = 0; r < n; ++r) {
        const int64_t base = ((int64_t)(seq * p.T + t + r) * p.Hkv + kvh) * D;
        for (int d = lane; d < D; d += 64) a = fmaxf(a, fabsf(new_value(p, src, base + d)));
      }
      a = wave_max(a);
      const float cand = a / kCodeMax;
      float* sp = p.scales + ((int64_t)blk * p.Hkv + kvh) * 2 + which;
      const float old = first > 0 ? *sp : 0.f;
      const float scale = first > 0 ? fmaxf(old, cand) : cand;
      if (first > 0 && scale > old) {
        // re-quantise the codes already in the block with the larger scale
        uint32_t* words = reinterpret_cast<uint32_t*>(pool + row0 * D);
        for (int w = lane; w < first * D / 4; w += 64) {
          const uint32_t c4 = words[w];
          uint32_t out = 0;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float c = code_value<FP8>((c4 >> (8 * k)) & 0xFFu);
            out |= encode_code<FP8>(c * old, scale) << (8 * k);
          }
          words[w] = out;
        }
      }
      for (int r = 0; r < n; ++r) {
        const int64_t base = ((int64_t)(seq * p.T + t + r) * p.Hkv + kvh) * D;
        uint32_t* words = reinterpret_cast<uint32_t*>(pool + (row0 + first + r) * D);
        for (int w = lane; w < D / 4; w += 64) {
          uint32_t out = 0;
#pragma unroll
          for (int k = 0; k < 4; ++k)
            out |= encode_code<FP8>(new_value(p, src, base + 4 * w + k), scale) << (8 * k);
          words[w] = out;
        }
      }
      if (lane == 0) *sp = scale;
      t += n;
    }
  }
}

}  // namespace

hipError_t launch_write_kv_int8(const pa_dims& d, const void* k_new, const void* v_new, int8_t* k_pool,
                                int8_t* v_pool, float* scales, const int32_t* block_tables,
                                const int32_t* positions, bool fp8, hipStream_t stream) {
  WriteInt8Params p;
  p.k_new = k_new;
  p.v_new = v_new;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.scales = scales;
  p.block_tables = block_tables;
  p.positions = positions;
  p.T = d.q_tokens;
  p.Hkv = d.num_kv_heads;
  p.MB = d.max_blocks_per_seq;
  p.block_size = d.block_size;
  p.D = d.head_dim;
  p.new_f32 = d.q_dtype == PA_F32;
  const int64_t grid = (int64_t)d.num_seqs * d.num_kv_heads;
  if (grid == 0) return hipSuccess;
  if (fp8)
    write_kv_int8_kernel<true><<<dim3((unsigned)grid), dim3(128), 0, stream>>>(p);
  else
    write_kv_int8_kernel<false><<<dim3((unsigned)grid), dim3(128), 0, stream>>>(p);
  return hipGetLastError();
}

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
