// Block copies for copy-on-write ([P1] "25. Paged attention and prefix caching", section "Sharing
// blocks: forks and copy-on-write": before a sequence writes into a block that others share, the
// block's contents are copied to a fresh block). One physical block of a pool [N, Hkv, b, D] is
// Hkv * b * D contiguous elements, so a copy is a plain contiguous move of that many bytes, for the
// K pool and the V pool. Each thread moves 16 bytes; a workgroup covers 4 KiB of one (pair, pool).
// 8-bit pools carry one K and one V scale per (block, kv head) ([P2] "Модуль 09: PagedAttention:
// пейджинг KV-кэша", section 6), 2 * Hkv contiguous floats per block in the [N, Hkv, 2] array: the
// K-pool workgroup of a pair's first chunk copies them too, so the copy is the whole block.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

struct CopyParams {
  char* k_pool;
  char* v_pool;
  float* scales;         // 8-bit pools: [N, Hkv, 2]; else null
  const int32_t* pairs;  // [n, 2]: source block, destination block
  int64_t block_bytes;   // Hkv * b * D * sizeof(dtype), a multiple of 16
  int32_t scale_floats;  // 2 * Hkv scales per block (8-bit pools)
  int32_t chunks;        // workgroups per (pair, pool): ceil(block_bytes / 4096)
};

__global__ __launch_bounds__(256) void copy_blocks_kernel(const CopyParams p) {
  const int c = blockIdx.x % p.chunks;
  const int which = (blockIdx.x / p.chunks) & 1;  // 0: K pool, 1: V pool
  const int pair = blockIdx.x / (2 * p.chunks);
  const int32_t src = p.pairs[2 * pair], dst = p.pairs[2 * pair + 1];
  if (p.scales && c == 0 && which == 0) {
    for (int i = threadIdx.x; i < p.scale_floats; i += 256)
      p.scales[(int64_t)dst * p.scale_floats + i] = p.scales[(int64_t)src * p.scale_floats + i];
  }
  const int64_t off = (int64_t)c * 4096 + threadIdx.x * 16;
  if (off >= p.block_bytes) return;
  char* pool = which ? p.v_pool : p.k_pool;
  const u32x4 v = load16(pool + (int64_t)src * p.block_bytes + off);
  *reinterpret_cast<u32x4*>(pool + (int64_t)dst * p.block_bytes + off) = v;
}

}  // namespace

hipError_t launch_copy_blocks(const pa_dims& d, void* k_pool, void* v_pool, float* scales, const int32_t* pairs,
                              int32_t num_pairs, hipStream_t stream) {
  if (num_pairs == 0) return hipSuccess;
  CopyParams p;
  p.k_pool = static_cast<char*>(k_pool);
  p.v_pool = static_cast<char*>(v_pool);
  p.scales = scales;
  p.pairs = pairs;
  p.scale_floats = 2 * d.num_kv_heads;
  p.block_bytes = (int64_t)d.num_kv_heads * d.block_size * d.head_dim * (d.kv_dtype == PA_F32 ? 4 : d.kv_dtype == PA_BF16 ? 2 : 1);
  p.chunks = (int32_t)((p.block_bytes + 4095) / 4096);
  const int64_t grid = (int64_t)num_pairs * 2 * p.chunks;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  copy_blocks_kernel<<<dim3((unsigned)grid), dim3(256), 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace pa
