// Measurement probes of libpa_probe.so (declared in include/pa_probe.h): a streaming-read kernel, the
// ceiling HBM reads reach on this GPU; a paged read of every K/V block a decode call reads, through the
// same block tables with no arithmetic, the ceiling of that access pattern; the dependent loads in
// front of a decode workgroup's first tile, the latency floor of a decode launch; and a register-only
// MFMA loop, the bf16 matrix rate this GPU sustains, alone and with vector-ALU work beside it. None of
// them is part of the decode path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// XOR of a workgroup's per-thread values, written by thread 0 (256 threads, 4 waves).
__device__ __forceinline__ void store_xor(uint32_t x, uint32_t* dst) {
  for (int m = 32; m >= 1; m >>= 1) x ^= __shfl_xor(x, m, 64);
  __shared__ uint32_t red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) *dst = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// Consecutive threads read consecutive 16-byte chunks; each thread takes U chunks one grid-stride apart
// per step, all in flight before any is used.
template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16, uint32_t* out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= src[i];
  store_xor(fold(acc), out + blockIdx.x);
}

struct ChainParams {
  const char* k_pool;
  const char* v_pool;
  const int32_t* tables;
  const int32_t* lens;
  int32_t hkv, mb, nblocks, bs, row_bytes, dependent;
  uint32_t* out;
};

__global__ __launch_bounds__(256) void first_tile_kernel(const ChainParams p) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kvh = blockIdx.x % p.hkv, seq = blockIdx.x / p.hkv;
  const int32_t* row = p.tables + (int64_t)seq * p.mb;
  const int L = p.lens[seq];
  int j;
  if (p.dependent) {
    j = min(min(w, max(0, (L + p.bs - 1) / p.bs - 1)), p.mb - 1);  // the index needs the length first
  } else {
    j = min(w, p.mb - 1);  // clamped to the row: issued with the length
  }
  const int blk = (int)min((uint32_t)row[j], (uint32_t)(p.nblocks - 1));
  const int tile = p.bs * p.row_bytes;
  const int64_t off = ((int64_t)blk * p.hkv + kvh) * tile;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int b = lane * 16; b < tile; b += 64 * 16) {
    acc ^= *reinterpret_cast<const u32x4*>(p.k_pool + off + b);
    acc ^= *reinterpret_cast<const u32x4*>(p.v_pool + off + b);
  }
  store_xor(fold(acc) ^ (uint32_t)L, p.out + blockIdx.x);
}

struct PagedParams {
  const char* k_pool;
  const char* v_pool;
  const int32_t* tables;
  const int32_t* lens;
  int32_t hkv, mb, nblocks, bs, blocks_per_wave, groups;
  uint32_t* out;
};

template <int NT>
__device__ __forceinline__ u32x4 load_policy(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  return *p;
}

// One workgroup of 4 waves per (sequence, group of 4 * blocks_per_wave blocks, kv head), the kv head
// fastest; wave w reads blocks [j0, j0 + blocks_per_wave) of its group, U blocks (K and V rows of its
// kv head, NL 16-byte loads per lane each) in flight per step, through the table. A wave past the
// sequence's last block leaves. Each wave folds what it read into the workgroup's XOR.
template <int U, int NL, int NT>
__global__ __launch_bounds__(256) void paged_read_kernel(const PagedParams p) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int bid = blockIdx.x;
  const int kvh = bid % p.hkv;
  bid /= p.hkv;
  const int grp = bid % p.groups, seq = bid / p.groups;
  const int32_t* row = p.tables + (int64_t)seq * p.mb;
  const int nb = min((p.lens[seq] + p.bs - 1) / p.bs, p.mb);
  const int j0 = (grp * 4 + w) * p.blocks_per_wave, j1 = min(nb, j0 + p.blocks_per_wave);
  const int64_t tile = (int64_t)NL * 1024;  // bytes of one block's rows of one kv head
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int j = j0; j < j1; j += U) {
    u32x4 v[U][2 * NL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int blk = (int)min((uint32_t)row[min(j + u, j1 - 1)], (uint32_t)(p.nblocks - 1));
      const int64_t off = ((int64_t)blk * p.hkv + kvh) * tile + lane * 16;
#pragma unroll
      for (int l = 0; l < NL; ++l) {
        v[u][l] = load_policy<NT>(reinterpret_cast<const u32x4*>(p.k_pool + off + l * 1024));
        v[u][NL + l] = load_policy<NT>(reinterpret_cast<const u32x4*>(p.v_pool + off + l * 1024));
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (j + u < j1) {
#pragma unroll
        for (int l = 0; l < 2 * NL; ++l) acc ^= v[u][l];
      }
  }
  store_xor(fold(acc), p.out + blockIdx.x);
}

template <int U, int NT>
hipError_t launch_paged_u(const PagedParams& p, int nl, dim3 grid, hipStream_t s) {
  switch (nl) {
    case 1: paged_read_kernel<U, 1, NT><<<grid, dim3(256), 0, s>>>(p); break;
    case 2: paged_read_kernel<U, 2, NT><<<grid, dim3(256), 0, s>>>(p); break;
    case 4: paged_read_kernel<U, 4, NT><<<grid, dim3(256), 0, s>>>(p); break;
    case 8: paged_read_kernel<U, 8, NT><<<grid, dim3(256), 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int NT>
hipError_t launch_paged(const PagedParams& p, int nl, int unroll, dim3 grid, hipStream_t s) {
  switch (unroll) {
    case 1: return launch_paged_u<1, NT>(p, nl, grid, s);
    case 2: return launch_paged_u<2, NT>(p, nl, grid, s);
    case 4: return launch_paged_u<4, NT>(p, nl, grid, s);
    default: return hipErrorInvalidValue;
  }
}

// Each wave: `iters` rounds of 8 independent v_mfma_f32_16x16x32_bf16 into 8 accumulators, each MFMA
// followed by NV independent fp32 FMAs; scheduling fences keep that order. Operands come from the lane
// index, so the loop touches no memory; every thread stores one float made of all it computed.
template <int NV>
__global__ __launch_bounds__(256) void mfma_rate_kernel(int32_t iters, float* out) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(lane + i));
    b[i] = (__bf16)(0.002f * (float)(lane - i));
  }
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = 0.01f * (float)lane + (float)k;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
#pragma unroll
      for (int k = 0; k < NV; ++k) v[(j * NV + k) & 7] = fmaf(v[(j * NV + k) & 7], 0.9999f, 0.5f);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float t = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) t += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
#pragma unroll
  for (int k = 0; k < 8; ++k) t += v[k];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = t;
}

}  // namespace

extern "C" {

int pa_probe_stream_read(const void* src, size_t bytes, int32_t workgroups, int32_t unroll, uint32_t* out,
                         pa_probe_stream_t stream) {
  if (!src || !out || bytes == 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15u) != 0) return -1;
  if (workgroups < 1) return -1;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t n16 = (int64_t)(bytes / 16);
  (void)hipGetLastError();
  switch (unroll) {
    case 1: stream_read_kernel<1><<<dim3(workgroups), dim3(256), 0, s>>>((const u32x4*)src, n16, out); break;
    case 2: stream_read_kernel<2><<<dim3(workgroups), dim3(256), 0, s>>>((const u32x4*)src, n16, out); break;
    case 4: stream_read_kernel<4><<<dim3(workgroups), dim3(256), 0, s>>>((const u32x4*)src, n16, out); break;
    case 8: stream_read_kernel<8><<<dim3(workgroups), dim3(256), 0, s>>>((const u32x4*)src, n16, out); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int pa_probe_first_tile(const void* k_pool, const void* v_pool, const int32_t* block_tables, const int32_t* seq_lens,
                        int32_t num_seqs, int32_t num_kv_heads, int32_t max_blocks, int32_t num_blocks,
                        int32_t block_size, int32_t row_bytes, int32_t dependent, uint32_t* out,
                        pa_probe_stream_t stream) {
  if (!k_pool || !v_pool || !block_tables || !seq_lens || !out) return -1;
  if (num_seqs < 1 || num_kv_heads < 1 || max_blocks < 1 || num_blocks < 1 || block_size < 1 || row_bytes < 16 ||
      row_bytes % 16 != 0 || (int64_t)block_size * row_bytes > 16384)
    return -1;
  ChainParams p = {static_cast<const char*>(k_pool), static_cast<const char*>(v_pool), block_tables, seq_lens,
                   num_kv_heads, max_blocks, num_blocks, block_size, row_bytes, dependent ? 1 : 0, out};
  (void)hipGetLastError();
  first_tile_kernel<<<dim3((unsigned)((int64_t)num_seqs * num_kv_heads)), dim3(256), 0,
                      reinterpret_cast<hipStream_t>(stream)>>>(p);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int pa_probe_paged_read(const void* k_pool, const void* v_pool, const int32_t* block_tables, const int32_t* seq_lens,
                        int32_t num_seqs, int32_t num_kv_heads, int32_t max_blocks, int32_t num_blocks,
                        int32_t block_size, int32_t row_bytes, int32_t blocks_per_wave, int32_t unroll,
                        int32_t nontemporal, uint32_t* out, pa_probe_stream_t stream) {
  if (!k_pool || !v_pool || !block_tables || !seq_lens || !out) return -1;
  if (num_seqs < 1 || num_kv_heads < 1 || max_blocks < 1 || num_blocks < 1 || block_size < 1 || row_bytes < 1 ||
      blocks_per_wave < 1)
    return -1;
  const int64_t block_bytes = (int64_t)block_size * row_bytes;  // one block's rows of one kv head
  const int nl = (int)(block_bytes / 1024);
  if (block_bytes % 1024 != 0 || (nl != 1 && nl != 2 && nl != 4 && nl != 8)) return -1;
  const int32_t groups = (int32_t)(((int64_t)max_blocks + 4 * blocks_per_wave - 1) / (4 * blocks_per_wave));
  const int64_t grid = (int64_t)num_seqs * groups * num_kv_heads;
  if (grid > INT32_MAX) return -1;
  const PagedParams p = {static_cast<const char*>(k_pool), static_cast<const char*>(v_pool), block_tables, seq_lens,
                         num_kv_heads, max_blocks, num_blocks, block_size, blocks_per_wave, groups, out};
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const hipError_t e = nontemporal ? launch_paged<1>(p, nl, unroll, dim3((unsigned)grid), s)
                                   : launch_paged<0>(p, nl, unroll, dim3((unsigned)grid), s);
  if (e == hipErrorInvalidValue) return -1;
  return e == hipSuccess ? 0 : -3;
}

int pa_probe_mfma(int32_t workgroups, int32_t iters, int32_t valu_per_mfma, float* out, pa_probe_stream_t stream) {
  if (!out || workgroups < 1 || iters < 1) return -1;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  switch (valu_per_mfma) {
    case 0: mfma_rate_kernel<0><<<dim3(workgroups), dim3(256), 0, s>>>(iters, out); break;
    case 2: mfma_rate_kernel<2><<<dim3(workgroups), dim3(256), 0, s>>>(iters, out); break;
    case 4: mfma_rate_kernel<4><<<dim3(workgroups), dim3(256), 0, s>>>(iters, out); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
