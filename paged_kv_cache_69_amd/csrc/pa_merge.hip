// Merge of split-context partials (the "final merge" of flash-decoding).
//
// Partition k of a query row left (m_k, l_k, acc_k[D]), with l_k and acc_k
// both relative to the reference m_k (base-2 exponent units). The three-step
// merge of [P5] "Chapter 7 Paged KV Cache and Memory Management", section 4.2
// gives the exact result:
//   M = max_k m_k,  l = sum_k l_k 2^(m_k - M),  o = sum_k acc_k 2^(m_k - M) / l.
// A partition whose l_k is 0 (no visible position for this row) contributes
// nothing and is skipped, so 2^(-inf - -inf) is never formed. One workgroup of
// four waves handles one query row. Wave w sums partitions w, w + 4, ...
// (each lane holds D/64 elements), then the waves combine in LDS.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kMergeWaves = 4;

template <int D>
__global__ __launch_bounds__(kMergeWaves * 64) void merge_partials_kernel(const DecodeParams p) {
  constexpr int PER_LANE = D / 64;
  __shared__ float part_sum[kMergeWaves][D];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row = blockIdx.x;  // (seq * T + t) * Hq + h
  const int seq = (int)(row / ((int64_t)p.T * p.Hq));
  const int L = p.seq_lens[seq];
  const int nparts = L > 0 ? min(p.parts, (L + p.part_tokens - 1) / p.part_tokens) : 0;
  const float* ml = p.part_ml + row * p.parts * 2;
  const float* acc = p.part_acc + row * p.parts * D;

  float M = kNegInf;
  for (int k = lane; k < nparts; k += 64)
    if (ml[2 * k + 1] > 0.f) M = fmaxf(M, ml[2 * k]);
  M = wave_max(M);
  float lsum = 0.f;
  for (int k = lane; k < nparts; k += 64) {
    const float lk = ml[2 * k + 1];
    if (lk > 0.f) lsum = fmaf(lk, exp2_fast(ml[2 * k] - M), lsum);
  }
  lsum = wave_sum(lsum);

  float o[PER_LANE];
#pragma unroll
  for (int c = 0; c < PER_LANE; ++c) o[c] = 0.f;
#pragma unroll 4
  for (int k = wave; k < nparts; k += kMergeWaves) {
    const float lk = ml[2 * k + 1];
    if (lk > 0.f) {
      const float w = exp2_fast(ml[2 * k] - M);
#pragma unroll
      for (int c = 0; c < PER_LANE; ++c) o[c] = fmaf(w, acc[(int64_t)k * D + lane + 64 * c], o[c]);
    }
  }
#pragma unroll
  for (int c = 0; c < PER_LANE; ++c) part_sum[wave][lane + 64 * c] = o[c];
  __syncthreads();
  for (int d = threadIdx.x; d < D; d += kMergeWaves * 64) {
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) a += part_sum[w][d];
    const float out = lsum > 0.f ? a / lsum : 0.f;
    if (p.out_dtype == PA_F32)
      static_cast<float*>(p.out)[row * D + d] = out;
    else
      static_cast<uint16_t*>(p.out)[row * D + d] = f32_to_bf16(out);
  }
}

}  // namespace

hipError_t launch_merge_partials(const DecodeParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.B * p.T * p.Hq;
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)rows), block(kMergeWaves * 64);
  if (p.D == 128)
    merge_partials_kernel<128><<<grid, block, 0, stream>>>(p);
  else if (p.D == 64)
    merge_partials_kernel<64><<<grid, block, 0, stream>>>(p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
