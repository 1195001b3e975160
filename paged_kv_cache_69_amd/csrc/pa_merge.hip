// Merge of split-context partials (the "final merge" of flash-decoding).
//
// Partition k of a query row left (m_k, l_k, acc_k[D]), with l_k and acc_k
// both relative to the reference m_k (base-2 exponent units). The three-step
// merge of [P5] "Chapter 7 Paged KV Cache and Memory Management", section 4.2
// gives the exact result:
//   M = max_k m_k,  l = sum_k l_k 2^(m_k - M),  o = sum_k acc_k 2^(m_k - M) / l.
// A partition whose l_k is 0 (no visible position for this row) contributes
// nothing and is skipped, so 2^(-inf - -inf) is never formed.
//
// The work is pure HBM traffic (each partial is read once), so the layout is
// chosen for bytes in flight: a workgroup of 256 threads serves RPW query rows;
// a row's threads form SLOTS groups of D/4, each thread reading a float4 of one
// partition's accumulator, so a row has SLOTS partitions in flight per step.
// Few partitions per row -> several rows per workgroup, so short splits do not
// launch one tiny workgroup per row.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kMergeThreads = 256;

template <int D, int RPW>
__global__ __launch_bounds__(kMergeThreads) void merge_partials_kernel(const DecodeParams p) {
  constexpr int LPC = D / 4;                   // threads per partition (one float4 each)
  constexpr int TPR = kMergeThreads / RPW;     // threads per row
  constexpr int SLOTS = TPR / LPC;             // partitions of a row in flight per step
  constexpr int WPR = TPR / 64;                // waves per row
  static_assert(TPR >= 64 && SLOTS >= 1, "a row needs at least one wave and one slot");
  __shared__ f32x4 part_sum[RPW][SLOTS][LPC];
  __shared__ float red_m[kMergeThreads / 64], red_l[kMergeThreads / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int r = tid / TPR, t = tid % TPR;
  const int slot = t / LPC, c = t % LPC;
  const int64_t rows = (int64_t)p.B * p.T * p.Hq;
  const int64_t row_raw = (int64_t)blockIdx.x * RPW + r;  // (seq * T + token) * Hq + head
  const int64_t row = min(row_raw, rows - 1);             // a padding row re-reads the last one
  const f32x2* ml = reinterpret_cast<const f32x2*>(p.part_ml) + row * p.parts;
  const float* acc = p.part_acc + row * p.parts * D + 4 * c;

  // Every load below depends only on the row: the (m, l) of partition t (the first TPR of them) and
  // the accumulators of this slot's first kBatch partitions are in flight together with the length.
  // Indices are clamped to the workspace's partition count; partitions at or past the sequence's
  // own count (never written) are masked out once the length is known.
  constexpr int kBatch = 8;
  const f32x2 ml_t = ml[min(t, p.parts - 1)];
  f32x4 a[kBatch];
  f32x2 v[kBatch];
#pragma unroll
  for (int j = 0; j < kBatch; ++j) {
    const int k = min(slot + j * SLOTS, p.parts - 1);
    v[j] = ml[k];
    a[j] = *reinterpret_cast<const f32x4*>(acc + (int64_t)k * D);
  }
  const int64_t seq = row / ((int64_t)p.T * p.Hq);
  const int L = p.seq_lens[seq];
  // slots written: the shared prefix's (cascade), then one per partition of the sequence's own positions,
  // or, after balanced ranges, the count that kernel wrote for the sequence
  const int own = p.slot_counts ? p.slot_counts[seq] : max(0, (L - p.prefix_tokens + p.part_tokens - 1) / p.part_tokens);
  const int nparts = row_raw < rows && L > 0 ? min(p.parts, p.prefix_parts + own) : 0;

  // M = max m_k over partitions with l_k > 0, then l = sum l_k 2^(m_k - M)
  float M = t < nparts && ml_t[1] > 0.f ? ml_t[0] : kNegInf;
  for (int k = t + TPR; k < nparts; k += TPR) {
    const f32x2 w = ml[k];
    if (w[1] > 0.f) M = fmaxf(M, w[0]);
  }
  M = wave_max(M);
  if constexpr (WPR > 1) {
    if (lane == 0) red_m[wave] = M;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < WPR; ++w) M = fmaxf(M, red_m[r * WPR + w]);
  }
  float lsum = t < nparts && ml_t[1] > 0.f ? ml_t[1] * exp2_fast(ml_t[0] - M) : 0.f;
  for (int k = t + TPR; k < nparts; k += TPR) {
    const f32x2 w = ml[k];
    if (w[1] > 0.f) lsum = fmaf(w[1], exp2_fast(w[0] - M), lsum);
  }
  lsum = wave_sum(lsum);
  if constexpr (WPR > 1) {
    if (lane == 0) red_l[wave] = lsum;
    __syncthreads();
    lsum = 0.f;
#pragma unroll
    for (int w = 0; w < WPR; ++w) lsum += red_l[r * WPR + w];
  }

  // o = sum acc_k 2^(m_k - M): slot s takes partitions s, s + SLOTS, ..., kBatch at a time.
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = slot;; k0 += kBatch * SLOTS) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (k0 + j * SLOTS < nparts && v[j][1] > 0.f) {
        const float w = exp2_fast(v[j][0] - M);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = fmaf(w, a[j][e], o[e]);
      }
    }
    if (k0 + kBatch * SLOTS >= nparts) break;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int k = min(k0 + kBatch * SLOTS + j * SLOTS, p.parts - 1);
      v[j] = ml[k];
      a[j] = *reinterpret_cast<const f32x4*>(acc + (int64_t)k * D);
    }
  }
  part_sum[r][slot][c] = o;
  __syncthreads();
  if (row_raw < rows && t < LPC) {
    f32x4 a = part_sum[r][0][t];
#pragma unroll
    for (int s = 1; s < SLOTS; ++s) a += part_sum[r][s][t];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float out = lsum > 0.f ? a[e] / lsum : 0.f;
      const int64_t idx = row * D + 4 * t + e;
      if (p.out_dtype == PA_F32)
        static_cast<float*>(p.out)[idx] = out;
      else
        static_cast<uint16_t*>(p.out)[idx] = f32_to_bf16(out);
    }
  }
}

template <int D, int RPW>
hipError_t launch_rpw(const DecodeParams& p, int64_t rows, hipStream_t stream) {
  const dim3 grid((unsigned)((rows + RPW - 1) / RPW)), block(kMergeThreads);
  merge_partials_kernel<D, RPW><<<grid, block, 0, stream>>>(p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeParams& p, int64_t rows, hipStream_t stream) {
  // Rows per workgroup: a row's threads load up to 8 partitions per slot in one go, so one wave per row
  // (2 slots for D = 128) covers 16 partitions; more partitions get more of the workgroup.
  constexpr int LPC = D / 4;
  // balanced ranges: the workspace rows hold 2P + 2 slots, but a row uses about two per range of its
  // sequence; two rows per workgroup prefetch 32 slots each and loop past that
  if (p.slot_counts) return launch_rpw<D, 2>(p, rows, stream);
  if (p.parts * LPC > 8 * kMergeThreads) return launch_rpw<D, 1>(p, rows, stream);
  if (p.parts * LPC > 4 * kMergeThreads) return launch_rpw<D, 2>(p, rows, stream);
  return launch_rpw<D, 4>(p, rows, stream);
}

}  // namespace

hipError_t launch_merge_partials(const DecodeParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.B * p.T * p.Hq;
  if (rows == 0) return hipSuccess;
  if (p.D == 128) return launch_d<128>(p, rows, stream);
  if (p.D == 64) return launch_d<64>(p, rows, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
