// Split-context decode over balanced, paired ranges, on the matrix cores (gfx950 MFMA), head_dim 128,
// bf16 or 8-bit (int8, E4M3) pools, up to 16 query rows per kv head.
//
// It computes what pa_decode_partitioned computes ([P1] "25. Paged attention and prefix caching",
// section "Attention that reads through the table": long contexts are cut into pieces whose partial
// results a second pass merges; [P5] "Chapter 7 Paged KV Cache and Memory Management", section 4.2:
// the exact merge of (m, l, acc) partials) with a division of the work that keeps every SIMD busy
// to the end:
//  * The 16-position tiles of every sequence, for one kv head, are taken as one list (sequence 0's
//    tiles, then sequence 1's, ...), cut into R equal contiguous ranges (R <= tiles / partition
//    tiles, so a range is at least one partition long), one per pair of waves.
//  * A workgroup is 8 waves, 4 pairs (w, w + 4), and its LDS keeps it alone on its CU, two waves per
//    SIMD. Of two waves on one SIMD the older one is served first and streams several times faster
//    while both run, so ranges fixed per wave end at very different times. Here the two waves of a
//    pair share their range instead: one takes tiles from the front and the other from the back,
//    through one 64-bit LDS word (front, back) that both update with an atomic add, and they meet
//    wherever their speeds put them, so both end within a few tiles of each other.
//  * A wave's tiles of one sequence form one piece with its own (m, l, acc). Its partial goes to
//    workspace slot 2 (r - r0) + side of each of the sequence's rows, r the pair's range, r0 the
//    range holding the sequence's first tile, side 0 for the front wave and 1 for the back wave. At
//    the end each wave marks the slots of the sequences of its range that it did not touch as empty
//    (m = -inf, l = 0), and the kernel writes each sequence's slot count for the merge kernel, which
//    combines the slots of each row exactly.
//  * A piece's first tile sets each row's reference max; a later score more than 2^64 above it
//    raises the reference and rescales that row's l and accumulator by 2^(old - new) (rare: scores
//    that climb by more than 64 base-2 units; o = acc / l does not depend on the reference).
//  * The q rows of the workgroup's kv head go to LDS; a wave crossing into another sequence takes
//    that sequence's q operand from there. Up to 63 sequences (with their q rows in four 16-byte
//    pieces per thread), every wave scans the lengths itself in registers, lane s holding sequence
//    s, and its first tiles are fixed without the shared word (the front wave takes up to PF + 2
//    from the front, the back wave up to PF + 2 from the back, halves of shorter ranges), so its
//    first block-id lookups and tile loads go out before the workgroup's one barrier, behind which
//    the q rows and the shared words are stored. Larger batches stage the prefix sums in LDS first.
// The per-tile arithmetic (S^T = K Q^T on the matrix cores, masking, probabilities split into bf16 hi
// and lo parts, V through a swizzled LDS tile and transposed reads, P.V on the matrix cores) and the
// 8-bit widenings are those of the other matrix-core kernels (pa_mfma_tile.h).
#include "pa_device.h"
#include "pa_internal.h"
#include "pa_mfma_tile.h"
#include "pa_wave_timeline.h"

PA_TIMELINE_BUFFER(balanced)

namespace pa {
namespace {

using namespace mfma;

constexpr int kBalWaves = 8;  // waves per workgroup: pairs (w, w + 4)
constexpr int kBalPairs = kBalWaves / 2;
#ifndef PA_BAL_PREFETCH
#define PA_BAL_PREFETCH 2
#endif
#ifndef PA_BAL_Q8_PREFETCH
#define PA_BAL_Q8_PREFETCH 2
#endif
constexpr int kBalPrefetch = PA_BAL_PREFETCH;  // bf16 tiles in flight ahead of the one computed
// 8-bit tiles are half the registers, but running them further ahead measured slower (long_int8 96.7 us
// at 4 ahead against 90.5 at 2 and 89.9 at 1): the deeper ring's block ids and scales spill the
// tile loop's scalar registers
constexpr int kBalQ8Prefetch = PA_BAL_Q8_PREFETCH;
constexpr int kBalMaxSeqs = 1024;
constexpr int kBalSeqsPerThread = kBalMaxSeqs / (kBalWaves * 64);
constexpr int kBalQBytes = 48 * 1024;  // q rows of the batch for one kv head: B * rows * 256 bytes at most
constexpr int kBalQRegs = 4;            // small batches: 16-byte pieces of q per thread held in registers

struct BalLds {
  char vt[kBalWaves][kTileBytes];        // per-wave V tile
  int pre[kBalMaxSeqs + 1];              // pre[s]: tiles of the sequences before s
  int len[kBalMaxSeqs];
  int wsum[kBalWaves];
  unsigned long long cursor[kBalPairs];  // per pair: next front tile (low word), back end (high word)
  char q[kBalQBytes];                    // [B][rows][256 B]: q rows of this kv head, bf16 as stored
};
// more than half of a CU's 160 KiB: one workgroup per CU, so a pair's two waves share a SIMD
static_assert(sizeof(BalLds) > 80 * 1024, "the workgroup must hold a CU alone");

template <int BS, bool Q8, bool F8, bool AP, int PF>
__global__ __launch_bounds__(kBalWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void balanced_kernel(const DecodeParams p) {
  static_assert(BS >= kTile, "a tile lies inside one block");
  static_assert(!(Q8 && AP), "8-bit pools append with the separate append kernel");
  constexpr int kKvRow = Q8 ? kD : kRowBytes;
  constexpr int NBUF = PF + 1;
  __shared__ __attribute__((aligned(16))) BalLds sh;
  WaveTimeline tl;
  tl.begin();

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave % kBalPairs, side = wave / kBalPairs;  // side 0 walks forward, 1 backward
  const int g = lane >> 4, c16 = lane & 15;
  const int kvh = blockIdx.x % p.Hkv;
  const int W = (int)(gridDim.x / p.Hkv) * kBalPairs;  // pairs per kv head
  const int r = (int)(blockIdx.x / p.Hkv) * kBalPairs + pair;
  const int T = p.T, B = p.B, rows = p.rows;
  const int pt = p.part_tokens / kTile;  // tiles per partition

  // ---- lengths and tile prefix sums: in registers for small batches (lane s: sequence s's length
  // and first tile), else in LDS
  auto q_src = [&](int idx) {  // 16-byte piece idx of the kv head's q rows, [B][rows][16]
    const int s = idx / (rows * 16), n = (idx / 16) % rows, c = idx % 16;
    return static_cast<const char*>(p.q) + ((int64_t)(s * T + n / p.G) * p.Hq + kvh * p.G + n % p.G) * kRowBytes +
           c * 16;
  };
  const int q_pieces = B * rows * 16;
  const bool small = B < 64 && q_pieces <= kBalQRegs * kBalWaves * 64;
  int r_len = 0, r_pre = 0;
  u32x4 qreg[kBalQRegs];
  if (small) {
    r_len = lane < B ? (int)read_only(p.seq_lens)[lane] : 0;
#pragma unroll
    for (int i = 0; i < kBalQRegs; ++i) {
      const int idx = tid + i * kBalWaves * 64;
      if (idx < q_pieces) qreg[i] = load16(q_src(idx));
    }
    const int cnt = r_len > 0 ? (r_len + kTile - 1) / kTile : 0;
    r_pre = wave_inclusive_sum(cnt) - cnt;  // lanes B..63 hold the total
  } else {
    int loc[kBalSeqsPerThread], sum = 0;
#pragma unroll
    for (int k = 0; k < kBalSeqsPerThread; ++k) {
      const int s = kBalSeqsPerThread * tid + k;
      const int L = s < B ? (int)read_only(p.seq_lens)[s] : 0;
      loc[k] = L > 0 ? (L + kTile - 1) / kTile : 0;
      if (s < B) sh.len[s] = L;
      sum += loc[k];
    }
    const int incl = wave_inclusive_sum(sum);  // over the wave, then over the waves
    if (lane == 63) sh.wsum[wave] = incl;
    for (int idx = tid; idx < q_pieces; idx += kBalWaves * 64)
      *reinterpret_cast<u32x4*>(sh.q + idx * 16) = load16(q_src(idx));
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += sh.wsum[w];
    int run_sum = base + incl - sum;  // exclusive prefix of this thread's first sequence
#pragma unroll
    for (int k = 0; k < kBalSeqsPerThread; ++k) {
      const int s = kBalSeqsPerThread * tid + k;
      if (s <= B) sh.pre[s] = run_sum;
      run_sum += loc[k];
    }
    if (tid == kBalWaves * 64 - 1 && B == kBalMaxSeqs) sh.pre[B] = run_sum;
    __syncthreads();
  }
  // pre[s] (s <= B) and the length of sequence s < B, wave-uniform
  auto pre_at = [&](int s) {
    return small ? __builtin_amdgcn_readlane(r_pre, s) : __builtin_amdgcn_readfirstlane(sh.pre[s]);
  };
  auto len_at = [&](int s) {
    return small ? __builtin_amdgcn_readlane(r_len, s) : __builtin_amdgcn_readfirstlane(sh.len[s]);
  };
  const int N = pre_at(B);
  const int R = min(W, max(1, N / pt));
  // range of tile t < N: the largest r with floor(r N / R) <= t
  auto range_of = [&](int t) { return (int)(((int64_t)(t + 1) * R - 1) / N); };
  // sequence of tile t: the largest s with pre[s] <= t (empty sequences are passed over)
  auto seq_of = [&](int t) {
    if (small) {
      const uint64_t at_or_before = __ballot(lane < B && r_pre <= t);
      return __builtin_amdgcn_readfirstlane(63 - __builtin_clzll(at_or_before));
    }
    int lo = 0, hi = B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pre_at(mid) <= t) lo = mid; else hi = mid;
    }
    return lo;
  };

  const int t0 = r < R ? (int)((int64_t)r * N / R) : 0;
  const int t1 = r < R ? (int)((int64_t)(r + 1) * N / R) : 0;
  // the first tiles of each wave, fixed: up to PF + 2 from its end, the halves of a shorter range
  constexpr int kFirst = PF + 2;
  const int n_range = t1 - t0;
  const int k_front = min(kFirst, (n_range + 1) / 2), k_back = min(kFirst, n_range - k_front);
  auto first_take = [&](int i) {
    return side == 0 ? (i < k_front ? t0 + i : -1) : (i < k_back ? t1 - 1 - i : -1);
  };

  // The next tile of this wave from the pair's shared word (front, back), which starts past both first
  // takes, or -1 once the two ends have met. The front wave adds 1 to the low word and takes the old
  // front; the back wave adds -1 to the high word and takes the old back - 1; a tile is taken when the
  // old front < the old back, compared as signed words (the back may pass below 0 after the last take).
  // Each wave stops at its first miss, so the front wave's tiles are [t0, m) and the back wave's
  // [m, t1) for one m.
  auto grab_issue = [&]() -> uint64_t {
    uint64_t old = 0;
    if (lane == 0)
      old = __hip_atomic_fetch_add(&sh.cursor[pair], side == 0 ? (uint64_t)1 : (uint64_t)(-(int64_t)1) << 32,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return old;
  };
  auto grab_take = [&](uint64_t old) -> int {
    const int f = __builtin_amdgcn_readfirstlane((int)(uint32_t)old);
    const int b = __builtin_amdgcn_readfirstlane((int)(uint32_t)(old >> 32));
    const int t = side == 0 ? f : b - 1;
    return t >= f && t < b ? t : -1;
  };
  const int64_t block_bytes = (int64_t)p.Hkv * BS * kKvRow;
  const char* kbase = static_cast<const char*>(p.k_pool) + (int64_t)kvh * BS * kKvRow;
  const char* vbase = static_cast<const char*>(p.v_pool) + (int64_t)kvh * BS * kKvRow;
  lds_char* vt = (lds_char*)sh.vt[wave];

  struct Meta {
    int t, s, j, L, blk;  // t < 0: no tile
    float ks, vs;
  };
  struct TileRegs {
    u32x4 k[Q8 ? 2 : 4];
    u32x4 v[Q8 ? 2 : 4];
  };
  const uint32_t k_lane_off = Q8 ? c16 * kD + 32 * g : c16 * kRowBytes + g * 16;
  const uint32_t v_lane_off = Q8 ? (lane >> 2) * kD + 32 * (lane & 3) : lane * 16;

  // Block id and scales of tile t; the lookup cursor only moves one way (forward or backward). The
  // cursor keeps its sequence's bounds and length in registers, so a lookup inside the same sequence
  // reads no LDS: an LDS read there would wait for the table loads still in flight (LDS and scalar
  // loads share one counter, and scalar loads complete out of order), and the block-id loads of
  // consecutive tiles would then go out one after another instead of together.
  int lk_s = 0, lk_beg = 0, lk_end = 0, lk_len = 0;
  if (first_take(0) >= 0) {
    lk_s = seq_of(first_take(0));
    lk_beg = pre_at(lk_s);
    lk_end = pre_at(lk_s + 1);
    lk_len = len_at(lk_s);
  }
  auto meta_of = [&](int t) -> Meta {
    Meta m;
    m.t = t;
    m.s = m.j = m.L = m.blk = 0;
    m.ks = m.vs = 1.f;
    if (t < 0) return m;
    if (t >= lk_end || t < lk_beg) {
      while (t >= lk_end) {
        ++lk_s;
        lk_beg = lk_end;
        lk_end = pre_at(lk_s + 1);
      }
      while (t < lk_beg) {
        --lk_s;
        lk_end = lk_beg;
        lk_beg = pre_at(lk_s);
      }
      lk_len = len_at(lk_s);
    }
    m.s = lk_s;
    m.j = t - lk_beg;
    m.L = lk_len;
    const auto* trow = read_only(p.block_tables + (int64_t)lk_s * p.MB);
    // the id is clamped into the pool: a table entry past the length is never used for the result
    m.blk = (int)min((uint32_t)trow[min(m.j * kTile / BS, p.MB - 1)], (uint32_t)(p.num_blocks - 1));
    if constexpr (Q8) {
      const f32x2 sc = read_only(reinterpret_cast<const f32x2*>(p.scales))[(int64_t)m.blk * p.Hkv + kvh];
      m.ks = sc[0];
      m.vs = sc[1];
    }
    return m;
  };
  // `live` false: a load past the wave's last tile (every step issues the same loads); its empty
  // descriptors fetch nothing.
  auto load_tile = [&](const Meta& m, TileRegs& tr, bool live) {
    const int tile_p0 = m.j * kTile;
    const int64_t boff = (int64_t)m.blk * block_bytes + (int64_t)(tile_p0 % BS) * kKvRow;
    // the descriptors end at the sequence's length: rows past it read as zeros, fetching nothing
    const int bytes = live ? min(kTile, m.L - tile_p0) * kKvRow : 0;
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(kbase + boff, bytes);
    const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(vbase + boff, bytes);
    if constexpr (Q8) {
#pragma unroll
      for (int c = 0; c < 2; ++c) tr.k[c] = buffer_load16(kr, k_lane_off + 16 * c);
#pragma unroll
      for (int c = 0; c < 2; ++c) tr.v[c] = buffer_load16(vr, v_lane_off + 16 * c);
    } else {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) tr.k[kc] = buffer_load16(kr, k_lane_off + kc * 64);
#pragma unroll
      for (int c = 0; c < 4; ++c) tr.v[c] = buffer_load16(vr, v_lane_off + c * 1024);
    }
    if constexpr (AP) {
      if (tile_p0 + kTile > m.L - T) {  // the tile holds new positions: their rows come from k_new / v_new
        auto new_row = [&](const void* base, int t) -> const char* {
          return static_cast<const char*>(base) + ((int64_t)(m.s * T + t) * p.Hkv + kvh) * kRowBytes;
        };
        const int tk = tile_p0 + c16 - (m.L - T);
        if (tk >= 0 && tk < T) {
#pragma unroll
          for (int kc = 0; kc < 4; ++kc) tr.k[kc] = load16(new_row(p.k_new, tk) + (kc * 4 + g) * 16);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int tv = tile_p0 + 4 * c + (lane >> 4) - (m.L - T);
          if (tv >= 0 && tv < T) tr.v[c] = load16(new_row(p.v_new, tv) + (lane & 15) * 16);
        }
      }
    }
  };

  // ---- the computed piece's sequence: q operand, row limits
  int cs = -1, L_c = 0, vis_all = 0, row_lim = -1, row_tok = 0;
  u32x4 qb[4];
  float qsum = 0.f, qk_mul = p.qk_scale_log2;
  const bool present = c16 < rows;
  const bool rows_all_present = rows == 16;
  auto switch_seq = [&](int s) {
    cs = s;
    L_c = len_at(s);
    vis_all = L_c - T + 1;
    row_tok = present ? c16 / p.G : 0;
    row_lim = present ? L_c - T + row_tok : -1;
    const lds_char* qrow = (const lds_char*)sh.q + (s * rows + (present ? c16 : 0)) * kRowBytes;
    if constexpr (F8) {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const u32x4 v = *(const lds_u32x4*)(qrow + 64 * g + 16 * kc);
        qb[kc] = present ? v : u32x4{0u, 0u, 0u, 0u};
      }
      qsum = 0.f;
      qk_mul = p.qk_scale_log2;
    } else if constexpr (Q8) {
      u32x4 raw[4];
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) raw[kc] = *(const lds_u32x4*)(qrow + 64 * g + 16 * kc);
      float amax = 0.f;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
#pragma unroll
        for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(raw[kc][e])), fabsf(bf16_hi(raw[kc][e]))));
      amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
      const int k = present && amax >= 32768.f ? (int)((__float_as_uint(amax) >> 23) & 0xffu) - 141 : 0;
      const float down = __uint_as_float((uint32_t)(127 - k) << 23);  // 2^-k
      qk_mul = p.qk_scale_log2 * __uint_as_float((uint32_t)(127 + k) << 23);
      float part = 0.f;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const u32x4 v = present ? raw[kc] : u32x4{0u, 0u, 0u, 0u};
        f16x8 h;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          h[2 * e] = (_Float16)(bf16_lo(v[e]) * down);
          h[2 * e + 1] = (_Float16)(bf16_hi(v[e]) * down);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) part += (float)h[e];
        qb[kc] = __builtin_bit_cast(u32x4, h);
      }
      part += __shfl_xor(part, 16, 64);
      part += __shfl_xor(part, 32, 64);
      qsum = part;
    } else {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const u32x4 v = *(const lds_u32x4*)(qrow + (kc * 4 + g) * 16);
        qb[kc] = present ? v : u32x4{0u, 0u, 0u, 0u};
      }
      qk_mul = p.qk_scale_log2;
    }
  };

  float m_ref = kNegInf, l_part = 0.f, vcorr = 0.f;
  f32x4 acc[8];
  bool have_ref = false;
  auto clear = [&]() {
    m_ref = kNegInf;
    have_ref = false;
    l_part = 0.f;
    vcorr = 0.f;
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) acc[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  // S^T of one tile (lane l: positions 4g + e of score row c16), scaled, masked.
  auto scores = [&](bool masked, int tile_p0, const TileRegs& tr, float kscale) -> f32x4 {
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
    if constexpr (Q8) {
      u32x4 kf[4];
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const int j = 2 * kc;
        const uint32_t w0 = tr.k[j >> 2][j & 3], w1 = tr.k[(j + 1) >> 2][(j + 1) & 3];
        const u32x2 a = F8 ? fp8_to_bf16(w0) : codes_to_f16(w0);
        const u32x2 b = F8 ? fp8_to_bf16(w1) : codes_to_f16(w1);
        kf[kc] = u32x4{a[0], a[1], b[0], b[1]};
      }
      if constexpr (F8) {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[kc]), as_bf16x8(qb[kc]), c, 0, 0, 0);
        c = c * (kscale * qk_mul);
      } else {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(kf[kc]), as_f16x8(qb[kc]), c, 0, 0, 0);
        c = (c - kKOffset * qsum) * (kscale * qk_mul);
      }
    } else {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(tr.k[kc]), as_bf16x8(qb[kc]), c, 0, 0, 0);
      c = c * qk_mul;
    }
    if (masked) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (tile_p0 + 4 * g + e > row_lim) c[e] = kNegInf;
    }
    return c;
  };
  // the row max of s, on every lane of the row's column c16
  auto row_max = [&](const f32x4& s) {
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    return fmaxf(mx, __shfl_xor(mx, 32, 64));
  };
  // A score above the reference by more than 2^64: the row's reference becomes its max, and l, the V
  // offset weight and the accumulator row are rescaled by 2^(old - new) (accumulator row 4g + e of a
  // lane takes the factor of lane 4g + e, whose column c16 is that row).
  auto rescale = [&](const f32x4& s) {
    const float m_new = fmaxf(m_ref, row_max(s));
    const float f = exp2_fast(m_ref - m_new);
    l_part *= f;
    vcorr *= f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float fe = __shfl(f, 4 * g + e, 64);
#pragma unroll
      for (int jb = 0; jb < 8; ++jb) acc[jb][e] *= fe;
    }
    m_ref = m_new;
  };
  // P.V of one tile: probabilities split into bf16 hi + lo parts, V through the swizzled LDS tile.
  auto accumulate = [&](bool masked, int tile_p0, const f32x4& s, const TileRegs& tr, float vscale) {
    float pr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = s[e];
      pr[e] = x == kNegInf ? 0.f : exp2_fast(x - m_ref);
      l_part += pr[e];
      if constexpr (Q8) {
        pr[e] *= vscale;
        if constexpr (!F8) vcorr += pr[e];
      }
    }
    const uint32_t h01 = cvt_pk_bf16(pr[0], pr[1]);
    const uint32_t h23 = cvt_pk_bf16(pr[2], pr[3]);
    const uint32_t l01 = cvt_pk_bf16(pr[0] - bf16_lo(h01), pr[1] - bf16_hi(h01));
    const uint32_t l23 = cvt_pk_bf16(pr[2] - bf16_lo(h23), pr[3] - bf16_hi(h23));
    const s16x4 a_hi = __builtin_bit_cast(s16x4, (uint64_t)h01 | ((uint64_t)h23 << 32));
    const s16x4 a_lo = __builtin_bit_cast(s16x4, (uint64_t)l01 | ((uint64_t)l23 << 32));
    if constexpr (Q8) {
      const int t = lane >> 2;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t w0 = tr.v[c >> 1][2 * (c & 1)], w1 = tr.v[c >> 1][2 * (c & 1) + 1];
        const u32x2 a = F8 ? fp8_to_bf16(w0) : codes_to_bf16(w0);
        const u32x2 b = F8 ? fp8_to_bf16(w1) : codes_to_bf16(w1);
        *(lds_u32x4*)(vt + v_swz(t, 64 * (lane & 3) + 16 * c)) = u32x4{a[0], a[1], b[0], b[1]};
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int t = 4 * c + (lane >> 4);
        u32x4 v = tr.v[c];
        if (masked && tile_p0 + t >= L_c) v = u32x4{0u, 0u, 0u, 0u};
        *(lds_u32x4*)(vt + v_swz(t, (lane & 15) * 16)) = v;
      }
    }
    wave_lds_order();
    const int rr = (lane >> 2) & 3, qq = lane & 3;
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) {
      const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vt + v_swz(4 * g + rr, (16 * jb + 4 * qq) * 2)));
      acc[jb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_hi, b, acc[jb], 0, 0, 0);
      acc[jb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_lo, b, acc[jb], 0, 0, 0);
    }
    wave_lds_order();
  };

  auto out_row = [&](int s, int n) -> int64_t { return (int64_t)(s * T + n / p.G) * p.Hq + kvh * p.G + n % p.G; };
  // slot of sequence s for this range and side; past the workspace's slots (lengths beyond the
  // call's max_seq_len) nothing is written
  auto slot_of = [&](int s) { return 2 * (r - range_of(pre_at(s))) + side; };
  // This wave's partial of sequence cs (its piece) into the sequence's slot for this range and side.
  auto flush = [&]() {
    if constexpr (Q8 && !F8) {  // remove the V offset: accumulator row 4g + e held 128 * sum(scaled P)
      float tot = vcorr;
      tot += __shfl_xor(tot, 16, 64);
      tot += __shfl_xor(tot, 32, 64);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ce = kVOffset * __shfl(tot, 4 * g + e, 64);
#pragma unroll
        for (int jb = 0; jb < 8; ++jb) acc[jb][e] -= ce;
      }
    }
    const int slot = slot_of(cs);
    if (slot >= p.parts) return;
    float l = l_part;
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (g == 0 && present)
      *reinterpret_cast<f32x2*>(p.part_ml + (out_row(cs, c16) * p.parts + slot) * 2) = f32x2{m_ref, l};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int na = 4 * g + e;
      if (na < rows) {
        float* dst = p.part_acc + (out_row(cs, na) * p.parts + slot) * kD + c16;
#pragma unroll
        for (int jb = 0; jb < 8; ++jb) dst[16 * jb] = acc[jb][e];
      }
    }
  };

  // ---- the pipeline: loads run PF tiles ahead of the tile computed, block ids one tile before their
  // loads, and grabs one tile before that. Past this wave's last tile every step still issues the same
  // loads, through empty descriptors that fetch nothing.
  int lo_tile = INT32_MAX, hi_tile = -1;  // this wave's part of the range, as it is taken
  {
    TileRegs ring[NBUF];
    Meta meta[NBUF];
    // the first takes: the PF tiles loaded ahead, the next block ids and the pending tile; their
    // block-id lookups go out together, before the workgroup's barrier
#pragma unroll
    for (int u = 0; u < PF; ++u) meta[u] = meta_of(first_take(u));
    Meta last_valid = meta[0];
    if (meta[0].t >= 0) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        if (meta[u].t >= 0) last_valid = meta[u];
        load_tile(last_valid, ring[u], meta[u].t >= 0);
      }
    }
    Meta m_next = meta_of(first_take(PF));
    int t_pending = first_take(PF + 1);

    // q rows (small batches), the pairs' shared words and the merge's slot counts; then the one barrier
    if (small) {
#pragma unroll
      for (int i = 0; i < kBalQRegs; ++i) {
        const int idx = tid + i * kBalWaves * 64;
        if (idx < q_pieces) *reinterpret_cast<u32x4*>(sh.q + idx * 16) = qreg[i];
      }
    }
    if (side == 0 && lane == 0)
      sh.cursor[pair] = (unsigned long long)(uint32_t)(t0 + k_front) |
                        ((unsigned long long)(uint32_t)(t1 - k_back) << 32);
    // slot counts for the merge, one per sequence (every kv head has the same ranges): written once
    if (blockIdx.x == 0) {
      if (small) {
        // pre[s + 1] from lane s + 1, read with every lane active (lane B <= 63 holds the total)
        const int a = r_pre, b = __shfl_down(r_pre, 1, 64);
        if (wave == 0 && lane < B) p.slot_counts[lane] = b > a ? 2 * (range_of(b - 1) - range_of(a) + 1) : 0;
      } else {
        for (int s = tid; s < B; s += kBalWaves * 64) {
          const int a = sh.pre[s], b = sh.pre[s + 1];
          p.slot_counts[s] = b > a ? 2 * (range_of(b - 1) - range_of(a) + 1) : 0;
        }
      }
    }
    __syncthreads();  // no barrier below this point

    if (meta[0].t >= 0) {
      for (bool more = true; more;) {
#pragma unroll
        for (int u = 0; u < NBUF; ++u) {
          if (more) {
            const Meta m = meta[u];
            if (m.t < 0) {
              more = false;
            } else {
              // the loads PF tiles ahead, the block ids of the tile after, the grab of the one after that
              if (m_next.t >= 0) last_valid = m_next;
              meta[(u + PF) % NBUF] = m_next;
              load_tile(last_valid, ring[(u + PF) % NBUF], m_next.t >= 0);
              m_next = meta_of(t_pending);
              const bool grab_live = t_pending >= 0;
              const uint64_t raw = grab_live ? grab_issue() : 0ull;

              tl.first_tile();
              lo_tile = min(lo_tile, m.t);
              hi_tile = max(hi_tile, m.t);
              if (m.s != cs) {  // a new piece: this wave's tiles of another sequence
                if (cs >= 0) flush();
                switch_seq(m.s);
                clear();
              }
              const int tile_p0 = m.j * kTile;
              const bool masked = !rows_all_present || tile_p0 + kTile > vis_all;
              const f32x4 s = scores(masked, tile_p0, ring[u], m.ks);
              if (!have_ref) {
                m_ref = row_max(s);  // the piece's first tile sets the reference
                have_ref = true;
              } else {
                bool over = false;
#pragma unroll
                for (int e = 0; e < 4; ++e) over |= s[e] > m_ref + kRefSlack;
                if (__builtin_expect(__any(over), 0)) rescale(s);
              }
              accumulate(masked, tile_p0, s, ring[u], m.vs);
              t_pending = grab_live ? grab_take(raw) : -1;
            }
          }
        }
      }
      flush();
    }
  }
  if (n_range <= 0) return;  // a range past the last (more pairs than ranges)
  tl.end_loop(hi_tile >= lo_tile ? hi_tile - lo_tile + 1 : 0);

  // ---- empty slots: the sequences of the range that this wave's part does not touch. The front
  // part is [t0, hi_tile], the back part [lo_tile, t1 - 1].
  {
    int skip_lo = seq_of(t0), skip_hi = seq_of(t1 - 1);
    if (hi_tile >= 0) {
      if (side == 0)
        skip_lo = seq_of(hi_tile) + 1;  // the sequences after the front part's last
      else
        skip_hi = seq_of(lo_tile) - 1;  // the sequences before the back part's first
    }
    for (int s = skip_lo; s <= skip_hi; ++s) {
      if (pre_at(s + 1) == pre_at(s)) continue;  // an empty sequence has no slots
      const int slot = slot_of(s);
      if (slot < p.parts && g == 0 && present)
        *reinterpret_cast<f32x2*>(p.part_ml + (out_row(s, c16) * p.parts + slot) * 2) = f32x2{kNegInf, 0.f};
    }
  }

  if constexpr (AP) {
    // the new rows (positions L - T .. L - 1) whose tiles this wave walked go to their pool slots
    if (hi_tile >= 0) {
      for (int s = seq_of(lo_tile); s < B && pre_at(s) <= hi_tile; ++s) {
        const int L = len_at(s);
        const auto* trow = read_only(p.block_tables + (int64_t)s * p.MB);
        for (int t = max(0, T - L); t < T; ++t) {
          const int pos = L - T + t;
          const int tile = pre_at(s) + pos / kTile;
          if (tile < lo_tile || tile > hi_tile) continue;
          const int blk = (int)min((uint32_t)trow[min(pos / BS, p.MB - 1)], (uint32_t)(p.num_blocks - 1));
          if (lane < 32) {
            const int which = lane >> 4, chunk = lane & 15;
            const int64_t dst = (int64_t)blk * block_bytes + (int64_t)(pos % BS) * kRowBytes + chunk * 16;
            const char* src = static_cast<const char*>(which ? p.v_new : p.k_new) +
                              ((int64_t)(s * T + t) * p.Hkv + kvh) * kRowBytes + chunk * 16;
            *reinterpret_cast<u32x4*>(const_cast<char*>(which ? vbase : kbase) + dst) = load16(src);
          }
        }
      }
    }
  }
  PA_TIMELINE_STORE(tl, blockIdx.x * kBalWaves + wave);
}

template <int BS, bool Q8, bool F8, bool AP>
hipError_t launch_bs_t(const DecodeParams& p, int grid, hipStream_t stream) {
  constexpr int PF = Q8 ? kBalQ8Prefetch : kBalPrefetch;
  balanced_kernel<BS, Q8, F8, AP, PF><<<dim3(grid), dim3(kBalWaves * 64), 0, stream>>>(p);
  return hipGetLastError();
}

template <bool Q8, bool F8, bool AP>
hipError_t launch_q(const DecodeParams& p, int grid, hipStream_t stream) {
  switch (p.block_size) {
    case 16: return launch_bs_t<16, Q8, F8, AP>(p, grid, stream);
    case 32: return launch_bs_t<32, Q8, F8, AP>(p, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

// Compute units of the current device (one workgroup each), read once per device.
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

}  // namespace

bool balanced_supported(const pa_dims& d) {
  const int rows = d.q_tokens * (d.num_q_heads / d.num_kv_heads);
  const bool pools = (d.kv_dtype == PA_BF16 || d.kv_dtype == PA_INT8 || d.kv_dtype == PA_FP8_E4M3) &&
                     d.q_dtype == PA_BF16;
  return pools && d.head_dim == kD && (d.block_size == 16 || d.block_size == 32) && rows <= 16 &&
         d.num_seqs <= kBalMaxSeqs && (int64_t)d.num_seqs * rows * kRowBytes <= kBalQBytes;
}

hipError_t launch_balanced(const DecodeParams& p, hipStream_t stream) {
  if (p.B == 0) return hipSuccess;
  if (!p.slot_counts || (p.append && p.kv_int8)) return hipErrorInvalidValue;
  // one workgroup (4 pairs) per CU, shared out over the kv heads; at least one per kv head
  const int grid = p.Hkv * max(1, device_cus() / p.Hkv);
  if (p.kv_int8)
    return p.kv_fp8 ? launch_q<true, true, false>(p, grid, stream) : launch_q<true, false, false>(p, grid, stream);
  return p.append ? launch_q<false, false, true>(p, grid, stream) : launch_q<false, false, false>(p, grid, stream);
}

}  // namespace pa
