// Split-context decode with balanced wave ranges, on the matrix cores (gfx950 MFMA), head_dim 128,
// bf16 or 8-bit (int8, E4M3) pools, up to 16 query rows per kv head.
//
// It computes what pa_decode_partitioned computes ([P1] "25. Paged attention and prefix caching",
// section "Attention that reads through the table": long contexts are cut into partitions whose
// partial results a second pass merges; [P5] "Chapter 7 Paged KV Cache and Memory Management",
// section 4.2: the exact merge of (m, l, acc) partials) with a different division of the work:
//  * The 16-position tiles of every sequence, for one kv head, are taken as one list (sequence 0's
//    tiles, then sequence 1's, ...), and the list is cut into R equal contiguous ranges, one per
//    wave. Every wave therefore streams the same number of tiles, however the lengths are spread.
//    The launch has one wave per SIMD (one round), and each wave keeps PF tiles in flight in
//    registers, so the bytes in flight per SIMD do not depend on another wave's progress.
//  * A range never holds less than one partition (R <= tiles / partition tiles), so a partition is
//    cut by at most one range boundary. Its first piece goes to workspace slot 2k of the row, its
//    second piece to slot 2k + 1; a partition that one wave walks whole writes its partial to slot
//    2k and an empty (m = -inf, l = 0) pair to slot 2k + 1. The merge kernel combines the 2P slots
//    of each row exactly as it combines P partitions.
//  * Each piece has its own reference max and restarts itself when a score outruns it by 2^64, as in
//    the other matrix-core kernels, so every slot holds what a wave of its own would have written.
//  * The workgroup stages the tile prefix sums of the batch, the lengths and the q rows of its kv
//    head in LDS before any wave starts; a wave crossing into the next sequence takes that
//    sequence's q operand from there.
// The per-tile arithmetic (S^T = K Q^T on the matrix cores, masking, probabilities split into bf16 hi
// and lo parts, V through a swizzled LDS tile and transposed reads, P.V on the matrix cores) and the
// 8-bit widenings are those of the other matrix-core kernels (pa_mfma_tile.h).
#include "pa_device.h"
#include "pa_internal.h"
#include "pa_mfma_tile.h"

namespace pa {
namespace {

using namespace mfma;

constexpr int kBalWaves = 4;  // waves per workgroup
#ifndef PA_BAL_WAVES_PER_SIMD
#define PA_BAL_WAVES_PER_SIMD 1
#endif
#ifndef PA_BAL_PREFETCH
#define PA_BAL_PREFETCH 6
#endif
#ifndef PA_BAL_Q8_PREFETCH
#define PA_BAL_Q8_PREFETCH 10
#endif
constexpr int kBalWavesPerSimd = PA_BAL_WAVES_PER_SIMD;
constexpr int kBalPrefetch = PA_BAL_PREFETCH;      // bf16 tiles in flight ahead of the one computed
constexpr int kBalQ8Prefetch = PA_BAL_Q8_PREFETCH;  // 8-bit tiles are half the registers
constexpr int kBalMaxSeqs = 1024;
constexpr int kBalQBytes = 48 * 1024;  // q rows of the batch for one kv head: B * rows * 256 bytes at most

struct BalLds {
  char vt[kBalWaves][kTileBytes];  // per-wave V tile
  int pre[kBalMaxSeqs + 1];        // pre[s]: tiles of the sequences before s
  int len[kBalMaxSeqs];
  int wsum[kBalWaves];
  char q[kBalQBytes];              // [B][rows][256 B]: q rows of this kv head, bf16 as stored
};

template <int BS, bool Q8, bool F8, bool AP, int PF>
__global__ __launch_bounds__(kBalWaves * 64) __attribute__((amdgpu_waves_per_eu(kBalWavesPerSimd)))
void balanced_kernel(const DecodeParams p) {
  static_assert(BS >= kTile, "a tile lies inside one block");
  static_assert(!(Q8 && AP), "8-bit pools append with the separate append kernel");
  constexpr int kKvRow = Q8 ? kD : kRowBytes;
  constexpr int kKvTile = kTile * kKvRow;
  constexpr int NBUF = PF + 1;
  __shared__ __attribute__((aligned(16))) BalLds sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const int kvh = blockIdx.x % p.Hkv;
  const int W = (int)(gridDim.x / p.Hkv) * kBalWaves;  // waves per kv head
  const int r = (int)(blockIdx.x / p.Hkv) * kBalWaves + wave;
  const int T = p.T, B = p.B, rows = p.rows;
  const int pt = p.part_tokens / kTile;  // tiles per partition

  // ---- lengths, tile prefix sums and this kv head's q rows into LDS (the whole workgroup)
  {
    int loc[4], sum = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int s = 4 * tid + k;
      const int L = s < B ? (int)read_only(p.seq_lens)[s] : 0;
      loc[k] = L > 0 ? (L + kTile - 1) / kTile : 0;
      if (s < B) sh.len[s] = L;
      sum += loc[k];
    }
    int incl = sum;  // inclusive scan over the wave, then over the waves
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d, 64);
      if (lane >= d) incl += y;
    }
    if (lane == 63) sh.wsum[wave] = incl;
    for (int idx = tid; idx < B * rows * 16; idx += kBalWaves * 64) {
      const int s = idx / (rows * 16), n = (idx / 16) % rows, c = idx % 16;
      const char* src = static_cast<const char*>(p.q) +
                        ((int64_t)(s * T + n / p.G) * p.Hq + kvh * p.G + n % p.G) * kRowBytes + c * 16;
      *reinterpret_cast<u32x4*>(sh.q + (s * rows + n) * kRowBytes + c * 16) = load16(src);
    }
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += sh.wsum[w];
    int run_sum = base + incl - sum;  // exclusive prefix of this thread's first sequence
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int s = 4 * tid + k;
      if (s <= B) sh.pre[s] = run_sum;
      run_sum += loc[k];
    }
    if (tid == kBalWaves * 64 - 1 && B == kBalMaxSeqs) sh.pre[B] = run_sum;
    __syncthreads();
  }
  const int N = sh.pre[B];
  const int R = min(W, max(1, N / pt));
  if (r >= R) return;  // no barrier below this point
  const int t0 = (int)((int64_t)r * N / R), t1 = (int)((int64_t)(r + 1) * N / R);
  if (t1 <= t0) return;

  auto pre_at = [&](int s) { return __builtin_amdgcn_readfirstlane(sh.pre[s]); };
  auto len_at = [&](int s) { return __builtin_amdgcn_readfirstlane(sh.len[s]); };
  // sequence of tile t: the largest s with pre[s] <= t (empty sequences are passed over)
  int s_first = 0;
  {
    int lo = 0, hi = B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pre_at(mid) <= t0) lo = mid; else hi = mid;
    }
    s_first = lo;
  }
  struct Cursor {
    int s, beg, end, L;  // sequence, its tiles [beg, end) in the list, its length
  };
  auto advance = [&](Cursor& c, int t) {
    while (t >= c.end) {
      ++c.s;
      c.beg = c.end;
      c.end = pre_at(c.s + 1);
      c.L = len_at(c.s);
    }
  };

  const int64_t block_bytes = (int64_t)p.Hkv * BS * kKvRow;
  const char* kbase = static_cast<const char*>(p.k_pool) + (int64_t)kvh * BS * kKvRow;
  const char* vbase = static_cast<const char*>(p.v_pool) + (int64_t)kvh * BS * kKvRow;
  lds_char* vt = (lds_char*)sh.vt[wave];

  struct Meta {
    int s, j, L, blk;
    float ks, vs;
  };
  struct TileRegs {
    u32x4 k[Q8 ? 2 : 4];
    u32x4 v[Q8 ? 2 : 4];
  };
  const uint32_t k_lane_off = Q8 ? c16 * kD + 32 * g : c16 * kRowBytes + g * 16;
  const uint32_t v_lane_off = Q8 ? (lane >> 2) * kD + 32 * (lane & 3) : lane * 16;

  // Block id and scales of tile t of the load cursor's sequence, then its loads.
  auto meta_of = [&](const Cursor& c, int t) -> Meta {
    Meta m;
    m.s = c.s;
    m.j = t - c.beg;
    m.L = c.L;
    const auto* trow = read_only(p.block_tables + (int64_t)c.s * p.MB);
    // the id is clamped into the pool: a table entry past the length is never used for the result
    m.blk = (int)min((uint32_t)trow[min(m.j * kTile / BS, p.MB - 1)], (uint32_t)(p.num_blocks - 1));
    m.ks = m.vs = 1.f;
    if constexpr (Q8) {
      const f32x2 sc = read_only(reinterpret_cast<const f32x2*>(p.scales))[(int64_t)m.blk * p.Hkv + kvh];
      m.ks = sc[0];
      m.vs = sc[1];
    }
    return m;
  };
  auto load_tile = [&](const Meta& m, TileRegs& tr) {
    const int tile_p0 = m.j * kTile;
    const int64_t boff = (int64_t)m.blk * block_bytes + (int64_t)(tile_p0 % BS) * kKvRow;
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(kbase + boff, kKvTile);
    const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(vbase + boff, kKvTile);
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

  // ---- the compute cursor's sequence: q operand, row limits
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
  auto raise_ref = [&](const f32x4& s) {
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    m_ref = fmaxf(m_ref, mx);
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

  // The partial of the piece [seg_i0, i_end) of sequence cs: slot 2k (the piece starts its partition)
  // or 2k + 1; a piece that is its whole partition also marks slot 2k + 1 empty.
  int seg_i0 = t0, seg_j0 = 0;
  auto flush = [&](int i_end) {
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
    const int k = seg_j0 / pt;
    const bool starts = seg_j0 % pt == 0;
    const int j_last = i_end - 1 - pre_at(cs);
    const int ntiles = pre_at(cs + 1) - pre_at(cs);
    const bool whole = starts && ((j_last + 1) % pt == 0 || j_last + 1 == ntiles);
    const int slot = 2 * k + (starts ? 0 : 1);
    auto out_row = [&](int n) -> int64_t { return (int64_t)(cs * T + n / p.G) * p.Hq + kvh * p.G + n % p.G; };
    float l = l_part;
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (g == 0 && present) {
      const int64_t pi = out_row(c16) * p.parts + slot;
      *reinterpret_cast<f32x2*>(p.part_ml + pi * 2) = f32x2{m_ref, l};
      if (whole) *reinterpret_cast<f32x2*>(p.part_ml + (pi + 1) * 2) = f32x2{kNegInf, 0.f};
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int na = 4 * g + e;
      if (na < rows) {
        float* dst = p.part_acc + (out_row(na) * p.parts + slot) * kD + c16;
#pragma unroll
        for (int jb = 0; jb < 8; ++jb) dst[16 * jb] = acc[jb][e];
      }
    }
  };

  const int last = t1 - 1;
  // Tiles [ib, t1) of the current piece onwards. Returns -1 when done, or the first tile of the piece
  // to run again when a score outran the reference (raised by then).
  auto run = [&](int ib) -> int {
    ib = __builtin_amdgcn_readfirstlane(ib);
    clear();
    TileRegs ring[NBUF];
    Meta meta[NBUF];
    Cursor lc = {cs, pre_at(cs), pre_at(cs + 1), L_c};
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int ti = min(ib + u, last);
      advance(lc, ti);
      meta[u] = meta_of(lc, ti);
      load_tile(meta[u], ring[u]);
    }
    // block ids (and scales) are fetched one tile before the loads that need them
    advance(lc, min(ib + PF, last));
    Meta m_next = meta_of(lc, min(ib + PF, last));
    int again = -1;
    for (int i0 = ib; i0 < t1 && again < 0; i0 += NBUF) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        const int i = i0 + u;
        if (i < t1 && again < 0) {
          const Meta m = meta[u];
          {
            meta[(u + PF) % NBUF] = m_next;
            load_tile(m_next, ring[(u + PF) % NBUF]);
            const int ti = min(i + PF + 1, last);
            advance(lc, ti);
            m_next = meta_of(lc, ti);
          }
          if (i != seg_i0 && (m.s != cs || m.j % pt == 0)) {  // a new piece starts at tile i
            flush(i);
            if (m.s != cs) switch_seq(m.s);
            seg_i0 = i;
            seg_j0 = m.j;
            m_ref = kNegInf;
            have_ref = false;
            clear();
          }
          const int tile_p0 = m.j * kTile;
          const bool masked = !rows_all_present || tile_p0 + kTile > vis_all;
          const f32x4 s = scores(masked, tile_p0, ring[u], m.ks);
          if (!have_ref) {
            raise_ref(s);
            have_ref = true;
          } else {
            bool over = false;
#pragma unroll
            for (int e = 0; e < 4; ++e) over |= s[e] > m_ref + kRefSlack;
            if (__builtin_expect(__any(over), 0)) {
              raise_ref(s);
              again = seg_i0;
            }
          }
          accumulate(masked, tile_p0, s, ring[u], m.vs);
        }
      }
    }
    return again;
  };

  switch_seq(s_first);
  seg_i0 = t0;
  seg_j0 = t0 - pre_at(s_first);
  for (int from = t0; (from = run(from)) >= 0;) {
  }
  flush(t1);

  if constexpr (AP) {
    // the new rows (positions L - T .. L - 1) whose tiles this wave walked go to their pool slots
    for (int s = s_first; s < B && pre_at(s) < t1; ++s) {
      const int L = len_at(s);
      const auto* trow = read_only(p.block_tables + (int64_t)s * p.MB);
      for (int t = max(0, T - L); t < T; ++t) {
        const int pos = L - T + t;
        const int tile = pre_at(s) + pos / kTile;
        if (tile < t0 || tile >= t1) continue;
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

}  // namespace

bool balanced_supported(const pa_dims& d) {
  const int rows = d.q_tokens * (d.num_q_heads / d.num_kv_heads);
  const bool pools = (d.kv_dtype == PA_BF16 || d.kv_dtype == PA_INT8 || d.kv_dtype == PA_FP8_E4M3) &&
                     d.q_dtype == PA_BF16;
  return pools && d.head_dim == kD && (d.block_size == 16 || d.block_size == 32) && rows <= 16 &&
         d.num_seqs <= kBalMaxSeqs && (int64_t)d.num_seqs * rows * kRowBytes <= kBalQBytes;
}

int balanced_waves() { return 1024 * kBalWavesPerSimd; }

hipError_t launch_balanced(const DecodeParams& p, hipStream_t stream) {
  if (p.B == 0) return hipSuccess;
  // one wave per SIMD of the chip (256 CUs x 4 SIMDs) per resident round, shared out over the kv heads
  const int per_head = max(kBalWaves, balanced_waves() / p.Hkv / kBalWaves * kBalWaves);
  const int grid = p.Hkv * (per_head / kBalWaves);
  if (p.append && p.kv_int8) return hipErrorInvalidValue;
  if (p.kv_int8)
    return p.kv_fp8 ? launch_q<true, true, false>(p, grid, stream) : launch_q<true, false, false>(p, grid, stream);
  return p.append ? launch_q<false, false, true>(p, grid, stream) : launch_q<false, false, false>(p, grid, stream);
}

}  // namespace pa
