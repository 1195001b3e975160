// Paged decode attention on the vector ALUs (gfx950, wave64).
//
// What is computed. For each query row (token t, head h) of a sequence of
// length L, scores s_p = scale * q . K[p] over the visible positions
// p <= L - T + t. K[p] and V[p] are read through the block table (physical
// block table[p / b], offset p % b). The result is o = sum_p softmax(s)_p V[p]
// ([P1] "25. Paged attention and prefix caching", section "Attention that
// reads through the table"; [P5] "Chapter 7 Paged KV Cache and Memory
// Management", sections 4.1-4.2). Softmax is online, per [P5] section 4.2: a
// running reference max m, a sum l and an accumulator acc that always share
// that reference, merged exactly at the end.
//
// Mapping onto the hardware. One workgroup of NW waves handles one
// (sequence, kv head, context partition, group of up to 8 query rows). All
// query rows of the GQA group share every K/V byte the workgroup loads. The
// partition's positions are cut into tiles of 16. A kv head's row is C
// 16-byte chunks: C = 8 (64 bf16), 16 (128 bf16 or 64 fp32) or 32 (128 fp32),
// so one tile of K is C KiB. Wave w takes tiles w, w + NW, ... and, while it
// computes tile i, its loads for the next tiles are already in flight. A
// tile's physical block id is a wave-uniform scalar load issued one tile
// before the K/V loads that need it, so the table lookup never sits on the
// critical path and never waits behind vector loads.
//  * K layout: lane = 4*ts + j holds token ts of the tile, 16-byte chunks
//    4*r + j (r = 0 .. C/4 - 1). Four adjacent lanes read 64 contiguous bytes.
//    q . k is C v_dot2_f32_bf16 per row (fp32: C FMAs), then a 2-step DPP
//    quad reduction.
//  * V layout: lane = C*R + cv holds chunk cv of tokens (C/4)*R + r. Each
//    lane accumulates a contiguous 8-element (bf16) or 4-element (fp32) slice
//    of head_dim for every row, so P.V needs no cross-lane reduction until
//    the end, where the 64/C lanes of a chunk add up. The probabilities move
//    from the K lanes to the V lanes through 16 * NR floats of LDS per wave.
//  * Lazy max: the reference max of a row is only raised when a score
//    exceeds it by more than 2^8 (base-2 units). That happens once per row in
//    practice, so the common path rescales nothing. acc and l stay within
//    fp32 range (p <= 256), and o = acc / l is unchanged because both share
//    the same reference ([P5] section 4.2).
//  * Masking: only tiles that reach past the fully visible prefix, and row
//    groups with absent rows, take the masked path. There, invisible scores
//    become -inf, and V chunks of positions >= L are zeroed before use, since
//    those slots may hold any bits (a 0 * NaN product would otherwise leak).
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kTile = 16;             // positions per wave tile
constexpr float kRescaleSlack = 8.0f; // lazy-max slack, base-2 exponent units

// Launch shape: waves per workgroup, tiles each wave keeps in flight ahead of
// the one it computes, q staged in LDS instead of registers, non-temporal K/V loads.
#ifndef PA_VALU_WAVES
#define PA_VALU_WAVES 4
#endif
#ifndef PA_VALU_PREFETCH
#define PA_VALU_PREFETCH 3
#endif
#ifndef PA_VALU_Q_IN_LDS
#define PA_VALU_Q_IN_LDS 1
#endif
#ifndef PA_VALU_NT_LOADS
#define PA_VALU_NT_LOADS 0
#endif
constexpr int kWaves = PA_VALU_WAVES;
constexpr int kPrefetch = PA_VALU_PREFETCH;
constexpr bool kQInLds = PA_VALU_Q_IN_LDS != 0;
constexpr bool kNtLoads = PA_VALU_NT_LOADS != 0;

template <bool BF16>
struct KvFmt {
  static constexpr int E = BF16 ? 8 : 4;  // elements per 16-byte chunk
};

// One tile held by a wave: C/4 K chunks (the lane's token) and C/4 V chunks (its chunk of C/4 tokens).
template <int KC>
struct Tile {
  u32x4 k[KC];
  u32x4 v[KC];
};

template <bool NT>
__device__ __forceinline__ u32x4 load_kv16(const char* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else
    return load16(p);
}

template <bool BF16, int C, int NR, int BS, int NW, int PF, bool QLDS, bool NT>
__global__ __launch_bounds__(NW * 64) void decode_valu_kernel(const DecodeParams p) {
  static_assert(C == 8 || C == 16 || C == 32, "a row is 8, 16 or 32 chunks of 16 bytes");
  constexpr int E = KvFmt<BF16>::E;
  constexpr int D = C * E;
  constexpr int RB = C * 16;                 // bytes of one kv head's K or V row (and of a q row)
  constexpr int KC = C / 4;                  // chunks per lane per tile, for K and for V
  constexpr int NPL = NR >= 4 ? NR / 4 : 1;  // rows each K lane turns into probabilities
  using TileT = Tile<KC>;

  __shared__ float p_lds[NW][kTile][NR];
  __shared__ u32x4 q_lds[QLDS ? NR : 1][C];
  __shared__ float red_acc[NW][NR][D];
  __shared__ float red_m[NW][NR];
  __shared__ float red_l[NW][NR];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Block id = ((seq * parts + part) * row_groups + rg) * Hkv + kvh: workgroups are dealt
  // round-robin to the 8 XCDs, so with Hkv = 8 every workgroup of one kv head shares an L2.
  int bid = blockIdx.x;
  const int kvh = bid % p.Hkv;
  bid /= p.Hkv;
  const int rg = bid % p.row_groups;
  bid /= p.row_groups;
  const int part = bid % p.parts;
  const int seq = bid / p.parts;

  const int L = p.seq_lens[seq];
  const int T = p.T;
  const int p_begin = part * p.part_tokens;
  if (p.partial && p_begin >= L) return;  // empty partition: the merge pass never reads it
  const int p_end = min(L, p_begin + p.part_tokens);
  const int ntiles = p_end > p_begin ? (p_end - p_begin + kTile - 1) / kTile : 0;
  const int vis_all = L - T + 1;  // positions below this are visible to every query row

  const int ts = lane >> 2, j = lane & 3;  // K lanes
  const int R = lane / C, cv = lane % C;   // V lanes: chunk cv of tokens KC*R .. KC*R + KC - 1

  // ---- query rows: row n of this group is global row rg*NR + n = t*G + g
  int row_lim[NR];  // last visible position; -1 for an absent row
  bool rows_all_present = true;
  u32x4 qv[QLDS ? 1 : NR][KC];
#pragma unroll
  for (int n = 0; n < NR; ++n) {
    const int r = rg * NR + n;
    row_lim[n] = r < p.rows ? L - T + r / p.G : -1;
    rows_all_present = rows_all_present && r < p.rows;
  }
  auto q_row_ptr = [&](int n) {
    const int r = rg * NR + n;
    return static_cast<const char*>(p.q) + ((int64_t)(seq * T + r / p.G) * p.Hq + kvh * p.G + r % p.G) * RB;
  };
  if constexpr (QLDS) {
    for (int idx = threadIdx.x; idx < NR * C; idx += NW * 64) {
      const int n = idx / C, c = idx % C;
      q_lds[n][c] = rg * NR + n < p.rows ? load16(q_row_ptr(n) + c * 16) : u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
  } else {
#pragma unroll
    for (int n = 0; n < NR; ++n) {
#pragma unroll
      for (int c = 0; c < KC; ++c)
        qv[QLDS ? 0 : n][c] = rg * NR + n < p.rows ? load16(q_row_ptr(n) + (c * 4 + j) * 16) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  auto q_chunk = [&](int n, int c) -> u32x4 {
    if constexpr (QLDS)
      return q_lds[n][c * 4 + j];
    else
      return qv[QLDS ? 0 : n][c];
  };

  const int32_t* trow = p.block_tables + (int64_t)seq * p.MB;
  const int64_t block_bytes = (int64_t)p.Hkv * BS * RB;
  const char* kbase = static_cast<const char*>(p.k_pool) + (int64_t)kvh * BS * RB;
  const char* vbase = static_cast<const char*>(p.v_pool) + (int64_t)kvh * BS * RB;
  const int my_tiles = wave < ntiles ? (ntiles - wave + NW - 1) / NW : 0;

  // Physical block of the wave's i-th tile when blocks hold >= 16 positions: a wave-uniform
  // index, so the lookup is a scalar load, fetched one tile ahead of the K/V loads that need it.
  auto phys_of = [&](int i) -> int { return trow[(p_begin + (wave + i * NW) * kTile) / BS]; };

  // A tile inside one block is read through a buffer descriptor built per tile in SGPRs plus a
  // lane offset that never changes, so its loads need no per-tile vector address arithmetic.
  const uint32_t k_lane_off = ts * RB + j * 16;        // + 64 * c
  const uint32_t v_lane_off = R * KC * RB + cv * 16;    // + RB * c
  auto load_tile = [&](int i, int phys32, TileT& tl) {
    const int tile_p0 = p_begin + (wave + i * NW) * kTile;
    if constexpr (BS >= kTile) {
      const int64_t off = (int64_t)phys32 * block_bytes + (int64_t)(tile_p0 % BS) * RB;
      const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(kbase + off, kTile * RB);
      const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(vbase + off, kTile * RB);
#pragma unroll
      for (int c = 0; c < KC; ++c) tl.k[c] = buffer_load16(kr, k_lane_off + c * 64);
#pragma unroll
      for (int c = 0; c < KC; ++c) tl.v[c] = buffer_load16(vr, v_lane_off + c * RB);
    } else {
      // Blocks shorter than a tile: each lane finds its own block. Positions past the
      // sequence are clamped to its last position (a valid slot), then masked.
      const int pk = min(tile_p0 + ts, L - 1);
      const char* kb = kbase + (int64_t)trow[pk / BS] * block_bytes + (int64_t)(pk % BS) * RB;
#pragma unroll
      for (int c = 0; c < KC; ++c) tl.k[c] = load_kv16<NT>(kb + (c * 4 + j) * 16);
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const int pv = min(tile_p0 + KC * R + c, L - 1);
        tl.v[c] = load_kv16<NT>(vbase + (int64_t)trow[pv / BS] * block_bytes + (int64_t)(pv % BS) * RB + cv * 16);
      }
    }
  };

  float m_ref[NR];
  float l_part[NPL];
  float acc[NR][E];
#pragma unroll
  for (int n = 0; n < NR; ++n) {
    m_ref[n] = kNegInf;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[n][e] = 0.f;
  }
#pragma unroll
  for (int nl = 0; nl < NPL; ++nl) l_part[nl] = 0.f;

  auto row_of = [&](int nl) { return NR >= 4 ? nl * 4 + j : j; };

  auto compute_tile = [&](auto masked_tag, int i, const TileT& tl) {
    constexpr bool masked = decltype(masked_tag)::value;
    const int tile_p0 = p_begin + (wave + i * NW) * kTile;

    // ---- scores of token ts for every row (all four lanes of the quad end up with them)
    float s[NR];
#pragma unroll
    for (int n = 0; n < NR; ++n) {
      float a = 0.f;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const u32x4 qc = q_chunk(n, c);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if constexpr (BF16)
            a = dot2_bf16(qc[w], tl.k[c][w], a);
          else
            a = fmaf(__uint_as_float(qc[w]), __uint_as_float(tl.k[c][w]), a);
        }
      }
      a += quad_xor1(a);
      a += quad_xor2(a);
      s[n] = a * p.qk_scale_log2;
    }
    if constexpr (masked) {
      const int pk = tile_p0 + ts;
#pragma unroll
      for (int n = 0; n < NR; ++n)
        if (pk > row_lim[n]) s[n] = kNegInf;
    }

    // ---- lazy reference max (wave-uniform per row)
    bool over = false;
#pragma unroll
    for (int n = 0; n < NR; ++n) over |= s[n] > m_ref[n] + kRescaleSlack;
    if (__builtin_expect(__any(over), 0)) {
#pragma unroll
      for (int n = 0; n < NR; ++n) {
        const float m_new = fmaxf(m_ref[n], wave_max(s[n]));
        if (m_new > m_ref[n]) {
          const float alpha = exp2_fast(m_ref[n] - m_new);  // 0 when m_ref was -inf
#pragma unroll
          for (int e = 0; e < E; ++e) acc[n][e] *= alpha;
#pragma unroll
          for (int nl = 0; nl < NPL; ++nl)
            if (row_of(nl) == n) l_part[nl] *= alpha;
          m_ref[n] = m_new;
        }
      }
    }

    // ---- probabilities of this lane's rows, handed to the V lanes through LDS
#pragma unroll
    for (int nl = 0; nl < NPL; ++nl) {
      constexpr int kSel = NR >= 4 ? 4 : NR;
      float x = s[NR >= 4 ? nl * 4 : 0];
      float m = m_ref[NR >= 4 ? nl * 4 : 0];
#pragma unroll
      for (int jj = 1; jj < kSel; ++jj) {
        if (j == jj) {
          x = s[(NR >= 4 ? nl * 4 : 0) + jj];
          m = m_ref[(NR >= 4 ? nl * 4 : 0) + jj];
        }
      }
      float pr = x == kNegInf ? 0.f : exp2_fast(x - m);
      if (NR < 4 && j >= NR) pr = 0.f;
      l_part[nl] += pr;
      if (NR >= 4 || j < NR) p_lds[wave][ts][row_of(nl)] = pr;
    }
    // One wave writes and reads its own LDS slice; its LDS operations execute in order.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- P.V on this lane's head_dim slice
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      float pv[NR];
#pragma unroll
      for (int n = 0; n < NR; ++n) pv[n] = p_lds[wave][KC * R + c][n];
      u32x4 v = tl.v[c];
      if constexpr (masked) {
        if (tile_p0 + KC * R + c >= L) v = u32x4{0u, 0u, 0u, 0u};
      }
      float vf[E];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if constexpr (BF16) {
          vf[2 * w] = bf16_lo(v[w]);
          vf[2 * w + 1] = bf16_hi(v[w]);
        } else {
          vf[w] = __uint_as_float(v[w]);
        }
      }
#pragma unroll
      for (int n = 0; n < NR; ++n)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[n][e] = fmaf(pv[n], vf[e], acc[n][e]);
    }
  };

  // ---- tile loop: a ring of PF + 1 register tiles, so tiles i+1 .. i+PF load while tile i computes.
  // Every iteration issues its prefetch unconditionally (past the end it re-reads the wave's last
  // tile, a cache hit that is never used), so the number of loads in flight is the same on every
  // path and the wait before each compute leaves the prefetched tiles outstanding.
  if (my_tiles > 0) {
    const int last = my_tiles - 1;
    TileT ring[PF + 1];
#pragma unroll
    for (int u = 0; u < PF; ++u) load_tile(min(u, last), BS >= kTile ? phys_of(min(u, last)) : 0, ring[u]);
    int phys_next = BS >= kTile ? phys_of(min(PF, last)) : 0;
    for (int i0 = 0; i0 < my_tiles; i0 += PF + 1) {
#pragma unroll
      for (int u = 0; u <= PF; ++u) {
        const int i = i0 + u;
        if (i < my_tiles) {
          const int ph = phys_next;
          if (BS >= kTile) phys_next = phys_of(min(i + PF + 1, last));
          load_tile(min(i + PF, last), ph, ring[(u + PF) % (PF + 1)]);
          const int tile_p0 = p_begin + (wave + i * NW) * kTile;
          if (!rows_all_present || tile_p0 + kTile > vis_all)
            compute_tile(std::true_type{}, i, ring[u]);
          else
            compute_tile(std::false_type{}, i, ring[u]);
        }
      }
    }
  }

  // ---- merge the 64/C V-lane groups, then the waves, then write out or emit the partial
#pragma unroll
  for (int n = 0; n < NR; ++n)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float a = acc[n][e];
#pragma unroll
      for (int m = C; m < 64; m <<= 1) a += __shfl_xor(a, m, 64);
      acc[n][e] = a;
    }
#pragma unroll
  for (int nl = 0; nl < NPL; ++nl) {
    float l = l_part[nl];
    l += __shfl_xor(l, 4, 64);
    l += __shfl_xor(l, 8, 64);
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (ts == 0 && (NR >= 4 || j < NR)) red_l[wave][row_of(nl)] = l;
  }
  if (lane == 0) {
#pragma unroll
    for (int n = 0; n < NR; ++n) red_m[wave][n] = m_ref[n];
  }
  if (R == 0) {
#pragma unroll
    for (int n = 0; n < NR; ++n)
#pragma unroll
      for (int e = 0; e < E; ++e) red_acc[wave][n][cv * E + e] = acc[n][e];
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < NR * D; idx += NW * 64) {
    const int n = idx / D, d = idx % D;
    const int r = rg * NR + n;
    if (r >= p.rows) continue;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, red_m[w][n]);
    float lsum = 0.f, a = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = red_m[w][n];
        if (mw != kNegInf) {
          const float sc = exp2_fast(mw - M);
          lsum = fmaf(sc, red_l[w][n], lsum);
          a = fmaf(sc, red_acc[w][n][d], a);
        }
      }
    }
    const int t = r / p.G, g = r % p.G;
    const int64_t orow = (int64_t)(seq * T + t) * p.Hq + kvh * p.G + g;
    if (p.partial) {
      const int64_t pi = orow * p.parts + part;
      p.part_acc[pi * D + d] = a;
      if (d == 0) {
        p.part_ml[pi * 2] = M;
        p.part_ml[pi * 2 + 1] = lsum;
      }
    } else {
      const float o = lsum > 0.f ? a / lsum : 0.f;
      if (p.out_dtype == PA_F32)
        static_cast<float*>(p.out)[orow * D + d] = o;
      else
        static_cast<uint16_t*>(p.out)[orow * D + d] = f32_to_bf16(o);
    }
  }
}

// Tiles kept in flight ahead of the one being computed: a 32-chunk row (fp32, head_dim 128) makes
// a tile 64 VGPRs per lane, so its ring keeps one tile ahead to stay at two waves per SIMD.
template <int C>
constexpr int prefetch_for() {
  return C == 32 ? 1 : kPrefetch;
}

template <bool BF16, int C, int NR, int BS>
hipError_t launch_t(const DecodeParams& p, hipStream_t stream) {
  const int64_t grid = (int64_t)p.B * p.parts * p.row_groups * p.Hkv;
  if (grid == 0) return hipSuccess;
  decode_valu_kernel<BF16, C, NR, BS, kWaves, prefetch_for<C>(), kQInLds, kNtLoads>
      <<<dim3((unsigned)grid), dim3(kWaves * 64), 0, stream>>>(p);
  return hipGetLastError();
}

template <bool BF16, int C, int NR>
hipError_t launch_bs(const DecodeParams& p, hipStream_t stream) {
  switch (p.block_size) {
    case 4: return launch_t<BF16, C, NR, 4>(p, stream);
    case 8: return launch_t<BF16, C, NR, 8>(p, stream);
    case 16: return launch_t<BF16, C, NR, 16>(p, stream);
    case 32: return launch_t<BF16, C, NR, 32>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool BF16, int C>
hipError_t launch_nr(const DecodeParams& p, hipStream_t stream) {
  switch (valu_rows_per_group(p.rows)) {
    case 1: return launch_bs<BF16, C, 1>(p, stream);
    case 2: return launch_bs<BF16, C, 2>(p, stream);
    case 4: return launch_bs<BF16, C, 4>(p, stream);
    default: return launch_bs<BF16, C, 8>(p, stream);
  }
}

}  // namespace

int valu_rows_per_group(int rows) {
  if (rows >= 8) return 8;
  int nr = 1;
  while (nr < rows) nr *= 2;
  return nr;
}

bool valu_supported(const pa_dims& d) {
  const bool dtype = d.kv_dtype == PA_BF16 || d.kv_dtype == PA_F32;
  const bool head = d.head_dim == 64 || d.head_dim == 128;
  const bool block = d.block_size == 4 || d.block_size == 8 || d.block_size == 16 || d.block_size == 32;
  return dtype && head && block && d.q_dtype == d.kv_dtype;
}

hipError_t launch_decode_valu(const DecodeParams& p, int kv_dtype, hipStream_t stream) {
  if (kv_dtype == PA_BF16) return p.D == 64 ? launch_nr<true, 8>(p, stream) : launch_nr<true, 16>(p, stream);
  return p.D == 64 ? launch_nr<false, 16>(p, stream) : launch_nr<false, 32>(p, stream);
}

}  // namespace pa
