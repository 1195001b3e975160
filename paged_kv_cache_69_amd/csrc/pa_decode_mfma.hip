// Paged decode attention on the matrix cores (gfx950 MFMA), bf16 K/V, head_dim 128.
//
// It computes exactly what the vector-ALU kernel computes (and what [P1] "25.
// Paged attention and prefix caching", section "Attention that reads through
// the table", and [P5] "Chapter 7 Paged KV Cache and Memory Management",
// sections 4.1-4.2 define): for each query row (token t, head h), softmax over
// the visible positions p <= L - T + t of scale * q . K[p], applied to V[p],
// with K/V gathered through the block table. It differs only in how the
// arithmetic is issued. The query rows of one kv head (T*G of them, padded to
// 16 or 32) become the N (q.k) and M (P.V) dimension of
// v_mfma_f32_16x16x32_bf16, so the vector ALU is left with the softmax alone.
//
// Per wave, positions are consumed in pairs of 16-position tiles (32
// positions, the K dimension of one P.V MFMA):
//  * S^T = K Q^T: the K tile is the A operand, loaded straight from the pool
//    (lane l: position l%16 of the tile, 16 bytes at head_dim 32*kc + 8*(l/16)).
//    q is the B operand, held in registers for the whole partition. Four
//    MFMAs per tile cover head_dim 128. The C layout leaves lane l with
//    positions 4*(l/16) + i of row l%16.
//  * Softmax: scaled scores in base-2 units, a lazy reference max per row
//    (raised only when a score exceeds it by more than 2^8), p = 2^(x - m).
//  * P.V: the C layout above is already the A-operand layout of P (row l%16,
//    8 positions). P is split into bf16 hi + lo parts, so P.V keeps about 16
//    mantissa bits of p, and each part gets its own MFMA. V goes through LDS:
//    the tile is written in its natural [position][head_dim] layout (32-byte
//    blocks XOR-swizzled by position to spread banks), and two
//    ds_read_b64_tr_b16 per 16-column block return 8 positions of one column
//    per lane, which is the B operand.
// Masked tail tiles (positions >= L, causal limits for T > 1, or a phantom
// second tile past the partition) select -inf scores and zero V before use,
// so garbage in unwritten slots can never reach the result.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kTile = 16;
constexpr int kRowBytes = 256;  // 128 bf16
constexpr int kD = 128;
constexpr float kRescaleSlack = 8.0f;
constexpr int kPairChunk = 32;  // tile pairs whose block ids one table fetch covers

#ifndef PA_MFMA_WAVES
#define PA_MFMA_WAVES 4
#endif
constexpr int kMfmaWaves = PA_MFMA_WAVES;

struct PairRegs {
  u32x4 k[2][4];  // A operands of S^T for the two tiles
  u32x4 v[2][4];  // V tiles, 16 bytes per lane per 1 KiB
};

// Byte offset of (position t of the pair, byte b of its 256-byte row) in a wave's V buffer.
__device__ __forceinline__ int v_lds_offset(int t, int b) { return t * kRowBytes + (b ^ ((t & 7) << 5)); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Round-to-nearest-even fp32 -> bf16 pair packing, and the residual x - bf16(x).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

template <int MT, int BS, int NW>
__global__ __launch_bounds__(NW * 64) void decode_mfma_kernel(const DecodeParams p) {
  constexpr int ROWS = 16 * MT;
  constexpr int kVBytes = 2 * kTile * kRowBytes;                  // one pair of V tiles per wave
  constexpr int kRedBytes = (NW * ROWS * kD + 2 * NW * ROWS) * 4;  // end-of-kernel merge buffers
  constexpr int kLdsBytes = (NW * kVBytes > kRedBytes) ? NW * kVBytes : kRedBytes;
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;    // 16-lane group: k slice of the MFMA operands
  const int c16 = lane & 15;  // column inside the group

  int bid = blockIdx.x;  // ((seq * parts + part) * Hkv + kvh)
  const int kvh = bid % p.Hkv;
  bid /= p.Hkv;
  const int part = bid % p.parts;
  const int seq = bid / p.parts;

  const int L = p.seq_lens[seq];
  const int T = p.T;
  const int p_begin = part * p.part_tokens;
  if (p.partial && p_begin >= L) return;
  const int p_end = min(L, p_begin + p.part_tokens);
  const int ntiles = p_end > p_begin ? (p_end - p_begin + kTile - 1) / kTile : 0;
  const int npairs = (ntiles + 1) >> 1;
  const int vis_all = L - T + 1;
  const bool rows_all_present = p.rows == ROWS;

  // ---- q rows as the B operand of S^T: lane (g, c16) holds row c16 + 16*mt, head_dim 32*kc + 8g .. +7
  u32x4 qb[MT][4];
  int row_lim[MT];  // last visible position of this lane's score row; -1 if absent
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = mt * 16 + c16;
    const bool present = r < p.rows;
    row_lim[mt] = present ? L - T + r / p.G : -1;
    const char* qrow = static_cast<const char*>(p.q) +
                       ((int64_t)(seq * T + (present ? r / p.G : 0)) * p.Hq + kvh * p.G + (present ? r % p.G : 0)) *
                           kRowBytes;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) qb[mt][kc] = present ? load16(qrow + (kc * 4 + g) * 16) : u32x4{0u, 0u, 0u, 0u};
  }

  const int32_t* trow = p.block_tables + (int64_t)seq * p.MB;
  const int64_t block_bytes = (int64_t)p.Hkv * BS * kRowBytes;
  const char* kbase = static_cast<const char*>(p.k_pool) + (int64_t)kvh * BS * kRowBytes;
  const char* vbase = static_cast<const char*>(p.v_pool) + (int64_t)kvh * BS * kRowBytes;
  const int my_pairs = wave < npairs ? (npairs - wave + NW - 1) / NW : 0;
  char* vbuf = lds + wave * kVBytes;

  // Block ids: lane 2*i + h of tab_v holds tile h of the wave's (tab_base + i)-th pair.
  int tab_base = 0;
  int tab_v = 0;
  auto refill_table = [&](int base) {
    tab_base = base;
    const int pair = wave + (base + (lane >> 1)) * NW;
    const int tile = 2 * pair + (lane & 1);
    tab_v = 0;
    if ((base + (lane >> 1)) < my_pairs && tile < ntiles) tab_v = trow[(p_begin + tile * kTile) / BS];
  };

  auto load_pair = [&](int i, PairRegs& pr) {
    const int pair = wave + i * NW;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int tile = 2 * pair + h;
      if (tile < ntiles) {  // uniform
        const int tile_p0 = p_begin + tile * kTile;
        if constexpr (BS >= kTile) {
          const int64_t phys = __builtin_amdgcn_readlane(tab_v, 2 * (i - tab_base) + h);
          const int64_t off = phys * block_bytes + (int64_t)(tile_p0 % BS) * kRowBytes;
#pragma unroll
          for (int kc = 0; kc < 4; ++kc) pr.k[h][kc] = load16(kbase + off + c16 * kRowBytes + (kc * 4 + g) * 16);
#pragma unroll
          for (int c = 0; c < 4; ++c) pr.v[h][c] = load16(vbase + off + c * 1024 + lane * 16);
        } else {
          const int pk = min(tile_p0 + c16, L - 1);
          const char* kb = kbase + (int64_t)trow[pk / BS] * block_bytes + (int64_t)(pk % BS) * kRowBytes;
#pragma unroll
          for (int kc = 0; kc < 4; ++kc) pr.k[h][kc] = load16(kb + (kc * 4 + g) * 16);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int pv = min(tile_p0 + c * 4 + (lane >> 4), L - 1);
            pr.v[h][c] = load16(vbase + (int64_t)trow[pv / BS] * block_bytes + (int64_t)(pv % BS) * kRowBytes +
                                (lane & 15) * 16);
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          pr.k[h][c] = u32x4{0u, 0u, 0u, 0u};
          pr.v[h][c] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  };

  float m_ref[MT];      // reference max of this lane's score row (row c16 + 16*mt)
  float l_part[MT];     // sum of p over the positions this lane has seen for that row
  f32x4 acc[MT][8];     // P.V: rows 4g + i (+16*mt), head_dim 16*j + c16
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    m_ref[mt] = kNegInf;
    l_part[mt] = 0.f;
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) acc[mt][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto compute_pair = [&](int i, const PairRegs& pr) {
    const int pair = wave + i * NW;
    const int pair_p0 = p_begin + pair * 2 * kTile;
    const bool masked = !rows_all_present || pair_p0 + 2 * kTile > vis_all || 2 * pair + 1 >= ntiles;

    // ---- S^T for both tiles (C layout: lane l has positions 4g + e of score row c16 + 16*mt)
    f32x4 s[2][MT];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(pr.k[h][kc]), as_bf16x8(qb[mt][kc]), c, 0, 0, 0);
        s[h][mt] = c * p.qk_scale_log2;
      }
    if (masked) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bool tile_ok = 2 * pair + h < ntiles;
        const int pos0 = pair_p0 + h * kTile + 4 * g;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (!tile_ok || pos0 + e > row_lim[mt]) s[h][mt][e] = kNegInf;
      }
    }

    // ---- lazy reference max per row
    bool over = false;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) over |= s[h][mt][e] > m_ref[mt] + kRescaleSlack;
    if (__builtin_expect(__any(over), 0)) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        float mx = m_ref[mt];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) mx = fmaxf(mx, s[h][mt][e]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // this lane's row changes reference: alpha = 2^(old - new) (0 from -inf, 1 when unchanged)
        const float alpha = mx == kNegInf ? 1.f : exp2_fast(m_ref[mt] - mx);
        l_part[mt] *= alpha;
        m_ref[mt] = mx;
        // acc rows 4g + e belong to score rows held by lanes c16 = 4g + e
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a_row = __shfl(alpha, 4 * g + e, 64);
#pragma unroll
          for (int jb = 0; jb < 8; ++jb) acc[mt][jb][e] *= a_row;
        }
      }
    }

    // ---- probabilities, split into bf16 hi + lo A operands of P.V
    u32x4 p_hi[MT], p_lo[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float pv[8];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = s[h][mt][e];
          const float pe = x == kNegInf ? 0.f : exp2_fast(x - m_ref[mt]);
          pv[h * 4 + e] = pe;
          l_part[mt] += pe;
        }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t hi = pack_bf16x2(pv[2 * w], pv[2 * w + 1]);
        p_hi[mt][w] = hi;
        p_lo[mt][w] = pack_bf16x2(pv[2 * w] - bf16_lo(hi), pv[2 * w + 1] - bf16_hi(hi));
      }
    }

    // ---- V pair into this wave's LDS buffer (zero where the position is not readable)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int t = h * kTile + c * 4 + (lane >> 4);
        u32x4 v = pr.v[h][c];
        if (masked && (2 * pair + h >= ntiles || pair_p0 + t >= L)) v = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(vbuf + v_lds_offset(t, (lane & 15) * 16)) = v;
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- P.V: B operand = 8 positions of head_dim column 16*jb + c16, via two transpose reads
    const int rr = (lane >> 2) & 3, qq = lane & 3;
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) {
      const int col_b = (16 * jb + 4 * qq) * 2;
      const s16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)((__attribute__((address_space(3))) char*)vbuf + v_lds_offset(4 * g + rr, col_b)));
      const s16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)((__attribute__((address_space(3))) char*)vbuf + v_lds_offset(kTile + 4 * g + rr, col_b)));
      const u32x4 bv = {__builtin_bit_cast(uint32_t, __builtin_shufflevector(b0, b0, 0, 1)),
                        __builtin_bit_cast(uint32_t, __builtin_shufflevector(b0, b0, 2, 3)),
                        __builtin_bit_cast(uint32_t, __builtin_shufflevector(b1, b1, 0, 1)),
                        __builtin_bit_cast(uint32_t, __builtin_shufflevector(b1, b1, 2, 3))};
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc[mt][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(p_hi[mt]), as_bf16x8(bv), acc[mt][jb], 0, 0, 0);
        acc[mt][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(p_lo[mt]), as_bf16x8(bv), acc[mt][jb], 0, 0, 0);
      }
    }
  };

  for (int chunk0 = 0; chunk0 < my_pairs; chunk0 += kPairChunk) {
    const int n_here = min(kPairChunk, my_pairs - chunk0);
    if constexpr (BS >= kTile) refill_table(chunk0);
    PairRegs ring[2];
    load_pair(chunk0, ring[0]);
    for (int i0 = 0; i0 < n_here; i0 += 2) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = i0 + u;
        if (i < n_here) {
          if (i + 1 < n_here) load_pair(chunk0 + i + 1, ring[u ^ 1]);
          compute_pair(chunk0 + i, ring[u]);
        }
      }
    }
  }

  // ---- merge: per-row (m, l) of each wave, then P.V accumulators across waves
  __syncthreads();  // every wave is done with its V buffer before the merge reuses the LDS
  float* red_acc = reinterpret_cast<float*>(lds);  // [NW][ROWS][kD]
  float* red_m = red_acc + NW * ROWS * kD;         // [NW][ROWS]
  float* red_l = red_m + NW * ROWS;                // [NW][ROWS]
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    float l = l_part[mt];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (g == 0) {
      red_l[wave * ROWS + mt * 16 + c16] = l;
      red_m[wave * ROWS + mt * 16 + c16] = m_ref[mt];
    }
#pragma unroll
    for (int jb = 0; jb < 8; ++jb)
#pragma unroll
      for (int e = 0; e < 4; ++e) red_acc[(wave * ROWS + mt * 16 + 4 * g + e) * kD + 16 * jb + c16] = acc[mt][jb][e];
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < ROWS * kD; idx += NW * 64) {
    const int n = idx / kD, d = idx % kD;
    if (n >= p.rows) continue;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, red_m[w * ROWS + n]);
    float lsum = 0.f, a = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = red_m[w * ROWS + n];
        if (mw != kNegInf) {
          const float sc = exp2_fast(mw - M);
          lsum = fmaf(sc, red_l[w * ROWS + n], lsum);
          a = fmaf(sc, red_acc[(w * ROWS + n) * kD + d], a);
        }
      }
    }
    const int t = n / p.G, gq = n % p.G;
    const int64_t orow = (int64_t)(seq * T + t) * p.Hq + kvh * p.G + gq;
    if (p.partial) {
      const int64_t pi = orow * p.parts + part;
      p.part_acc[pi * kD + d] = a;
      if (d == 0) {
        p.part_ml[pi * 2] = M;
        p.part_ml[pi * 2 + 1] = lsum;
      }
    } else {
      const float o = lsum > 0.f ? a / lsum : 0.f;
      if (p.out_dtype == PA_F32)
        static_cast<float*>(p.out)[orow * kD + d] = o;
      else
        static_cast<uint16_t*>(p.out)[orow * kD + d] = f32_to_bf16(o);
    }
  }
}

template <int MT, int BS>
hipError_t launch_t(const DecodeParams& p, hipStream_t stream) {
  const int64_t grid = (int64_t)p.B * p.parts * p.Hkv;
  if (grid == 0) return hipSuccess;
  decode_mfma_kernel<MT, BS, kMfmaWaves><<<dim3((unsigned)grid), dim3(kMfmaWaves * 64), 0, stream>>>(p);
  return hipGetLastError();
}

template <int MT>
hipError_t launch_bs(const DecodeParams& p, hipStream_t stream) {
  switch (p.block_size) {
    case 4: return launch_t<MT, 4>(p, stream);
    case 8: return launch_t<MT, 8>(p, stream);
    case 16: return launch_t<MT, 16>(p, stream);
    case 32: return launch_t<MT, 32>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool mfma_supported(const pa_dims& d) {
  const int rows = d.q_tokens * (d.num_q_heads / d.num_kv_heads);
  const bool block = d.block_size == 4 || d.block_size == 8 || d.block_size == 16 || d.block_size == 32;
  return d.kv_dtype == PA_BF16 && d.q_dtype == PA_BF16 && d.head_dim == kD && block && rows <= 32;
}

hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t stream) {
  return p.rows <= 16 ? launch_bs<1>(p, stream) : launch_bs<2>(p, stream);
}

}  // namespace pa
