// Paged prefill on the matrix cores (gfx950 MFMA), bf16 K/V, head_dim 128.
//
// What it computes ([P1] "25. Paged attention and prefix caching", stretch
// exercise 4; [P4] "Prefill vs decode under paging"; [P5] "Chapter 7 Paged KV
// Cache and Memory Management" section 4.1): sequence i brings a chunk of n_i
// new query tokens, packed as rows q_start[i] .. q_start[i+1]-1 of q, which
// are its newest positions L_i - n_i .. L_i - 1. Token j, query head h,
// attends causally to positions 0 .. L_i - n_i + j of kv head h / G: the
// sequence's paged history and the chunk itself, gathered through the block
// table (the chunk's K/V rows are already in the pools).
//
// Unlike decode, this is a dense contraction: a workgroup takes 128 query rows
// (floor(128 / G) tokens x the G heads that share one kv head) of one
// sequence, and every K/V row it reads serves all of them. Design:
//  * Workgroup = 4 waves x 32 query rows; row r is token r / G, head r % G.
//    q rows are the resident B operand of S^T = K Q^T, as in the decode
//    kernel.
//  * Positions go in tiles of 32. The whole workgroup loads a tile's K and V
//    (8 KiB each) from the pool straight into LDS, two tiles ahead of the one
//    whose scores are computed (four buffers, one barrier per tile). Each
//    thread loads 16-byte chunks of two positions; the block ids come from the
//    table one step before the loads are issued, and for b < 16 a lane picks
//    its own position's block, so any block size works.
//  * The LDS operand reads of a tile run one stretch of work ahead of the
//    MFMAs that use them (the next tile's K and half of this tile's V behind
//    the softmax, the other half of V behind the scores), kept there by
//    scheduling fences: the matrix cores otherwise wait on LDS latency.
//  * K sits in LDS as [position][256 B] with its 16-byte chunks XOR-swizzled
//    by position, so the A operand reads (16 positions x the same chunk) hit
//    16 different bank groups.
//  * P.V: the C layout of the two 16-position halves of S^T gives a lane
//    positions 4g .. 4g+3 of each half; taken together they are the 8 k-slots
//    of one v_mfma_f32_16x16x32_bf16 A operand, and the matching B operand is
//    two transposed LDS reads (ds_read_b64_tr_b16) of V, one per half. P goes
//    in as bf16 hi + lo parts, as in the decode kernel.
//  * Online softmax with a lazy reference ([P5] section 4.2): each row keeps a
//    reference max; a tile whose score exceeds it by more than 2^64 (base-2
//    units) raises it and rescales that wave's accumulators once. Otherwise
//    the accumulators are only touched by MFMAs.
//  * Causal mask by selection (-inf, never computed), only in the tiles that
//    cross a row's limit; V rows at or past L are zeroed in LDS, so garbage in
//    unwritten slots never reaches the result.
//  * Consecutive workgroups are consecutive kv heads, so with 8 kv heads all
//    workgroups of one kv head run on one XCD; along the grid, one sequence's
//    query blocks (last block first: the longest rows) come before the next
//    sequence's, so the workgroups an XCD holds at a time read the K/V of one
//    or two sequences, which stays in its L2.
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr int kD = 128;
constexpr int kRowBytes = 256;          // one bf16 row of head_dim 128
constexpr int kNW = 4;                  // waves per workgroup
constexpr int kWaveRows = 32;           // query rows per wave (two 16-row MFMA tiles)
constexpr int kWgRows = kNW * kWaveRows;
constexpr int kKT = 32;                 // positions per K/V tile
constexpr int kKBytes = kKT * kRowBytes;  // 8 KiB of K (or V) per tile
constexpr int kBufBytes = 2 * kKBytes;    // K then V
constexpr float kSlack = 64.0f;

struct PrefillParams {
  const char* q;
  const char* k_pool;
  const char* v_pool;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* q_start;
  void* out;
  float qk_scale_log2;
  int32_t B, Hq, Hkv, G, MB, num_blocks, out_dtype;
  int32_t qb_tokens;  // query tokens per workgroup: floor(128 / G)
  int32_t n_qblocks;  // query blocks of the longest chunk
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Largest of eight scores (IEEE maximum: v_maximum3_f32, no canonicalising moves; a NaN would
// propagate, and then fails every comparison).
__device__ __forceinline__ float max8(const f32x4& a, const f32x4& b) {
  const float x = __builtin_elementwise_maximum(__builtin_elementwise_maximum(a[0], a[1]), a[2]);
  const float y = __builtin_elementwise_maximum(__builtin_elementwise_maximum(a[3], b[0]), b[1]);
  const float z = __builtin_elementwise_maximum(__builtin_elementwise_maximum(b[2], b[3]), x);
  return __builtin_elementwise_maximum(y, z);
}

typedef __attribute__((address_space(3))) void lds_void;

// A row of zeros in global memory: the source of tile rows at or past a sequence's length.
__device__ __attribute__((aligned(16))) const char kZeroRow[kRowBytes] = {};

// Wait until at most N vector-memory operations of this wave are outstanding (vmcnt only).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Keeps the compiler's scheduler from moving any instruction across it: the LDS operand reads of the
// tile loop then stay one stretch of work ahead of the MFMAs that consume them (left to itself, the
// scheduler moves each read down to its first use, and the MFMA waits for the LDS).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Workgroup barrier with no implied wait for outstanding memory operations; the memory clobber keeps
// the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// V tile half (16 positions x 256 B): 32-byte blocks XOR-swizzled by position, as the transposed
// reads expect.
__device__ __forceinline__ int v_swz(int t, int byte) { return t * kRowBytes + (byte ^ ((t & 7) << 5)); }
// K tile (32 positions x 256 B): 16-byte chunk c of position t at chunk c ^ (t % 16).
__device__ __forceinline__ int k_swz(int t, int chunk) { return t * kRowBytes + ((chunk ^ (t & 15)) << 4); }

template <int BS>
__global__ __launch_bounds__(kNW * 64) void prefill_mfma_kernel(const PrefillParams p) {
  // four tile buffers, separate LDS objects: the compiler then tracks the direct-to-LDS loads into
  // each one apart and does not wait for all of them before reading any buffer
  __shared__ __attribute__((aligned(16))) char lds0[kBufBytes];
  __shared__ __attribute__((aligned(16))) char lds1[kBufBytes];
  __shared__ __attribute__((aligned(16))) char lds2[kBufBytes];
  __shared__ __attribute__((aligned(16))) char lds3[kBufBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;

  int bid = blockIdx.x;
  const int kvh = bid % p.Hkv;
  bid /= p.Hkv;
  const int qblk = p.n_qblocks - 1 - bid % p.n_qblocks;  // a sequence's longest rows first
  const int seq = bid / p.n_qblocks;

  const int q0 = p.q_start[seq];
  const int n = p.q_start[seq + 1] - q0;
  const int QB = p.qb_tokens, G = p.G;
  const int tok0 = qblk * QB;
  if (tok0 >= n) return;  // the whole workgroup: this sequence's chunk is shorter
  const int L = p.seq_lens[seq];
  const int hist = L - n;
  const int tok_end = min(n, tok0 + QB);

  // ---- this lane's query rows (score layout: row c16 + 16 mt of the wave)
  int row_lim[2];  // last visible position of the row; -1 for padding rows
  u32x4 qb[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int r = wave * kWaveRows + mt * 16 + c16;
    const int tr = r / G;
    const bool present = r < QB * G && tok0 + tr < tok_end;
    row_lim[mt] = present ? hist + tok0 + tr : -1;
    const int64_t qrow = present ? (int64_t)(q0 + tok0 + tr) * p.Hq + kvh * G + r % G : (int64_t)q0 * p.Hq;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const u32x4 v = load16(p.q + qrow * kRowBytes + (kc * 4 + g) * 16);
      qb[mt][kc] = present ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // the wave's rows: tokens tok0 + w*32/G .. ; lowest and highest visible limits
  const int w_first = wave * kWaveRows;
  const int w_last_tok = min(min((w_first + kWaveRows - 1) / G, QB - 1), tok_end - 1 - tok0);
  const bool wave_rows = w_first < QB * G && tok0 + w_first / G < tok_end;
  const int wave_lo = hist + tok0 + w_first / G;
  const int wave_hi = wave_rows ? hist + tok0 + w_last_tok : -1;

  const int ntiles = (hist + tok_end + kKT - 1) / kKT;

  // ---- tile loads, straight from the pools into LDS (global_load_lds_dwordx4: lane l of one
  // instruction fills bytes 16 l .. 16 l + 15 of a 1 KiB slot). A tile buffer is 16 slots: K rows 0-31
  // (4 per slot, K layout), then V halves 0 and 1 (4 rows per slot, V layout). Wave w fills K slots
  // w and 4 + w and V slots 8 + w and 12 + w: rows 4w .. 4w + 3 of each 16-position half. Each lane
  // picks the source chunk that its LDS chunk holds under the swizzle; positions at or past L read a
  // row of zeros instead of the pool (unwritten slots may hold anything).
  // The table is read through the constant address space: its wave-uniform lookups become scalar
  // loads (counted by lgkmcnt), so waiting for one never waits for the tile loads in flight.
  const __attribute__((address_space(4))) int32_t* trow =
      (const __attribute__((address_space(4))) int32_t*)(p.block_tables + (int64_t)seq * p.MB);
  const int64_t block_bytes = (int64_t)p.Hkv * BS * kRowBytes;
  const char* kbase = p.k_pool + (int64_t)kvh * BS * kRowBytes;
  const char* vbase = p.v_pool + (int64_t)kvh * BS * kRowBytes;
  const int tq = 4 * wave + (lane >> 4);                // row inside a 16-position half
  const int lc_k = (lane & 15) ^ (tq & 15);              // K chunk this lane's LDS chunk holds
  const int lc_v = (lane & 15) ^ ((tq & 7) << 1);        // V chunk (32-byte blocks swizzled)
  constexpr int kHalfBlocks = BS >= 16 ? 1 : 16 / BS;    // blocks one half spans
  const uint32_t lane_k = (uint32_t)(tq * kRowBytes + lc_k * 16);  // this lane's chunk within a half
  const uint32_t lane_v = (uint32_t)(tq * kRowBytes + lc_v * 16);
  // Block ids of a tile's two 16-position halves (b >= 16), read one step before the tile's loads
  // are issued so that the issue does not wait for the table; the index is clamped to the table row.
  auto fetch_blocks = [&](int tile, int (&nb)[2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      nb[h] = trow[min((tile * kKT + 16 * h) / BS, p.MB - 1)];  // clamped to the pool where used
  };
  auto issue = [&](lds_char* buf, int tile, const int (&nb)[2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int p0 = tile * kKT + 16 * h;
      // block of this lane's row (scalar table loads; a lane selects among them for b < 16)
      int64_t row_off;
      if constexpr (BS >= 16) {
        const int blk = (int)min((uint32_t)nb[h], (uint32_t)(p.num_blocks - 1));
        const int64_t base_off = (int64_t)blk * block_bytes + (int64_t)(p0 % BS) * kRowBytes;
        if (p0 + 16 <= L) {
          // every row of the half is below the length: a scalar base plus this lane's fixed offset
          __builtin_amdgcn_global_load_lds((const void*)(kbase + base_off + lane_k),
                                           (lds_void*)(buf + (4 * h + wave) * 1024), 16, 0, 0);
          __builtin_amdgcn_global_load_lds((const void*)(vbase + base_off + lane_v),
                                           (lds_void*)(buf + (8 + 4 * h + wave) * 1024), 16, 0, 0);
          continue;
        }
        row_off = (int64_t)blk * block_bytes + (int64_t)(p0 % BS + tq) * kRowBytes;
      } else {
        int ids[kHalfBlocks];
#pragma unroll
        for (int j = 0; j < kHalfBlocks; ++j)
          ids[j] = (int)min((uint32_t)trow[min(p0 / BS + j, p.MB - 1)], (uint32_t)(p.num_blocks - 1));
        int blk = ids[0];
#pragma unroll
        for (int j = 1; j < kHalfBlocks; ++j)
          if (tq / BS == j) blk = ids[j];
        row_off = (int64_t)blk * block_bytes + (int64_t)(tq % BS) * kRowBytes;
      }
      const bool live = p0 + tq < L;
      const char* ksrc = live ? kbase + row_off + lc_k * 16 : kZeroRow + lc_k * 16;
      const char* vsrc = live ? vbase + row_off + lc_v * 16 : kZeroRow + lc_v * 16;
      __builtin_amdgcn_global_load_lds((const void*)ksrc, (lds_void*)(buf + (4 * h + wave) * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)vsrc, (lds_void*)(buf + (8 + 4 * h + wave) * 1024), 16, 0, 0);
    }
  };
  int rd_k[4];  // K A operand: position c16 (+16 for half 1), chunk 4kc + g
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) rd_k[kc] = k_swz(c16, kc * 4 + g);
  int rd_v[8];  // V B operand (transposed read): positions 4g .. 4g+3, head_dim 16 jb + c16
  {
    const int rr = (lane >> 2) & 3, qq = lane & 3;
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) rd_v[jb] = kKBytes + v_swz(4 * g + rr, (16 * jb + 4 * qq) * 2);
  }

  const float c = p.qk_scale_log2;  // > 0: scores are kept raw and scaled inside the exponent
  float m_ref[2] = {kNegInf, kNegInf};  // base-2 units
  float l_part[2] = {0.f, 0.f};
  f32x4 acc[2][8];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) acc[mt][jb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // K operands of a tile: position c16 (+16 for half 1), chunk 4kc + g.
  auto read_k = [&](const lds_char* buf, u32x4 (&ka)[4][2]) {
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      ka[kc][0] = *(const lds_u32x4*)(buf + rd_k[kc]);
      ka[kc][1] = *(const lds_u32x4*)(buf + kKBytes / 2 + rd_k[kc]);
    }
  };
  // Raw S^T of a tile for both 16-position halves: lane (g, c16) holds positions 16h + 4g + e of
  // row c16 + 16 mt. Four independent accumulation chains, interleaved, so no MFMA waits for the one
  // before it.
  auto scores = [&](const u32x4 (&ka)[4][2], f32x4 (&s)[2][2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) s[h][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        s[0][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka[kc][0]), as_bf16x8(qb[mt][kc]), s[0][mt], 0, 0, 0);
        s[1][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka[kc][1]), as_bf16x8(qb[mt][kc]), s[1][mt], 0, 0, 0);
      }
  };
  // Softmax and P.V of a tile whose raw scores are s and whose V rows are in buf.
  // Mask, reference check and (rarely) rescale for a tile whose raw scores are s.
  auto head = [&](int tile, f32x4 (&s)[2][2]) {
    const int tile_p0 = tile * kKT;
    if (tile_p0 + kKT - 1 > wave_lo) {  // the tile crosses some row's causal limit
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (tile_p0 + 16 * h + 4 * g + e > row_lim[mt]) s[h][mt][e] = kNegInf;
    }
    // Lazy reference: each lane checks its own 8 scores of a row against the row's reference; only
    // when one outruns it does the wave reduce the row maxima and rescale what it accumulated.
    float lmx[2];
    bool over = false;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      lmx[mt] = max8(s[0][mt], s[1][mt]);
      over |= lmx[mt] * c > m_ref[mt] + kSlack;
    }
    if (__builtin_expect(__any(over), 0)) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        float x = lmx[mt];
        x = fmaxf(x, __shfl_xor(x, 16, 64));
        x = fmaxf(x, __shfl_xor(x, 32, 64));
        const float m_new = fmaxf(m_ref[mt], x * c);
        const float alpha = m_ref[mt] == kNegInf ? 0.f : exp2_fast(m_ref[mt] - m_new);
        m_ref[mt] = m_new;
        l_part[mt] *= alpha;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ae = __shfl(alpha, 4 * g + e, 64);  // accumulator row 4g + e
#pragma unroll
          for (int jb = 0; jb < 8; ++jb) acc[mt][jb][e] *= ae;
        }
      }
    }
  };
  // The bf16 pairs (-1, 0) and (0, -1), materialised in registers: as an operand of the packed-bf16
  // dot product the compiler encodes the first as the inline constant -1.0, and the results were
  // then wrong (the products did not use that pair).
  uint32_t neg_lo, neg_hi;
  asm("v_mov_b32 %0, 0xbf80" : "=v"(neg_lo));
  asm("v_mov_b32 %0, 0xbf800000" : "=v"(neg_hi));
  // P of a tile (hi and lo operands) and its row sums.
  auto probs = [&](const f32x4 (&s)[2][2], u32x4 (&a_hi)[2], u32x4 (&a_lo)[2]) {
    // P = 2^(c s - m), masked positions exactly 0. Split P = hi + lo: hi is P truncated to bf16 (its
    // top 16 bits, picked with one byte permute per pair), lo = P - hi exactly, rounded to bf16.
    // k-slots 8g .. 8g+3 hold half 0 and 8g+4 .. 8g+7 half 1.
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      float pr[8];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pr[4 * h + e] = exp2_fast(fmaf(s[h][mt][e], c, -m_ref[mt]));
          l_part[mt] += pr[4 * h + e];
        }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t u0 = __float_as_uint(pr[2 * w]), u1 = __float_as_uint(pr[2 * w + 1]);
        const uint32_t hp = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
        a_hi[mt][w] = hp;
        // P - hi, exact, as one packed-bf16 dot product each: (hi0, hi1) . (-1, 0) + P0 and
        // (hi0, hi1) . (0, -1) + P1 (the products are exact in fp32 and so is the difference)
        a_lo[mt][w] = cvt_pk_bf16(dot2_bf16(hp, neg_lo, pr[2 * w]), dot2_bf16(hp, neg_hi, pr[2 * w + 1]));
      }
    }
  };
  // V operands (transposed reads) of head_dim blocks jb0 .. jb0+3 of a tile.
  auto read_v = [&](const lds_char* buf, int jb0, u32x4 (&bv)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const s16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(buf + rd_v[jb0 + j]));
      const s16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(buf + kKBytes / 2 + rd_v[jb0 + j]));
      const uint64_t w0 = __builtin_bit_cast(uint64_t, b0), w1 = __builtin_bit_cast(uint64_t, b1);
      bv[j] = u32x4{(uint32_t)w0, (uint32_t)(w0 >> 32), (uint32_t)w1, (uint32_t)(w1 >> 32)};
    }
  };
  // P.V of head_dim blocks jb0 .. jb0+3. Two blocks at a time: their hi MFMAs for both row tiles, then
  // their lo MFMAs, so an accumulator's two updates are four instructions apart.
  auto pv = [&](const u32x4 (&bv)[4], int jb0, const u32x4 (&a_hi)[2], const u32x4 (&a_lo)[2]) {
#pragma unroll
    for (int j0 = 0; j0 < 4; j0 += 2) {
#pragma unroll
      for (int j = j0; j < j0 + 2; ++j)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          acc[mt][jb0 + j] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a_hi[mt]), as_bf16x8(bv[j]), acc[mt][jb0 + j], 0, 0, 0);
#pragma unroll
      for (int j = j0; j < j0 + 2; ++j)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          acc[mt][jb0 + j] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a_lo[mt]), as_bf16x8(bv[j]), acc[mt][jb0 + j], 0, 0, 0);
    }
  };

  // Software pipeline, step i: wait for this wave's loads of tile i+1 (tile i+2 may stay in flight),
  // barrier (every wave's part of tile i+1 is in LDS, and every wave is done with tile i-1); the LDS
  // reads of tile i+1's K operands and of half of tile i's V operands; issue tile i+3 into the buffer
  // tile i-1 used (and read the table for tile i+4); the mask and reference check of tile i; then,
  // fenced apart so that each group of LDS reads has a stretch of work to hide behind: tile i's P on
  // the vector ALUs, tile i+1's scores, the other half of the V reads, and tile i's P.V. Unrolled by
  // four so that each buffer is a fixed LDS object.
  lds_char* const bufs[4] = {(lds_char*)lds0, (lds_char*)lds1, (lds_char*)lds2, (lds_char*)lds3};
  int nb[2] = {0, 0};
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    if constexpr (BS >= 16) fetch_blocks(min(t, ntiles - 1), nb);
    if (t < ntiles) issue(bufs[t], t, nb);
  }
  if constexpr (BS >= 16) fetch_blocks(min(3, ntiles - 1), nb);
  // tile 0 in LDS: the loads of tiles 1 and 2 may stay in flight
  if (ntiles > 2)
    wait_vmem<8>();
  else if (ntiles > 1)
    wait_vmem<4>();
  else
    wait_vmem<0>();
  lds_barrier();
  f32x4 s_a[2][2], s_b[2][2];
  {
    u32x4 ka[4][2];
    read_k(bufs[0], ka);
    scores(ka, s_a);
  }
  // Every scalar value the loop reads (the kernel arguments above all) is in its register before the
  // loop starts: otherwise the wait for such a load lands inside the loop, where it would also wait
  // for every LDS read in flight, on every step.
  asm volatile("" ::"s"(c));  // the scale's load is issued above this point
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  for (int i0 = 0; i0 < ntiles; i0 += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u;
      if (i < ntiles) {
        f32x4(&s_cur)[2][2] = (u & 1) ? s_b : s_a;
        f32x4(&s_next)[2][2] = (u & 1) ? s_a : s_b;
        u32x4 ka[4][2], bv0[4], bv1[4], a_hi[2], a_lo[2];
        if (i + 1 < ntiles) {
          if (i + 2 < ntiles)
            wait_vmem<4>();
          else
            wait_vmem<0>();
          lds_barrier();
        }
        // Past the last tile the K reads and scores use a stale buffer and are never used; tiles past
        // a wave's rows are fully masked and add nothing.
        read_k(bufs[(u + 1) & 3], ka);
        read_v(bufs[u], 0, bv0);
        if (i + 1 < ntiles) {
          if (i + 3 < ntiles) issue(bufs[(u + 3) & 3], i + 3, nb);
          if constexpr (BS >= 16) fetch_blocks(min(i + 4, ntiles - 1), nb);
        }
        head(i, s_cur);
        sched_fence();
        probs(s_cur, a_hi, a_lo);  // behind it: the K reads and the first V reads
        sched_fence();
        scores(ka, s_next);
        sched_fence();
        read_v(bufs[u], 4, bv1);
        sched_fence();
        pv(bv0, 0, a_hi, a_lo);  // behind it (and the scores): the second V reads
        sched_fence();
        pv(bv1, 4, a_hi, a_lo);
      }
    }
  }

  // ---- o = acc / l; accumulator row 4g + e of the wave's 16-row tile mt
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    float l = l_part[mt];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);  // row c16's sum, on every lane of column c16
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float le = __shfl(l, 4 * g + e, 64);
      const int r = wave * kWaveRows + mt * 16 + 4 * g + e;
      const int tr = r / G;
      if (r >= QB * G || tok0 + tr >= tok_end) continue;
      const int64_t orow = (int64_t)(q0 + tok0 + tr) * p.Hq + kvh * G + r % G;
      const float inv = le > 0.f ? 1.f / le : 0.f;
#pragma unroll
      for (int jb = 0; jb < 8; ++jb) {
        const float o = acc[mt][jb][e] * inv;
        const int64_t idx = orow * kD + 16 * jb + c16;
        if (p.out_dtype == PA_F32)
          static_cast<float*>(p.out)[idx] = o;
        else
          static_cast<uint16_t*>(p.out)[idx] = f32_to_bf16(o);
      }
    }
  }
}

// ---- the chunk's scatter: row q_start[i] + j of k_new / v_new ([Q, Hkv, D]) to position
// L_i - n_i + j of sequence i. Grid: (chunks of the longest chunk's rows, sequences).
struct VarlenWriteParams {
  const char* k_new;
  const char* v_new;
  char* k_pool;
  char* v_pool;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* q_start;
  int32_t Hkv, MB, block_size, num_blocks;
  int32_t chunks_per_row;  // D * sizeof(dtype) / 16
  int32_t row_bytes;
  int64_t block_bytes;
};

__global__ __launch_bounds__(256) void write_kv_varlen_kernel(const VarlenWriteParams p) {
  const int seq = blockIdx.y;
  const int q0 = p.q_start[seq];
  const int n = p.q_start[seq + 1] - q0;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int chunk = (int)(idx % p.chunks_per_row);
  const int64_t row = idx / p.chunks_per_row;  // (j * 2 + which) * Hkv + kvh
  const int kvh = (int)(row % p.Hkv);
  const int which = (int)(row / p.Hkv) & 1;
  const int64_t j = row / (2 * p.Hkv);
  if (j >= n) return;
  const int64_t src = ((q0 + j) * p.Hkv + kvh) * p.row_bytes + chunk * 16;
  const u32x4 v = load16((which ? p.v_new : p.k_new) + src);
  const int pos = p.seq_lens[seq] - n + (int)j;
  const int phys = p.block_tables[(int64_t)seq * p.MB + pos / p.block_size];
  const int64_t dst = (int64_t)phys * p.block_bytes +
                      ((int64_t)kvh * p.block_size + pos % p.block_size) * p.row_bytes + chunk * 16;
  *reinterpret_cast<u32x4*>((which ? p.v_pool : p.k_pool) + dst) = v;
}

template <int BS>
hipError_t launch_bs(const PrefillParams& p, hipStream_t stream) {
  const int64_t grid = (int64_t)p.n_qblocks * p.B * p.Hkv;
  if (grid == 0) return hipSuccess;
  prefill_mfma_kernel<BS><<<dim3((unsigned)grid), dim3(kNW * 64), 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace

bool prefill_supported(const pa_dims& d) {
  const int G = d.num_q_heads / d.num_kv_heads;
  return d.q_dtype == PA_BF16 && d.kv_dtype == PA_BF16 && d.head_dim == kD && G <= kWgRows &&
         (d.block_size == 4 || d.block_size == 8 || d.block_size == 16 || d.block_size == 32) &&
         (d.out_dtype == PA_F32 || d.out_dtype == PA_BF16);
}

hipError_t launch_prefill(const pa_dims& d, const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_tables, const int32_t* seq_lens, const int32_t* q_start, float scale,
                          void* out, hipStream_t stream) {
  PrefillParams p = {};
  p.q = static_cast<const char*>(q);
  p.k_pool = static_cast<const char*>(k_pool);
  p.v_pool = static_cast<const char*>(v_pool);
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  p.q_start = q_start;
  p.out = out;
  p.qk_scale_log2 = scale * kLog2eHost;
  p.B = d.num_seqs;
  p.Hq = d.num_q_heads;
  p.Hkv = d.num_kv_heads;
  p.G = d.num_q_heads / d.num_kv_heads;
  p.MB = d.max_blocks_per_seq;
  p.num_blocks = d.num_blocks;
  p.out_dtype = d.out_dtype;
  p.qb_tokens = kWgRows / p.G;
  p.n_qblocks = (d.q_tokens + p.qb_tokens - 1) / p.qb_tokens;
  switch (d.block_size) {
    case 4: return launch_bs<4>(p, stream);
    case 8: return launch_bs<8>(p, stream);
    case 16: return launch_bs<16>(p, stream);
    case 32: return launch_bs<32>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_write_kv_varlen(const pa_dims& d, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                  const int32_t* block_tables, const int32_t* seq_lens, const int32_t* q_start,
                                  hipStream_t stream) {
  VarlenWriteParams p = {};
  p.k_new = static_cast<const char*>(k_new);
  p.v_new = static_cast<const char*>(v_new);
  p.k_pool = static_cast<char*>(k_pool);
  p.v_pool = static_cast<char*>(v_pool);
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  p.q_start = q_start;
  p.Hkv = d.num_kv_heads;
  p.MB = d.max_blocks_per_seq;
  p.block_size = d.block_size;
  p.num_blocks = d.num_blocks;
  p.row_bytes = d.head_dim * (d.kv_dtype == PA_F32 ? 4 : 2);
  p.chunks_per_row = p.row_bytes / 16;
  p.block_bytes = (int64_t)d.num_kv_heads * d.block_size * p.row_bytes;
  const int64_t per_seq = (int64_t)d.q_tokens * 2 * d.num_kv_heads * p.chunks_per_row;
  const int64_t blocks_x = (per_seq + 255) / 256;
  if (blocks_x == 0 || d.num_seqs == 0) return hipSuccess;
  if (blocks_x > 0x7fffffff || d.num_seqs > 65535) return hipErrorInvalidValue;
  write_kv_varlen_kernel<<<dim3((unsigned)blocks_x, (unsigned)d.num_seqs), dim3(256), 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace pa
