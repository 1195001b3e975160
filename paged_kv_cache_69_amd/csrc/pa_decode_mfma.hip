// Paged decode attention on the matrix cores (gfx950 MFMA), bf16 or int8 K/V, head_dim 128.
//
// It computes what the vector-ALU kernel computes (and what [P1] "25. Paged
// attention and prefix caching", section "Attention that reads through the
// table", and [P5] "Chapter 7 Paged KV Cache and Memory Management", sections
// 4.1-4.2 define): for each query row (token t, head h), the softmax over the
// visible positions p <= L - T + t of scale * q . K[p], applied to V[p], with
// K/V gathered through the block table. The query rows of one kv head (T*G of
// them, padded to 16 or 32) form one side of each MFMA, so the vector ALU
// only runs the softmax.
//
// Per wave, positions are consumed in tiles of 16 (4 KiB of K, 4 KiB of V):
//  * S^T = K Q^T, four v_mfma_f32_16x16x32_bf16 per 16 query rows. The K tile
//    is the A operand, loaded straight from the pool into registers (lane l:
//    position l%16, 16 bytes at head_dim 32*kc + 8*(l/16)). q is the B
//    operand, resident for the whole kernel. The C layout leaves lane l with
//    positions 4*(l/16) + i of query row l%16.
//  * That C layout is exactly the A-operand layout of v_mfma_f32_16x16x16_bf16
//    (row l%16, positions 4*(l/16) .. +3), so P.V needs no cross-lane move.
//    P is split into bf16 hi + lo parts, which keeps about 16 mantissa bits
//    of each probability, and each part gets its own MFMA.
//  * V is loaded into registers with the K tile (16 bytes per lane per KiB,
//    fully contiguous), then written to a 4 KiB per-wave LDS tile in natural
//    [position][head_dim] order, its 32-byte blocks XOR-swizzled by position
//    to spread LDS banks. One ds_read_b64_tr_b16 per 16-column block then
//    gives each lane 4 positions of one head_dim column, the B operand.
//  * Tiles inside one block are read through a buffer descriptor built per
//    tile in SGPRs plus a fixed lane offset: no per-tile vector address math.
//    The descriptor of a sequence's last tile ends at its length, so the rows
//    past it are never fetched (they read as zeros and are masked anyway).
//  * Softmax reference: a wave's first tile sets each row's reference max m.
//    Later tiles use p = 2^(x - m) with x in base-2 units. If a score ever
//    exceeds m by more than 2^64, the wave restarts its range with the larger
//    reference instead of rescaling, so the accumulators are only ever touched
//    by MFMAs. 2^64 headroom keeps l and acc far inside fp32 range, and
//    o = acc / l does not depend on the reference ([P5] section 4.2).
//  * Loads run PF tiles ahead. Every iteration issues the same 8 vector loads
//    (past the wave's last tile through empty descriptors, which fetch nothing),
//    so the compiler's wait before a tile is used leaves the younger tiles'
//    loads in flight. In the single pass a wave with few tiles asks for its
//    second tile only after its first has been computed: a smaller first
//    burst, which the waves with many tiles get through sooner.
// Masked tail tiles (positions >= L, causal limits when T > 1, absent padded
// rows) select -inf scores and zero the V rows past L before they are stored
// to LDS, so garbage in unwritten slots never reaches the result.
//
// int8 pools (Q8): codes with one fp32 scale per (block, kv head) ([P2]
// "Модуль 09: PagedAttention: пейджинг KV-кэша", section 6). The codes stay
// exact on the matrix cores and the scales are applied in fp32:
//  * K: code + 128 as an unsigned byte u, placed under the fp16 exponent byte
//    0x64, is the fp16 value 1024 + u = 1152 + code (one v_perm_b32 per two
//    codes). S^T runs as v_mfma_f32_16x16x32_f16 against q converted to fp16,
//    and the 1152 * sum(q) offset of each row is removed before the tile's
//    K scale multiplies the scores. fp16 holds every bf16 value of magnitude
//    2^-14 .. 2^15 exactly; a query row whose largest |q| reaches 2^15 is
//    first multiplied by a power of two 2^-k that brings it below, and its
//    scores by 2^k, so any finite q converts without overflow. Operand kc of lane (g, c16) takes head_dim
//    32g + 8kc .. +7, so each lane reads 32 contiguous bytes of its K row; q's
//    B operand is laid out the same way, so the dot products are unchanged.
//  * V: code + 128 converted to bf16 (exact below 256) goes through the same
//    LDS tile and transposed reads; P is multiplied by the tile's V scale
//    before its hi/lo split, and 128 * (sum of those scaled P) is removed from
//    each accumulator row at the end.
//  * A tile lies in one block (b >= 16), so one K and one V scale per tile,
//    one 8-byte scalar load (the scales are [N, Hkv, 2]) issued with the
//    block id. int8 codes are always finite, so tail V rows need no zeroing:
//    their P is exactly 0.
//
// Fused append (APPEND, bf16 pools only): the call also stores this step's new K/V
// rows, at positions L - T .. L - 1, into their pool slots ([P4] "Block table
// and allocator": a decode step writes the new token's K and V, then
// attends). The workgroup of (sequence, kv head) stores that head's rows
// itself: in a single pass the last wave, after its tiles, from rows and slots
// it fetched at the start (wave 0 before its tiles when T > 2); split, the
// wave whose partition holds them. No
// wave waits for those stores: in the tile that holds a new position, the
// lanes of that position take its K/V chunks from k_new / v_new instead of the
// pool, so the result is bit for bit the one a separate append followed by a
// decode gives.
//
// Cascade over a shared prefix (CASCADE, split context): when every sequence's
// first prefix_tokens positions map to the same physical blocks (a forked or
// prefix-cached prompt: [P1] "Sharing blocks"), the prefix is attended once
// per kv head for the query rows of all sequences together: the rows of one
// wave come from many sequences, so each K/V tile of the prefix is read by
// B*T*G / 32 waves instead of B workgroups. The prefix is cut into chunks of
// prefix_part_tokens, small enough for the prefix items to fill the chip; the
// NW waves of a prefix workgroup take NW consecutive chunks for the same 32
// rows and merge them through LDS like the single pass, writing one of the
// first prefix_parts partition slots; the sequences' own positions (from
// prefix_tokens on) run as ordinary split items in the slots after them, in
// the same launch (cascade_kernel), and the merge kernel combines all slots
// exactly ([P5] section 4.2).
//
// Two ways of sharing the work:
//  * Single pass (WAVE_ITEMS = false): one workgroup per (sequence, kv head).
//    Wave w takes tiles w, w + NW, ..., and the waves' (m, l, acc) are merged
//    through LDS at the end. Batches large enough to need several rounds of
//    workgroups are dealt longest sequence first (p.lpt).
//  * Split context (WAVE_ITEMS = true): every wave owns one partition of
//    part_tokens positions of one (sequence, kv head) and is independent of
//    the other waves of its workgroup (no barrier anywhere). It writes its
//    partition's (m, l, acc) partial to the workspace straight from
//    registers; the merge kernel that follows on the stream combines the
//    partials. When one partition per wave would need more waves than the
//    GPU holds at once (MULTI, bf16), a wave walks two consecutive
//    partitions with one unbroken load pipeline and parks the first
//    partition's partial in LDS until its end; each partition keeps its own
//    reference, so every partial is the one a wave of its own would write.
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"
#include "pa_mfma_tile.h"
#include "pa_wave_timeline.h"

PA_TIMELINE_BUFFER(mfma)

namespace pa {
namespace {

using namespace mfma;

#ifndef PA_MFMA_WAVES
#define PA_MFMA_WAVES 4
#endif
#ifndef PA_MFMA_PREFETCH
#define PA_MFMA_PREFETCH 1
#endif
#ifndef PA_MFMA_SPLIT_PREFETCH
#define PA_MFMA_SPLIT_PREFETCH 2
#endif
#ifndef PA_MFMA_Q8_PREFETCH
#define PA_MFMA_Q8_PREFETCH 1
#endif
#ifndef PA_MFMA_Q8_SPLIT_PREFETCH
#define PA_MFMA_Q8_SPLIT_PREFETCH 3
#endif
#ifndef PA_MFMA_WAVES_PER_EU
#define PA_MFMA_WAVES_PER_EU 1
#endif
#ifndef PA_CASCADE_WAVES_PER_EU
#define PA_CASCADE_WAVES_PER_EU 2
#endif
#ifndef PA_MFMA_F8_SPLIT_PREFETCH
#define PA_MFMA_F8_SPLIT_PREFETCH 1
#endif
#ifndef PA_MFMA_F8_SPLIT_WAVES_PER_EU
#define PA_MFMA_F8_SPLIT_WAVES_PER_EU 4
#endif
// prefix items hold every wave of the grid at once only at two waves per SIMD; FP8 split waves of 16 rows
// fit four per SIMD with one tile ahead (a long-context batch's waves then run in one round, not two)
#define PA_MFMA_OCCUPANCY                                                                             \
  __attribute__((amdgpu_waves_per_eu(CASCADE && BS >= 16 ? PA_CASCADE_WAVES_PER_EU                  \
                                     : F8 && WAVE_ITEMS && MT == 1 ? PA_MFMA_F8_SPLIT_WAVES_PER_EU   \
                                                         : PA_MFMA_WAVES_PER_EU)))
constexpr int kMfmaWaves = PA_MFMA_WAVES;
constexpr int kLptMaxSeqs = 512;  // largest batch the single pass orders longest first
constexpr int kMfmaPrefetch = PA_MFMA_PREFETCH;            // single pass: few tiles per wave
constexpr int kMfmaSplitPrefetch = PA_MFMA_SPLIT_PREFETCH;  // split context: a whole partition per wave
// int8 tiles are half the bytes and half the registers, so they run further ahead
constexpr int kMfmaQ8Prefetch = PA_MFMA_Q8_PREFETCH;
constexpr int kMfmaQ8SplitPrefetch = PA_MFMA_Q8_SPLIT_PREFETCH;
constexpr int kMfmaF8SplitPrefetch = PA_MFMA_F8_SPLIT_PREFETCH;
#ifndef PA_MFMA_DEFER_TILES
#define PA_MFMA_DEFER_TILES 4
#endif
// Single pass, one tile ahead: a wave with at most this many tiles computes its first tile before it
// asks for the second, so the launch's first burst of loads is smaller and the waves with many tiles
// (the longest sequences, which end the call) get their first tiles sooner. Measured on batch64: int8
// pools 15.00 -> 14.18 us, FP8 13.32 -> 12.98 us, bf16 with the append fused 19.28 -> 19.23 us.
constexpr int kMfmaDeferTiles = PA_MFMA_DEFER_TILES;
#ifndef PA_CASCADE_PREFIX_PREFETCH
#define PA_CASCADE_PREFIX_PREFETCH 1
#endif
#ifndef PA_CASCADE_SUFFIX_PREFETCH
#define PA_CASCADE_SUFFIX_PREFETCH 1
#endif
// The cascade launch runs its shared-prefix items and the sequences' own partitions one tile ahead: its
// waves outnumber the GPU's slots, and one tile ahead measured faster than two (prefix workload 82.7 ->
// 81.0 us per call, most of it from the own partitions)
constexpr int kCascadePrefixPrefetch = PA_CASCADE_PREFIX_PREFETCH;
constexpr int kCascadeSuffixPrefetch = PA_CASCADE_SUFFIX_PREFETCH;

__device__ __forceinline__ void store_out(const DecodeParams& p, int64_t idx, float o) {
  if (p.out_dtype == PA_F32)
    static_cast<float*>(p.out)[idx] = o;
  else
    static_cast<uint16_t*>(p.out)[idx] = f32_to_bf16(o);
}

// A wave's registers of one partition's partial (acc, then each lane's (m, l)), parked in LDS.
template <int MT>
constexpr int stash_bytes() {
  return MT * (8 * 64 * 16 + 64 * 8);
}

// The single pass of 16-row tiles merges its waves with one barrier: each wave writes its (m, l, acc) to
// LDS of its own as soon as its tiles are done, beside the V tiles rather than over them.
template <int MT, bool WAVE_ITEMS, bool CASCADE>
constexpr bool one_barrier_merge() {
  return !WAVE_ITEMS && !CASCADE && MT == 1;
}

// LDS of one workgroup: a V tile per wave, or the waves' (m, l, acc) when they merge in LDS (after the V
// tiles and the longest-first ranking's lengths for a one-barrier merge, over the V tiles otherwise);
// waves that walk two partitions (MULTI) also park the first one's partial after the V tiles.
template <int MT, int NW, bool WAVE_ITEMS, bool CASCADE, bool MULTI = false>
constexpr int decode_lds_bytes() {
  const int v = NW * kTileBytes + (MULTI ? NW * stash_bytes<MT>() : 0);
  const int red = (!WAVE_ITEMS || CASCADE) ? (NW * 16 * MT * kD + 2 * NW * 16 * MT) * 4 : 0;
  if (one_barrier_merge<MT, WAVE_ITEMS, CASCADE>()) return v + (kLptMaxSeqs + 4) * 4 + red;
  return v > red ? v : red;
}

// The work of one workgroup, `block` being its index in its kind of work (the launch's block index, or
// its place among the cascade launch's blocks of the same kind).
template <int MT, int BS, int NW, int PF, bool WAVE_ITEMS, bool Q8, bool APPEND, bool CASCADE, bool F8,
          bool MULTI = false>
__device__ __forceinline__ void decode_body(const DecodeParams& p, char* lds, int block, WaveTimeline& tl) {
  static_assert(!MULTI || (WAVE_ITEMS && !CASCADE && !Q8), "two partitions per wave are for bf16 split items");
  static_assert(!CASCADE || (WAVE_ITEMS && !Q8 && !APPEND), "prefix items are split-context bf16 items");
  static_assert(!Q8 || BS >= kTile, "int8 pools need a tile inside one block");
  static_assert(!(Q8 && APPEND), "8-bit pools append with the separate append kernel");
  static_assert(!F8 || Q8, "FP8 pools are 8-bit pools");
  constexpr int kKvRow = Q8 ? kD : kRowBytes;  // bytes of one K or V row in the pool
  constexpr int ROWS = 16 * MT;
  constexpr int NBUF = PF + 1;
  constexpr bool kLdsMerge = !WAVE_ITEMS || CASCADE;  // the waves' (m, l, acc) meet in LDS at the end

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;    // 16-lane group
  const int c16 = lane & 15;  // column inside the group

  // Single pass: block = seq * Hkv + kvh. Split context: block = j * Hkv + kvh, where j counts the
  // (sequence, group cg) pairs that hold work (see below), wave w owning item cg * NW + w of the
  // sequence's own partitions (the slots after the prefix_parts prefix slots). Cascade prefix items:
  // `seq` is a group of ROWS query rows over all sequences and the wave owns prefix partition
  // cg * NW + w. Consecutive blocks are consecutive kv heads, and blocks are dealt round-robin to the
  // 8 XCDs, so with Hkv = 8 one kv head's blocks share an L2.
  int bid = block;
  const int kvh = bid % p.Hkv;
  bid /= p.Hkv;
  // prefix items: NW chunks per workgroup, merged into one workspace slot per workgroup. Split items: KP
  // consecutive partitions per wave (one partial each), so that a long-context batch needs fewer waves
  // than the GPU holds at once.
  const int KP = MULTI && p.wave_parts > 1 ? 2 : 1;
  const int item_parts = !WAVE_ITEMS ? 1
                         : CASCADE ? (p.prefix_tokens + p.prefix_part_tokens - 1) / p.prefix_part_tokens
                                   : (p.parts - p.prefix_parts + KP - 1) / KP;
  const int groups = WAVE_ITEMS ? (item_parts + NW - 1) / NW : 1;
  int cg = bid % groups;
  int seq = bid / groups;
  int L_item = 0;  // split items: the sequence's length, found with it
  if constexpr (WAVE_ITEMS && !CASCADE) {
    // Split items are packed: workgroup index j (per kv head) is the j-th (sequence, group of NW
    // items) that holds work, sequence by sequence, and the grid's bound on their number leaves
    // only its tail empty. The dispatcher deals an XCD's workgroups to its shader engines in strict
    // rotation and waits when the next one's engine is full, so empty workgroups spread through the
    // grid would pile the real ones onto some engines while others idle.
    const int pt = p.part_tokens, pre = p.prefix_tokens, cap = p.parts - p.prefix_parts;
    auto count = [&](int len) {  // capped at the workspace's partitions, like the grid's bound
      const int own_parts = min(cap, max(0, (len - pre + pt - 1) / pt));
      return ((own_parts + KP - 1) / KP + NW - 1) / NW;
    };
    if (!find_item(p.seq_lens, p.B, bid, count, seq, cg, L_item)) return;
  }
  // Longest first (p.lpt, single pass): when the grid takes several rounds of workgroups, the j-th
  // workgroup of each kv head takes the sequence of length rank j (ties by index), so the rounds end
  // with the short sequences and the last workgroups to start are the quickest to finish. The ranking
  // reads every length once through LDS, past the V tiles' part of it.
  if constexpr (!WAVE_ITEMS && !CASCADE) {
    if (p.lpt) {
      int* lens = reinterpret_cast<int*>(lds + NW * kTileBytes);  // [kLptMaxSeqs], then the winner
      // (with a one-barrier merge the waves' partials go after these lengths, so no wave overwrites them
      // while another still reads its winner)
      const int b4 = (p.B + 3) / 4;
      for (int t = threadIdx.x; t < 4 * b4; t += NW * 64) lens[t] = t < p.B ? p.seq_lens[t] : INT32_MIN;
      __syncthreads();
      const int j = seq;
      for (int t = threadIdx.x; t < p.B; t += NW * 64) {
        const int lt = lens[t];
        int rank = 0;  // sequences ahead of t: longer, or as long with a lower index
#pragma unroll 4
        for (int i = 0; i < b4; ++i) {
          const int4 v = reinterpret_cast<const int4*>(lens)[i];
          rank += (v.x > lt || (v.x == lt && 4 * i < t)) + (v.y > lt || (v.y == lt && 4 * i + 1 < t)) +
                  (v.z > lt || (v.z == lt && 4 * i + 2 < t)) + (v.w > lt || (v.w == lt && 4 * i + 3 < t));
        }
        if (rank == j) lens[kLptMaxSeqs] = t;
      }
      __syncthreads();
      seq = __builtin_amdgcn_readfirstlane(lens[kLptMaxSeqs]);
    }
  }
  const int part_local = WAVE_ITEMS ? cg * NW + wave : 0;
  // workspace slot (of the item's first partition)
  const int part = !WAVE_ITEMS ? 0 : CASCADE ? cg : p.prefix_parts + part_local * KP;
  const int part_tiles = p.part_tokens / kTile;  // split items: tiles per partition

  const int T = p.T;
  const int p_begin = !WAVE_ITEMS ? 0 : CASCADE ? part_local * p.prefix_part_tokens
                                                : p.prefix_tokens + part_local * KP * p.part_tokens;

  // Query row n (< ROWS) of this wave: row n of sequence seq, or, for prefix items, row seq*ROWS + n of
  // all sequences' rows taken together.
  auto row_seq = [&](int n) { return CASCADE ? (seq * ROWS + n) / p.rows : seq; };
  auto row_in_seq = [&](int n) { return CASCADE ? (seq * ROWS + n) % p.rows : n; };
  auto row_present = [&](int n) { return CASCADE ? seq * ROWS + n < p.B * p.rows : n < p.rows; };

  // ---- q rows as the B operand of S^T: lane (g, c16) holds row c16 + 16*mt, head_dim 32*kc + 8g .. +7.
  // Issued first and unconditionally (an absent row reads row 0, then selects zero): they depend on
  // nothing else the kernel loads.
  u32x4 qb[MT][4];
  int row_tok[MT];  // query token of this lane's score row
  float qsum[MT];   // int8 pools: sum over head_dim of the row's fp16 q (weight of the K offset)
  float qk_mul[MT];  // base-2 score scale of this lane's score row (int8: times the row's 2^k)
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = mt * 16 + c16;
    const bool present = row_present(r);
    const int rr = present ? row_in_seq(r) : 0;
    const int rs = present ? row_seq(r) : 0;
    row_tok[mt] = rr / p.G;
    const char* qrow =
        static_cast<const char*>(p.q) + ((int64_t)(rs * T + row_tok[mt]) * p.Hq + kvh * p.G + rr % p.G) * kRowBytes;
    if constexpr (F8) {
      // lane (g, c16): head_dim 32g .. 32g+31 of the row, bf16 as stored; operand kc = 32g + 8kc .. +7
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const u32x4 v = load16(qrow + 64 * g + 16 * kc);
        qb[mt][kc] = present ? v : u32x4{0u, 0u, 0u, 0u};
      }
      qsum[mt] = 0.f;
      qk_mul[mt] = p.qk_scale_log2;
    } else if constexpr (Q8) {
      // lane (g, c16): head_dim 32g .. 32g+31 of the row, as fp16; operand kc = 32g + 8kc .. +7
      u32x4 raw[4];
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) raw[kc] = load16(qrow + 64 * g + 16 * kc);
      // the row's largest |q| (the four 16-lane groups hold a quarter each); a row at or above 2^15
      // is scaled by 2^-k (k = its exponent - 14) so that its fp16 values stay finite and exact
      float amax = 0.f;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
#pragma unroll
        for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(raw[kc][e])), fabsf(bf16_hi(raw[kc][e]))));
      amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
      const int k = present && amax >= 32768.f ? (int)((__float_as_uint(amax) >> 23) & 0xffu) - 141 : 0;
      const float down = __uint_as_float((uint32_t)(127 - k) << 23);  // 2^-k, k <= 114
      qk_mul[mt] = p.qk_scale_log2 * __uint_as_float((uint32_t)(127 + k) << 23);
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
        qb[mt][kc] = __builtin_bit_cast(u32x4, h);
      }
      part += __shfl_xor(part, 16, 64);
      part += __shfl_xor(part, 32, 64);
      qsum[mt] = part;
    } else {
      qk_mul[mt] = p.qk_scale_log2;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const u32x4 v = load16(qrow + (kc * 4 + g) * 16);
        qb[mt][kc] = present ? v : u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  // Prefix items: the row groups that share a chunk start at different tiles of it (and wrap round), so
  // at any moment they read different lines rather than all queueing on the same L2 channel.
  const int c_tiles =
      CASCADE ? max(1, (min(p.prefix_tokens, p_begin + p.prefix_part_tokens) - p_begin + kTile - 1) / kTile) : 1;
  const int rot = CASCADE ? seq % c_tiles : 0;
  auto tile_p0_of = [&](int i) {
    if constexpr (CASCADE) {
      const int j = i + rot;
      return p_begin + (j >= c_tiles ? j - c_tiles : j) * kTile;
    }
    return WAVE_ITEMS ? p_begin + i * kTile : (wave + i * NW) * kTile;
  };

  // Physical block ids of the wave's i-th tile, as wave-uniform scalar loads. A tile lies in one
  // block when BS >= 16, or spans 16 / BS whole blocks otherwise. The table index is clamped to the
  // row and the id to the pool, so a lookup never depends on the length and any entry (padding
  // included) gives an address inside the pool; positions at or past L are masked out of the
  // result whatever they hold. That lets the first tile's lookup go out together with the length.
  const auto* trow = read_only(p.block_tables + (CASCADE ? 0 : (int64_t)seq * p.MB));  // prefix: every row's blocks
  constexpr int kBlocksPerTile = BS >= kTile ? 1 : kTile / BS;
  struct TileIds {
    int b[kBlocksPerTile];
    float ks, vs;  // int8 pools: the block's K and V scales
  };
  auto ids_of = [&](int i) -> TileIds {
    TileIds ids;
    const int first = tile_p0_of(i) / BS;
#pragma unroll
    for (int jj = 0; jj < kBlocksPerTile; ++jj)
      ids.b[jj] = (int)min((uint32_t)trow[min(first + jj, p.MB - 1)], (uint32_t)(p.num_blocks - 1));
    if constexpr (Q8) {
      const f32x2 sc = read_only(reinterpret_cast<const f32x2*>(p.scales))[(int64_t)ids.b[0] * p.Hkv + kvh];
      ids.ks = sc[0];
      ids.vs = sc[1];
    } else {
      ids.ks = ids.vs = 1.f;
    }
    return ids;
  };
  const TileIds ids0 = ids_of(0);
  // prefix items: every prefix position is visible
  const int L = CASCADE ? p.prefix_tokens : WAVE_ITEMS ? L_item : read_only(p.seq_lens)[seq];
  // an empty split partition's wave leaves (the merge never reads its slot); a prefix item's wave with
  // no chunk stays for the workgroup's merge, with nothing to add
  if (WAVE_ITEMS && !CASCADE && (part_local >= item_parts || p_begin >= L)) return;
  const bool idle = CASCADE && (part_local >= item_parts || p_begin >= L);
  const int p_end = WAVE_ITEMS ? min(L, p_begin + (CASCADE ? p.prefix_part_tokens : KP * p.part_tokens)) : L;
  const int ntiles = !idle && p_end > p_begin ? (p_end - p_begin + kTile - 1) / kTile : 0;
  const int vis_all = CASCADE ? L : L - T + 1;
  const bool rows_all_present = CASCADE ? (seq + 1) * ROWS <= p.B * p.rows : p.rows == ROWS;
  const int my_tiles = WAVE_ITEMS ? ntiles : (wave < ntiles ? (ntiles - wave + NW - 1) / NW : 0);

  int row_lim[MT];  // last visible position of this lane's score row; -1 if the row is padding
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    row_lim[mt] = !row_present(mt * 16 + c16) ? -1 : CASCADE ? L - 1 : L - T + row_tok[mt];

  const int64_t block_bytes = (int64_t)p.Hkv * BS * kKvRow;
  const char* kbase = static_cast<const char*>(p.k_pool) + (int64_t)kvh * BS * kKvRow;
  const char* vbase = static_cast<const char*>(p.v_pool) + (int64_t)kvh * BS * kKvRow;
  lds_char* vt = (lds_char*)lds + wave * kTileBytes;
  lds_char* stash = (lds_char*)lds + NW * kTileBytes + wave * stash_bytes<MT>();  // MULTI only
  bool stashed = false;  // the wave's first partition's partial waits in its stash

  // Row t of this sequence's new K or V rows ([B, T, Hkv, D]), for this kv head.
  auto new_row = [&](const void* base, int t) -> const char* {
    return static_cast<const char*>(base) + ((int64_t)(seq * T + t) * p.Hkv + kvh) * kRowBytes;
  };

  // Byte offset, inside this kv head's view of the pool, of position `pos` of a tile whose blocks are `ids`.
  auto pos_offset = [&](const TileIds& ids, int tile_p0, int pos) -> int64_t {
    if constexpr (BS >= kTile) {
      return (int64_t)ids.b[0] * block_bytes + (int64_t)(pos % BS) * kRowBytes;
    } else {
      const int jj = (pos - tile_p0) / BS;  // tile_p0 is a multiple of 16, hence of BS
      int phys = ids.b[0];
#pragma unroll
      for (int k = 1; k < kBlocksPerTile; ++k)
        if (jj == k) phys = ids.b[k];
      return (int64_t)phys * block_bytes + (int64_t)(pos % BS) * kRowBytes;
    }
  };

  struct TileRegs {
    u32x4 k[Q8 ? 2 : 4];  // bf16: A operands of S^T; int8: 32 code bytes of row c16 at head_dim 32g
    u32x4 v[Q8 ? 2 : 4];  // bf16: position 4c + lane/16, chunk lane%16; int8: row lane/4, bytes 32 (lane%4)
  };
  const uint32_t k_lane_off = Q8 ? c16 * kD + 32 * g : c16 * kRowBytes + g * 16;
  const uint32_t v_lane_off = Q8 ? (lane >> 2) * kD + 32 * (lane & 3) : lane * 16;
  // `live` false: a load past the wave's last tile, issued only so that every step issues the same
  // loads; its descriptors are empty, so it fetches nothing and reads zeros.
  auto load_tile = [&](int i, const TileIds& ids, TileRegs& tr, bool live) {
    const int tile_p0 = tile_p0_of(i);
    if constexpr (BS >= kTile) {
      const int64_t boff = (int64_t)ids.b[0] * block_bytes + (int64_t)(tile_p0 % BS) * kKvRow;
      // the descriptors end at the sequence's length: rows past it read as zeros and cost no memory
      // traffic (they are masked out of the result in any case)
      const int bytes = live ? min(kTile, L - tile_p0) * kKvRow : 0;
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
    } else {
      const int64_t koff = pos_offset(ids, tile_p0, tile_p0 + c16);
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) tr.k[kc] = load16(kbase + koff + (kc * 4 + g) * 16);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        tr.v[c] = load16(vbase + pos_offset(ids, tile_p0, tile_p0 + 4 * c + (lane >> 4)) + (lane & 15) * 16);
    }
    if constexpr (APPEND && !Q8) {
      if (tile_p0 + kTile > L - T) {  // the tile holds new positions: their rows come from k_new / v_new
        const int tk = tile_p0 + c16 - (L - T);
        if (tk >= 0 && tk < T) {
#pragma unroll
          for (int kc = 0; kc < 4; ++kc) tr.k[kc] = load16(new_row(p.k_new, tk) + (kc * 4 + g) * 16);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int tv = tile_p0 + 4 * c + (lane >> 4) - (L - T);
          if (tv >= 0 && tv < T) tr.v[c] = load16(new_row(p.v_new, tv) + (lane & 15) * 16);
        }
      }
    }
  };

  float m_ref[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) m_ref[mt] = kNegInf;
  float l_part[MT];
  float vcorr[MT];  // int8 pools: this lane's sum of V-scaled P (weight of the V offset)
  f32x4 acc[MT][8];
  bool have_ref = false;

  // S^T of one tile (C layout: lane l has positions 4g + e of score row c16 + 16*mt), scaled and masked.
  auto scores = [&](bool masked, int tile_p0, const TileRegs& tr, float kscale, f32x4 (&s)[MT]) {
    u32x4 kf[4];  // 8-bit pools: the K codes as fp16 (int8) or bf16 (FP8) operands
    if constexpr (Q8) {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const int j = 2 * kc;  // dwords j, j + 1 of the lane's 32 code bytes
        const uint32_t w0 = tr.k[j >> 2][j & 3], w1 = tr.k[(j + 1) >> 2][(j + 1) & 3];
        const u32x2 a = F8 ? fp8_to_bf16(w0) : codes_to_f16(w0);
        const u32x2 b = F8 ? fp8_to_bf16(w1) : codes_to_f16(w1);
        kf[kc] = u32x4{a[0], a[1], b[0], b[1]};
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
      if constexpr (F8) {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[kc]), as_bf16x8(qb[mt][kc]), c, 0, 0, 0);
        s[mt] = c * (kscale * qk_mul[mt]);
      } else if constexpr (Q8) {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(kf[kc]), as_f16x8(qb[mt][kc]), c, 0, 0, 0);
        s[mt] = (c - kKOffset * qsum[mt]) * (kscale * qk_mul[mt]);
      } else {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(tr.k[kc]), as_bf16x8(qb[mt][kc]), c, 0, 0, 0);
        s[mt] = c * qk_mul[mt];
      }
      if (masked) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (tile_p0 + 4 * g + e > row_lim[mt]) s[mt][e] = kNegInf;
      }
    }
  };

  // Raise each row's reference to at least the row max of s.
  auto raise_ref = [&](const f32x4 (&s)[MT]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float mx = fmaxf(fmaxf(s[mt][0], s[mt][1]), fmaxf(s[mt][2], s[mt][3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      m_ref[mt] = fmaxf(m_ref[mt], mx);
    }
  };

  // P.V of one tile whose scores are s and whose V rows are in vreg. Masked positions have
  // score -inf (p = 0, selected, never computed from -inf) and V rows past L are zeroed.
  auto accumulate = [&](bool masked, int tile_p0, const f32x4 (&s)[MT], const TileRegs& tr, float vscale) {
    s16x4 a_hi[MT], a_lo[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float pr[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = s[mt][e];
        pr[e] = x == kNegInf ? 0.f : exp2_fast(x - m_ref[mt]);
        l_part[mt] += pr[e];
        if constexpr (Q8) {
          pr[e] *= vscale;  // from here on P carries the block's V scale
          if constexpr (!F8) vcorr[mt] += pr[e];
        }
      }
      const uint32_t h01 = cvt_pk_bf16(pr[0], pr[1]);
      const uint32_t h23 = cvt_pk_bf16(pr[2], pr[3]);
      const uint32_t l01 = cvt_pk_bf16(pr[0] - bf16_lo(h01), pr[1] - bf16_hi(h01));
      const uint32_t l23 = cvt_pk_bf16(pr[2] - bf16_lo(h23), pr[3] - bf16_hi(h23));
      a_hi[mt] = __builtin_bit_cast(s16x4, (uint64_t)h01 | ((uint64_t)h23 << 32));
      a_lo[mt] = __builtin_bit_cast(s16x4, (uint64_t)l01 | ((uint64_t)l23 << 32));
    }

    if constexpr (Q8) {
      // V codes of row lane/4, head_dim 32 (lane%4) .. +31, as bf16 (int8: 128 + code; FP8: its value),
      // into the LDS tile
      const int t = lane >> 2;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t w0 = tr.v[c >> 1][2 * (c & 1)], w1 = tr.v[c >> 1][2 * (c & 1) + 1];
        const u32x2 a = F8 ? fp8_to_bf16(w0) : codes_to_bf16(w0);
        const u32x2 b = F8 ? fp8_to_bf16(w1) : codes_to_bf16(w1);
        const u32x4 w = {a[0], a[1], b[0], b[1]};
        *(lds_u32x4*)(vt + v_swz(t, 64 * (lane & 3) + 16 * c)) = w;
      }
    } else {
      // V tile into this wave's LDS tile (positions >= L zeroed: those slots may hold anything)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int t = 4 * c + (lane >> 4);
        u32x4 v = tr.v[c];
        if (masked && tile_p0 + t >= L) v = u32x4{0u, 0u, 0u, 0u};
        *(lds_u32x4*)(vt + v_swz(t, (lane & 15) * 16)) = v;
      }
    }
    wave_lds_order();

    // B operand = positions 4g .. 4g+3 of head_dim column 16*jb + c16 (one transpose read)
    const int rr = (lane >> 2) & 3, qq = lane & 3;
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) {
      const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vt + v_swz(4 * g + rr, (16 * jb + 4 * qq) * 2)));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc[mt][jb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_hi[mt], b, acc[mt][jb], 0, 0, 0);
        acc[mt][jb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_lo[mt], b, acc[mt][jb], 0, 0, 0);
      }
    }
    // the next tile overwrites this LDS tile after these reads, in this wave's order
    wave_lds_order();
  };

  auto out_row = [&](int n) -> int64_t {  // flat (seq, token, q head) index of query row n
    const int rs = row_seq(n), m = row_in_seq(n);
    return (int64_t)(rs * T + m / p.G) * p.Hq + kvh * p.G + m % p.G;
  };
  auto clear = [&]() {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      l_part[mt] = 0.f;
      vcorr[mt] = 0.f;
#pragma unroll
      for (int jb = 0; jb < 8; ++jb) acc[mt][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  // Split context: this partition's (m, l, acc) partial, straight from registers. Lanes of column
  // c16 hold parts of row c16 (+16*mt)'s l; the four 16-lane groups are summed first.
  auto flush = [&](int slot) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float l = l_part[mt];
      l += __shfl_xor(l, 16, 64);
      l += __shfl_xor(l, 32, 64);
      const int n = mt * 16 + c16;
      if (g == 0 && row_present(n)) {
        const int64_t pi = out_row(n) * p.parts + slot;
        *reinterpret_cast<f32x2*>(p.part_ml + pi * 2) = f32x2{m_ref[mt], l};
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int na = mt * 16 + 4 * g + e;  // accumulator row of this lane
        if (row_present(na)) {
          float* dst = p.part_acc + (out_row(na) * p.parts + slot) * kD + c16;
#pragma unroll
          for (int jb = 0; jb < 8; ++jb) dst[16 * jb] = acc[mt][jb][e];
        }
      }
    }
  };
  // int8 pools: remove the V offset (accumulator row 4g + e (+16 mt) held 128 * sum(scaled P) of that row too)
  auto remove_v_offset = [&]() {
    if constexpr (Q8 && !F8) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        float tot = vcorr[mt];
        tot += __shfl_xor(tot, 16, 64);
        tot += __shfl_xor(tot, 32, 64);  // row c16's total, on every lane of column c16
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ce = kVOffset * __shfl(tot, 4 * g + e, 64);
#pragma unroll
          for (int jb = 0; jb < 8; ++jb) acc[mt][jb][e] -= ce;
        }
      }
    }
  };
  // Process the wave's tiles from tile ib on. Returns -1 when done, or the tile to run again from when a
  // score outran the reference: m_ref has then been raised and the caller runs again from the start of
  // that tile's partition (its first tile, or ib) with cleared accumulators (the tile that outran was
  // still accumulated, into values that are discarded). With KP > 1 the loads run on across the end of
  // a partition: its partial is written there and the next partition starts with cleared accumulators
  // and a reference of its own.
  auto run = [&](int ib) -> int {
    ib = __builtin_amdgcn_readfirstlane(ib);  // uniform, so the table lookups below stay scalar loads
    clear();
    if (ib >= my_tiles) return -1;
    const int last = my_tiles - 1;
    TileRegs ring[NBUF];
    TileIds cur[NBUF];  // block ids (and scales) of the tile in each ring slot
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      cur[u] = ib + u == 0 ? ids0 : ids_of(min(ib + u, last));
      load_tile(min(ib + u, last), cur[u], ring[u], ib + u <= last);
    }
    TileIds ids_next = ids_of(min(ib + PF, last));
    const int ib_first = ib;  // a restart runs again from here
    // (the separate bf16 pass is left as it is: the extra code costs it a wave per SIMD)
    if constexpr (!WAVE_ITEMS && !CASCADE && PF == 1 && (APPEND || Q8)) {
      if (ib == 0 && !have_ref && my_tiles <= kMfmaDeferTiles) {
        // the first tile, computed before the next one is asked for; then tile 1 goes into ring slot 0
        // and the loop below starts from it as if it had been issued there
        tl.first_tile();
        const int tile_p0 = tile_p0_of(ib);
        const bool masked = !rows_all_present || tile_p0 + kTile > vis_all;
        f32x4 s[MT];
        scores(masked, tile_p0, ring[0], cur[0].ks, s);
        raise_ref(s);  // the wave's first tile sets the reference
        have_ref = true;
        accumulate(masked, tile_p0, s, ring[0], cur[0].vs);
        cur[0] = ids_next;
        load_tile(min(ib + 1, last), cur[0], ring[0], ib + 1 <= last);
        ids_next = ids_of(min(ib + 2, last));
        ib += 1;
      }
    }
    int again = -1;
    int part_end = KP > 1 ? (ib / part_tiles + 1) * part_tiles : my_tiles;  // tile after this partition
    for (int i0 = ib; i0 < my_tiles && again < 0; i0 += NBUF) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        const int i = i0 + u;
        if (i < my_tiles && again < 0) {
          const TileIds ids = ids_next;
          ids_next = ids_of(min(i + PF + 1, last));
          load_tile(min(i + PF, last), ids, ring[(u + PF) % NBUF], i + PF <= last);
          const TileIds ids_cur = cur[u];  // the scales of tile i
          cur[(u + PF) % NBUF] = ids;
          tl.first_tile();
          const int tile_p0 = tile_p0_of(i);
          const bool masked = !rows_all_present || tile_p0 + kTile > vis_all;
          const float kscale = ids_cur.ks, vscale = ids_cur.vs;
          f32x4 s[MT];
          scores(masked, tile_p0, ring[u], kscale, s);
          if (!have_ref) {
            raise_ref(s);  // the wave's first tile sets the reference
            have_ref = true;
          } else {
            bool over = false;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
              for (int e = 0; e < 4; ++e) over |= s[mt][e] > m_ref[mt] + kRefSlack;
            if (__builtin_expect(__any(over), 0)) {
              raise_ref(s);
              again = KP > 1 ? part_end - part_tiles : ib_first;
            }
          }
          accumulate(masked, tile_p0, s, ring[u], vscale);
          if (KP > 1 && i + 1 == part_end && i + 1 < my_tiles && again < 0) {
            // the first partition ends here: its partial waits in LDS until the wave's end. Written to
            // memory now, its stores would be younger than the tile loads in flight, and the waits for
            // those tiles would then wait for the stores too.
            if constexpr (MULTI) {
#pragma unroll
              for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
                for (int jb = 0; jb < 8; ++jb)
                  *(__attribute__((address_space(3))) f32x4*)(stash + ((mt * 8 + jb) * 64 + lane) * 16) = acc[mt][jb];
                *(__attribute__((address_space(3))) f32x2*)(stash + MT * 8192 + (mt * 64 + lane) * 8) =
                    f32x2{m_ref[mt], l_part[mt]};
              }
              stashed = true;
            }
            clear();
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) m_ref[mt] = kNegInf;
            have_ref = false;
            part_end += part_tiles;
          }
        }
      }
    }
    return again;
  };

  // Single pass: the last waves (the fewest tiles) store the new rows after their tiles, two rows each
  // (wave NW - 1 rows 0-1, wave NW - 2 rows 2-3, ...). Their data and slots are fetched now, ahead of the
  // tiles, so those stores wait on nothing by then. Split items with T <= 2: the wave whose range holds a
  // new row stores it the same way, after its own tiles.
  const bool late = APPEND && !Q8 && !CASCADE && (WAVE_ITEMS ? T <= 2 : T <= 2 * NW);
  u32x4 late_row = {0u, 0u, 0u, 0u};
  int64_t late_dst = -1;
  if constexpr (APPEND && !Q8 && !CASCADE) {
    const int t_base = WAVE_ITEMS ? 0 : 2 * (NW - 1 - wave);  // this wave's first row
    if (late && t_base < T) {
      // lane: row t_base + lane / 32; K (lanes 0-15 of the half) or V (16-31); 16-byte chunk lane % 16
      const int t = t_base + (lane >> 5), which = (lane >> 4) & 1, chunk = lane & 15;
      const int pos0 = L - T + t_base, pos1 = min(pos0 + 1, L - 1);  // the two rows' positions
      const int blk0 = (int)min((uint32_t)trow[min(max(pos0, 0) / BS, p.MB - 1)], (uint32_t)(p.num_blocks - 1));
      const int blk1 = (int)min((uint32_t)trow[min(max(pos1, 0) / BS, p.MB - 1)], (uint32_t)(p.num_blocks - 1));
      const int pos = L - T + t;
      const bool mine = !WAVE_ITEMS || (pos >= p_begin && pos < p_end);
      if (t < T && pos >= 0 && mine) {
        late_row = load16(new_row(which ? p.v_new : p.k_new, t) + chunk * 16);
        late_dst = (int64_t)(t > t_base ? blk1 : blk0) * block_bytes + (int64_t)(pos % BS) * kRowBytes + chunk * 16;
      }
    }
  }
  if constexpr (APPEND && !Q8) {
    // store the new rows this wave owns (positions L - T .. L - 1 in its range) into the pools
    // One row per step, so its position and block are wave-uniform (a scalar table load); lanes 0-15
    // copy the K row's 16-byte chunks and lanes 16-31 the V row's.
    const int t_lo = WAVE_ITEMS ? max(0, p_begin - (L - T)) : 0;
    const int t_hi = late ? 0 : WAVE_ITEMS ? min(T, p_end - (L - T)) : (wave == 0 ? T : 0);
    for (int t = max(t_lo, T - L); t < t_hi; ++t) {
      const int pos = L - T + t;
      const int blk = (int)min((uint32_t)trow[min(pos / BS, p.MB - 1)], (uint32_t)(p.num_blocks - 1));
      if (lane < 32) {
        const int which = lane >> 4, chunk = lane & 15;
        const int64_t dst = (int64_t)blk * block_bytes + (int64_t)(pos % BS) * kRowBytes + chunk * 16;
        const u32x4 v = load16(new_row(which ? p.v_new : p.k_new, t) + chunk * 16);
        *reinterpret_cast<u32x4*>(const_cast<char*>(which ? vbase : kbase) + dst) = v;
      }
    }
  }

  for (int from = 0; (from = run(from)) >= 0;) {
  }
  tl.end_loop(my_tiles);
  if constexpr (APPEND && !Q8 && !CASCADE) {
    if (late_dst >= 0) {
      const bool v_half = (lane >> 4) & 1;
      *reinterpret_cast<u32x4*>(const_cast<char*>(v_half ? vbase : kbase) + late_dst) = late_row;
    }
  }

  remove_v_offset();

  if constexpr (!kLdsMerge) {
    flush(part + (KP > 1 ? (my_tiles - 1) / part_tiles : 0));
    if constexpr (MULTI) {
      if (stashed) {  // the first partition's partial, back from LDS
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
          for (int jb = 0; jb < 8; ++jb)
            acc[mt][jb] = *(__attribute__((address_space(3))) f32x4*)(stash + ((mt * 8 + jb) * 64 + lane) * 16);
          const f32x2 ml = *(__attribute__((address_space(3))) f32x2*)(stash + MT * 8192 + (mt * 64 + lane) * 8);
          m_ref[mt] = ml[0];
          l_part[mt] = ml[1];
        }
        flush(part);
      }
    }
  } else {
    // per-row l of this wave: lanes of column c16 hold row c16 (+16*mt); sum the four 16-lane groups
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      l_part[mt] += __shfl_xor(l_part[mt], 16, 64);
      l_part[mt] += __shfl_xor(l_part[mt], 32, 64);
    }
    // ---- merge the waves' (m, l, acc) through LDS ([P5] section 4.2, three-step merge):
    // M = max_w m_w;  l = sum_w l_w 2^(m_w - M);  acc = sum_w acc_w 2^(m_w - M).
    constexpr bool kOneBarrier = one_barrier_merge<MT, WAVE_ITEMS, CASCADE>();
    float* red_acc = reinterpret_cast<float*>(lds + (kOneBarrier ? NW * kTileBytes + (kLptMaxSeqs + 4) * 4 : 0));
    float* red_m = red_acc + NW * ROWS * kD;  // [ROWS][NW]
    float* red_l = red_m + NW * ROWS;         // [ROWS][NW]
    // [NW][ROWS][kD]: one barrier, each wave's accumulators as they are (the final pass scales them); else
    // each wave rescales its own in registers once every m is known, and the final pass only sums
    if constexpr (!kOneBarrier) __syncthreads();  // every wave is done with its V tile before the merge reuses the LDS
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (g == 0) {
        red_l[(mt * 16 + c16) * NW + wave] = l_part[mt];
        red_m[(mt * 16 + c16) * NW + wave] = m_ref[mt];
      }
    }
    if constexpr (kOneBarrier) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 4 * g + e;
#pragma unroll
        for (int jb = 0; jb < 8; ++jb) red_acc[(wave * ROWS + row) * kD + 16 * jb + c16] = acc[0][jb][e];
      }
    } else {
      __syncthreads();
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = mt * 16 + 4 * g + e;
          float M = kNegInf;
#pragma unroll
          for (int w = 0; w < NW; ++w) M = fmaxf(M, red_m[row * NW + w]);
          const float mw = red_m[row * NW + wave];
          const float sc = mw == kNegInf ? 0.f : exp2_fast(mw - M);
#pragma unroll
          for (int jb = 0; jb < 8; ++jb) red_acc[(wave * ROWS + row) * kD + 16 * jb + c16] = acc[mt][jb][e] * sc;
        }
    }
    __syncthreads();

    // Each thread finishes 4 consecutive head_dim values of a row at a time: the normalised output, or
    // (prefix items) the workgroup's partial (M, l, acc) for its slot.
    for (int idx = threadIdx.x; idx < ROWS * (kD / 4); idx += NW * 64) {
      const int n = idx / (kD / 4), d4 = (idx % (kD / 4)) * 4;
      if (!row_present(n)) continue;
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, red_m[n * NW + w]);
      float lsum = 0.f;
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
      if (M != kNegInf) {
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const float mw = red_m[n * NW + w];
          const float sc = mw == kNegInf ? 0.f : exp2_fast(mw - M);
          lsum = fmaf(sc, red_l[n * NW + w], lsum);
          const f32x4 aw = *reinterpret_cast<const f32x4*>(red_acc + (w * ROWS + n) * kD + d4);
          if constexpr (kOneBarrier)
            a += sc * aw;
          else
            a += aw;
        }
      }
      const int64_t orow = out_row(n);
      if constexpr (CASCADE) {
        const int64_t pi = orow * p.parts + part;
        *reinterpret_cast<f32x4*>(p.part_acc + pi * kD + d4) = a;
        if (d4 == 0) *reinterpret_cast<f32x2*>(p.part_ml + pi * 2) = f32x2{M, lsum};
      } else {
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = lsum > 0.f ? a[e] / lsum : 0.f;
        if (p.out_dtype == PA_F32) {  // one 16-byte store (out is 16-byte aligned, d4 a multiple of 4)
          *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + orow * kD + d4) = o;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) store_out(p, orow * kD + d4 + e, o[e]);
        }
      }
    }
  }
}

template <int MT, int BS, int NW, int PF, bool WAVE_ITEMS, bool Q8, bool APPEND, bool CASCADE, bool F8, bool MULTI>
__global__ __launch_bounds__(NW * 64) PA_MFMA_OCCUPANCY void decode_mfma_kernel(const DecodeParams p) {
  __shared__ __attribute__((aligned(16))) char lds[decode_lds_bytes<MT, NW, WAVE_ITEMS, CASCADE, MULTI>()];
  WaveTimeline tl;
  tl.begin();
  decode_body<MT, BS, NW, PF, WAVE_ITEMS, Q8, APPEND, CASCADE, F8, MULTI>(p, lds, blockIdx.x, tl);
  PA_TIMELINE_STORE(tl, blockIdx.x * NW + (threadIdx.x >> 6));
}

// Cascade in one launch: the shared prefix's items (32 rows of many sequences per wave, L2-bound) and
// the sequences' own partitions (HBM-bound) run side by side instead of one launch after the other.
// Blocks alternate between the two kinds in runs of Hkv (one run is one index of every kv head, so
// each kind keeps its kv head = XCD placement), and whichever kind has more runs takes the tail.
template <int MT, int BS, bool AP>
__global__ __launch_bounds__(kMfmaWaves * 64) __attribute__((amdgpu_waves_per_eu(PA_CASCADE_WAVES_PER_EU)))
void cascade_kernel(const DecodeParams p, int pre_runs, int suf_runs) {
  constexpr int kPre = decode_lds_bytes<2, kMfmaWaves, true, true>();
  constexpr int kSuf = decode_lds_bytes<MT, kMfmaWaves, true, false>();
  __shared__ __attribute__((aligned(16))) char lds[kPre > kSuf ? kPre : kSuf];
  const int run = blockIdx.x / p.Hkv, r = blockIdx.x % p.Hkv;
  const int both = min(pre_runs, suf_runs);
  const bool prefix = run < 2 * both ? (run & 1) == 0 : pre_runs > suf_runs;
  const int idx = (run < 2 * both ? run / 2 : both + (run - 2 * both)) * p.Hkv + r;
  WaveTimeline tl;
  tl.begin();
  if (prefix)
    decode_body<2, BS, kMfmaWaves, kCascadePrefixPrefetch, true, false, false, true, false>(p, lds, idx, tl);
  else
    decode_body<MT, BS, kMfmaWaves, kCascadeSuffixPrefetch, true, false, AP, false, false>(p, lds, idx, tl);
  PA_TIMELINE_STORE(tl, blockIdx.x * kMfmaWaves + (threadIdx.x >> 6));
}

template <int MT, int BS, bool WI, bool Q8, bool AP, bool CAS = false, bool F8 = false>
hipError_t launch_t(const DecodeParams& p, hipStream_t stream) {
  // two partitions per wave: a kernel of its own (the extra flush costs registers), bf16 16-row tiles only
  constexpr bool kMultiOk = WI && !CAS && MT == 1 && !Q8;
  const int64_t kp = kMultiOk && p.wave_parts > 1 ? p.wave_parts : 1;
  const int64_t item_parts = !WI ? 1
                             : CAS ? (p.prefix_tokens + p.prefix_part_tokens - 1) / p.prefix_part_tokens
                                   : (p.parts - p.prefix_parts + kp - 1) / kp;
  const int64_t groups = WI ? (item_parts + kMfmaWaves - 1) / kMfmaWaves : 1;
  const int64_t units = CAS ? ((int64_t)p.B * p.rows + 16 * MT - 1) / (16 * MT) : p.B;  // row groups or sequences
  const int64_t grid = units * groups * p.Hkv;
  if (grid == 0) return hipSuccess;
  constexpr int PF = Q8 ? (WI ? (F8 && MT == 1 ? kMfmaF8SplitPrefetch : kMfmaQ8SplitPrefetch) : kMfmaQ8Prefetch)
                        : (WI ? kMfmaSplitPrefetch : kMfmaPrefetch);
  if (kp > 1)
    decode_mfma_kernel<MT, BS, kMfmaWaves, PF, WI, Q8, AP, CAS, F8, kMultiOk>
        <<<dim3((unsigned)grid), dim3(kMfmaWaves * 64), 0, stream>>>(p);
  else
    decode_mfma_kernel<MT, BS, kMfmaWaves, PF, WI, Q8, AP, CAS, F8, false>
        <<<dim3((unsigned)grid), dim3(kMfmaWaves * 64), 0, stream>>>(p);
  return hipGetLastError();
}

template <int MT, bool WI>
hipError_t launch_bs(const DecodeParams& p, hipStream_t stream) {
  if (p.kv_int8 && p.append) return hipErrorInvalidValue;  // 8-bit pools append with the append kernel
  if (p.kv_int8 && p.kv_fp8) {
    switch (p.block_size) {
      case 16: return launch_t<MT, 16, WI, true, false, false, true>(p, stream);
      case 32: return launch_t<MT, 32, WI, true, false, false, true>(p, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (p.kv_int8) {
    switch (p.block_size) {
      case 16: return launch_t<MT, 16, WI, true, false>(p, stream);
      case 32: return launch_t<MT, 32, WI, true, false>(p, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (p.append) {
    switch (p.block_size) {
      case 4: return launch_t<MT, 4, WI, false, true>(p, stream);
      case 8: return launch_t<MT, 8, WI, false, true>(p, stream);
      case 16: return launch_t<MT, 16, WI, false, true>(p, stream);
      case 32: return launch_t<MT, 32, WI, false, true>(p, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (p.block_size) {
    case 4: return launch_t<MT, 4, WI, false, false>(p, stream);
    case 8: return launch_t<MT, 8, WI, false, false>(p, stream);
    case 16: return launch_t<MT, 16, WI, false, false>(p, stream);
    case 32: return launch_t<MT, 32, WI, false, false>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool mfma_supported(const pa_dims& d) {
  const int rows = d.q_tokens * (d.num_q_heads / d.num_kv_heads);
  const bool block = d.block_size == 4 || d.block_size == 8 || d.block_size == 16 || d.block_size == 32;
  return d.kv_dtype == PA_BF16 && d.q_dtype == PA_BF16 && d.head_dim == kD && block && rows <= 32;
}

bool mfma_int8_supported(const pa_dims& d) {
  const int rows = d.q_tokens * (d.num_q_heads / d.num_kv_heads);
  return (d.kv_dtype == PA_INT8 || d.kv_dtype == PA_FP8_E4M3) && d.q_dtype == PA_BF16 && d.head_dim == kD &&
         (d.block_size == 16 || d.block_size == 32) && rows <= 32;
}

template <int MT, bool AP>
hipError_t launch_cascade_bs(const DecodeParams& p, hipStream_t stream, int pre_runs, int suf_runs) {
  const dim3 grid((unsigned)((int64_t)(pre_runs + suf_runs) * p.Hkv)), block(kMfmaWaves * 64);
  switch (p.block_size) {
    case 4: cascade_kernel<MT, 4, AP><<<grid, block, 0, stream>>>(p, pre_runs, suf_runs); break;
    case 8: cascade_kernel<MT, 8, AP><<<grid, block, 0, stream>>>(p, pre_runs, suf_runs); break;
    case 16: cascade_kernel<MT, 16, AP><<<grid, block, 0, stream>>>(p, pre_runs, suf_runs); break;
    case 32: cascade_kernel<MT, 32, AP><<<grid, block, 0, stream>>>(p, pre_runs, suf_runs); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_cascade(const DecodeParams& p, hipStream_t stream) {
  // runs (of Hkv blocks) of each kind, from the same grid arithmetic as the separate launches
  const int64_t pre_items = (p.prefix_tokens + p.prefix_part_tokens - 1) / p.prefix_part_tokens;
  const int64_t pre_runs = ((int64_t)p.B * p.rows + 31) / 32 * ((pre_items + kMfmaWaves - 1) / kMfmaWaves);
  const int64_t suf_runs = (int64_t)p.B * ((p.parts - p.prefix_parts + kMfmaWaves - 1) / kMfmaWaves);
  if (pre_runs + suf_runs == 0) return hipSuccess;
  // fused append: the suffix items hold every new row (they follow the shared prefix)
  if (p.append)
    return p.rows <= 16 ? launch_cascade_bs<1, true>(p, stream, (int)pre_runs, (int)suf_runs)
                        : launch_cascade_bs<2, true>(p, stream, (int)pre_runs, (int)suf_runs);
  return p.rows <= 16 ? launch_cascade_bs<1, false>(p, stream, (int)pre_runs, (int)suf_runs)
                      : launch_cascade_bs<2, false>(p, stream, (int)pre_runs, (int)suf_runs);
}

int mfma_waves() { return kMfmaWaves; }
int mfma_lpt_max_seqs() { return kLptMaxSeqs; }

hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t stream) {
  if (p.partial) return p.rows <= 16 ? launch_bs<1, true>(p, stream) : launch_bs<2, true>(p, stream);
  return p.rows <= 16 ? launch_bs<1, false>(p, stream) : launch_bs<2, false>(p, stream);
}

}  // namespace pa
