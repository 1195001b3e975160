// Device helpers for the gfx950 kernels: 16-byte chunks, bf16 bit tricks,
// wave64 cross-lane steps and the base-2 exponential.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;

// bf16 is the top half of an fp32: widening is a shift or a mask.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 with round-to-nearest-even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// c + a.lo*b.lo + a.hi*b.hi with bf16 inputs and fp32 accumulation (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                         c, false);
}

// 2^x on the hardware transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP quad permutes: lane i of each group of 4 reads lane i^1 or lane i^2.
__device__ __forceinline__ float quad_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
}

// Full-wave reductions (ds_bpermute based); used outside the per-tile fast path.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Inclusive prefix sum over the 64 lanes of a wave (Hillis-Steele through lane shuffles).
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

// Item `item` of a list in which sequence s (s < B, in order) owns count(L_s) consecutive items, L_s =
// lens[s]: sets seq, the item's rank inside its sequence and L, all wave-uniform, and returns false
// when the list has fewer than item + 1 items. One lens entry per lane, 64 sequences per step, the
// next step's lengths loaded while this step's counts are summed.
template <typename Count>
__device__ __forceinline__ bool find_item(const int32_t* lens, int B, int item, Count count, int& seq, int& rank,
                                          int& L) {
  const int lane = threadIdx.x & 63;
  int carry = 0;
  int len = lane < B ? lens[lane] : 0;
  for (int base = 0; base < B; base += 64) {
    const int next = base + 64 + lane < B ? lens[base + 64 + lane] : 0;
    const int c = base + lane < B ? count(len) : 0;
    const int incl = wave_inclusive_sum(c);
    const int excl = incl - c;
    const uint64_t hit = __ballot(c > 0 && item >= carry + excl && item < carry + incl);
    if (hit) {
      const int l = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
      seq = base + l;
      rank = __builtin_amdgcn_readfirstlane(item - carry - __shfl(excl, l, 64));
      L = __builtin_amdgcn_readfirstlane(__shfl(len, l, 64));
      return true;
    }
    carry += __shfl(incl, 63, 64);
    len = next;
  }
  return false;
}

// Raw buffer descriptor for `bytes` bytes at a wave-uniform `base` (gfx9 format word 0x00020000).
// Loads through it take a 32-bit lane offset, so no 64-bit vector address is formed per load, and
// any offset at or past `bytes` reads zeros instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t offset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, 0));
}

// ---- codes of 8-bit pools, as the append decides them: the scale amax / 127 (int8) or amax / 448
// (E4M3), the quotient x / scale (correctly rounded), then round half to even and clip (int8) or the
// E4M3 rounding below, every step in fp32.
__device__ __forceinline__ int quantise(float x, float scale) {
  if (scale == 0.f) return 0;
  return (int)fminf(fmaxf(__builtin_rintf(x / scale), -127.f), 127.f);
}

// E4M3 (OCP: 4 exponent bits, bias 7, 3 mantissa bits, largest finite 448) code of a float32 y,
// rounded to the nearest value with ties to the even code, saturated at +-448; the sign bit is y's.
// Below 2^-6 the values are the multiples of 2^-9, so y * 512 rounded is the code itself (8 is the
// smallest normal, 0x08); above, the top 3 mantissa bits are rounded on the other 20, and a carry
// out of the mantissa steps the exponent, which the code's layout does by itself.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fminf(fabsf(y), 448.f);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)__builtin_rintf(a * 512.f);
  } else {
    const uint32_t bits = __float_as_uint(a);
    const uint32_t m = (bits >> 20) & 7u, rest = bits & 0xFFFFFu;
    code = ((((bits >> 23) - 120u) << 3) | m) + ((rest > 0x80000u || (rest == 0x80000u && (m & 1u))) ? 1u : 0u);
    code = min(code, 126u);
  }
  return code | sign;
}

// Value of an E4M3 code (exact in float32).
__device__ __forceinline__ float e4m3_value(uint32_t code) {
  const uint32_t e = (code >> 3) & 0xFu, m = code & 7u;
  const float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (code & 0x80u) ? -v : v;
}

// One code of an 8-bit pool: int8 (x / scale rounded to an integer) or E4M3.
template <bool FP8>
__device__ __forceinline__ uint32_t encode_code(float x, float scale) {
  if constexpr (FP8) return scale == 0.f ? 0u : e4m3_encode(x / scale);
  return (uint32_t)(uint8_t)quantise(x, scale);
}
template <bool FP8>
__device__ __forceinline__ float code_value(uint32_t byte) {
  if constexpr (FP8) return e4m3_value(byte);
  return (float)(int8_t)byte;
}

}  // namespace pa
