// Matrix-core tile helpers shared by the decode kernels of libpa.so (gfx950): the operand types, the
// per-wave V tile layout in LDS, the exact widenings of 8-bit codes into MFMA operands, and the
// constants of a 16-position tile of 128-element rows.
#pragma once

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace mfma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr int kTile = 16;
constexpr int kRowBytes = 256;  // 128 bf16
constexpr int kD = 128;
constexpr int kTileBytes = kTile * kRowBytes;
constexpr float kRefSlack = 64.0f;  // base-2 units a score may exceed the reference max by

// A view of memory no part of the launch writes (tables, lengths, scales), in the constant address
// space: uniform loads through it stay scalar loads even after the launch's own stores (partials, the
// fused append's rows), which would otherwise make the compiler fall back to vector loads and waits.
template <class T>
__device__ __forceinline__ const __attribute__((address_space(4))) T* read_only(const T* ptr) {
  return (const __attribute__((address_space(4))) T*)ptr;
}

// Byte offset of (position t, byte b of its 256-byte row) inside one V tile in LDS.
__device__ __forceinline__ int v_swz(int t, int b) { return t * kRowBytes + (b ^ ((t & 7) << 5)); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

// Four int8 codes (one dword) -> two dwords of fp16 values 1152 + code: flip the sign bit of each
// byte (code + 128 as unsigned u), then pair each u with the exponent byte 0x64 (fp16 1024 + u).
__device__ __forceinline__ u32x2 codes_to_f16(uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;
  return u32x2{__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u),   // bytes u0, 0x64, u1, 0x64
               __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)};  // bytes u2, 0x64, u3, 0x64
}

// Four int8 codes -> two dwords of bf16 values 128 + code (exact: integers below 256).
__device__ __forceinline__ u32x2 codes_to_bf16(uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;
  const bf16x2v a = {(__bf16)(float)(u & 0xffu), (__bf16)(float)((u >> 8) & 0xffu)};
  const bf16x2v b = {(__bf16)(float)((u >> 16) & 0xffu), (__bf16)(float)(u >> 24)};
  return u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
}

// Four E4M3 codes (one dword) -> two dwords of bf16, exactly: every E4M3 value is a bf16 value
// (v_cvt_scalef32_pk_bf16_fp8 with scale 1; bytes 0-1, then bytes 2-3).
__device__ __forceinline__ u32x2 fp8_to_bf16(uint32_t w) {
  return u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))};
}

constexpr float kKOffset = 1152.f;  // fp16 K code value minus the code
constexpr float kVOffset = 128.f;   // bf16 V code value minus the code

// Round-to-nearest-even packing of two fp32 into bf16 (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  const bf16x2v v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ void wave_lds_order() {
  // one wave reads back LDS it wrote; its LDS operations execute in order
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace mfma
}  // namespace pa
