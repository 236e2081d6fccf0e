// gqa_device.h -- device-side types and helpers shared by the kernels of libgqa (decode, cache
// append, prefill): vector types, buffer descriptors and cache policies, bf16 and fp8 conversions,
// cross-lane reductions, uniform values and output stores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace gqa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

#define GQA_LDS __attribute__((address_space(3)))
// Constant address space: a uniform read through it is a scalar load, which waits on no vector load.
#define GQA_CONST __attribute__((address_space(4)))

// Raw-buffer descriptor word 3 for gfx950 (32-bit data format, no swizzle, range checked).
constexpr int kBufferFlags = 0x00020000;
// Cache policy of the cache-streaming loads: non-temporal (each byte is read once per step).
constexpr int kStreamPolicy = 2;
// Cache policy of workspace traffic between workgroups: agent scope (sc1), the bits the compiler
// gives agent-scope atomic loads and stores, coherent across the per-XCD L2 caches.
constexpr int kAgentScope = 16;
// Byte offset used for loads of tiles that do not exist: beyond every descriptor's range, so the
// load returns zeros without touching memory.
constexpr uint32_t kNoTile = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufferFlags);
}

__device__ __forceinline__ u32x4_t load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kStreamPolicy));
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) {
  return __builtin_bit_cast(float, h << 16);
}

// Round-to-nearest-even float -> bf16 bit pattern (NaN stays NaN).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u | ((u >> 16) & 0x8000u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats to a bf16 pair (round to nearest even), one v_cvt_pk_bf16_f32; lo in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// Two fp8-e4m3fn codes (the low or high 16 bits of `w`) -> two bf16 in one dword.  Exact: every
// e4m3fn value is representable in bf16.  The result is used as a whole dword only.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

__device__ __forceinline__ u32x4_t fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  return u32x4_t{fp8x2_to_bf16x2<false>(lo), fp8x2_to_bf16x2<true>(lo), fp8x2_to_bf16x2<false>(hi),
                 fp8x2_to_bf16x2<true>(hi)};
}

__device__ __forceinline__ float wave_max_xor_16_32(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_sum_xor_16_32(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

// Values every lane agrees on are moved to scalar registers, so that everything derived from them
// (buffer descriptors in particular) stays uniform in the compiler's view.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

template <typename OutT>
__device__ __forceinline__ void store_out(OutT* p, float x);
template <>
__device__ __forceinline__ void store_out<float>(float* p, float x) { *p = x; }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* p, float x) {
  *p = (uint16_t)float_to_bf16_bits(x);
}
// Four consecutive outputs (16-byte aligned for f32, 8-byte aligned for bf16).
template <typename OutT>
__device__ __forceinline__ void store_out4(OutT* p, f32x4_t x);
template <>
__device__ __forceinline__ void store_out4<float>(float* p, f32x4_t x) {
  *reinterpret_cast<f32x4_t*>(p) = x;
}
template <>
__device__ __forceinline__ void store_out4<uint16_t>(uint16_t* p, f32x4_t x) {
  *reinterpret_cast<u32x2_t*>(p) = u32x2_t{float_to_bf16_bits(x[0]) | (float_to_bf16_bits(x[1]) << 16),
                                           float_to_bf16_bits(x[2]) | (float_to_bf16_bits(x[3]) << 16)};
}

// e4m3fn code of x / descale: binary32 division, then round to nearest even, saturating at +-448
// (infinities included); a NaN x gives 0x7F with its sign bit.
__device__ __forceinline__ uint32_t float_to_fp8_e4m3_bits(float x, float descale) {
  const uint32_t ux = __builtin_bit_cast(uint32_t, x);
  if ((ux & 0x7fffffffu) > 0x7f800000u) return 0x7fu | ((ux >> 24) & 0x80u);  // NaN
  const float y = __fdiv_rn(x, descale);
  const uint32_t u = __builtin_bit_cast(uint32_t, y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a >= 0x43e00000u) return 0x7eu | sign;  // |y| >= 448
  if (a < 0x3c800000u) {                      // |y| < 2^-6: multiples of 2^-9 (8 is the smallest normal)
    return sign | (uint32_t)__builtin_rintf(__builtin_bit_cast(float, a) * 512.0f);
  }
  // keep three mantissa bits, rounding to nearest even, then move the exponent bias from 127 to 7
  const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
  return sign | (r - (120u << 3));
}

}  // namespace gqa
