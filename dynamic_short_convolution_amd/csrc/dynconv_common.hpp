// Device helpers shared by the dynamic short convolution kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dynconv {

// Storage element types. bf16 and fp16 travel as raw 16-bit patterns; every product and
// sum is float32; 16-bit results are rounded to nearest even (v_cvt_pk_bf16_f32,
// v_cvt_f16_f32).
struct bf16_t {
  uint16_t bits;
};
struct f16_t {
  uint16_t bits;
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Conversions of a 16-bit storage type: the low / high half of a 32-bit word to float, a
// pair of floats to a word, one float to its bits (round to nearest even).
template <typename ET>
struct Cvt;

template <>
struct Cvt<bf16_t> {
  static __device__ __forceinline__ float lo(uint32_t u) { return bf16_lo(u); }
  static __device__ __forceinline__ float hi(uint32_t u) { return bf16_hi(u); }
  static __device__ __forceinline__ float of_bits(uint32_t h) { return __uint_as_float(h << 16); }
  static __device__ __forceinline__ uint32_t pack2(float l, float h) { return pack_bf16x2(l, h); }
  static __device__ __forceinline__ uint16_t bits(float f) { return to_bf16_bits(f); }
};

template <>
struct Cvt<f16_t> {
  static __device__ __forceinline__ float of_bits(uint32_t h) {
    return float(__builtin_bit_cast(_Float16, uint16_t(h)));
  }
  static __device__ __forceinline__ float lo(uint32_t u) { return of_bits(u & 0xffffu); }
  static __device__ __forceinline__ float hi(uint32_t u) { return of_bits(u >> 16); }
  static __device__ __forceinline__ uint16_t bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
  static __device__ __forceinline__ uint32_t pack2(float l, float h) {
    return uint32_t(bits(l)) | (uint32_t(bits(h)) << 16);
  }
};

// ---------------------------------------------------------------------------------
// Workgroups are dispatched round-robin over the 8 XCDs (workgroup i runs on XCD i % 8),
// and each XCD has its own L2. This bijection renumbers workgroups so that consecutive
// logical ids run on the same XCD, which lets neighbouring time tiles (which share a
// W-1 token halo) meet in the same L2.
// ---------------------------------------------------------------------------------
constexpr int kNumXcd = 8;

__device__ __forceinline__ uint32_t xcd_logical_block(uint32_t bid, uint32_t nblocks) {
  const uint32_t q = nblocks / kNumXcd;
  const uint32_t r = nblocks % kNumXcd;
  const uint32_t x = bid % kNumXcd;
  return x * q + (x < r ? x : r) + bid / kNumXcd;
}

}  // namespace dynconv
