// Device helpers shared by the dynamic short convolution kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dynconv {

// Storage element types. bf16 travels as raw 16-bit patterns; every product and sum
// is float32; bf16 results are rounded to nearest even by v_cvt_pk_bf16_f32.
struct bf16_t {
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

// ---------------------------------------------------------------------------------
// N contiguous elements starting at an address aligned to min(16, N * sizeof) bytes
// (4 bytes at least), converted to float.
// ---------------------------------------------------------------------------------
template <typename ET, int N>
struct Vec;

template <int N>
struct Vec<bf16_t, N> {
  static_assert(N % 2 == 0, "bf16 vectors hold an even number of elements");
  static __device__ __forceinline__ void load(const bf16_t* p, float (&o)[N]) {
    if constexpr (N == 8) {
      u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[2 * i] = bf16_lo(u[i]);
        o[2 * i + 1] = bf16_hi(u[i]);
      }
    } else {
      const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
      for (int i = 0; i < N / 2; ++i) {
        uint32_t u = q[i];
        o[2 * i] = bf16_lo(u);
        o[2 * i + 1] = bf16_hi(u);
      }
    }
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float (&v)[N]) {
    if constexpr (N == 8) {
      u32x4 u;
#pragma unroll
      for (int i = 0; i < 4; ++i) u[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
      *reinterpret_cast<u32x4*>(p) = u;
    } else {
      uint32_t* q = reinterpret_cast<uint32_t*>(p);
#pragma unroll
      for (int i = 0; i < N / 2; ++i) q[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    }
  }
};

template <int N>
struct Vec<float, N> {
  static __device__ __forceinline__ void load(const float* p, float (&o)[N]) {
    if constexpr (N == 4) {
      float4 u = *reinterpret_cast<const float4*>(p);
      o[0] = u.x;
      o[1] = u.y;
      o[2] = u.z;
      o[3] = u.w;
    } else {
#pragma unroll
      for (int i = 0; i < N; ++i) o[i] = p[i];
    }
  }
  static __device__ __forceinline__ void store(float* p, const float (&v)[N]) {
    if constexpr (N == 4) {
      *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
      for (int i = 0; i < N; ++i) p[i] = v[i];
    }
  }
};

// N contiguous elements with only natural (element) alignment.
template <typename ET, int N>
__device__ __forceinline__ void load_unaligned(const ET* p, float (&o)[N]) {
  if constexpr (sizeof(ET) == 2) {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(p);
#pragma unroll
    for (int i = 0; i < N; ++i) o[i] = __uint_as_float(uint32_t(q[i]) << 16);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) o[i] = reinterpret_cast<const float*>(p)[i];
  }
}

template <typename ET, int N>
__device__ __forceinline__ void store_unaligned(ET* p, const float (&v)[N]) {
  if constexpr (sizeof(ET) == 2) {
    uint16_t* q = reinterpret_cast<uint16_t*>(p);
#pragma unroll
    for (int i = 0; i < N; ++i) q[i] = to_bf16_bits(v[i]);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) reinterpret_cast<float*>(p)[i] = v[i];
  }
}

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
