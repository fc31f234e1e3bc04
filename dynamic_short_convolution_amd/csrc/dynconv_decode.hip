// Inference kernels of the dynamic short convolution, gfx950: decoding one token at a
// time ("Dynamic Short Convolutions Improve Transformers", reading note, section
// "Parameterization", eq. 2 + eq. 3; the note lists inference as not yet optimised).
//
// A sequence keeps its last W-1 inputs in a ring: token s sits in slot s mod (W-1), and
// slots of positions before 0 hold zeros (the causal zero padding). A step at token t
// reads the ring for taps k = 1..W-1 (slots (t-k) mod (W-1)), then writes x_t into slot
// t mod (W-1) - the slot of token t-(W-1), which the same thread has already read.
// The work per step is a few bytes per channel, so every kernel here is launch bound;
// threads own one channel and loads are coalesced along the channels.
#include <type_traits>

#include "dynconv_common.hpp"
#include "dynconv_decode_internal.hpp"
#include "dynconv_internal.hpp"

namespace dynconv {

namespace {

template <typename ET>
__device__ __forceinline__ float ldf(const void* p, int64_t i) {
  if constexpr (sizeof(ET) == 2) {
    return Cvt<ET>::of_bits(static_cast<const uint16_t*>(p)[i]);
  } else {
    return static_cast<const float*>(p)[i];
  }
}

template <typename ET>
__device__ __forceinline__ void stf(void* p, int64_t i, float v) {
  if constexpr (sizeof(ET) == 2) {
    static_cast<uint16_t*>(p)[i] = Cvt<ET>::bits(v);
  } else {
    static_cast<float*>(p)[i] = v;
  }
}

// Cache fill after a prompt of T = p.t tokens: slot m receives the prompt token s in
// T-(W-1) .. T-1 with s mod (W-1) == m, or zero when s < 0. For a packed prompt, decoding
// continues its last document, so tokens of other segments than token T-1 count as zero
// too. One thread per (b, m, d).
template <typename ET, int W>
__global__ __launch_bounds__(256) void k_cache_fill(const DecodeParams p) {
  constexpr int S = W - 1;
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= int64_t(p.B) * S * p.D) return;
  const int d = int(idx % p.D);
  const int m = int((idx / p.D) % S);
  const int b = int(idx / (int64_t(p.D) * S));
  const int64_t s0 = p.t - S;
  const int64_t s = s0 + (((m - s0) % S) + S) % S;
  bool keep = s >= 0;
  if (keep && p.seg != nullptr) {
    const int32_t* sg = p.seg + b * p.ss0;
    keep = sg[s * p.ss1] == sg[(p.t - 1) * p.ss1];
  }
  const float v = keep ? ldf<ET>(p.x, b * p.xs0 + s * p.xs1 + d) : 0.f;
  stf<ET>(p.cache, b * p.cs0 + int64_t(m) * p.cs1 + d, v);
}

// The step for channel d of sequence b given its taps w[0..W-1] (float32): y = x_t +
// sum_k w_k x_{t-k} (+ the optional convolution bias), the ring updated with x_t.
template <typename ET, int W>
__device__ __forceinline__ void decode_channel(const DecodeParams& p, int b, int d, const float (&w)[W]) {
  constexpr int S = W - 1;
  const float xt = ldf<ET>(p.x, b * p.xs0 + d);
  const float cb = p.cbias != nullptr ? ldf<ET>(p.cbias, d) : 0.f;
  float acc = fmaf(w[0], xt, xt + cb);
  if constexpr (S > 0) {
    const int64_t cb = b * p.cs0 + d;
#pragma unroll
    for (int k = 1; k < W; ++k) {
      const int slot = int((p.t - k) % S + S) % S;
      acc = fmaf(w[k], ldf<ET>(p.cache, cb + slot * p.cs1), acc);
    }
    stf<ET>(p.cache, cb + (p.t % S) * p.cs1, xt);
  }
  stf<ET>(p.y, b * p.ys0 + d, acc);
}

// Materialised (per-token, head-wise or static) filters: one thread per (b, d).
template <typename ET, int W>
__global__ __launch_bounds__(256) void k_decode_step(const DecodeParams p) {
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= int64_t(p.B) * p.D) return;
  const int d = int(idx % p.D);
  const int b = int(idx / p.D);
  const int64_t wb = b * p.ws0 + int64_t(d / p.H) * W;
  float w[W];
#pragma unroll
  for (int k = 0; k < W; ++k) w[k] = ldf<ET>(p.w, wb + k);
  decode_channel<ET, W>(p, b, d, w);
}

// Low-rank filters w[b,c,k] = sum_r z[b,r] U[r,gW+k] + bias[gW+k] with g = c / H (H = 1 per
// channel, H > 1 head-wise: the H channels of a group read the same columns), generated per step on the
// matrix cores. One wave owns 16 sequences x 16 channels. For each tap k the product of the
// z rows and the columns cW+k of U is a 16x16 tile whose lane holds 4 sequences of a single
// channel, so after the W products a lane holds every tap of its 4 (sequence, channel) pairs
// and applies them from registers: no LDS and no barrier. Every global load of the wave (z,
// U, bias, x and the cache) is issued before the first product, so a step costs one memory
// latency. Lane (l, q) = (lane % 16, lane / 16) carries ranks 32s + 8q + e, e < 8, of rank
// step s, for both operands.
typedef __bf16 dec_bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 dec_f16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t dec_u16x8_t __attribute__((ext_vector_type(8)));
typedef float dec_f32x8_t __attribute__((ext_vector_type(8)));
typedef float dec_f32x4_t __attribute__((ext_vector_type(4)));

template <typename ET>
struct DecMma;

template <>
struct DecMma<bf16_t> {
  using RT = uint16_t;        // an element as stored
  using Frag = dec_u16x8_t;   // 8 ranks of one operand row / column
  static __device__ __forceinline__ float to_f(RT v) { return __uint_as_float(uint32_t(v) << 16); }
  static __device__ __forceinline__ Frag load8(const RT* p) {
    return __builtin_bit_cast(Frag, *reinterpret_cast<const u32x4*>(p));
  }
  // 32 ranks in one 16x16x32 product.
  static __device__ __forceinline__ dec_f32x4_t mma(const Frag& a, const Frag& b, dec_f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(dec_bf16x8_t, a),
                                                   __builtin_bit_cast(dec_bf16x8_t, b), c, 0, 0, 0);
  }
};

template <>
struct DecMma<f16_t> {
  using RT = uint16_t;
  using Frag = dec_u16x8_t;
  static __device__ __forceinline__ float to_f(RT v) { return Cvt<f16_t>::of_bits(v); }
  static __device__ __forceinline__ Frag load8(const RT* p) {
    return __builtin_bit_cast(Frag, *reinterpret_cast<const u32x4*>(p));
  }
  static __device__ __forceinline__ dec_f32x4_t mma(const Frag& a, const Frag& b, dec_f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(dec_f16x8_t, a),
                                                  __builtin_bit_cast(dec_f16x8_t, b), c, 0, 0, 0);
  }
};

template <>
struct DecMma<float> {
  using RT = float;
  using Frag = dec_f32x8_t;
  static __device__ __forceinline__ float to_f(RT v) { return v; }
  static __device__ __forceinline__ Frag load8(const RT* p) {
    const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
    return Frag{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  }
  // 32 ranks in eight 16x16x4 products: product e takes rank 32s + 8q + e from lane group q.
  static __device__ __forceinline__ dec_f32x4_t mma(const Frag& a, const Frag& b, dec_f32x4_t c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
    return c;
  }
};

// W consecutive elements at p (one channel's taps); with VEC, W in {2, 4} is one vector load.
template <typename RT, int W, bool VEC>
__device__ __forceinline__ void load_taps(const RT* p, RT (&o)[W]) {
  if constexpr (VEC && (W == 2 || W == 4) && W * sizeof(RT) <= 16) {
    typedef RT V __attribute__((ext_vector_type(W)));
    const V v = *reinterpret_cast<const V*>(p);
#pragma unroll
    for (int k = 0; k < W; ++k) o[k] = v[k];
  } else {
#pragma unroll
    for (int k = 0; k < W; ++k) o[k] = p[k];
  }
}

// VEC: z rows, U rows and bias are aligned for vector loads and R % 8 == 0 (chosen on the
// host, so that each variant's loads form one straight run before the first wait).
template <typename ET, int W, int NK, bool VEC>
__global__ __launch_bounds__(64) void k_lowrank_decode_step(const DecodeParams p) {
  using M = DecMma<ET>;
  using RT = typename M::RT;
  using Frag = typename M::Frag;
  constexpr int S = W - 1;
  const int lane = threadIdx.x, l = lane & 15, q = lane >> 4;
  const int c0 = blockIdx.x * 16, b0 = blockIdx.y * 16;
  const int ca = min(c0 + l, p.D - 1);  // channel of the lane's column (clamped; see stores)
  const int R = p.R;
  const RT* z = static_cast<const RT*>(p.z);
  const RT* U = static_cast<const RT*>(p.U);

  // The lane's pairs: sequences b0 + 4q + i, channel ca; x_t and the cached inputs.
  int slot[W] = {};
  if constexpr (S > 0) {
#pragma unroll
    for (int k = 1; k < W; ++k) slot[k] = int((p.t - k) % S + S) % S;
  }
  float xv[4], cv[4][W];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t b = min(b0 + 4 * q + i, p.B - 1);
    xv[i] = ldf<ET>(p.x, b * p.xs0 + ca);
#pragma unroll
    for (int k = 1; k < W; ++k) cv[i][k] = ldf<ET>(p.cache, b * p.cs0 + slot[k] * p.cs1 + ca);
  }

  // z rows b0 + l (rows past B are clamped, computed and dropped), as the A operand.
  const RT* zr = z + int64_t(min(b0 + l, p.B - 1)) * p.zs0;
  Frag a[NK];
#pragma unroll
  for (int s = 0; s < NK; ++s) {
    const int k0 = 32 * s + 8 * q;
    if constexpr (VEC) {
      const Frag v = M::load8(zr + min(k0, R - 8));
      a[s] = k0 < R ? v : Frag{};
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const RT v = zr[min(k0 + e, R - 1)];
        a[s][e] = k0 + e < R ? v : RT(0);
      }
    }
  }

  // Columns cW + k of U, ranks of step s, as the B operands of tap k.
  Frag bt[NK][W];
#pragma unroll
  for (int s = 0; s < NK; ++s) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = 32 * s + 8 * q + e;
      RT u[W];
      load_taps<RT, W, VEC>(U + int64_t(min(r, R - 1)) * p.ldu + int64_t(ca / p.H) * W, u);
#pragma unroll
      for (int k = 0; k < W; ++k) bt[s][k][e] = r < R ? u[k] : RT(0);
    }
  }
  RT bias[W];
  if (p.bias != nullptr) {
    load_taps<RT, W, VEC>(static_cast<const RT*>(p.bias) + int64_t(ca / p.H) * W, bias);
  } else {
#pragma unroll
    for (int k = 0; k < W; ++k) bias[k] = RT(0);
  }

  const float cb = p.cbias != nullptr ? ldf<ET>(p.cbias, ca) : 0.f;  // optional convolution bias

  // Every load is in flight before the first wait.
  __builtin_amdgcn_sched_barrier(0);

  // Filters (float32, bias as the initial accumulator) and the convolution.
  float y[4];
#pragma unroll
  for (int k = 0; k < W; ++k) {
    const float bk = M::to_f(bias[k]);
    dec_f32x4_t acc = {bk, bk, bk, bk};
#pragma unroll
    for (int s = 0; s < NK; ++s) acc = M::mma(a[s], bt[s][k], acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = k == 0 ? fmaf(acc[i], xv[i], xv[i] + cb) : fmaf(acc[i], cv[i][k], y[i]);
  }
  if (c0 + l >= p.D) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = b0 + 4 * q + i;
    if (b >= p.B) break;
    stf<ET>(p.y, int64_t(b) * p.ys0 + ca, y[i]);
    if constexpr (S > 0) stf<ET>(p.cache, int64_t(b) * p.cs0 + (p.t % S) * p.cs1 + ca, xv[i]);
  }
}

template <int W, typename F>
hipError_t by_dtype(dynconv_dtype dt, F&& f) {
  return dt == DYNCONV_BF16  ? f(bf16_t{}, std::integral_constant<int, W>{})
         : dt == DYNCONV_F16 ? f(f16_t{}, std::integral_constant<int, W>{})
                             : f(float{}, std::integral_constant<int, W>{});
}

template <typename F>
hipError_t by_w(int W, dynconv_dtype dt, F&& f) {
  switch (W) {
    case 1: return by_dtype<1>(dt, f);
    case 2: return by_dtype<2>(dt, f);
    case 3: return by_dtype<3>(dt, f);
    case 4: return by_dtype<4>(dt, f);
    case 5: return by_dtype<5>(dt, f);
    case 6: return by_dtype<6>(dt, f);
    case 7: return by_dtype<7>(dt, f);
    case 8: return by_dtype<8>(dt, f);
    default: return hipErrorInvalidValue;
  }
}

dynconv_status status_of(hipError_t e) { return e == hipSuccess ? DYNCONV_OK : record_hip_error(e); }

}  // namespace

dynconv_status launch_cache_fill(const DecodeParams& p, int W, dynconv_dtype dt, hipStream_t s) {
  if (W == 1) return DYNCONV_OK;
  const int64_t n = int64_t(p.B) * (W - 1) * p.D;
  const unsigned blocks = unsigned((n + 255) / 256);
  return status_of(by_w(W, dt, [&](auto et, auto wc) {
    using ET = decltype(et);
    constexpr int WV = decltype(wc)::value;
    if constexpr (WV > 1) hipLaunchKernelGGL((k_cache_fill<ET, WV>), dim3(blocks), dim3(256), 0, s, p);
    return hipGetLastError();
  }));
}

dynconv_status launch_decode_step(const DecodeParams& p, int W, dynconv_dtype dt, hipStream_t s) {
  const int64_t n = int64_t(p.B) * p.D;
  const unsigned blocks = unsigned((n + 255) / 256);
  return status_of(by_w(W, dt, [&](auto et, auto wc) {
    using ET = decltype(et);
    hipLaunchKernelGGL((k_decode_step<ET, decltype(wc)::value>), dim3(blocks), dim3(256), 0, s, p);
    return hipGetLastError();
  }));
}

dynconv_status launch_lowrank_decode_step(const DecodeParams& p, int W, dynconv_dtype dt, hipStream_t s) {
  const unsigned gy = unsigned((p.B + 15) / 16);
  if (gy > 65535u) return DYNCONV_ERR_UNSUPPORTED;
  const dim3 grid(unsigned((p.D + 15) / 16), gy);
  const int nk = (p.R + 31) / 32;
  const size_t eb = dt == DYNCONV_F32 ? 4 : 2;
  const auto al = [](const void* q, size_t a) { return reinterpret_cast<uintptr_t>(q) % a == 0; };
  const bool vec = p.R % 8 == 0 && (p.zs0 * eb) % 16 == 0 && al(p.z, 16) && p.ldu % W == 0 && al(p.U, W * eb) &&
                   (p.bias == nullptr || al(p.bias, W * eb));
  return status_of(by_w(W, dt, [&](auto et, auto wc) {
    using ET = decltype(et);
    constexpr int WV = decltype(wc)::value;
    const auto go = [&](auto nkc) {
      constexpr int NK = decltype(nkc)::value;
      if constexpr (WV > kMaxLowrankW) {
        return hipErrorInvalidValue;  // rejected by the C ABI before this point
      } else {
        if (vec) {
          hipLaunchKernelGGL((k_lowrank_decode_step<ET, WV, NK, true>), grid, dim3(64), 0, s, p);
        } else {
          hipLaunchKernelGGL((k_lowrank_decode_step<ET, WV, NK, false>), grid, dim3(64), 0, s, p);
        }
        return hipGetLastError();
      }
    };
    switch (nk) {
      case 1: return go(std::integral_constant<int, 1>{});
      case 2: return go(std::integral_constant<int, 2>{});
      case 3: return go(std::integral_constant<int, 3>{});
      case 4: return go(std::integral_constant<int, 4>{});
      default: return hipErrorInvalidValue;
    }
  }));
}

}  // namespace dynconv
