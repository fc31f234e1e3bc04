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
    return __uint_as_float(uint32_t(static_cast<const uint16_t*>(p)[i]) << 16);
  } else {
    return static_cast<const float*>(p)[i];
  }
}

template <typename ET>
__device__ __forceinline__ void stf(void* p, int64_t i, float v) {
  if constexpr (sizeof(ET) == 2) {
    static_cast<uint16_t*>(p)[i] = to_bf16_bits(v);
  } else {
    static_cast<float*>(p)[i] = v;
  }
}

// Cache fill after a prompt of T = p.t tokens: slot m receives the prompt token s in
// T-(W-1) .. T-1 with s mod (W-1) == m, or zero when s < 0. One thread per (b, m, d).
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
  const float v = s >= 0 ? ldf<ET>(p.x, b * p.xs0 + s * p.xs1 + d) : 0.f;
  stf<ET>(p.cache, b * p.cs0 + int64_t(m) * p.cs1 + d, v);
}

// The step for channel d of sequence b given its taps w[0..W-1] (float32): y = x_t +
// sum_k w_k x_{t-k}, the ring updated with x_t.
template <typename ET, int W>
__device__ __forceinline__ void decode_channel(const DecodeParams& p, int b, int d, const float (&w)[W]) {
  constexpr int S = W - 1;
  const float xt = ldf<ET>(p.x, b * p.xs0 + d);
  float acc = fmaf(w[0], xt, xt);
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

// Low-rank filters w[b,c,k] = sum_r z[b,r] U[r,cW+k] + bias[cW+k], generated per step.
// A workgroup owns 32 channels (32 W filter columns) and up to 16 sequences. z of those
// sequences and the workgroup's columns of U are staged in LDS as float32 (loads issued
// in batches, so each batch costs one memory latency); two threads per column form it for
// 8 sequences each from LDS; the filters go through LDS to the threads that apply them.
constexpr int kDecCh = 32;
constexpr int kDecSeq = 16;
constexpr int kDecBatch = 32;  // independent loads per thread in flight while staging

// dst[i] = src(i) for i < n, element loads issued kDecBatch at a time per thread.
template <typename F, typename G>
__device__ __forceinline__ void stage(int n, F&& load, G&& store) {
  for (int base = 0; base < n; base += 256 * kDecBatch) {
    float v[kDecBatch];
#pragma unroll
    for (int e = 0; e < kDecBatch; ++e) {
      const int i = base + e * 256 + int(threadIdx.x);
      v[e] = load(i < n ? i : n - 1);
    }
#pragma unroll
    for (int e = 0; e < kDecBatch; ++e) {
      const int i = base + e * 256 + int(threadIdx.x);
      if (i < n) store(i, v[e]);
    }
  }
}

template <typename ET, int W>
__global__ __launch_bounds__(256) void k_lowrank_decode_step(const DecodeParams p) {
  constexpr int HS = kDecSeq / 2;  // sequences per thread
  constexpr int NC = kDecCh * W;   // filter columns of a workgroup
  __shared__ __align__(16) float zs[kDecSeq][128];
  __shared__ float us[128][NC];
  __shared__ float wt[kDecSeq][NC];
  const int tid = threadIdx.x;
  const int c0 = blockIdx.x * kDecCh;
  const int b0 = blockIdx.y * kDecSeq;
  const int nb = min(kDecSeq, p.B - b0);
  const int ncol = min(kDecCh, p.D - c0) * W;
  const int R4 = (p.R + 3) / 4 * 4;  // ranks padded with zeros to whole vectors
  const int64_t j0 = int64_t(c0) * W;
  stage(kDecSeq * R4,
        [&](int i) {
          const int bb = i / R4, r = i % R4;
          return ldf<ET>(p.z, int64_t(b0 + min(bb, nb - 1)) * p.zs0 + min(r, p.R - 1));
        },
        [&](int i, float v) {
          const int bb = i / R4, r = i % R4;
          zs[bb][r] = (bb < nb && r < p.R) ? v : 0.f;
        });
  stage(p.R * ncol, [&](int i) { return ldf<ET>(p.U, int64_t(i / ncol) * p.ldu + j0 + i % ncol); },
        [&](int i, float v) { us[i / ncol][i % ncol] = v; });
  __syncthreads();
  for (int task = tid; task < 2 * ncol; task += 256) {
    const int col = task % ncol, half = task / ncol;
    float acc[HS];
    const float bv = p.bias != nullptr ? ldf<ET>(p.bias, j0 + col) : 0.f;
#pragma unroll
    for (int i = 0; i < HS; ++i) acc[i] = bv;
    for (int r = 0; r < p.R; r += 4) {
      float u[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) u[e] = r + e < p.R ? us[r + e][col] : 0.f;
#pragma unroll
      for (int i = 0; i < HS; ++i) {
        const float4 zv = *reinterpret_cast<const float4*>(&zs[half * HS + i][r]);
        acc[i] = fmaf(zv.x, u[0], fmaf(zv.y, u[1], fmaf(zv.z, u[2], fmaf(zv.w, u[3], acc[i]))));
      }
    }
#pragma unroll
    for (int i = 0; i < HS; ++i) wt[half * HS + i][col] = acc[i];
  }
  __syncthreads();
  for (int i = tid; i < nb * kDecCh; i += 256) {
    const int bb = i / kDecCh, cl = i % kDecCh;
    const int d = c0 + cl;
    if (d >= p.D) continue;
    float w[W];
#pragma unroll
    for (int k = 0; k < W; ++k) w[k] = wt[bb][cl * W + k];
    decode_channel<ET, W>(p, b0 + bb, d, w);
  }
}

template <int W, typename F>
hipError_t by_dtype(dynconv_dtype dt, F&& f) {
  return dt == DYNCONV_BF16 ? f(bf16_t{}, std::integral_constant<int, W>{})
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
  const dim3 grid(unsigned((p.D + kDecCh - 1) / kDecCh), unsigned((p.B + kDecSeq - 1) / kDecSeq));
  return status_of(by_w(W, dt, [&](auto et, auto wc) {
    using ET = decltype(et);
    hipLaunchKernelGGL((k_lowrank_decode_step<ET, decltype(wc)::value>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
  }));
}

}  // namespace dynconv
