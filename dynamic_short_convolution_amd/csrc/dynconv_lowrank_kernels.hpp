// General low-rank kernels, instantiated once per storage type by
// dynconv_lowrank_{f32,bf16,f16}.hip so that the three compile in parallel.
#pragma once

// Low-rank dynamic short convolution for gfx950: the filters w = z U + b are formed on
// the matrix cores and consumed on-chip; they never reach HBM.
//
// From "Dynamic Short Convolutions Improve Transformers" (reading note): section
// "Parameterization" (low-rank generator D -> R -> W*D, affine; eq. 2 and eq. 3) and
// section "Efficient training (Triton kernels)" (the fused kernel reads z and U,
// generates z U on-chip and applies the convolution at once).
//
// Kernels
//   k_lowrank_fwd   per (sequence, token range, 64-channel slice) workgroup, per 16-token
//                   tile: z tile -> LDS; MFMA  W^T[j][n] = sum_r U[r][j] z[n][r] + b[j]
//                   (M = filter columns j = c*W + k, N = tokens, K = rank); the filter tile
//                   goes to LDS as float32; the conv + residual reads x from an LDS ring
//                   that keeps the W-1 previous tokens.
//   k_lowrank_bwd   same decomposition, one tile behind the filter regeneration so that
//                   the future halo of dx (w and dy of the next W-1 tokens) is on-chip;
//                   produces dx, the per-token filter gradient g = dw (LDS only), and
//                   accumulates dU += z^T g (MFMA, K = tokens) and db += g in registers
//                   over the token range; writes one float32 partial per token range.
//   k_lowrank_dz    per (sequence, 64-token block): dz = g U^T (MFMA, K = filter columns)
//                   with g recomputed from x and dy, looping over channel chunks, so dz is
//                   complete without partial sums (register-staged: any type and shape).
//   k_lowrank_dz_dma the same for bf16 whole token blocks, staged by LDS DMA; head-wise
//                   groups of 2 or 4 channels are summed before the matrix step.
//   partial sums of dU and db are then added in a fixed order (run-to-run deterministic).
#include <type_traits>

#include "dynconv_common.hpp"
#include "dynconv_internal.hpp"
#include "dynconv_lowrank_internal.hpp"

namespace dynconv {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int TT = kLowrankTT;  // tokens per tile (the N, or K, extent of one MFMA)
// Rows staged before a token range or step: the W - 1 earlier tokens a filter reaches (at
// least 4, so that the tilings of W <= 5 stay as they are).
constexpr int lr_halo(int W) { return W <= 5 ? 4 : W - 1; }

// Raw storage of an element in LDS / fragments: bf16 bits or float32.
template <typename ET>
struct Raw;
template <>
struct Raw<bf16_t> {
  using type = uint16_t;
  static __device__ __forceinline__ uint16_t from_mem(const bf16_t* p, int64_t i) {
    return reinterpret_cast<const uint16_t*>(p)[i];
  }
  static __device__ __forceinline__ uint16_t from_float(float f) { return to_bf16_bits(f); }
  static __device__ __forceinline__ float to_float(uint16_t u) { return __uint_as_float(uint32_t(u) << 16); }
  static __device__ __forceinline__ uint16_t zero() { return 0; }
};
template <>
struct Raw<f16_t> {
  using type = uint16_t;
  static __device__ __forceinline__ uint16_t from_mem(const f16_t* p, int64_t i) {
    return reinterpret_cast<const uint16_t*>(p)[i];
  }
  static __device__ __forceinline__ uint16_t from_float(float f) { return Cvt<f16_t>::bits(f); }
  static __device__ __forceinline__ float to_float(uint16_t u) { return Cvt<f16_t>::of_bits(u); }
  static __device__ __forceinline__ uint16_t zero() { return 0; }
};
template <>
struct Raw<float> {
  using type = float;
  static __device__ __forceinline__ float from_mem(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ float from_float(float f) { return f; }
  static __device__ __forceinline__ float to_float(float f) { return f; }
  static __device__ __forceinline__ float zero() { return 0.f; }
};

// MFMA flavours. Fragment element e of lane l (q = l / 16) holds K index kNN(q, e):
//   bf16: v_mfma_f32_16x16x32_bf16 (K = 32, 8 elements per lane, k = 8q + e) and
//         v_mfma_f32_16x16x16_bf16 (K = 16, 4 elements per lane, k = 4q + e);
//   f32:  v_mfma_f32_16x16x4_f32 issued 8 (or 4) times, k = 4e + q.
// A is indexed [row = l % 16][k], B is [k][col = l % 16]; the 16x16 float32 result has
// lane l holding rows 4q + i (i < 4) of column l % 16.
template <typename ET>
struct Mfma;

template <>
struct Mfma<bf16_t> {
  struct F32k {
    u16x8_t v;
  };
  struct F16k {
    u16x4_t v;
  };
  static __device__ __forceinline__ int k32(int q, int e) { return 8 * q + e; }
  static __device__ __forceinline__ int k16(int q, int e) { return 4 * q + e; }
  static __device__ __forceinline__ f32x4_t mma32(const F32k& a, const F32k& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.v), __builtin_bit_cast(bf16x8_t, b.v),
                                                   c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t mma16(const F16k& a, const F16k& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a.v), __builtin_bit_cast(s16x4_t, b.v),
                                                     c, 0, 0, 0);
  }
};

template <>
struct Mfma<f16_t> {
  struct F32k {
    u16x8_t v;
  };
  struct F16k {
    u16x4_t v;
  };
  static __device__ __forceinline__ int k32(int q, int e) { return 8 * q + e; }
  static __device__ __forceinline__ int k16(int q, int e) { return 4 * q + e; }
  static __device__ __forceinline__ f32x4_t mma32(const F32k& a, const F32k& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a.v), __builtin_bit_cast(f16x8_t, b.v),
                                                  c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t mma16(const F16k& a, const F16k& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a.v), __builtin_bit_cast(f16x4_t, b.v),
                                                 c, 0, 0, 0);
  }
};

template <>
struct Mfma<float> {
  struct F32k {
    float v[8];
  };
  struct F16k {
    float v[4];
  };
  static __device__ __forceinline__ int k32(int q, int e) { return 4 * e + q; }
  static __device__ __forceinline__ int k16(int q, int e) { return 4 * e + q; }
  static __device__ __forceinline__ f32x4_t mma32(const F32k& a, const F32k& b, f32x4_t c) {
#pragma unroll
    for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[s], b.v[s], c, 0, 0, 0);
    return c;
  }
  static __device__ __forceinline__ f32x4_t mma16(const F16k& a, const F16k& b, f32x4_t c) {
#pragma unroll
    for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[s], b.v[s], c, 0, 0, 0);
    return c;
  }
};

// Block -> (sequence b, token range tr, channel slice cs), channel slice fastest, so the
// workgroups that share a z tile run on the same XCD at about the same time. A launch
// covers the channel slices cs0 .. cs0 + nCsL - 1.
struct LrBlock {
  int b, tr, cs;
};
__device__ __forceinline__ LrBlock lr_block(const LowRankParams& p) {
  uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
  LrBlock r;
  r.cs = p.cs0 + int(lb % uint32_t(p.nCsL));
  lb /= uint32_t(p.nCsL);
  r.tr = lb % p.nTr;
  r.b = lb / p.nTr;
  return r;
}

// Slot of token t in the x ring of one workgroup (tokens t_first - HALO .. kept).
template <int HALO, int RING>
__device__ __forceinline__ int ring_slot(int t, int t_first) { return (t - t_first + HALO) % RING; }

// ---------------------------------------------------------------------------------
// 16-byte staging of activation / z rows: one chunk = 16 bytes of consecutive elements.
// Vector load when the tensor allows it and the chunk is whole; element loads (zero
// past `limit`) otherwise.
// ---------------------------------------------------------------------------------
template <typename ET>
__device__ __forceinline__ u32x4 load_chunk(const ET* row, int c, int limit, bool vec_ok) {
  constexpr int E = 16 / int(sizeof(ET));
  if (vec_ok && c + E <= limit) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + c));
  u32x4 r = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (c + e < limit) {
      if constexpr (sizeof(ET) == 2) {
        const uint32_t h = reinterpret_cast<const uint16_t*>(row)[c + e];
        r[e / 2] |= (e & 1) ? (h << 16) : h;
      } else {
        r[e] = __float_as_uint(reinterpret_cast<const float*>(row)[c + e]);
      }
    }
  }
  return r;
}

// Head-wise low-rank: 16 bytes of per-channel filter columns jj = j0 .. of the channels from
// c0 (column jj is tap jj % W of channel c0 + jj / W), read from the U row of their groups
// (column ((c0 + jj / W) / H) * W + jj % W); the first `limit` (>= 1) are valid.
template <typename ET>
__device__ __forceinline__ u32x4 load_group_cols(const ET* urow, int c0, int j0, int limit, int W, int H) {
  constexpr int E = 16 / int(sizeof(ET));
  u32x4 r = {0u, 0u, 0u, 0u};
  uint32_t h[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int jj = j0 + min(e, limit - 1);
    const int64_t col = int64_t((c0 + jj / W) / H) * W + jj % W;
    if constexpr (sizeof(ET) == 2) {
      h[e] = reinterpret_cast<const uint16_t*>(urow)[col];
    } else {
      h[e] = __float_as_uint(reinterpret_cast<const float*>(urow)[col]);
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t v = e < limit ? h[e] : 0u;
    if constexpr (sizeof(ET) == 2) {
      r[e / 2] |= (e & 1) ? (v << 16) : v;
    } else {
      r[e] = v;
    }
  }
  return r;
}

// The first `limit` (>= 1) of the 16 bytes at row[0 ..] by element loads, all issued
// before any is used (indices clamped into the row, the tail masked afterwards).
template <typename ET>
__device__ __forceinline__ u32x4 load_elems16(const ET* row, int limit) {
  constexpr int E = 16 / int(sizeof(ET));
  u32x4 r = {0u, 0u, 0u, 0u};
  uint32_t h[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = min(e, limit - 1);
    if constexpr (sizeof(ET) == 2) {
      h[e] = reinterpret_cast<const uint16_t*>(row)[i];
    } else {
      h[e] = __float_as_uint(reinterpret_cast<const float*>(row)[i]);
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t v = e < limit ? h[e] : 0u;
    if constexpr (sizeof(ET) == 2) {
      r[e / 2] |= (e & 1) ? (v << 16) : v;
    } else {
      r[e] = v;
    }
  }
  return r;
}

// A run of N contiguous elements in LDS, aligned to min(16, N * sizeof) bytes.
template <typename ET, int N>
__device__ __forceinline__ void lds_read_run(const ET* p, float (&o)[N]) {
  constexpr int BYTES = N * int(sizeof(ET));
  const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
  uint32_t u[BYTES / 4];
  if constexpr (BYTES % 16 == 0) {
#pragma unroll
    for (int i = 0; i < BYTES / 16; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(q + 4 * i);
      u[4 * i] = v[0];
      u[4 * i + 1] = v[1];
      u[4 * i + 2] = v[2];
      u[4 * i + 3] = v[3];
    }
  } else if constexpr (BYTES == 8) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(q);
    u[0] = v[0];
    u[1] = v[1];
  } else {
#pragma unroll
    for (int i = 0; i < BYTES / 4; ++i) u[i] = q[i];
  }
#pragma unroll
  for (int e = 0; e < N; ++e) {
    if constexpr (sizeof(ET) == 2) {
      o[e] = (e & 1) ? Cvt<ET>::hi(u[e >> 1]) : Cvt<ET>::lo(u[e >> 1]);
    } else {
      o[e] = __uint_as_float(u[e]);
    }
  }
}

// A run of N contiguous elements to global memory: vector stores when `vec` (the address
// is then aligned to min(16, N * sizeof) bytes), element stores of the first `count`
// elements otherwise.
template <typename ET, int N>
__device__ __forceinline__ void global_store_run(ET* p, const float (&v)[N], bool vec, int count) {
  constexpr int BYTES = N * int(sizeof(ET));
  if (vec && count >= N) {
    uint32_t u[BYTES / 4];
#pragma unroll
    for (int i = 0; i < BYTES / 4; ++i) {
      if constexpr (sizeof(ET) == 2) {
        u[i] = Cvt<ET>::pack2(v[2 * i], v[2 * i + 1]);
      } else {
        u[i] = __float_as_uint(v[i]);
      }
    }
    uint32_t* q = reinterpret_cast<uint32_t*>(p);
    if constexpr (BYTES % 16 == 0) {
#pragma unroll
      for (int i = 0; i < BYTES / 16; ++i)
        *reinterpret_cast<u32x4*>(q + 4 * i) = u32x4{u[4 * i], u[4 * i + 1], u[4 * i + 2], u[4 * i + 3]};
    } else if constexpr (BYTES == 8) {
      *reinterpret_cast<u32x2*>(q) = u32x2{u[0], u[1]};
    } else {
#pragma unroll
      for (int i = 0; i < BYTES / 4; ++i) q[i] = u[i];
    }
    return;
  }
#pragma unroll
  for (int e = 0; e < N; ++e) {
    if (e < count) {
      if constexpr (sizeof(ET) == 2) {
        reinterpret_cast<uint16_t*>(p)[e] = Cvt<ET>::bits(v[e]);
      } else {
        reinterpret_cast<float*>(p)[e] = v[e];
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// Forward
//
// Filter generation (MFMA, M = filter rows, N = 16 tokens, K = rank): the rows of the
// wave's MT tiles are assigned so that, in the result, lane (token n = l % 16, group
// q = l / 16) holds for each tile mt the taps 4*(q % LPC) .. +3 of channel
//   cw0 + (q / LPC) * MT + mt,
// i.e. every lane ends up with the filters of a run of MT contiguous channels of one
// token. The conv then reads 16-byte rows of x from an LDS ring (the tile's 16 tokens
// plus 4 earlier ones) and writes MT contiguous outputs of y per lane.
// ---------------------------------------------------------------------------------
template <typename ET, int W, int KS>
__global__ __launch_bounds__(kBlockThreads) void k_lowrank_fwd(const LowRankParams p) {
  using RT = typename Raw<ET>::type;
  constexpr int EB = int(sizeof(ET));
  constexpr int MT = lowrank_fwd_mt(KS);
  constexpr int LPC = lowrank_rows_per_channel(W) / 4;  // lane groups per channel
  constexpr int CPW = MT * 4 / LPC;                      // channels per wave
  constexpr int DC = 4 * CPW;                            // channels per workgroup
  constexpr int RP = 32 * KS;
  constexpr int ZP = RP + 16 / EB;                       // z row pitch (elements)
  constexpr int XP = DC + 16 / EB;                       // x row pitch (elements)
  constexpr int CE = 16 / EB;                            // elements per 16-byte chunk
  constexpr int XCH = (TT * DC / CE + kBlockThreads - 1) / kBlockThreads;  // x chunks per thread
  constexpr int ZCH = (TT * RP / CE + kBlockThreads - 1) / kBlockThreads;  // z chunks per thread
  static_assert(DC % CE == 0 && RP % CE == 0, "tiles hold whole 16-byte chunks");
  constexpr int HALO = lr_halo(W);
  constexpr int RING = TT + HALO;
  __shared__ __align__(16) RT zl[TT * ZP];
  __shared__ __align__(16) ET xl[RING * XP];
  __shared__ int sl[RING];  // segment ids of the ring's tokens (packed sequences)

  const LrBlock blk = lr_block(p);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int q = lane >> 4;
  const int n = lane & 15;
  const int wv = tid >> 6;
  const int c_base = blk.cs * DC;
  const int t_first = blk.tr * p.Ltok;
  const int t_end = min(p.T, t_first + p.Ltok);
  if (t_first >= p.T) return;
  const ET* x = static_cast<const ET*>(p.x) + blk.b * p.xs0;
  const ET* z = static_cast<const ET*>(p.z) + blk.b * p.zs0;
  ET* y = static_cast<ET*>(p.out) + blk.b * p.os0;
  const bool act16 = p.act16 != 0;
  const bool z16 = p.z16 != 0;
  // packed sequences: tap k of token t is present only when token t-k has t's segment id
  const bool segs = p.seg != nullptr;
  const int32_t* sgp = segs ? p.seg + blk.b * p.ss0 : nullptr;

  // A operands (U columns in the lane-run order above) and bias, once per workgroup.
  const int cw0 = c_base + wv * CPW;
  typename Mfma<ET>::F32k afr[MT][KS];
  f32x4_t binit[MT];
  {
    const ET* U = static_cast<const ET*>(p.U);
    const ET* bias = static_cast<const ET*>(p.bias);
    const int m = n;  // A row held by this lane
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int ch = cw0 + ((m >> 2) / LPC) * MT + mt;
      const int tap = 4 * ((m >> 2) % LPC) + (m & 3);
      const bool ok = ch < p.D && tap < W;
      const int64_t col = int64_t(ch / p.H) * W + tap;  // group ch / H (head-wise: H > 1)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 32 * ks + Mfma<ET>::k32(q, e);
          afr[mt][ks].v[e] = (ok && r < p.R) ? Raw<ET>::from_mem(U, int64_t(r) * p.ldu + col) : Raw<ET>::zero();
        }
      const int chq = cw0 + (q / LPC) * MT + mt;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tq = 4 * (q % LPC) + i;
        binit[mt][i] = (bias != nullptr && chq < p.D && tq < W)
                           ? Raw<ET>::to_float(Raw<ET>::from_mem(bias, int64_t(chq / p.H) * W + tq))
                           : 0.f;
      }
    }
  }

  // Staging of one tile: z rows (zero past the range / R) and x rows (zero past D); the
  // loads of tile i+1 are issued before tile i is computed.
  u32x4 zpre_s[1][ZCH], xpre_s[1][XCH];
  int spre = INT32_MIN;
  auto prefetch = [&](u32x4 (&zpre)[ZCH], u32x4 (&xpre)[XCH], int t0) {
    if (segs && tid < TT) spre = t0 + tid < t_end ? sgp[int64_t(t0 + tid) * p.ss1] : INT32_MIN;
#pragma unroll
    for (int i = 0; i < ZCH; ++i) {
      const int ck = tid + i * kBlockThreads;
      zpre[i] = u32x4{0u, 0u, 0u, 0u};
      if (ck < TT * RP / CE) {
        const int row = ck / (RP / CE);
        const int c = (ck % (RP / CE)) * CE;
        const int t = t0 + row;
        if (t < t_end) zpre[i] = load_chunk<ET>(z + int64_t(t) * p.zs1, c, p.R, z16);
      }
    }
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int ck = tid + i * kBlockThreads;
      xpre[i] = u32x4{0u, 0u, 0u, 0u};
      if (ck < TT * DC / CE) {
        const int row = ck / (DC / CE);
        const int c = (ck % (DC / CE)) * CE;
        const int t = t0 + row;
        if (t < t_end) xpre[i] = load_chunk<ET>(x + int64_t(t) * p.xs1 + c_base, c, p.D - c_base, act16);
      }
    }
  };
  auto commit = [&](const u32x4 (&zpre)[ZCH], const u32x4 (&xpre)[XCH], int t0) {
#pragma unroll
    for (int i = 0; i < ZCH; ++i) {
      const int ck = tid + i * kBlockThreads;
      if (ck < TT * RP / CE)
        *reinterpret_cast<u32x4*>(&zl[(ck / (RP / CE)) * ZP + (ck % (RP / CE)) * CE]) = zpre[i];
    }
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int ck = tid + i * kBlockThreads;
      if (ck < TT * DC / CE) {
        const int row = ck / (DC / CE);
        *reinterpret_cast<u32x4*>(&xl[ring_slot<HALO, RING>(t0 + row, t_first) * XP + (ck % (DC / CE)) * CE]) = xpre[i];
      }
    }
    if (segs && tid < TT) sl[ring_slot<HALO, RING>(t0 + tid, t_first)] = spre;
  };

  // halo: the HALO tokens before the range
  for (int ck = tid; ck < HALO * DC / CE; ck += kBlockThreads) {
    const int row = ck / (DC / CE);
    const int c = (ck % (DC / CE)) * CE;
    const int t = t_first - HALO + row;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (t >= 0) v = load_chunk<ET>(x + int64_t(t) * p.xs1 + c_base, c, p.D - c_base, act16);
    *reinterpret_cast<u32x4*>(&xl[ring_slot<HALO, RING>(t, t_first) * XP + c]) = v;
  }
  if (segs && tid < HALO) {
    const int t = t_first - HALO + tid;
    sl[ring_slot<HALO, RING>(t, t_first)] = t >= 0 ? sgp[int64_t(t) * p.ss1] : INT32_MIN;
  }
  prefetch(zpre_s[0], xpre_s[0], t_first);
  commit(zpre_s[0], xpre_s[0], t_first);
  __syncthreads();

  const int lane_c = (q / LPC) * MT;  // first channel of this lane's run, within the wave
  // optional convolution bias of the lane's channels (zero without one, or past D)
  float cbv[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int ch = cw0 + lane_c + mt;
    cbv[mt] = (p.cbias != nullptr && ch < p.D) ? Raw<ET>::to_float(Raw<ET>::from_mem(static_cast<const ET*>(p.cbias), ch))
                                                : 0.f;
  }
  for (int t0 = t_first; t0 < t_end; t0 += TT) {
    const bool more = t0 + TT < t_end;
    if (more) prefetch(zpre_s[0], xpre_s[0], t0 + TT);
    // generate the filters of this tile (the z fragments are shared by the MT tiles)
    typename Mfma<ET>::F32k bfr[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (EB == 2) {
        bfr[ks].v = *reinterpret_cast<const u16x8_t*>(&zl[n * ZP + 32 * ks + 8 * q]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) bfr[ks].v[e] = zl[n * ZP + 32 * ks + Mfma<ET>::k32(q, e)];
      }
    }
    f32x4_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc[mt] = binit[mt];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc[mt] = Mfma<ET>::mma32(afr[mt][ks], bfr[ks], acc[mt]);
    }
    // conv + residual for token t0 + n, channels cw0 + lane_c .. + MT - 1
    const int t = t0 + n;
    const int sc = segs ? sl[ring_slot<HALO, RING>(t, t_first)] : 0;
    float sum[MT], xcur[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      sum[mt] = 0.f;
      xcur[mt] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tap = 4 * (q % LPC) + i;
      if (tap < W && (!segs || sl[ring_slot<HALO, RING>(t - tap, t_first)] == sc)) {
        float xv[MT];
        lds_read_run<ET, MT>(&xl[ring_slot<HALO, RING>(t - tap, t_first) * XP + wv * CPW + lane_c], xv);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          sum[mt] = fmaf(acc[mt][i], xv[mt], sum[mt]);
          if (tap == 0) xcur[mt] = xv[mt];
        }
      }
    }
    if constexpr (LPC == 2) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) sum[mt] += __shfl_xor(sum[mt], 16, 64);
    }
    const int cg = cw0 + lane_c;
    if ((q % LPC) == 0 && t < t_end && cg < p.D) {
      float yv[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) yv[mt] = xcur[mt] + sum[mt] + cbv[mt];
      global_store_run<ET, MT>(y + int64_t(t) * p.os1 + cg, yv, act16, p.D - cg);
    }
    __syncthreads();
    if (more) commit(zpre_s[0], xpre_s[0], t0 + TT);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------
// Backward main kernel: dx, and float32 partial sums of dU and db per token range.
//
// Same workgroup decomposition and filter regeneration as the forward (MT tiles per
// wave, so lane (token n, group q) holds the filter taps of a run of MT contiguous
// channels for one token). The pipeline advances S = 64 tokens (four 16-token tiles)
// per step, with the loads of the next two steps in flight; a step's x and dy rows sit
// in a tile that starts HALO tokens early (those rows are copied from the previous
// tile), so every LDS address is a per-lane base plus a compile-time offset. Per tile:
//  * P_k = w_k^(t) dy_t for the lane's token; dx_s = dy_s + sum_k P_k(s + k) is formed
//    for s = t - (W-1): the terms of later tokens come from the lanes to the right
//    (DPP row_shr) and, for the first lanes, from the previous tile (DPP row_ror). The
//    tiles past the range supply the last W-1 rows (the future halo).
//  * g_k(t) = dy_t x_{t-k} for the lane's token and channels; db is summed per lane; g
//    is written token-contiguous to a wave-private LDS tile.
// Per step the matrix cores then accumulate dU += z^T g (K = 32 tokens per instruction)
// in registers over the whole range, reading z from a token-contiguous copy staged next
// to the row-major one that feeds the regeneration.
// ---------------------------------------------------------------------------------
template <int K>
__device__ __forceinline__ float shift_lanes(float cur, float prev) {
  if constexpr (K == 0) {
    return cur;
  } else {
    const int from_prev = __builtin_amdgcn_mov_dpp(__float_as_int(prev), 0x120 | K, 0xf, 0xf, false);
    return __int_as_float(__builtin_amdgcn_update_dpp(from_prev, __float_as_int(cur), 0x110 | K, 0xf, 0xf, false));
  }
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// 16 bytes at base + off (elements) for a lane whose chunk is valid (`ok`). FAST: one
// 16-byte load whatever `ok` (lanes that must not read load `safe`, a valid address),
// so every thread issues the same number of loads; the value of a !ok lane is dropped
// later, by keep_if() when it is stored, so that nothing waits for the load here. The
// caller guarantees 16-byte alignment and whole chunks. Otherwise element loads of the
// first `limit` elements behind a branch, zero-filled (keep_if() changes nothing).
template <bool FAST, typename ET>
__device__ __forceinline__ u32x4 stage16(const ET* base, int off, bool ok, int limit, const ET* safe) {
  if constexpr (FAST) {
    const ET* a = ok ? base + off : safe;
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a));
  } else {
    u32x4 r = {0u, 0u, 0u, 0u};
    if (ok) r = load_elems16<ET>(base + off, limit);
    return r;
  }
}

__device__ __forceinline__ u32x4 keep_if(const u32x4& v, uint32_t okmask, int bit) {
  return ((okmask >> bit) & 1u) ? v : u32x4{0u, 0u, 0u, 0u};
}
__device__ __forceinline__ u32x4 keep_if(const u32x4& v, uint64_t okmask, int bit) {
  return ((okmask >> bit) & 1u) ? v : u32x4{0u, 0u, 0u, 0u};
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// K = 32 MFMA fragment (element e <-> k = 8q + e) of column col0 + (lane % 16) of a
// row-major 16-bit LDS tile whose row k0 + k holds index k, by two transposing 8-byte
// reads (ds_read_b64_tr_b16: in each 16-lane group, lane i receives element i % 4 of
// the 4 values loaded by lanes i / 4 + 4 e', e' = 0..3). Lane j of group q loads row
// k0 + 8q + j / 4 (+ 4 for the second half), columns col0 + 4 (j % 4) .. + 3.
__device__ __forceinline__ u16x8_t lds_colfrag_tr(const uint16_t* tile, int pitch, int k0, int col0) {
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4, j = lane & 15;
  const uint16_t* a = tile + (k0 + 8 * q + (j >> 2)) * pitch + col0 + 4 * (j & 3);
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(a));
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(a + 4 * pitch));
  u16x8_t r;
  r[0] = uint16_t(lo[0]); r[1] = uint16_t(lo[1]); r[2] = uint16_t(lo[2]); r[3] = uint16_t(lo[3]);
  r[4] = uint16_t(hi[0]); r[5] = uint16_t(hi[1]); r[6] = uint16_t(hi[2]); r[7] = uint16_t(hi[3]);
  return r;
}

// The same fragment for float32 tiles (element e <-> k = k32(q, e)), element reads.
template <typename ET>
__device__ __forceinline__ void lds_colfrag(typename Mfma<ET>::F32k& f, const typename Raw<ET>::type* tile, int pitch,
                                            int k0, int col0) {
  const int lane = threadIdx.x & 63;
  if constexpr (sizeof(ET) == 2) {
    f.v = lds_colfrag_tr(tile, pitch, k0, col0);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = tile[(k0 + Mfma<ET>::k32(lane >> 4, e)) * pitch + col0 + (lane & 15)];
  }
}

// Tile shape of the backward main kernel (shared by its LDS layout and its code).
template <typename ET, int W, int KS>
struct LrBwdShape {
  using RT = typename Raw<ET>::type;
  static constexpr int EB = int(sizeof(ET));
  static constexpr int MT = lowrank_bwd_mt(KS);
  static constexpr int WP = lowrank_rows_per_channel(W);  // padded taps per channel
  static constexpr int LPC = WP / 4;
  static constexpr int CPW = MT * 4 / LPC;  // channels per wave
  static constexpr int DC = 4 * CPW;        // channels per workgroup
  static constexpr int RP = 32 * KS;
  static constexpr int CE = 16 / EB;
  static constexpr int S = kLowrankBwdStep;  // tokens per pipeline step
  static constexpr int HALO = lr_halo(W);
  static constexpr int XR = S + HALO;        // rows of a step's x / dy tile
  static constexpr int ZP = RP + CE;         // z row pitch (elements)
  static constexpr int XP = DC + CE;
  static constexpr int GC = CPW * WP;        // padded filter columns of a wave
  static constexpr int GP = GC + 4;          // g row pitch (8-byte rows, spread banks)
  // two z buffers (one barrier per step) when they fit next to the rest
  static constexpr int LDS_REST = 4 * XR * XP * EB + 4 * S * GP * EB;
  static constexpr int ZB = (2 * S * ZP * EB + LDS_REST) <= 96 * 1024 ? 2 : 1;
};

template <typename ET, int W, int KS>
struct LrBwdSmem {
  using Sh = LrBwdShape<ET, W, KS>;
  using RT = typename Sh::RT;
  __align__(16) RT zl[Sh::ZB][Sh::S * Sh::ZP];
  __align__(16) ET xl[2][Sh::XR * Sh::XP];
  __align__(16) ET dyl[2][Sh::XR * Sh::XP];
  __align__(16) RT gl[4][Sh::S * Sh::GP];
  int sgl[2][Sh::XR];  // segment ids of the x / dy tile rows (packed sequences)
};

template <bool FAST, typename ET, int W, int KS>
__device__ __forceinline__ void lowrank_bwd_body(const LowRankParams& p, LrBwdSmem<ET, W, KS>& sm) {
  using Sh = LrBwdShape<ET, W, KS>;
  using RT = typename Raw<ET>::type;
  using R_ = Raw<ET>;
  constexpr int EB = Sh::EB, MT = Sh::MT, WP = Sh::WP, LPC = Sh::LPC, CPW = Sh::CPW, DC = Sh::DC;
  constexpr int RP = Sh::RP, CE = Sh::CE, S = Sh::S, XR = Sh::XR, ZP = Sh::ZP, XP = Sh::XP;
  constexpr int GC = Sh::GC, GP = Sh::GP, ZB = Sh::ZB, HALO = Sh::HALO;
  constexpr int NSUB = S / TT;
  constexpr int RTN = RP / 16;        // r tiles of dU
  constexpr int JTN = GC / 16;        // column tiles of dU
  constexpr int ZCH = S * RP / CE;    // 16-byte chunks of a step's z rows
  constexpr int XCH = S * DC / CE;    // ... of its x (and dy) rows
  constexpr int ZS = (ZCH + kBlockThreads - 1) / kBlockThreads;
  constexpr int XS = (XCH + kBlockThreads - 1) / kBlockThreads;
  constexpr int HCH = HALO * DC / CE;  // chunks of the HALO rows of x (and dy)
  static_assert(GC % 16 == 0 && S % 32 == 0 && 2 * HCH <= kBlockThreads && XR <= 2 * S, "tiling");
  auto& zl = sm.zl;
  auto& xl = sm.xl;
  auto& dyl = sm.dyl;
  auto& gl = sm.gl;

  const LrBlock blk = lr_block(p);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int q = lane >> 4;
  const int n = lane & 15;
  const int wv = tid >> 6;
  const int c_base = blk.cs * DC;
  const int t_first = blk.tr * p.Ltok;
  const int t_end = min(p.T, t_first + p.Ltok);
  const int t_need = min(p.T, t_end + HALO);  // z and dy rows feed dx up to t_end + W - 2
  const int range = blk.b * p.nTr + blk.tr;
  const ET* x = static_cast<const ET*>(p.x) + blk.b * p.xs0 + c_base;
  const ET* z = static_cast<const ET*>(p.z) + blk.b * p.zs0;
  const ET* dy = static_cast<const ET*>(p.dy) + blk.b * p.dys0 + c_base;
  ET* dx = static_cast<ET*>(p.out) + blk.b * p.os0;
  const ET* xsafe = static_cast<const ET*>(p.x);
  const ET* zsafe = static_cast<const ET*>(p.z);
  const ET* dysafe = static_cast<const ET*>(p.dy);
  const bool act16 = p.act16 != 0;
  const int xlimit = p.D - c_base;
  const int cw0 = c_base + wv * CPW;
  const int lane_c = (q / LPC) * MT;  // first channel of the lane's run, within the wave
  const int cl = cw0 + lane_c;
  const int cl_count = p.D - cl;
  const int xcol = wv * CPW + lane_c;  // the lane's column in the x / dy tiles
  // packed sequences: tap k of token t is present only when token t-k has t's segment id
  const bool segs = p.seg != nullptr;
  const int32_t* sgp = segs ? p.seg + blk.b * p.ss0 : nullptr;
  auto& sgl = sm.sgl;

  // regeneration operands, as in the forward
  typename Mfma<ET>::F32k afr[MT][KS];
  f32x4_t binit[MT];
  {
    const ET* U = static_cast<const ET*>(p.U);
    const ET* bias = static_cast<const ET*>(p.bias);
    const int m = n;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int ch = cw0 + ((m >> 2) / LPC) * MT + mt;
      const int tap = 4 * ((m >> 2) % LPC) + (m & 3);
      const bool ok = ch < p.D && tap < W;
      const int64_t col = int64_t(ch / p.H) * W + tap;  // group ch / H (head-wise: H > 1)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 32 * ks + Mfma<ET>::k32(q, e);
          afr[mt][ks].v[e] = (ok && r < p.R) ? R_::from_mem(U, int64_t(r) * p.ldu + col) : R_::zero();
        }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tq = 4 * (q % LPC) + i;
        binit[mt][i] = (bias != nullptr && cl + mt < p.D && tq < W)
                           ? R_::to_float(R_::from_mem(bias, int64_t((cl + mt) / p.H) * W + tq))
                           : 0.f;
      }
    }
  }

  // Loads of one step (tokens t0 .. t0 + S - 1): z rows below t_need, x rows below
  // t_end, dy rows below t_need; zeros elsewhere. Each thread always stages the same
  // (row, column) slots, so only the uniform base pointers move from step to step.
  struct Stage {
    u32x4 z[ZS], x[XS], d[XS];
    uint32_t ok;  // bit i: z[i]; bit ZS + i: x[i]; bit ZS + XS + i: d[i]
    bool full;    // every row of the step lies in the range: no masks
    int sid;      // segment id of token t0 + tid (tid < S)
  };
  static_assert(ZS + 2 * XS <= 32, "valid bits");
  auto prefetch = [&](Stage& st, int t0) {
    const ET* zb = z + int64_t(t0) * p.zs1;
    const ET* xb = x + int64_t(t0) * p.xs1;
    const ET* db_ = dy + int64_t(t0) * p.dys1;
    if (segs && tid < S) st.sid = t0 + tid < t_need ? sgp[int64_t(t0 + tid) * p.ss1] : INT32_MIN;
    st.full = FAST && t0 + S <= t_end;
    if (FAST && t0 + S <= t_end) {
      // same loads as below with every chunk valid (z chunks are whole: R % 32 == 0). A
      // thread past the step's chunks (XCH not a multiple of the block: W = 5 slices of
      // 16-bit channels) would address rows beyond the step, past the tensor's end on the
      // last steps; it loads the tensor's first chunk instead, which commit never stores.
      static_assert(ZCH % kBlockThreads == 0, "every thread owns z chunks of the step");
#pragma unroll
      for (int i = 0; i < ZS; ++i) {
        const int ck = tid + i * kBlockThreads;
        st.z[i] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(zb + (ck / (RP / CE)) * int(p.zs1) + (ck % (RP / CE)) * CE));
      }
#pragma unroll
      for (int i = 0; i < XS; ++i) {
        const int ck = tid + i * kBlockThreads;
        const bool in = XCH % kBlockThreads == 0 || ck < XCH;
        const int row = ck / (DC / CE), c = (ck % (DC / CE)) * CE;
        st.x[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(in ? xb + row * int(p.xs1) + c : xsafe));
        st.d[i] =
            __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(in ? db_ + row * int(p.dys1) + c : dysafe));
      }
      st.ok = ~0u;
      return;
    }
    uint32_t okm = 0;
#pragma unroll
    for (int i = 0; i < ZS; ++i) {
      const int ck = tid + i * kBlockThreads;
      const int row = ck / (RP / CE), c = (ck % (RP / CE)) * CE;
      const bool ok = ck < ZCH && t0 + row < t_need && c < p.R;
      st.z[i] = stage16<FAST, ET>(zb, row * int(p.zs1) + c, ok, p.R - c, zsafe);
      okm |= uint32_t(ok) << i;
    }
#pragma unroll
    for (int i = 0; i < XS; ++i) {
      const int ck = tid + i * kBlockThreads;
      const int row = ck / (DC / CE), c = (ck % (DC / CE)) * CE;
      const bool ok = ck < XCH && c < xlimit;
      const bool okx = ok && t0 + row < t_end, okd = ok && t0 + row < t_need;
      st.x[i] = stage16<FAST, ET>(xb, row * int(p.xs1) + c, okx, xlimit - c, xsafe);
      st.d[i] = stage16<FAST, ET>(db_, row * int(p.dys1) + c, okd, xlimit - c, dysafe);
      okm |= (uint32_t(okx) << (ZS + i)) | (uint32_t(okd) << (ZS + XS + i));
    }
    st.ok = okm;
  };
  // Writes a step's loads to x / dy buffer `buf` and z buffer `zbuf`; with `halo`, copies
  // the HALO rows that precede the step from the last rows of the other x / dy buffer.
  auto commit = [&](const Stage& st, int buf, int zbuf, bool halo) {
    const uint32_t okm = st.full ? ~0u : st.ok;  // uniform choice: folded for full steps
    auto put = [&](const uint32_t mask) {
#pragma unroll
      for (int i = 0; i < ZS; ++i) {
        const int ck = tid + i * kBlockThreads;
        if (ck < ZCH)
          *reinterpret_cast<u32x4*>(&zl[zbuf][(ck / (RP / CE)) * ZP + (ck % (RP / CE)) * CE]) = keep_if(st.z[i], mask, i);
      }
#pragma unroll
      for (int i = 0; i < XS; ++i) {
        const int ck = tid + i * kBlockThreads;
        if (ck < XCH) {
          const int o = (HALO + ck / (DC / CE)) * XP + (ck % (DC / CE)) * CE;
          *reinterpret_cast<u32x4*>(&xl[buf][o]) = keep_if(st.x[i], mask, ZS + i);
          *reinterpret_cast<u32x4*>(&dyl[buf][o]) = keep_if(st.d[i], mask, ZS + XS + i);
        }
      }
    };
    if (st.full) {
      put(~0u);
    } else {
      put(okm);
    }
    if (segs) {
      if (tid < S) sgl[buf][HALO + tid] = st.sid;
      if (halo && tid < HALO) sgl[buf][tid] = sgl[buf ^ 1][tid + S];
    }
    if (halo && tid < 2 * HCH) {
      const int k2 = tid % HCH;
      const int o = (k2 / (DC / CE)) * XP + (k2 % (DC / CE)) * CE;
      ET* dst = tid < HCH ? xl[buf] : dyl[buf];
      const ET* src = tid < HCH ? xl[buf ^ 1] : dyl[buf ^ 1];
      *reinterpret_cast<u32x4*>(dst + o) = *reinterpret_cast<const u32x4*>(src + o + S * XP);
    }
  };

  // first tile: its HALO rows come from memory (zeros before t = 0)
  if (segs && tid < HALO) {
    const int t = t_first - HALO + tid;
    sgl[0][tid] = t >= 0 ? sgp[int64_t(t) * p.ss1] : INT32_MIN;
  }
  if (tid < 2 * HCH) {
    const int k2 = tid % HCH;
    const int row = k2 / (DC / CE), c = (k2 % (DC / CE)) * CE, t = t_first - HALO + row;
    const ET* src = tid < HCH ? x + int64_t(t) * p.xs1 : dy + int64_t(t) * p.dys1;
    const bool ok = t >= 0 && c < xlimit;
    *reinterpret_cast<u32x4*>(&(tid < HCH ? xl : dyl)[0][row * XP + c]) =
        keep_if(stage16<FAST, ET>(src, c, ok, xlimit - c, tid < HCH ? xsafe : dysafe), uint32_t(ok), 0);
  }
  Stage stA, stB;
  prefetch(stA, t_first);
  commit(stA, 0, 0, false);
  __syncthreads();
  // prefetches are issued unconditionally (past the range every chunk reads as zero) so
  // that the number of loads in flight, and with it each wait, is the same on every path
  prefetch(stA, t_first + S);

  f32x4_t dU[RTN][JTN];
#pragma unroll
  for (int a = 0; a < RTN; ++a)
#pragma unroll
    for (int b = 0; b < JTN; ++b) dU[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float db[MT][4], Pprev[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      db[mt][i] = 0.f;
      Pprev[mt][i] = 0.f;
    }

  RT* gw = gl[wv];
  // one step: `cur` holds the loads of step t0 + S (in flight), `nxt` receives step t0 + 2S
  auto step = [&](int t0, Stage& cur, Stage& nxt, const int buf) {
    const int zbuf = ZB == 2 ? buf : 0;
    const bool more = t0 + S - (W - 1) < t_end;
    const bool do_g = t0 < t_end;
    prefetch(nxt, t0 + 2 * S);
    const ET* xt = &xl[buf][(HALO + n) * XP + xcol];   // x row of token t0 + n
    const ET* dyt = &dyl[buf][(HALO + n) * XP + xcol];  // dy row of token t0 + n
    ET* dxb = dx + int64_t(t0) * p.os1;
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      const int ts = t0 + sub * TT;
      const bool do_dx = ts - (W - 1) < t_end;
      if (!do_dx && !do_g) break;
      const int t = ts + n;
      // presence of the lane's taps for token t (packed sequences)
      bool tp[4];
      {
        const int* srow = &sgl[buf][HALO + sub * TT + n];
        const int sc = segs ? srow[0] : 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tap = 4 * (q % LPC) + i;
          tp[i] = !segs || tap >= W || srow[-tap] == sc;
        }
      }
      float dyn[MT];
      lds_read_run<ET, MT>(dyt + sub * TT * XP, dyn);
      if (do_dx) {
        // regenerate the filters of tokens ts .. ts + 15
        typename Mfma<ET>::F32k bfr[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if constexpr (EB == 2) {
            bfr[ks].v = *reinterpret_cast<const u16x8_t*>(&zl[zbuf][(sub * TT + n) * ZP + 32 * ks + 8 * q]);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) bfr[ks].v[e] = zl[zbuf][(sub * TT + n) * ZP + 32 * ks + Mfma<ET>::k32(q, e)];
          }
        }
        float P[MT][4], dxs[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          f32x4_t a = binit[mt];
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) a = Mfma<ET>::mma32(afr[mt][ks], bfr[ks], a);
#pragma unroll
          for (int i = 0; i < 4; ++i) P[mt][i] = tp[i] ? a[i] * dyn[mt] : 0.f;
        }
        // dx for token s = t - (W - 1)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          float acc;
          if constexpr (LPC == 1) {
            acc = shift_lanes<W - 1>(P[mt][0], Pprev[mt][0]);
            if constexpr (W > 1) acc += shift_lanes<(W > 1 ? W - 2 : 0)>(P[mt][1], Pprev[mt][1]);
            if constexpr (W > 2) acc += shift_lanes<(W > 2 ? W - 3 : 0)>(P[mt][2], Pprev[mt][2]);
            if constexpr (W > 3) acc += shift_lanes<(W > 3 ? W - 4 : 0)>(P[mt][3], Pprev[mt][3]);
          } else {
            // even groups hold taps 0..3 (from W-1..W-4 tokens back), odd groups taps
            // 4..W-1 (from W-5..0 tokens back)
            const float even = shift_lanes<W - 1>(P[mt][0], Pprev[mt][0]) + shift_lanes<W - 2>(P[mt][1], Pprev[mt][1]) +
                               shift_lanes<W - 3>(P[mt][2], Pprev[mt][2]) + shift_lanes<W - 4>(P[mt][3], Pprev[mt][3]);
            float odd = shift_lanes<(W > 4 ? W - 5 : 0)>(P[mt][0], Pprev[mt][0]);
            if constexpr (W > 5) odd += shift_lanes<(W > 5 ? W - 6 : 0)>(P[mt][1], Pprev[mt][1]);
            if constexpr (W > 6) odd += shift_lanes<(W > 6 ? W - 7 : 0)>(P[mt][2], Pprev[mt][2]);
            if constexpr (W > 7) odd += shift_lanes<(W > 7 ? W - 8 : 0)>(P[mt][3], Pprev[mt][3]);
            const float mine = (q & 1) ? odd : even;
            acc = mine + __shfl_xor(mine, 16, 64);
          }
          dxs[mt] = acc;
        }
        const int s = t - (W - 1);
        if ((q % LPC) == 0 && s >= t_first && s < t_end && cl_count > 0) {
          float dys[MT];
          lds_read_run<ET, MT>(dyt + (sub * TT - (W - 1)) * XP, dys);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) dxs[mt] += dys[mt];
          global_store_run<ET, MT>(dxb + (sub * TT + n - (W - 1)) * int(p.os1) + cl, dxs, act16, cl_count);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) Pprev[mt][i] = P[mt][i];
      }
      if (do_g) {
        // g_k(t) = dy_t x_{t-k}, zero past the range; row t - t0 of the wave's g tile
        // holds the lane's 4 taps of each of its MT channels
        // tokens of a step that ends inside the range need no mask
        const bool tok_ok = t0 + S <= t_end || t < t_end;
        float dyg[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) dyg[mt] = tok_ok ? dyn[mt] : 0.f;
        float g[MT][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tap = 4 * (q % LPC) + i;
          // padded taps (tap >= W) of the odd lane groups read a valid row (tap 0) and
          // zero the result
          const int rtap = tap < W ? tap : 0;
          float xr[MT] = {};
          if (LPC == 2 || tap < W) lds_read_run<ET, MT>(xt + (sub * TT - rtap) * XP, xr);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            g[mt][i] = (tap < W && tp[i]) ? dyg[mt] * xr[mt] : 0.f;
            db[mt][i] += g[mt][i];
          }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          RT* dst = &gw[(sub * TT + n) * GP + (lane_c + mt) * WP + 4 * (q % LPC)];
          if constexpr (EB == 2) {
            *reinterpret_cast<u32x2*>(dst) =
                u32x2{Cvt<ET>::pack2(g[mt][0], g[mt][1]), Cvt<ET>::pack2(g[mt][2], g[mt][3])};
          } else {
            *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{g[mt][0], g[mt][1], g[mt][2], g[mt][3]};
          }
        }
      }
    }
    if (do_g) {
      wave_lds_sync();
      // dU[r][col] += sum_t z_t[r] g_t[col] over the S tokens of the step (K = tokens;
      // both operands are read down the columns of row-major tiles)
#pragma unroll
      for (int kk = 0; kk < S / 32; ++kk) {
        typename Mfma<ET>::F32k gfr[JTN];
#pragma unroll
        for (int jt = 0; jt < JTN; ++jt) lds_colfrag<ET>(gfr[jt], gw, GP, 32 * kk, jt * 16);
#pragma unroll
        for (int rt = 0; rt < RTN; ++rt) {
          typename Mfma<ET>::F32k zfr;
          lds_colfrag<ET>(zfr, zl[zbuf], ZP, 32 * kk, rt * 16);
#pragma unroll
          for (int jt = 0; jt < JTN; ++jt) dU[rt][jt] = Mfma<ET>::mma32(zfr, gfr[jt], dU[rt][jt]);
        }
      }
    }
    // with two z buffers the other one was last read in the previous step, before the
    // last barrier; with one, every wave must be done with it first
    if constexpr (ZB == 1) __syncthreads();
    if (more) commit(cur, buf ^ 1, ZB == 2 ? (buf ^ 1) : 0, true);
    __syncthreads();
  };
  for (int t0 = t_first; t0 - (W - 1) < t_end; t0 += 2 * S) {
    step(t0, stA, stB, 0);
    if (!(t0 + S - (W - 1) < t_end)) break;
    step(t0 + S, stB, stA, 1);
  }

  // db partial: sum over the 16 token lanes of each row, written by lane n == 0
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = db[mt][i];
      v += __shfl_xor(v, 1, 64);
      v += __shfl_xor(v, 2, 64);
      v += __shfl_xor(v, 4, 64);
      v += __shfl_xor(v, 8, 64);
      const int tap = 4 * (q % LPC) + i;
      // head-wise: one partial per (range, channel of the group), summed by the reduce
      const int c = cl + mt;
      if (p.part_db != nullptr && n == 0 && tap < W && c < p.D)
        p.part_db[(int64_t(range) * p.H + c % p.H) * p.J + int64_t(c / p.H) * W + tap] = v;
    }
  // dU partial: lane holds rows rt*16 + 4q + ii of padded column jt*16 + n
#pragma unroll
  for (int rt = 0; rt < RTN; ++rt)
#pragma unroll
    for (int jt = 0; jt < JTN; ++jt) {
      const int pc = jt * 16 + n;
      const int ch = cw0 + pc / WP;
      const int tap = pc % WP;
      if (tap < W && ch < p.D) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int r = rt * 16 + 4 * q + ii;
          if (r < p.R)
            p.part_dU[((int64_t(range) * p.H + ch % p.H) * p.R + r) * p.J + int64_t(ch / p.H) * W + tap] =
                dU[rt][jt][ii];
        }
      }
    }
}

// FAST: 16-byte loads throughout (the launch covers channel slices that lie inside D,
// with aligned rows and R % 32 == 0); otherwise element loads where a chunk is partial.
template <typename ET, int W, int KS, bool FAST>
__global__ __launch_bounds__(kBlockThreads) void k_lowrank_bwd(const LowRankParams p) {
  __shared__ LrBwdSmem<ET, W, KS> sm;
  lowrank_bwd_body<FAST, ET, W, KS>(p, sm);
}

// ---------------------------------------------------------------------------------
// dz[t][r] = sum_j g_t[j] U[r][j], with g recomputed from x and dy.
// A workgroup owns kLowrankDzTokens tokens of one sequence (16 per wave) and walks the
// channels in chunks of CH = 32: the chunk's U columns (all ranks), the x rows (with the
// HALO tokens before) and the dy rows are staged in LDS, double-buffered when they fit,
// with the loads of the next two chunks in flight.
// Matrix cores: M = r, N = tokens, K = filter columns. Lane group q supplies g for the
// run of CR = 8 channels q*CR .. (all W taps, CR*W consecutive columns j), so the
// K step ks of group q covers columns q*CR*W + 8 ks .. + 7: the same map indexes the U
// rows in LDS, and the channel / tap of each element is a compile-time constant.
// ---------------------------------------------------------------------------------
template <typename ET, int W, int KS>
struct LrDzShape {
  using RT = typename Raw<ET>::type;
  static constexpr int EB = int(sizeof(ET));
  static constexpr int RP = 32 * KS;
  static constexpr int CH = kLowrankDzChunk;
  static constexpr int UC = CH * W;          // columns of a chunk
  static constexpr int CE = 16 / EB;
  static constexpr int UP = UC + CE;         // U row pitch (elements)
  static constexpr int TB = kLowrankDzTokens;
  static constexpr int HALO = lr_halo(W);
  static constexpr int XR = TB + HALO;
  static constexpr int XP = CH + CE;
  static constexpr int STAGE = (RP * UP + XR * XP + TB * XP) * EB;
  static constexpr int NBUF = 2 * STAGE <= 80 * 1024 ? 2 : 1;
};

template <typename ET, int W, int KS>
struct LrDzSmem {
  using Sh = LrDzShape<ET, W, KS>;
  __align__(16) typename Sh::RT Ul[Sh::NBUF][Sh::RP * Sh::UP];
  __align__(16) ET xl[Sh::NBUF][Sh::XR * Sh::XP];
  __align__(16) ET dyl[Sh::NBUF][Sh::TB * Sh::XP];
};

template <typename ET, int W, int KS>
__device__ __forceinline__ void lowrank_dz_body(const LowRankParams& p, LrDzSmem<ET, W, KS>& sm) {
  using Sh = LrDzShape<ET, W, KS>;
  using RT = typename Raw<ET>::type;
  constexpr int EB = Sh::EB, RP = Sh::RP, CH = Sh::CH, UC = Sh::UC, CE = Sh::CE, UP = Sh::UP;
  constexpr int TB = Sh::TB, XR = Sh::XR, XP = Sh::XP, NBUF = Sh::NBUF, HALO = Sh::HALO;
  constexpr int RTN = RP / 16;
  constexpr int CR = CH / 4;          // channels of a lane group
  constexpr int RUN = CR * W;         // columns of a lane group
  constexpr int KST = RUN / 8;        // K steps per chunk
  constexpr int UCH = RP * UC / CE;   // 16-byte chunks of U per stage
  constexpr int XCH = XR * CH / CE;
  constexpr int DCH = TB * CH / CE;
  constexpr int US = (UCH + kBlockThreads - 1) / kBlockThreads;
  constexpr int AS = (XCH + DCH + kBlockThreads - 1) / kBlockThreads;  // x and dy slots
  constexpr int ND = CR * EB / 4;     // 32-bit words of a lane's run of one row
  static_assert(RUN % 8 == 0 && UC % CE == 0 && TB == 64, "dz tiling");
  auto& Ul = sm.Ul;
  auto& xl = sm.xl;
  auto& dyl = sm.dyl;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int q = lane >> 4;
  const int n = lane & 15;
  const int wv = tid >> 6;
  const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int b = int(lb / uint32_t(p.nTbL));
  const int tb0 = (p.tbb0 + int(lb % uint32_t(p.nTbL))) * TB;
  // x rows from tb0 - HALO, dy rows from tb0 (row offsets below stay small)
  const ET* x = static_cast<const ET*>(p.x) + b * p.xs0 + int64_t(tb0 - HALO) * p.xs1;
  const ET* dy = static_cast<const ET*>(p.dy) + b * p.dys0 + int64_t(tb0) * p.dys1;
  const ET* U = static_cast<const ET*>(p.U);
  const ET* xsafe = static_cast<const ET*>(p.x);
  const ET* dysafe = static_cast<const ET*>(p.dy);
  const int nchunk = (p.D + CH - 1) / CH;

  // bit i: u[i]; bit US + i: a[i] (64 bits for float32 U at W >= 7 with 128 ranks)
  using Mask = typename std::conditional<(US + AS <= 32), uint32_t, uint64_t>::type;
  struct Stage {
    u32x4 u[US], a[AS];
    Mask ok;
  };
  static_assert(US + AS <= 64, "valid bits");
  auto prefetch = [&](Stage& st, int c0) {
    const int climit = p.D - c0;
    const int jlimit = climit * W;  // filter columns (channel, tap) of the chunk inside D
    const ET* ub = U + int64_t(c0) * W;
    Mask okm = 0;
#pragma unroll
    for (int i = 0; i < US; ++i) {
      const int ck = tid + i * kBlockThreads;
      const int r = ck / (UC / CE), c = (ck % (UC / CE)) * CE;
      const bool ok = ck < UCH && r < p.R && c < jlimit;
      if (p.H == 1) {
        st.u[i] = stage16<false, ET>(ub, r * int(p.ldu) + c, ok, jlimit - c, U);
      } else {
        // head-wise: column (c0 + cc) / H * W + k of U for the chunk's column cc * W + k
        st.u[i] = ok ? load_group_cols<ET>(U + int64_t(r) * p.ldu, c0, c, jlimit - c, W, p.H) : u32x4{0u, 0u, 0u, 0u};
      }
      okm |= Mask(ok) << i;
    }
#pragma unroll
    for (int i = 0; i < AS; ++i) {
      const int ck = tid + i * kBlockThreads;
      // x rows tb0 - HALO .. (ck < XCH), then dy rows tb0 ..
      const bool isx = ck < XCH;
      const int k2 = isx ? ck : ck - XCH;
      const int row = k2 / (CH / CE), c = (k2 % (CH / CE)) * CE;
      const int t = isx ? tb0 - HALO + row : tb0 + row;
      const bool ok = (isx || k2 < DCH) && t >= 0 && t < p.T && c < climit;
      st.a[i] = stage16<false, ET>(isx ? x + c0 : dy + c0, row * int(isx ? p.xs1 : p.dys1) + c, ok, climit - c,
                                  isx ? xsafe : dysafe);
      okm |= Mask(ok) << (US + i);
    }
    st.ok = okm;
  };
  auto commit = [&](const Stage& st, int buf) {
#pragma unroll
    for (int i = 0; i < US; ++i) {
      const int ck = tid + i * kBlockThreads;
      if (ck < UCH)
        *reinterpret_cast<u32x4*>(&Ul[buf][(ck / (UC / CE)) * UP + (ck % (UC / CE)) * CE]) = keep_if(st.u[i], st.ok, i);
    }
#pragma unroll
    for (int i = 0; i < AS; ++i) {
      const int ck = tid + i * kBlockThreads;
      const u32x4 v = keep_if(st.a[i], st.ok, US + i);
      if (ck < XCH) {
        *reinterpret_cast<u32x4*>(&xl[buf][(ck / (CH / CE)) * XP + (ck % (CH / CE)) * CE]) = v;
      } else if (ck - XCH < DCH) {
        const int k2 = ck - XCH;
        *reinterpret_cast<u32x4*>(&dyl[buf][(k2 / (CH / CE)) * XP + (k2 % (CH / CE)) * CE]) = v;
      }
    }
  };

  f32x4_t acc[RTN];
#pragma unroll
  for (int j = 0; j < RTN; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  Stage stA, stB;
  prefetch(stA, 0);
  commit(stA, 0);
  __syncthreads();
  // prefetches are issued unconditionally (past the last chunk every chunk reads as
  // zero) so that the number of loads in flight, and with it each wait, is the same on
  // every path
  prefetch(stA, CH);
  const int nt = wv * TT + n;  // the lane's token within the block
  // packed sequences: taps of the lane's token that reach into another segment
  bool tp[W];
#pragma unroll
  for (int k = 0; k < W; ++k) tp[k] = true;
  if (p.seg != nullptr) {
    const int32_t* sgp = p.seg + b * p.ss0;
    const int t = min(tb0 + nt, p.T - 1);
    const int cur = sgp[int64_t(t) * p.ss1];
#pragma unroll
    for (int k = 1; k < W; ++k) tp[k] = t - k < 0 || sgp[int64_t(t - k) * p.ss1] == cur;
  }
  // chunk ci: `cur` holds chunk ci + 1 (in flight), `nxt` receives chunk ci + 2
  auto chunk = [&](int ci, Stage& cur, Stage& nxt) {
    const int buf = NBUF == 2 ? (ci & 1) : 0;
    const bool more = ci + 1 < nchunk;
    prefetch(nxt, (ci + 2) * CH);
    // the lane's dy row and x rows (taps 0 .. W-1) for its run of CR channels, as words
    uint32_t dw_[ND], xw[W][ND];
    {
      const uint32_t* d = reinterpret_cast<const uint32_t*>(&dyl[buf][nt * XP + q * CR]);
#pragma unroll
      for (int i = 0; i < ND; i += 4) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(d + i);
        dw_[i] = v[0]; dw_[i + 1] = v[1]; dw_[i + 2] = v[2]; dw_[i + 3] = v[3];
      }
#pragma unroll
      for (int k = 0; k < W; ++k) {
        const uint32_t* xs = reinterpret_cast<const uint32_t*>(&xl[buf][(nt + HALO - k) * XP + q * CR]);
#pragma unroll
        for (int i = 0; i < ND; i += 4) {
          const u32x4 v = tp[k] ? *reinterpret_cast<const u32x4*>(xs + i) : u32x4{0u, 0u, 0u, 0u};
          xw[k][i] = v[0]; xw[k][i + 1] = v[1]; xw[k][i + 2] = v[2]; xw[k][i + 3] = v[3];
        }
      }
    }
    auto elem = [&](const uint32_t* w, int c) -> float {
      if constexpr (EB == 2) {
        return (c & 1) ? Cvt<ET>::hi(w[c >> 1]) : Cvt<ET>::lo(w[c >> 1]);
      } else {
        return __uint_as_float(w[c]);
      }
    };
    float dyf[CR];
#pragma unroll
    for (int c = 0; c < CR; ++c) dyf[c] = elem(dw_, c);
#pragma unroll
    for (int ks = 0; ks < KST; ++ks) {
      typename Mfma<ET>::F32k bfr;
      if constexpr (EB == 2) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int c0_ = (8 * ks + e) / W, k0_ = (8 * ks + e) % W;
          const int c1_ = (8 * ks + e + 1) / W, k1_ = (8 * ks + e + 1) % W;
          const uint32_t w2 = Cvt<ET>::pack2(dyf[c0_] * elem(xw[k0_], c0_), dyf[c1_] * elem(xw[k1_], c1_));
          bfr.v[e] = uint16_t(w2 & 0xffffu);
          bfr.v[e + 1] = uint16_t(w2 >> 16);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int c_ = (8 * ks + e) / W, k_ = (8 * ks + e) % W;
          bfr.v[e] = dyf[c_] * elem(xw[k_], c_);
        }
      }
#pragma unroll
      for (int rt = 0; rt < RTN; ++rt) {
        typename Mfma<ET>::F32k afr;
        const RT* src = &Ul[buf][(rt * 16 + n) * UP + q * RUN + 8 * ks];
        if constexpr (EB == 2) {
          afr.v = *reinterpret_cast<const u16x8_t*>(src);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) afr.v[e] = src[e];
        }
        acc[rt] = Mfma<ET>::mma32(afr, bfr, acc[rt]);
      }
    }
    if constexpr (NBUF == 1) __syncthreads();
    if (more) commit(cur, NBUF == 2 ? (buf ^ 1) : 0);
    __syncthreads();
  };
  for (int ci = 0; ci < nchunk; ci += 2) {
    chunk(ci, stA, stB);
    if (ci + 1 < nchunk) chunk(ci + 1, stB, stA);
  }
  // lane holds dz[token n][r = rt*16 + 4q + ii]
  ET* dz = static_cast<ET*>(p.dz) + b * p.dzs0;
  const int t = tb0 + nt;
  if (t < p.T) {
#pragma unroll
    for (int rt = 0; rt < RTN; ++rt)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int r = rt * 16 + 4 * q + ii;
        if (r < p.R) {
          const int64_t o = int64_t(t) * p.dzs1 + r;
          if constexpr (EB == 2) {
            reinterpret_cast<uint16_t*>(dz)[o] = Cvt<ET>::bits(acc[rt][ii]);
          } else {
            dz[o] = acc[rt][ii];
          }
        }
      }
  }
}

// ---------------------------------------------------------------------------------
// dz, bf16 interior blocks: the same computation as lowrank_dz_body, staged by LDS DMA
// (global_load_lds_dwordx4: each lane's 16 bytes land at the wave's LDS base + 16 *
// lane, no registers involved) into a ring of NST stages, NST - 1 chunks ahead of the one
// being computed. Each wave waits for its own transfers (vmcnt) and a barrier publishes
// the stage; nothing else needs the loads, so no other wait is tied to them. Two stages
// (one chunk ahead) leave room for 3 workgroups per CU at H = 1 (R = 64: 51 KiB each);
// measured against three stages: low-rank backward 213.7 -> 208.2 us at B8 T4096 D2048
// W4 R64, head-wise H = 4 194.3 -> 191.1 us.
// A lane owns GL filter groups (GL = 8 for HG <= 4, 32 / HG for HG = 8, 16), a chunk the
// 4 GL groups of the 4 lane groups: 32 channels per-channel, 32 * HG channels when HG
// consecutive channels share a filter (HG = 2, 4), 128 channels for HG = 8, 16. The filter
// columns of consecutive groups are consecutive in U, so a chunk's U tile is 4 GL W whole
// columns; a lane reads GL * HG / 8 16-byte runs of x and dy per row and sums its products
// over the HG channels of a group before the matrix-core step (1/HG of the per-channel
// matrix work, and U read 1/HG as often). Its GL * W columns must fill whole K steps of 8.
// LDS placement. The bank-conflict counts measured on this kernel (4 extra cycles per
// colliding 16-byte read) fit 16-byte reads served in passes of 16 lanes over 256 bytes:
// lanes 0-7 with 16-23, 8-15 with 24-31, 32-39 with 48-55, 40-47 with 56-63. A pass thus
// reads 8 consecutive rows, each at two logical chunks (of lane groups q and q + 1).
// LdsPlace<CPR> maps logical chunk c of row r to a slot:
//   CPR == 16 (256-byte rows: U at W = 4, x / dy at H = 4): rotate by
//     r % 4 + 8 * ((r / 4) % 2), which puts the 16 reads of a pass on distinct slots;
//   CPR % 8 == 4 (rows of 64, 192, 320, 448 bytes) and CPR == 24 (U at W = 6): rotate by
//     r / 2 (conflict-free for 64-byte rows, x / dy at H = 1; two-way for the others);
//   CPR == 8 and CPR == 32 (128- and 512-byte rows, U at W = 2 and W = 8): rotate by r
//     (r < 16: the 8 rows of a pass take 8 consecutive slots, the two chunks 8 apart).
// U rows use r % 16 (the row within a 16-row tile), so every tile has the same slots.
// ---------------------------------------------------------------------------------
constexpr bool lds_place_ok(int cpr) { return cpr % 8 == 4 || cpr == 8 || cpr == 16 || cpr == 24 || cpr == 32; }

template <int CPR>
struct LdsPlace {
  static_assert(lds_place_ok(CPR), "LDS row length of the dz kernel");
  static __device__ __forceinline__ int slot(int r, int c) {
    if constexpr (CPR == 16) return (c + r % 4 + 8 * ((r / 4) % 2)) % 16;
    else if constexpr (CPR == 8 || CPR == 32) return (c + r) % CPR;
    else return (c + r / 2) % CPR;
  }
  static __device__ __forceinline__ int chunk(int r, int p) {  // inverse of slot for row r
    if constexpr (CPR == 16) return (p - r % 4 - 8 * ((r / 4) % 2) + 16) % 16;
    else if constexpr (CPR == 8 || CPR == 32) return ((p - r % CPR) % CPR + CPR) % CPR;
    else return ((p - (r / 2) % CPR) % CPR + CPR) % CPR;
  }
};

#ifndef LRDZ_NST
#define LRDZ_NST 2
#endif
template <int W, int KS, int HG>
struct LrDzDma {
  static_assert(HG == 1 || HG == 2 || HG == 4 || HG == 8 || HG == 16, "group size of the DMA dz path");
  static constexpr int HALO = lr_halo(W);
  static constexpr int RP = 32 * KS;
  static constexpr int GL = HG <= 4 ? 8 : 32 / HG;  // filter groups of a lane
  static constexpr int RUNS = GL * HG / 8;          // 16-byte runs of a lane's row
  static constexpr int CH = 4 * GL;            // filter groups of a chunk
  static constexpr int CHC = CH * HG;          // channels of a chunk
  static constexpr int UC = CH * W;            // filter columns of a chunk
  static constexpr int UCPR = UC / 8;          // 16-byte chunks of a U row
  static constexpr int TB = kLowrankDzTokens;
  static constexpr int XR = TB + HALO;
  static constexpr int XCPR = CHC / 8;         // 16-byte chunks of an x / dy row
  static constexpr bool SHAPE_OK = (GL * W) % 8 == 0 && lds_place_ok(UCPR) && lds_place_ok(XCPR);
  static constexpr int UCH = RP * UCPR, XCH = XR * XCPR, DCH = TB * XCPR;
  static constexpr int NI_U = (UCH + 63) / 64, NI_X = (XCH + 63) / 64, NI_D = (DCH + 63) / 64;
  static constexpr int NI = NI_U + NI_X + NI_D;  // wave-wide transfers per stage
  static constexpr int X_OFF = NI_U * 64 * 16;   // byte offsets inside a stage
  static constexpr int D_OFF = X_OFF + NI_X * 64 * 16;
  static constexpr int STAGE = D_OFF + NI_D * 64 * 16;
  static constexpr int NST = LRDZ_NST;  // stages of the ring (2: one chunk ahead, 3: two)
  static constexpr int BYTES = NST * STAGE;
  static_assert(XCPR == 4 * RUNS && UC % 8 == 0, "dz DMA tiling");
  using UPlace = LdsPlace<UCPR>;
  using XPlace = LdsPlace<XCPR>;
};

__device__ __forceinline__ void dma16(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)(lds_wave_base), 16, 0, 0);
}

// Source of the U rows from R up to 32 KS (the padding of the matrix-core extent): zeros.
__device__ __align__(16) uint32_t g_dz_zero16[4];

// Waits until at most N of this wave's vector memory operations are outstanding, then
// joins the workgroup barrier; the memory clobber keeps LDS accesses on their side.
template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("s_barrier" ::: "memory");
}

template <typename ET, int W, int KS, int HG>
__device__ __forceinline__ void lowrank_dz_dma(const LowRankParams& p, unsigned char* smem, int b, int tb0) {
  using D = LrDzDma<W, KS, HG>;
  constexpr int RP = D::RP, CH = D::CH, UC = D::UC, UCPR = D::UCPR, XCPR = D::XCPR, HALO = D::HALO;
  constexpr int RTN = RP / 16;
  constexpr int GL = D::GL, RUNS = D::RUNS;
  constexpr int KST = GL * W / 8;  // K steps per chunk: the lane's GL * W columns / 8
  static_assert(D::SHAPE_OK, "whole K steps");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int q = lane >> 4;
  const int n = lane & 15;
  const int wv = tid >> 6;
  const int nchunk = p.D / D::CHC;
  const ET* U = static_cast<const ET*>(p.U);
  const ET* xb = static_cast<const ET*>(p.x) + b * p.xs0 + int64_t(tb0 - HALO) * p.xs1;
  const ET* dyb = static_cast<const ET*>(p.dy) + b * p.dys0 + int64_t(tb0) * p.dys1;

  // this wave's transfers of a stage: instructions wv, wv + 4, ... of each region; per
  // lane the element offset of its source chunk relative to the chunk's base
  constexpr int SU = (D::NI_U + 3) / 4, SX = (D::NI_X + 3) / 4, SD = (D::NI_D + 3) / 4;
  int uoffg[SU], xoffg[SX], doffg[SD];
  bool uact[SU], xact[SX], dact[SD], uzero[SU];
#pragma unroll
  for (int i = 0; i < SU; ++i) {
    const int pidx = (wv + 4 * i) * 64 + lane;
    const int r = pidx / UCPR, pc = pidx % UCPR;
    const int c = D::UPlace::chunk(r & 15, pc);
    uact[i] = pidx < D::UCH;
    uzero[i] = r >= p.R;  // a padding rank: zeros, never a row past U
    uoffg[i] = r * int(p.ldu) + c * 8;
  }
  const ET* uzsrc = reinterpret_cast<const ET*>(g_dz_zero16);
#pragma unroll
  for (int i = 0; i < SX; ++i) {
    const int pidx = (wv + 4 * i) * 64 + lane;
    const int row = pidx / XCPR, c = D::XPlace::chunk(row, pidx % XCPR);
    xact[i] = pidx < D::XCH;
    // rows before token 0 read token 0 instead (their products are zeroed below)
    xoffg[i] = max(row, HALO - tb0) * int(p.xs1) + c * 8;
  }
#pragma unroll
  for (int i = 0; i < SD; ++i) {
    const int pidx = (wv + 4 * i) * 64 + lane;
    const int row = pidx / XCPR, c = D::XPlace::chunk(row, pidx % XCPR);
    dact[i] = pidx < D::DCH;
    doffg[i] = row * int(p.dys1) + c * 8;
  }
  // every wave issues at least this many transfers per stage
  constexpr int NMIN = D::NI_U / 4 + D::NI_X / 4 + D::NI_D / 4;
  auto issue = [&](int st, int ci) {
    ci = min(ci, nchunk - 1);  // past the last chunk: reload it (never read)
    const int c0 = ci * D::CHC;  // first channel; the chunk's filter columns start at ci * CH * W
    unsigned char* stage = smem + st * D::STAGE;
    const ET* ub = U + int64_t(ci) * (CH * W);
#pragma unroll
    for (int i = 0; i < SU; ++i)
      if (uact[i]) dma16(uzero[i] ? uzsrc : ub + uoffg[i], stage + (wv + 4 * i) * 1024);
#pragma unroll
    for (int i = 0; i < SX; ++i)
      if (xact[i]) dma16(xb + c0 + xoffg[i], stage + D::X_OFF + (wv + 4 * i) * 1024);
#pragma unroll
    for (int i = 0; i < SD; ++i)
      if (dact[i]) dma16(dyb + c0 + doffg[i], stage + D::D_OFF + (wv + 4 * i) * 1024);
  };

  // per-lane LDS byte offsets inside a stage
  const int nt = wv * TT + n;  // the lane's token within the block
  // the lane's runs are logical chunks q * RUNS + h of its rows
  int dy_off[RUNS], x_off[W][RUNS];
#pragma unroll
  for (int h = 0; h < RUNS; ++h) {
    dy_off[h] = D::D_OFF + nt * (XCPR * 16) + D::XPlace::slot(nt, q * RUNS + h) * 16;
#pragma unroll
    for (int k = 0; k < W; ++k) {
      const int row = nt + HALO - k;
      x_off[k][h] = D::X_OFF + row * (XCPR * 16) + D::XPlace::slot(row, q * RUNS + h) * 16;
    }
  }
  int u_off[KST];  // row rt * 16 + n adds rt * 16 * UC * 2 bytes (same rotation)
#pragma unroll
  for (int ks = 0; ks < KST; ++ks) u_off[ks] = n * UC * 2 + D::UPlace::slot(n, q * KST + ks) * 16;

  f32x4_t acc[RTN];
#pragma unroll
  for (int j = 0; j < RTN; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Taps of the lane's token whose x row is zero: before t = 0 and, for packed
  // sequences, in another segment. The ids are read (and waited for) before the first
  // transfer, so that every wait below counts LDS transfers only.
  bool tp[W];
  const bool cut = tb0 < HALO || p.seg != nullptr;
#pragma unroll
  for (int k = 0; k < W; ++k) tp[k] = tb0 + nt - k >= 0;
  if (p.seg != nullptr) {
    const int32_t* sgp = p.seg + b * p.ss0;
    const int t = tb0 + nt;  // whole token blocks inside T
    const int cur = sgp[int64_t(t) * p.ss1];
#pragma unroll
    for (int k = 1; k < W; ++k) tp[k] = tp[k] && sgp[int64_t(max(t - k, 0)) * p.ss1] == cur;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  issue(0, 0);
  if constexpr (D::NST == 3) issue(1, 1);
  for (int ci = 0; ci < nchunk; ++ci) {
    if constexpr (D::NST == 3) {
      // this wave's transfers of stage ci were followed by at least NMIN newer ones
      vm_wait_barrier<NMIN>();
      issue((ci + 2) % D::NST, ci + 2);
    } else {
      vm_wait_barrier<0>();
      issue((ci + 1) % D::NST, ci + 1);
    }
    const unsigned char* stage = smem + (ci % D::NST) * D::STAGE;
    // words of the lane's dy run and x runs (taps 0 .. W-1); channel j of the lane is
    // word (j % 8) / 2 of run j / 8
    uint32_t dw_[RUNS][4], xw[W][RUNS][4];
#pragma unroll
    for (int h = 0; h < RUNS; ++h) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + dy_off[h]);
      dw_[h][0] = v[0]; dw_[h][1] = v[1]; dw_[h][2] = v[2]; dw_[h][3] = v[3];
#pragma unroll
      for (int k = 0; k < W; ++k) {
        const u32x4 u = *reinterpret_cast<const u32x4*>(stage + x_off[k][h]);
        xw[k][h][0] = u[0]; xw[k][h][1] = u[1]; xw[k][h][2] = u[2]; xw[k][h][3] = u[3];
      }
    }
    if (cut) {
#pragma unroll
      for (int k = 1; k < W; ++k)
#pragma unroll
        for (int h = 0; h < RUNS; ++h)
          if (!tp[k]) xw[k][h][0] = xw[k][h][1] = xw[k][h][2] = xw[k][h][3] = 0u;
    }
    float dyf[8 * RUNS];
#pragma unroll
    for (int j = 0; j < 8 * RUNS; ++j) dyf[j] = (j & 1) ? Cvt<ET>::hi(dw_[j >> 3][(j & 7) >> 1]) : Cvt<ET>::lo(dw_[j >> 3][(j & 7) >> 1]);
    // column (group g of the lane, tap k): the sum over the group's HG channels
    auto col = [&](int g, int k) -> float {
      auto prod = [&](int j) {
        const uint32_t wd = xw[k][j >> 3][(j & 7) >> 1];
        return dyf[j] * ((j & 1) ? Cvt<ET>::hi(wd) : Cvt<ET>::lo(wd));
      };
      float v = prod(g * HG);
#pragma unroll
      for (int h = 1; h < HG; ++h) v += prod(g * HG + h);
      return v;
    };
#pragma unroll
    for (int ks = 0; ks < KST; ++ks) {
      typename Mfma<ET>::F32k bfr;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int c0_ = (8 * ks + e) / W, k0_ = (8 * ks + e) % W;
        const int c1_ = (8 * ks + e + 1) / W, k1_ = (8 * ks + e + 1) % W;
        const uint32_t w2 = Cvt<ET>::pack2(col(c0_, k0_), col(c1_, k1_));
        bfr.v[e] = uint16_t(w2 & 0xffffu);
        bfr.v[e + 1] = uint16_t(w2 >> 16);
      }
#pragma unroll
      for (int rt = 0; rt < RTN; ++rt) {
        typename Mfma<ET>::F32k afr;
        afr.v = *reinterpret_cast<const u16x8_t*>(stage + u_off[ks] + rt * 16 * UC * 2);
        acc[rt] = Mfma<ET>::mma32(afr, bfr, acc[rt]);
      }
    }
  }
  // drain this wave's remaining transfers (into stages nobody reads) before leaving
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
  ET* dz = static_cast<ET*>(p.dz) + b * p.dzs0;
  const int t = tb0 + nt;
#pragma unroll
  for (int rt = 0; rt < RTN; ++rt)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int r = rt * 16 + 4 * q + ii;
      if (r < p.R) reinterpret_cast<uint16_t*>(dz)[int64_t(t) * p.dzs1 + r] = Cvt<ET>::bits(acc[rt][ii]);
    }
}

// The LDS DMA path serves 16-bit (bf16, float16) token blocks that lie inside T when its
// stages fit.
template <typename ET, int W, int KS, int HG>
constexpr bool lowrank_dz_dma_ok() {
  return (std::is_same<ET, bf16_t>::value || std::is_same<ET, f16_t>::value) && LrDzDma<W, KS, HG>::SHAPE_OK &&
         LrDzDma<W, KS, HG>::BYTES <= 150 * 1024;
}

// The register-staged path: any storage type, ragged token blocks, unaligned rows, any
// group size (head-wise: each channel's column of U loaded element by element).
template <typename ET, int W, int KS>
__global__ __launch_bounds__(kBlockThreads) void k_lowrank_dz(const LowRankParams p) {
  __shared__ LrDzSmem<ET, W, KS> sm;
  lowrank_dz_body<ET, W, KS>(p, sm);
}

// The LDS DMA path: the launch covers whole token blocks; aligned rows, D % (32 * HG) == 0;
// R zero-padded to 32 KS (the U rows past R read zeros, dz columns past R are not stored).
template <typename ET, int W, int KS, int HG>
__global__ __launch_bounds__(kBlockThreads) void k_lowrank_dz_dma(const LowRankParams p) {
  __shared__ __align__(16) unsigned char smem[LrDzDma<W, KS, HG>::BYTES];
  const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
  lowrank_dz_dma<ET, W, KS, HG>(p, smem, int(lb / uint32_t(p.nTbL)),
                            (p.tbb0 + int(lb % uint32_t(p.nTbL))) * kLowrankDzTokens);
}

// Launches the DMA dz kernel for group size HG over q.nTbL whole token blocks per sequence.
template <typename ET, int W, int KS, int HG>
hipError_t launch_dz_dma(const LowRankParams& q, hipStream_t s) {
  if constexpr (lowrank_dz_dma_ok<ET, W, KS, HG>()) {
    hipLaunchKernelGGL((k_lowrank_dz_dma<ET, W, KS, HG>), dim3(unsigned(int64_t(q.B) * q.nTbL)), dim3(kBlockThreads), 0,
                       s, q);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------------
template <typename ET, int W, int KS>
hipError_t lr_fwd_inst(const LowRankParams& p, const LowRankPlan& pl, hipStream_t s) {
  LowRankParams q = p;
  q.cs0 = 0;
  q.nCsL = pl.nCs;
  hipLaunchKernelGGL((k_lowrank_fwd<ET, W, KS>), dim3(unsigned(pl.blocks)), dim3(kBlockThreads), 0, s, q);
  return hipGetLastError();
}

template <typename ET, int W, int KS>
hipError_t lr_bwd_inst(const LowRankParams& p, const LowRankPlan& pl, hipStream_t s) {
  // bf16 fast path: dx, then the partial sums of dU and db, each by its own kernel;
  // otherwise one main kernel (the channel slices inside D on the 16-byte path, the rest on
  // the other)
  // (packed sequences: with contiguous, aligned id rows and T % 4 == 0)
  constexpr bool h16 = std::is_same<ET, bf16_t>::value || std::is_same<ET, f16_t>::value;
  constexpr dynconv_dtype dt = std::is_same<ET, f16_t>::value ? DYNCONV_F16 : DYNCONV_BF16;
  const bool fast = h16 && lowrank_bwd_fast(p, W, dt);
  LowRankParams q = p;
  const int64_t per_slice = int64_t(p.B) * pl.nTr;
  const bool vec = p.act16 != 0 && p.z16 != 0 && p.R % 32 == 0;
  const int nfull = fast ? pl.nCs : vec ? p.D / lowrank_bwd_dc(W, KS) : 0;
  if (fast) {
    const hipError_t e = launch_lowrank_bwd_fused(p, W, dt, s);
    if (e != hipSuccess) return e;
  } else if (nfull > 0) {
    q.cs0 = 0;
    q.nCsL = nfull;
    hipLaunchKernelGGL((k_lowrank_bwd<ET, W, KS, true>), dim3(unsigned(per_slice * nfull)), dim3(kBlockThreads), 0, s,
                       q);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (nfull < pl.nCs) {
    q.cs0 = nfull;
    q.nCsL = pl.nCs - nfull;
    hipLaunchKernelGGL((k_lowrank_bwd<ET, W, KS, false>), dim3(unsigned(per_slice * q.nCsL)), dim3(kBlockThreads), 0,
                       s, q);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // dz: token blocks inside T on the DMA path (group sizes 1, 2, 4 whose stages fit), the
  // rest on the register path
  const int nblk = (p.T + kLowrankDzTokens - 1) / kLowrankDzTokens;
  const bool hg_ok = p.H == 1    ? lowrank_dz_dma_ok<ET, W, KS, 1>()
                     : p.H == 2  ? lowrank_dz_dma_ok<ET, W, KS, 2>()
                     : p.H == 4  ? lowrank_dz_dma_ok<ET, W, KS, 4>()
                     : p.H == 8  ? lowrank_dz_dma_ok<ET, W, KS, 8>()
                     : p.H == 16 ? lowrank_dz_dma_ok<ET, W, KS, 16>()
                                 : false;
  const int chunk_channels = p.H <= 4 ? kLowrankDzChunk * p.H : 128;
  const bool dma = hg_ok && p.act16 != 0 && p.u16 != 0 && p.D % chunk_channels == 0;
  const int nfb = dma ? p.T / kLowrankDzTokens : 0;
  if (nfb > 0) {
    q.tbb0 = 0;
    q.nTbL = nfb;
    const hipError_t e = p.H == 1   ? launch_dz_dma<ET, W, KS, 1>(q, s)
                         : p.H == 2 ? launch_dz_dma<ET, W, KS, 2>(q, s)
                         : p.H == 4 ? launch_dz_dma<ET, W, KS, 4>(q, s)
                         : p.H == 8 ? launch_dz_dma<ET, W, KS, 8>(q, s)
                                    : launch_dz_dma<ET, W, KS, 16>(q, s);
    if (e != hipSuccess) return e;
  }
  if (nfb < nblk) {
    q.tbb0 = nfb;
    q.nTbL = nblk - nfb;
    hipLaunchKernelGGL((k_lowrank_dz<ET, W, KS>), dim3(unsigned(int64_t(p.B) * q.nTbL)), dim3(kBlockThreads), 0, s, q);
  }
  return hipGetLastError();
}

template <bool BWD, typename ET, int W>
hipError_t lr_dispatch_ks(const LowRankParams& p, const LowRankPlan& pl, hipStream_t s) {
  const int ks = (p.R + 31) / 32;
  switch (ks) {
    case 1: return BWD ? lr_bwd_inst<ET, W, 1>(p, pl, s) : lr_fwd_inst<ET, W, 1>(p, pl, s);
    case 2: return BWD ? lr_bwd_inst<ET, W, 2>(p, pl, s) : lr_fwd_inst<ET, W, 2>(p, pl, s);
    case 3: return BWD ? lr_bwd_inst<ET, W, 3>(p, pl, s) : lr_fwd_inst<ET, W, 3>(p, pl, s);
    case 4: return BWD ? lr_bwd_inst<ET, W, 4>(p, pl, s) : lr_fwd_inst<ET, W, 4>(p, pl, s);
    default: return hipErrorInvalidValue;
  }
}

template <bool BWD, typename ET>
hipError_t lr_dispatch_w(const LowRankParams& p, const LowRankPlan& pl, int W, hipStream_t s) {
  switch (W) {
    case 1: return lr_dispatch_ks<BWD, ET, 1>(p, pl, s);
    case 2: return lr_dispatch_ks<BWD, ET, 2>(p, pl, s);
    case 3: return lr_dispatch_ks<BWD, ET, 3>(p, pl, s);
    case 4: return lr_dispatch_ks<BWD, ET, 4>(p, pl, s);
    case 5: return lr_dispatch_ks<BWD, ET, 5>(p, pl, s);
    case 6: return lr_dispatch_ks<BWD, ET, 6>(p, pl, s);
    case 7: return lr_dispatch_ks<BWD, ET, 7>(p, pl, s);
    case 8: return lr_dispatch_ks<BWD, ET, 8>(p, pl, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Launches the general forward (bwd == false) or backward kernels for storage type ET.
template <typename ET>
hipError_t lowrank_dispatch(const LowRankParams& p, const LowRankPlan& pl, int W, bool bwd, hipStream_t s) {
  return bwd ? lr_dispatch_w<true, ET>(p, pl, W, s) : lr_dispatch_w<false, ET>(p, pl, W, s);
}

}  // namespace dynconv
