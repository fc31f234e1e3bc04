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
//                   complete without partial sums.
//   partial sums of dU and db are then added in a fixed order (run-to-run deterministic).
#include "dynconv_common.hpp"
#include "dynconv_internal.hpp"

namespace dynconv {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int TT = 16;    // tokens per tile (the N, or K, extent of one MFMA)
constexpr int HALO = 4;   // W - 1 for the widest filter (W = 5)
constexpr int RING = TT + HALO;

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
// workgroups that share a z tile run on the same XCD at about the same time.
struct LrBlock {
  int b, tr, cs;
};
__device__ __forceinline__ LrBlock lr_block(const LowRankParams& p) {
  uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
  LrBlock r;
  r.cs = lb % p.nCs;
  lb /= p.nCs;
  r.tr = lb % p.nTr;
  r.b = lb / p.nTr;
  return r;
}

// U^T fragments of this wave's filter-column tiles, loaded once per workgroup, and the
// bias as the accumulator's initial value. Columns past J and ranks past R read as 0.
template <typename ET, int KS, int MTW>
struct GenFrags {
  typename Mfma<ET>::F32k a[MTW][KS];
  f32x4_t binit[MTW];

  __device__ __forceinline__ void load(const LowRankParams& p, int j_base, int wv, int mt_total) {
    using R_ = Raw<ET>;
    const int lane = threadIdx.x & 63;
    const int q = lane >> 4;
    const ET* U = static_cast<const ET*>(p.U);
    const ET* bias = static_cast<const ET*>(p.bias);
#pragma unroll
    for (int i = 0; i < MTW; ++i) {
      const int mt = wv + 4 * i;
      const bool mt_ok = mt < mt_total;
      const int j = j_base + mt * 16 + (lane & 15);
      const bool j_ok = mt_ok && j < p.J;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 32 * ks + Mfma<ET>::k32(q, e);
          const auto v = (j_ok && r < p.R) ? R_::from_mem(U, int64_t(r) * p.ldu + j) : R_::zero();
          a[i][ks].v[e] = v;
        }
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int jr = j_base + mt * 16 + 4 * q + ii;
        binit[i][ii] = (mt_ok && bias != nullptr && jr < p.J) ? R_::to_float(R_::from_mem(bias, jr)) : 0.f;
      }
    }
  }
};

// One 16 x 16 block of generated filters: rows are filter columns (mt*16 ..), columns are
// the 16 tokens of the tile; z tile row n starts at zl + n * ZP.
template <typename ET, int KS, int ZP>
__device__ __forceinline__ f32x4_t gen_tile(const typename Mfma<ET>::F32k (&a)[KS], f32x4_t acc,
                                            const typename Raw<ET>::type* zl) {
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4;
  const int n = lane & 15;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    typename Mfma<ET>::F32k bfr;
    if constexpr (sizeof(ET) == 2) {
      bfr.v = *reinterpret_cast<const u16x8_t*>(zl + n * ZP + 32 * ks + 8 * q);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) bfr.v[e] = zl[n * ZP + 32 * ks + Mfma<ET>::k32(q, e)];
    }
    acc = Mfma<ET>::mma32(a[ks], bfr, acc);
  }
  return acc;
}

// Slot of token t in the x ring of one workgroup (tokens t_first - HALO .. kept).
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
      o[e] = (e & 1) ? bf16_hi(u[e >> 1]) : bf16_lo(u[e >> 1]);
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
        u[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
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
        reinterpret_cast<uint16_t*>(p)[e] = to_bf16_bits(v[e]);
      } else {
        reinterpret_cast<float*>(p)[e] = v[e];
      }
    }
  }
}

template <typename ET>
__device__ __forceinline__ float chunk_elem(const u32x4& v, int e) {
  if constexpr (sizeof(ET) == 2) {
    return (e & 1) ? bf16_hi(v[e >> 1]) : bf16_lo(v[e >> 1]);
  } else {
    return __uint_as_float(v[e]);
  }
}

// DPP / register-run helpers shared by the kernels below.
template <typename ET, int N>
struct RunWords {  // N contiguous elements as raw 32-bit words
  static constexpr int ND = N * int(sizeof(ET)) / 4;
  uint32_t u[ND];
};

template <typename ET, int N>
__device__ __forceinline__ void load_run(RunWords<ET, N>& r, const ET* p, bool vec, int count) {
  constexpr int ND = RunWords<ET, N>::ND;
  if (vec && count >= N) {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
    if constexpr (ND % 4 == 0) {
#pragma unroll
      for (int i = 0; i < ND / 4; ++i) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q) + i);
        r.u[4 * i] = v[0];
        r.u[4 * i + 1] = v[1];
        r.u[4 * i + 2] = v[2];
        r.u[4 * i + 3] = v[3];
      }
    } else if constexpr (ND == 2) {
      const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(q));
      r.u[0] = v[0];
      r.u[1] = v[1];
    } else {
#pragma unroll
      for (int i = 0; i < ND; ++i) r.u[i] = __builtin_nontemporal_load(q + i);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < ND; ++i) r.u[i] = 0u;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    if (e < count) {
      if constexpr (sizeof(ET) == 2) {
        const uint32_t h = reinterpret_cast<const uint16_t*>(p)[e];
        r.u[e >> 1] |= (e & 1) ? (h << 16) : h;
      } else {
        r.u[e] = __float_as_uint(reinterpret_cast<const float*>(p)[e]);
      }
    }
  }
}

template <typename ET, int N>
__device__ __forceinline__ float run_elem(const RunWords<ET, N>& r, int e) {
  if constexpr (sizeof(ET) == 2) {
    return (e & 1) ? bf16_hi(r.u[e >> 1]) : bf16_lo(r.u[e >> 1]);
  } else {
    return __uint_as_float(r.u[e]);
  }
}

// Lane i of each 16-lane row gets cur from lane i - K, or prev from lane i - K + 16.
template <int K, typename ET, int N>
__device__ __forceinline__ RunWords<ET, N> shift_rows(const RunWords<ET, N>& cur, const RunWords<ET, N>& prev) {
  static_assert(K >= 1 && K <= 15, "row shifts are 1..15 lanes");
  RunWords<ET, N> r;
#pragma unroll
  for (int i = 0; i < RunWords<ET, N>::ND; ++i) {
    const int from_prev = __builtin_amdgcn_mov_dpp(int(prev.u[i]), 0x120 | K, 0xf, 0xf, false);
    r.u[i] = uint32_t(__builtin_amdgcn_update_dpp(from_prev, int(cur.u[i]), 0x110 | K, 0xf, 0xf, false));
  }
  return r;
}

// z fragment of one K step for lane (token row, group q): z[row][32 ks + k32(q, e)].
template <typename ET>
__device__ __forceinline__ void load_zfrag(typename Mfma<ET>::F32k& f, const ET* zrow, int ks, int q, int R,
                                           bool vec, bool row_ok) {
  if constexpr (sizeof(ET) == 2) {
    const int r0 = 32 * ks + 8 * q;
    if (row_ok && vec && r0 + 8 <= R) {
      f.v = __builtin_nontemporal_load(reinterpret_cast<const u16x8_t*>(zrow + r0));
      return;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
      f.v[e] = (row_ok && r0 + e < R) ? reinterpret_cast<const uint16_t*>(zrow)[r0 + e] : uint16_t(0);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = 32 * ks + Mfma<ET>::k32(q, e);
      f.v[e] = (row_ok && r < R) ? reinterpret_cast<const float*>(zrow)[r] : 0.f;
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
  __shared__ __align__(16) RT zl[TT * ZP];
  __shared__ __align__(16) ET xl[RING * XP];

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
      const int64_t col = int64_t(ch) * W + tap;
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
                           ? Raw<ET>::to_float(Raw<ET>::from_mem(bias, int64_t(chq) * W + tq))
                           : 0.f;
      }
    }
  }

  // Staging of one tile: z rows (zero past the range / R) and x rows (zero past D); the
  // loads of tile i+1 are issued before tile i is computed.
  u32x4 zpre_s[1][ZCH], xpre_s[1][XCH];
  auto prefetch = [&](u32x4 (&zpre)[ZCH], u32x4 (&xpre)[XCH], int t0) {
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
        *reinterpret_cast<u32x4*>(&xl[ring_slot(t0 + row, t_first) * XP + (ck % (DC / CE)) * CE]) = xpre[i];
      }
    }
  };

  // halo: the HALO tokens before the range
  for (int ck = tid; ck < HALO * DC / CE; ck += kBlockThreads) {
    const int row = ck / (DC / CE);
    const int c = (ck % (DC / CE)) * CE;
    const int t = t_first - HALO + row;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (t >= 0) v = load_chunk<ET>(x + int64_t(t) * p.xs1 + c_base, c, p.D - c_base, act16);
    *reinterpret_cast<u32x4*>(&xl[ring_slot(t, t_first) * XP + c]) = v;
  }
  prefetch(zpre_s[0], xpre_s[0], t_first);
  commit(zpre_s[0], xpre_s[0], t_first);
  __syncthreads();

  const int lane_c = (q / LPC) * MT;  // first channel of this lane's run, within the wave
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
    float sum[MT], xcur[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      sum[mt] = 0.f;
      xcur[mt] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tap = 4 * (q % LPC) + i;
      if (tap < W) {
        float xv[MT];
        lds_read_run<ET, MT>(&xl[ring_slot(t - tap, t_first) * XP + wv * CPW + lane_c], xv);
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
      for (int mt = 0; mt < MT; ++mt) yv[mt] = xcur[mt] + sum[mt];
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
// Same workgroup decomposition and filter regeneration as the forward (with MT tiles
// per wave, so lane (token n, group q) holds the filter taps of a run of MT contiguous
// channels for token t0 + n). Per 16-token tile:
//  * P_k = w_k^(t) dy_t for the lane's token; dx_s = dy_s + sum_k P_k(s + k) is formed
//    for s = t0 + n - (W-1): the terms of later tokens come from the lanes to the right
//    (DPP row_shr) and, for the first lanes, from the previous tile (DPP row_ror). One
//    extra tile past the range supplies the last W-1 rows (the future halo).
//  * g_k(t) = dy_t x_{t-k} for the lane's token and channels (x from the LDS ring); db
//    is summed per lane; g goes to a wave-private LDS tile, from which the matrix cores
//    accumulate dU += z^T g (K = the 16 tokens) in registers over the whole range.
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

template <typename ET, int W, int KS>
__global__ __launch_bounds__(kBlockThreads) void k_lowrank_bwd(const LowRankParams p) {
  using RT = typename Raw<ET>::type;
  using R_ = Raw<ET>;
  constexpr int EB = int(sizeof(ET));
  constexpr int MT = lowrank_bwd_mt(KS);
  constexpr int WP = lowrank_rows_per_channel(W);  // padded taps per channel
  constexpr int LPC = WP / 4;
  constexpr int CPW = MT * 4 / LPC;  // channels per wave
  constexpr int DC = 4 * CPW;        // channels per workgroup
  constexpr int RP = 32 * KS;
  constexpr int CE = 16 / EB;
  constexpr int ZP = RP + CE;
  constexpr int XP = DC + CE;
  constexpr int GC = CPW * WP;       // padded filter columns of a wave
  constexpr int GP = GC + 8 / EB;    // g row pitch
  constexpr int RTN = RP / 16;       // r tiles of dU
  constexpr int JTN = GC / 16;       // column tiles of dU
  constexpr int ZCH = TT * RP / CE;
  constexpr int XCH = TT * DC / CE;
  constexpr int NCH = ZCH + 2 * XCH;
  constexpr int CPT = (NCH + kBlockThreads - 1) / kBlockThreads;
  static_assert(GC % 16 == 0, "whole column tiles per wave");
  __shared__ __align__(16) RT zl[TT * ZP];
  __shared__ __align__(16) ET xl[RING * XP];
  __shared__ __align__(16) ET dyl[RING * XP];
  __shared__ __align__(16) RT gl[4][TT * GP];

  const LrBlock blk = lr_block(p);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int q = lane >> 4;
  const int n = lane & 15;
  const int wv = tid >> 6;
  const int c_base = blk.cs * DC;
  const int t_first = blk.tr * p.Ltok;
  const int t_end = min(p.T, t_first + p.Ltok);
  const int range = blk.b * p.nTr + blk.tr;
  const ET* x = static_cast<const ET*>(p.x) + blk.b * p.xs0;
  const ET* z = static_cast<const ET*>(p.z) + blk.b * p.zs0;
  const ET* dy = static_cast<const ET*>(p.dy) + blk.b * p.dys0;
  ET* dx = static_cast<ET*>(p.out) + blk.b * p.os0;
  const bool act16 = p.act16 != 0;
  const bool z16 = p.z16 != 0;
  const int cw0 = c_base + wv * CPW;
  const int lane_c = (q / LPC) * MT;  // first channel of the lane's run, within the wave
  const int cl = cw0 + lane_c;
  const int cl_count = p.D - cl;

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
      const int64_t col = int64_t(ch) * W + tap;
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
                           ? R_::to_float(R_::from_mem(bias, int64_t(cl + mt) * W + tq))
                           : 0.f;
      }
    }
  }

  // staging: z and dy rows of a tile up to T (dy/w of later tokens complete dx), x rows
  // up to the end of the range
  u32x4 pre[CPT];
  auto prefetch = [&](int t0) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ck = tid + i * kBlockThreads;
      pre[i] = u32x4{0u, 0u, 0u, 0u};
      if (ck < ZCH) {
        const int row = ck / (RP / CE), c = (ck % (RP / CE)) * CE, t = t0 + row;
        if (t < p.T) pre[i] = load_chunk<ET>(z + int64_t(t) * p.zs1, c, p.R, z16);
      } else if (ck < ZCH + XCH) {
        const int k2 = ck - ZCH;
        const int row = k2 / (DC / CE), c = (k2 % (DC / CE)) * CE, t = t0 + row;
        if (t < t_end) pre[i] = load_chunk<ET>(x + int64_t(t) * p.xs1 + c_base, c, p.D - c_base, act16);
      } else if (ck < NCH) {
        const int k2 = ck - ZCH - XCH;
        const int row = k2 / (DC / CE), c = (k2 % (DC / CE)) * CE, t = t0 + row;
        if (t < p.T) pre[i] = load_chunk<ET>(dy + int64_t(t) * p.dys1 + c_base, c, p.D - c_base, act16);
      }
    }
  };
  auto commit = [&](int t0) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ck = tid + i * kBlockThreads;
      if (ck < ZCH) {
        *reinterpret_cast<u32x4*>(&zl[(ck / (RP / CE)) * ZP + (ck % (RP / CE)) * CE]) = pre[i];
      } else if (ck < ZCH + XCH) {
        const int k2 = ck - ZCH;
        const int row = k2 / (DC / CE);
        *reinterpret_cast<u32x4*>(&xl[ring_slot(t0 + row, t_first) * XP + (k2 % (DC / CE)) * CE]) = pre[i];
      } else if (ck < NCH) {
        const int k2 = ck - ZCH - XCH;
        const int row = k2 / (DC / CE);
        *reinterpret_cast<u32x4*>(&dyl[ring_slot(t0 + row, t_first) * XP + (k2 % (DC / CE)) * CE]) = pre[i];
      }
    }
  };

  // halo rows before the range: x (for g) and dy (rows of dx that other ranges store)
  for (int ck = tid; ck < 2 * HALO * DC / CE; ck += kBlockThreads) {
    const bool is_dy = ck >= HALO * DC / CE;
    const int k2 = is_dy ? ck - HALO * DC / CE : ck;
    const int row = k2 / (DC / CE), c = (k2 % (DC / CE)) * CE, t = t_first - HALO + row;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (t >= 0) v = load_chunk<ET>((is_dy ? dy + int64_t(t) * p.dys1 : x + int64_t(t) * p.xs1) + c_base, c,
                                   p.D - c_base, act16);
    *reinterpret_cast<u32x4*>(&(is_dy ? dyl : xl)[ring_slot(t, t_first) * XP + c]) = v;
  }
  prefetch(t_first);
  commit(t_first);
  __syncthreads();

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
  for (int t0 = t_first; t0 - (W - 1) < t_end; t0 += TT) {
    const bool more = t0 + TT - (W - 1) < t_end;
    if (more) prefetch(t0 + TT);
    // regenerate the filters of tokens t0 .. t0 + 15
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
    float wv_[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4_t a = binit[mt];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) a = Mfma<ET>::mma32(afr[mt][ks], bfr[ks], a);
#pragma unroll
      for (int i = 0; i < 4; ++i) wv_[mt][i] = a[i];
    }
    const int t = t0 + n;
    float dyn[MT];
    lds_read_run<ET, MT>(&dyl[ring_slot(t, t_first) * XP + wv * CPW + lane_c], dyn);
    // dx for token s = t - (W - 1)
    float P[MT][4], dxs[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) P[mt][i] = wv_[mt][i] * dyn[mt];
      float acc;
      if constexpr (LPC == 1) {
        acc = shift_lanes<W - 1>(P[mt][0], Pprev[mt][0]);
        if constexpr (W > 1) acc += shift_lanes<(W > 1 ? W - 2 : 0)>(P[mt][1], Pprev[mt][1]);
        if constexpr (W > 2) acc += shift_lanes<(W > 2 ? W - 3 : 0)>(P[mt][2], Pprev[mt][2]);
        if constexpr (W > 3) acc += shift_lanes<(W > 3 ? W - 4 : 0)>(P[mt][3], Pprev[mt][3]);
      } else {
        // even groups hold taps 0..3 (later by 4..1 tokens), odd groups tap 4 (same token)
        const float even = shift_lanes<4>(P[mt][0], Pprev[mt][0]) + shift_lanes<3>(P[mt][1], Pprev[mt][1]) +
                           shift_lanes<2>(P[mt][2], Pprev[mt][2]) + shift_lanes<1>(P[mt][3], Pprev[mt][3]);
        const float mine = (q & 1) ? P[mt][0] : even;
        acc = mine + __shfl_xor(mine, 16, 64);
      }
      dxs[mt] = acc;
    }
    const int s = t - (W - 1);
    if ((q % LPC) == 0 && s >= t_first && s < t_end && cl_count > 0) {
      float dys[MT];
      lds_read_run<ET, MT>(&dyl[ring_slot(s, t_first) * XP + wv * CPW + lane_c], dys);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) dxs[mt] += dys[mt];
      global_store_run<ET, MT>(dx + int64_t(s) * p.os1 + cl, dxs, act16, cl_count);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) Pprev[mt][i] = P[mt][i];

    if (t0 < t_end) {
      // g_k(t) = dy_t x_{t-k}, zero past the range
      const bool tok_ok = t < t_end;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tap = 4 * (q % LPC) + i;
        float xr[MT];
        if (tap < W) {
          lds_read_run<ET, MT>(&xl[ring_slot(t - tap, t_first) * XP + wv * CPW + lane_c], xr);
        } else {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) xr[mt] = 0.f;
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const float g = (tok_ok && tap < W) ? dyn[mt] * xr[mt] : 0.f;
          db[mt][i] += g;
          P[mt][i] = g;  // reuse as the g tile of this lane
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        RT* dst = &gw[n * GP + (lane_c + mt) * WP + 4 * (q % LPC)];
        if constexpr (EB == 2) {
          *reinterpret_cast<u32x2*>(dst) =
              u32x2{pack_bf16x2(P[mt][0], P[mt][1]), pack_bf16x2(P[mt][2], P[mt][3])};
        } else {
          *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{P[mt][0], P[mt][1], P[mt][2], P[mt][3]};
        }
      }
      wave_lds_sync();
      // dU[r][col] += sum_n z_n[r] g_n[col] over the 16 tokens of the tile
#pragma unroll
      for (int rt = 0; rt < RTN; ++rt) {
        typename Mfma<ET>::F16k afr16;
#pragma unroll
        for (int e = 0; e < 4; ++e) afr16.v[e] = zl[Mfma<ET>::k16(q, e) * ZP + rt * 16 + n];
#pragma unroll
        for (int jt = 0; jt < JTN; ++jt) {
          typename Mfma<ET>::F16k bfr16;
#pragma unroll
          for (int e = 0; e < 4; ++e) bfr16.v[e] = gw[Mfma<ET>::k16(q, e) * GP + jt * 16 + n];
          dU[rt][jt] = Mfma<ET>::mma16(afr16, bfr16, dU[rt][jt]);
        }
      }
    }
    __syncthreads();
    if (more) commit(t0 + TT);
    __syncthreads();
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
      if (p.part_db != nullptr && n == 0 && tap < W && cl + mt < p.D)
        p.part_db[int64_t(range) * p.J + int64_t(cl + mt) * W + tap] = v;
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
          if (r < p.R) p.part_dU[(int64_t(range) * p.R + r) * p.J + int64_t(ch) * W + tap] = dU[rt][jt][ii];
        }
      }
    }
}

// ---------------------------------------------------------------------------------
// dz[t][r] = sum_j g_t[j] U[r][j], with g recomputed from x and dy.
// A workgroup owns kLowrankDzTokens tokens of one sequence (each wave two 16-token
// tiles) and walks the channels in chunks of CH: the chunk's U columns are staged in LDS
// (padded to WP taps per channel); x (with its 4-token halo) and dy rows of the chunk
// are staged in LDS too. Matrix cores: M = r, N = tokens, K = padded filter columns.
// Lane (token n, group q) supplies g for a run of CH/4 (W <= 4) or CH/8 channels.
// ---------------------------------------------------------------------------------
template <typename ET, int W, int KS>
__global__ __launch_bounds__(kBlockThreads) void k_lowrank_dz(const LowRankParams p) {
  using RT = typename Raw<ET>::type;
  using R_ = Raw<ET>;
  constexpr int EB = int(sizeof(ET));
  constexpr int RP = 32 * KS;
  constexpr int RTN = RP / 16;
  constexpr int CH = lowrank_dz_chunk(KS, EB, W);
  constexpr int WP = lowrank_rows_per_channel(W);
  constexpr int CPK = 8 / WP * 1;            // channels per lane per K step (2 or 1)
  constexpr int CR = CH / 4;                 // channels of a lane group's run
  constexpr int KSTEPS = CR / CPK;           // K steps per chunk
  constexpr int UC = CH * WP;                // padded columns of a chunk
  constexpr int UP = UC + 8;                 // U row pitch (elements)
  constexpr int TB = kLowrankDzTokens;
  constexpr int CE = 16 / EB;
  constexpr int XP = CH + CE;
  constexpr int TPW = TB / 64;               // 16-token tiles per wave
  static_assert(CR % CPK == 0 && TB % 64 == 0, "dz tiling");
  __shared__ __align__(16) RT Ul[RP * UP];
  __shared__ __align__(16) ET xl[(TB + HALO) * XP];
  __shared__ __align__(16) ET dyl[TB * XP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int q = lane >> 4;
  const int n = lane & 15;
  const int wv = tid >> 6;
  const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int nblk = (p.T + TB - 1) / TB;
  const int b = lb / nblk;
  const int tb0 = (lb % nblk) * TB;
  const ET* x = static_cast<const ET*>(p.x) + b * p.xs0;
  const ET* dy = static_cast<const ET*>(p.dy) + b * p.dys0;
  const ET* U = static_cast<const ET*>(p.U);
  const bool act16 = p.act16 != 0;

  f32x4_t acc[TPW][RTN];
#pragma unroll
  for (int i = 0; i < TPW; ++i)
#pragma unroll
    for (int j = 0; j < RTN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int c0 = 0; c0 < p.D; c0 += CH) {
    const int climit = p.D - c0;
    // stage U columns of channels c0 .. c0 + CH - 1, padded to WP taps, ranks to RP
    for (int idx = tid; idx < RP * CH; idx += kBlockThreads) {
      const int r = idx / CH, cc = idx % CH;
      RT v[WP];
#pragma unroll
      for (int k = 0; k < WP; ++k)
        v[k] = (r < p.R && cc < climit && k < W) ? R_::from_mem(U, int64_t(r) * p.ldu + int64_t(c0 + cc) * W + k)
                                                 : R_::zero();
#pragma unroll
      for (int k = 0; k < WP; ++k) Ul[r * UP + cc * WP + k] = v[k];
    }
    // stage x rows tb0 - HALO .. tb0 + TB - 1 and dy rows tb0 .. tb0 + TB - 1 of the chunk
    for (int ck = tid; ck < (2 * TB + HALO) * (CH / CE); ck += kBlockThreads) {
      const int row = ck / (CH / CE), c = (ck % (CH / CE)) * CE;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < TB + HALO) {
        const int t = tb0 - HALO + row;
        if (t >= 0 && t < p.T) v = load_chunk<ET>(x + int64_t(t) * p.xs1 + c0, c, climit, act16);
        *reinterpret_cast<u32x4*>(&xl[row * XP + c]) = v;
      } else {
        const int r2 = row - TB - HALO;
        const int t = tb0 + r2;
        if (t < p.T) v = load_chunk<ET>(dy + int64_t(t) * p.dys1 + c0, c, climit, act16);
        *reinterpret_cast<u32x4*>(&dyl[r2 * XP + c]) = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int tile = 0; tile < TPW; ++tile) {
      const int nt = (wv * TPW + tile) * 16 + n;  // token within the block
      // the lane's dy and x rows for its channel run
      float dyr[CR], xr[W][CR];
      lds_read_run<ET, CR>(&dyl[nt * XP + q * CR], dyr);
#pragma unroll
      for (int k = 0; k < W; ++k) lds_read_run<ET, CR>(&xl[(nt + HALO - k) * XP + q * CR], xr[k]);
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        typename Mfma<ET>::F32k bfr;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // slot e of lane group q <-> column (channel q*CR + ks*CPK + e / WP, tap e % WP);
          // A below uses the same slot -> column map, which is all the contraction needs
          const int cr = ks * CPK + e / WP;  // channel within the run
          const int tap = e % WP;
          const float g = tap < W ? dyr[cr] * xr[tap < W ? tap : 0][cr] : 0.f;
          bfr.v[e] = R_::from_float(g);
        }
#pragma unroll
        for (int rt = 0; rt < RTN; ++rt) {
          typename Mfma<ET>::F32k afr;
          const RT* src = &Ul[(rt * 16 + n) * UP + (q * CR + ks * CPK) * WP];
          if constexpr (EB == 2) {
            afr.v = *reinterpret_cast<const u16x8_t*>(src);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) afr.v[e] = src[e];
          }
          acc[tile][rt] = Mfma<ET>::mma32(afr, bfr, acc[tile][rt]);
        }
      }
    }
    __syncthreads();
  }
  // lane holds dz[token n][r = rt*16 + 4q + ii] of each tile
  ET* dz = static_cast<ET*>(p.dz) + b * p.dzs0;
#pragma unroll
  for (int tile = 0; tile < TPW; ++tile) {
    const int t = tb0 + (wv * TPW + tile) * 16 + n;
    if (t >= p.T) continue;
#pragma unroll
    for (int rt = 0; rt < RTN; ++rt)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int r = rt * 16 + 4 * q + ii;
        if (r < p.R) {
          const int64_t o = int64_t(t) * p.dzs1 + r;
          if constexpr (EB == 2) {
            reinterpret_cast<uint16_t*>(dz)[o] = to_bf16_bits(acc[tile][rt][ii]);
          } else {
            dz[o] = acc[tile][rt][ii];
          }
        }
      }
  }
}

// ---------------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------------
template <typename ET, int W, int KS>
hipError_t lr_fwd_inst(const LowRankParams& p, const LowRankPlan& pl, hipStream_t s) {
  hipLaunchKernelGGL((k_lowrank_fwd<ET, W, KS>), dim3(unsigned(pl.blocks)), dim3(kBlockThreads), 0, s, p);
  return hipGetLastError();
}

template <typename ET, int W, int KS>
hipError_t lr_bwd_inst(const LowRankParams& p, const LowRankPlan& pl, hipStream_t s) {
  hipLaunchKernelGGL((k_lowrank_bwd<ET, W, KS>), dim3(unsigned(pl.blocks)), dim3(kBlockThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t zblocks = int64_t(p.B) * ((p.T + kLowrankDzTokens - 1) / kLowrankDzTokens);
  hipLaunchKernelGGL((k_lowrank_dz<ET, W, KS>), dim3(unsigned(zblocks)), dim3(kBlockThreads), 0, s, p);
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
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

LowRankPlan plan_lowrank(int64_t B, int64_t T, int64_t D, int W, int H, int R, bool bwd) {
  LowRankPlan pl{};
  const int ks = (R + 31) / 32;
  const int DC = !bwd ? lowrank_fwd_dc(W, ks) : lowrank_bwd_dc(W, ks);
  pl.nCs = int((D + DC - 1) / DC);
  // about 1024 (forward) or 2048 (backward) workgroups, ranges in whole 16-token tiles
  const int64_t target = bwd ? 2048 : 1024;
  int64_t per_seq = (target + B * pl.nCs - 1) / (B * pl.nCs);
  const int64_t max_ranges = (T + TT - 1) / TT;
  if (per_seq > max_ranges) per_seq = max_ranges;
  if (per_seq < 1) per_seq = 1;
  int64_t L = (T + per_seq - 1) / per_seq;
  L = (L + TT - 1) / TT * TT;
  pl.Ltok = int(L);
  pl.nTr = int((T + L - 1) / L);
  pl.blocks = B * int64_t(pl.nTr) * pl.nCs;
  const int64_t J = (D / H) * W;
  const int64_t nR = B * int64_t(pl.nTr);
  pl.ws_dU = 0;
  pl.ws_db = size_t(nR) * size_t(R) * size_t(J) * sizeof(float);
  pl.ws_dz = pl.ws_db + size_t(nR) * size_t(J) * sizeof(float);
  pl.ws_total = bwd ? pl.ws_dz : 0;
  (void)H;
  return pl;
}

dynconv_status launch_lowrank_fwd(const LowRankParams& p, const LowRankPlan& plan, int W, dynconv_dtype dt,
                                  hipStream_t stream) {
  const hipError_t e = dt == DYNCONV_BF16 ? lr_dispatch_w<false, bf16_t>(p, plan, W, stream)
                                          : lr_dispatch_w<false, float>(p, plan, W, stream);
  return e == hipSuccess ? DYNCONV_OK : record_hip_error(e);
}

dynconv_status launch_lowrank_bwd(const LowRankParams& p, const LowRankPlan& plan, int W, dynconv_dtype dt,
                                  float* dU, float* db, hipStream_t stream) {
  const hipError_t e = dt == DYNCONV_BF16 ? lr_dispatch_w<true, bf16_t>(p, plan, W, stream)
                                          : lr_dispatch_w<true, float>(p, plan, W, stream);
  if (e != hipSuccess) return record_hip_error(e);
  const int64_t nR = int64_t(p.B) * plan.nTr;
  dynconv_status st = launch_reduce_partials(p.part_dU, nR, int64_t(p.R) * p.J, dU, stream);
  if (st != DYNCONV_OK || db == nullptr) return st;
  return launch_reduce_partials(p.part_db, nR, p.J, db, stream);
}

}  // namespace dynconv
