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
// Forward
// ---------------------------------------------------------------------------------
template <typename ET, int W, int KS>
__global__ __launch_bounds__(kBlockThreads) void k_lowrank_fwd(const LowRankParams p) {
  using RT = typename Raw<ET>::type;
  using R_ = Raw<ET>;
  constexpr int DC = 64;
  constexpr int JC = DC * W;
  constexpr int MT = JC / 16;
  constexpr int MTW = (MT + 3) / 4;
  constexpr int RP = 32 * KS;
  constexpr int ZP = RP + 8;
  constexpr int JP = JC + 4;
  __shared__ __align__(16) RT zl[TT * ZP];
  __shared__ __align__(16) float wl[TT * JP];
  __shared__ float xl[RING * DC];

  const LrBlock blk = lr_block(p);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int c_base = blk.cs * DC;
  const int j_base = c_base * W;
  const int t_first = blk.tr * p.Ltok;
  const int t_end = min(p.T, t_first + p.Ltok);
  if (t_first >= p.T) return;
  const ET* x = static_cast<const ET*>(p.x) + blk.b * p.xs0;
  const ET* z = static_cast<const ET*>(p.z) + blk.b * p.zs0;
  ET* y = static_cast<ET*>(p.out) + blk.b * p.os0;

  GenFrags<ET, KS, MTW> gf;
  gf.load(p, j_base, wv, MT);

  // x halo: the HALO tokens before the range
  for (int idx = tid; idx < HALO * DC; idx += kBlockThreads) {
    const int t = t_first - HALO + idx / DC;
    const int c = idx % DC;
    float v = 0.f;
    if (t >= 0 && c_base + c < p.D) v = R_::to_float(R_::from_mem(x, int64_t(t) * p.xs1 + c_base + c));
    xl[ring_slot(t, t_first) * DC + c] = v;
  }

  for (int t0 = t_first; t0 < t_end; t0 += TT) {
    for (int idx = tid; idx < TT * RP; idx += kBlockThreads) {
      const int n = idx / RP;
      const int r = idx % RP;
      const int t = t0 + n;
      zl[n * ZP + r] = (t < t_end && r < p.R) ? R_::from_mem(z, int64_t(t) * p.zs1 + r) : R_::zero();
    }
    for (int idx = tid; idx < TT * DC; idx += kBlockThreads) {
      const int n = idx / DC;
      const int c = idx % DC;
      const int t = t0 + n;
      float v = 0.f;
      if (t < t_end && c_base + c < p.D) v = R_::to_float(R_::from_mem(x, int64_t(t) * p.xs1 + c_base + c));
      xl[ring_slot(t, t_first) * DC + c] = v;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < MTW; ++i) {
      const int mt = wv + 4 * i;
      if (mt < MT) {
        const f32x4_t acc = gen_tile<ET, KS, ZP>(gf.a[i], gf.binit[i], zl);
        *reinterpret_cast<f32x4_t*>(&wl[(lane & 15) * JP + mt * 16 + 4 * (lane >> 4)]) = acc;
      }
    }
    __syncthreads();
    // conv + residual: thread -> 2 channels x 2 tokens
    {
      const int cp = tid & 31;
      const int tg = tid >> 5;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int n = 2 * tg + u;
        const int t = t0 + n;
        if (t >= t_end) continue;
        float yv[2];
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          const int c = 2 * cp + v;
          float acc = xl[ring_slot(t, t_first) * DC + c];
#pragma unroll
          for (int k = 0; k < W; ++k) acc = fmaf(wl[n * JP + c * W + k], xl[ring_slot(t - k, t_first) * DC + c], acc);
          yv[v] = acc;
        }
        const int cg = c_base + 2 * cp;
        if constexpr (sizeof(ET) == 2) {
          if (cg + 1 < p.D) {
            *reinterpret_cast<uint32_t*>(y + int64_t(t) * p.os1 + cg) = pack_bf16x2(yv[0], yv[1]);
          } else if (cg < p.D) {
            reinterpret_cast<uint16_t*>(y)[int64_t(t) * p.os1 + cg] = to_bf16_bits(yv[0]);
          }
        } else {
          if (cg < p.D) y[int64_t(t) * p.os1 + cg] = yv[0];
          if (cg + 1 < p.D) y[int64_t(t) * p.os1 + cg + 1] = yv[1];
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------
// Backward: dx, and float32 partial sums of dU and db per token range
// ---------------------------------------------------------------------------------
template <typename ET, int W, int KS, int DC>
__global__ __launch_bounds__(kBlockThreads) void k_lowrank_bwd(const LowRankParams p) {
  using RT = typename Raw<ET>::type;
  using R_ = Raw<ET>;
  constexpr int JC = DC * W;
  constexpr int MT = JC / 16;
  constexpr int MTW = (MT + 3) / 4;
  constexpr int RP = 32 * KS;
  constexpr int ZP = RP + 8;
  constexpr int JP = JC + 4;
  constexpr int TP = TT + 4;               // pitch of token-minor (transposed) tiles
  constexpr int NT = (RP / 16) * (JC / 16);  // dU tiles of the workgroup
  constexpr int NTW = NT / 4;
  static_assert(NT % 4 == 0, "dU tiles must split over 4 waves");
  constexpr int CPT = DC / 32;                        // channels per thread in the elementwise phase
  constexpr int TPT = TT * DC / (kBlockThreads * CPT);  // ... and tokens per thread
  static_assert(TPT * kBlockThreads * CPT == TT * DC, "elementwise phase must cover the tile");

  __shared__ __align__(16) RT zl[2][TT * ZP];
  __shared__ __align__(16) RT zT[2][RP * TP];
  __shared__ __align__(16) float wl[2][TT * JP];
  __shared__ float dyl[2][TT * DC];
  __shared__ float xl[RING * DC];
  __shared__ __align__(16) RT gT[JC * TP];

  const LrBlock blk = lr_block(p);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int q = lane >> 4;
  const int wv = tid >> 6;
  const int c_base = blk.cs * DC;
  const int j_base = c_base * W;
  const int t_first = blk.tr * p.Ltok;
  const int t_end = min(p.T, t_first + p.Ltok);
  const int range = blk.b * p.nTr + blk.tr;
  const ET* x = static_cast<const ET*>(p.x) + blk.b * p.xs0;
  const ET* z = static_cast<const ET*>(p.z) + blk.b * p.zs0;
  const ET* dy = static_cast<const ET*>(p.dy) + blk.b * p.dys0;
  ET* dx = static_cast<ET*>(p.out) + blk.b * p.os0;

  GenFrags<ET, KS, MTW> gf;
  gf.load(p, j_base, wv, MT);

  f32x4_t dU[NTW];
#pragma unroll
  for (int i = 0; i < NTW; ++i) dU[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // elementwise-phase ownership: channels cp*CPT .. +CPT-1, tokens tg*TPT .. +TPT-1
  const int cp = tid % (DC / CPT);
  const int tg = tid / (DC / CPT);
  float dbacc[CPT][W];
#pragma unroll
  for (int v = 0; v < CPT; ++v)
#pragma unroll
    for (int k = 0; k < W; ++k) dbacc[v][k] = 0.f;

  const bool range_ok = t_first < p.T;
  if (range_ok) {
    for (int idx = tid; idx < HALO * DC; idx += kBlockThreads) {
      const int t = t_first - HALO + idx / DC;
      const int c = idx % DC;
      float v = 0.f;
      if (t >= 0 && c_base + c < p.D) v = R_::to_float(R_::from_mem(x, int64_t(t) * p.xs1 + c_base + c));
      xl[ring_slot(t, t_first) * DC + c] = v;
    }
  }
  const int ntiles = range_ok ? (t_end - t_first + TT - 1) / TT : 0;
  for (int i = 0; i <= ntiles && range_ok; ++i) {
    const int cur = i & 1;
    const int prv = cur ^ 1;
    const int t_lead = t_first + TT * i;  // tile whose filters are regenerated
    const int t_work = t_lead - TT;       // tile whose dx, g, dU, db are produced
    // stage z and dy of the lead tile (rows past T read as 0), x of the work tile
    for (int idx = tid; idx < TT * RP; idx += kBlockThreads) {
      const int n = idx / RP;
      const int r = idx % RP;
      const int t = t_lead + n;
      const RT v = (t < p.T && r < p.R) ? R_::from_mem(z, int64_t(t) * p.zs1 + r) : R_::zero();
      zl[cur][n * ZP + r] = v;
      zT[cur][r * TP + n] = v;
    }
    for (int idx = tid; idx < TT * DC; idx += kBlockThreads) {
      const int n = idx / DC;
      const int c = idx % DC;
      const int t = t_lead + n;
      float v = 0.f;
      if (t < p.T && c_base + c < p.D) v = R_::to_float(R_::from_mem(dy, int64_t(t) * p.dys1 + c_base + c));
      dyl[cur][n * DC + c] = v;
      if (i > 0) {
        const int tw = t_work + n;
        float xv = 0.f;
        if (tw < t_end && c_base + c < p.D) xv = R_::to_float(R_::from_mem(x, int64_t(tw) * p.xs1 + c_base + c));
        xl[ring_slot(tw, t_first) * DC + c] = xv;
      }
    }
    __syncthreads();
#pragma unroll
    for (int ii = 0; ii < MTW; ++ii) {
      const int mt = wv + 4 * ii;
      if (mt < MT) {
        const f32x4_t acc = gen_tile<ET, KS, ZP>(gf.a[ii], gf.binit[ii], zl[cur]);
        *reinterpret_cast<f32x4_t*>(&wl[cur][(lane & 15) * JP + mt * 16 + 4 * q]) = acc;
      }
    }
    __syncthreads();
    if (i == 0) continue;
    // elementwise phase on the work tile
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int n = tg * TPT + u;
      const int s = t_work + n;
#pragma unroll
      for (int v = 0; v < CPT; ++v) {
        const int c = cp * CPT + v;
        const bool ok = s < t_end && c_base + c < p.D;
        float g[W];
        if (ok) {
          const float dys = dyl[prv][n * DC + c];
          float acc = dys;
#pragma unroll
          for (int k = 0; k < W; ++k) {
            const int nk = n + k;
            const float wk = nk < TT ? wl[prv][nk * JP + c * W + k] : wl[cur][(nk - TT) * JP + c * W + k];
            const float dk = nk < TT ? dyl[prv][nk * DC + c] : dyl[cur][(nk - TT) * DC + c];
            acc = fmaf(wk, dk, acc);
            g[k] = dys * xl[ring_slot(s - k, t_first) * DC + c];
          }
          const int64_t o = int64_t(s) * p.os1 + c_base + c;
          if constexpr (sizeof(ET) == 2) {
            reinterpret_cast<uint16_t*>(dx)[o] = to_bf16_bits(acc);
          } else {
            dx[o] = acc;
          }
#pragma unroll
          for (int k = 0; k < W; ++k) dbacc[v][k] += g[k];
        } else {
#pragma unroll
          for (int k = 0; k < W; ++k) g[k] = 0.f;
        }
#pragma unroll
        for (int k = 0; k < W; ++k) gT[(c * W + k) * TP + n] = R_::from_float(g[k]);
      }
    }
    __syncthreads();
    // dU += z^T g over the 16 tokens of the work tile
#pragma unroll
    for (int ti = 0; ti < NTW; ++ti) {
      const int id = wv + 4 * ti;
      const int rt = id / (JC / 16);
      const int jt = id % (JC / 16);
      typename Mfma<ET>::F16k afr, bfr;
      const int r = rt * 16 + (lane & 15);
      const int j = jt * 16 + (lane & 15);
      if constexpr (sizeof(ET) == 2) {
        afr.v = *reinterpret_cast<const u16x4_t*>(&zT[prv][r * TP + 4 * q]);
        bfr.v = *reinterpret_cast<const u16x4_t*>(&gT[j * TP + 4 * q]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          afr.v[e] = zT[prv][r * TP + Mfma<ET>::k16(q, e)];
          bfr.v[e] = gT[j * TP + Mfma<ET>::k16(q, e)];
        }
      }
      dU[ti] = Mfma<ET>::mma16(afr, bfr, dU[ti]);
    }
    __syncthreads();
  }

  // db partial: sum the per-thread sums over the threads that share a channel
  float* red = &wl[0][0];  // reused: (256 / (DC / CPT)) rows of JC floats
#pragma unroll
  for (int v = 0; v < CPT; ++v)
#pragma unroll
    for (int k = 0; k < W; ++k) red[tg * JC + (cp * CPT + v) * W + k] = dbacc[v][k];
  __syncthreads();
  constexpr int NTG = kBlockThreads / (DC / CPT);
  if (p.part_db != nullptr) {
    for (int j = tid; j < JC; j += kBlockThreads) {
      float s = 0.f;
      for (int r = 0; r < NTG; ++r) s += red[r * JC + j];
      if (j_base + j < p.J) p.part_db[int64_t(range) * p.J + j_base + j] = s;
    }
  }
  // dU partial: lane holds rows rt*16 + 4q + ii of column jt*16 + lane%16
#pragma unroll
  for (int ti = 0; ti < NTW; ++ti) {
    const int id = wv + 4 * ti;
    const int rt = id / (JC / 16);
    const int jt = id % (JC / 16);
    const int j = j_base + jt * 16 + (lane & 15);
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int r = rt * 16 + 4 * q + ii;
      if (r < p.R && j < p.J) p.part_dU[(int64_t(range) * p.R + r) * p.J + j] = dU[ti][ii];
    }
  }
}

// ---------------------------------------------------------------------------------
// dz = g U^T, g recomputed from x and dy; one workgroup per 64 tokens of a sequence.
// ---------------------------------------------------------------------------------
template <typename ET, int W, int KS>
__global__ __launch_bounds__(kBlockThreads) void k_lowrank_dz(const LowRankParams p) {
  using RT = typename Raw<ET>::type;
  using R_ = Raw<ET>;
  constexpr int RP = 32 * KS;
  constexpr int DCZ = (KS * sizeof(ET) <= 4) ? 64 : (KS * sizeof(ET) <= 8) ? 32 : 16;
  constexpr int JCZ = DCZ * W;
  constexpr int JK = (JCZ + 31) / 32 * 32;  // K extent padded to whole MFMA steps
  constexpr int UP = JK + 8;
  constexpr int TB = 64;
  __shared__ float xl[(TB + HALO) * DCZ];
  __shared__ float dyl[TB * DCZ];
  __shared__ __align__(16) RT Ul[RP * UP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int q = lane >> 4;
  const int wv = tid >> 6;
  const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int nblk = (p.T + TB - 1) / TB;
  const int b = lb / nblk;
  const int t0 = (lb % nblk) * TB;
  const ET* x = static_cast<const ET*>(p.x) + b * p.xs0;
  const ET* dy = static_cast<const ET*>(p.dy) + b * p.dys0;
  const ET* U = static_cast<const ET*>(p.U);

  f32x4_t acc[RP / 16];
#pragma unroll
  for (int i = 0; i < RP / 16; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int n = lane & 15;     // A row: token within the wave's 16
  const int nw = wv * 16 + n;  // token within the block

  for (int c0 = 0; c0 < p.D; c0 += DCZ) {
    for (int idx = tid; idx < (TB + HALO) * DCZ; idx += kBlockThreads) {
      const int rr = idx / DCZ;
      const int c = idx % DCZ;
      const int t = t0 - HALO + rr;
      float v = 0.f;
      if (t >= 0 && t < p.T && c0 + c < p.D) v = R_::to_float(R_::from_mem(x, int64_t(t) * p.xs1 + c0 + c));
      xl[idx] = v;
    }
    for (int idx = tid; idx < TB * DCZ; idx += kBlockThreads) {
      const int rr = idx / DCZ;
      const int c = idx % DCZ;
      const int t = t0 + rr;
      float v = 0.f;
      if (t < p.T && c0 + c < p.D) v = R_::to_float(R_::from_mem(dy, int64_t(t) * p.dys1 + c0 + c));
      dyl[idx] = v;
    }
    for (int idx = tid; idx < RP * JK; idx += kBlockThreads) {
      const int r = idx / JK;
      const int jl = idx % JK;
      const int j = c0 * W + jl;
      Ul[r * UP + jl] = (r < p.R && jl < JCZ && j < p.J) ? R_::from_mem(U, int64_t(r) * p.ldu + j) : R_::zero();
    }
    __syncthreads();
#pragma unroll
    for (int j0 = 0; j0 < JK; j0 += 32) {
      typename Mfma<ET>::F32k afr;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int jl = j0 + Mfma<ET>::k32(q, e);
        const int c = jl / W;
        const int k = jl % W;
        float g = 0.f;
        if (jl < JCZ) g = dyl[nw * DCZ + c] * xl[(nw + HALO - k) * DCZ + c];
        afr.v[e] = R_::from_float(g);
      }
#pragma unroll
      for (int rt = 0; rt < RP / 16; ++rt) {
        typename Mfma<ET>::F32k bfr;
        const int r = rt * 16 + (lane & 15);
        if constexpr (sizeof(ET) == 2) {
          bfr.v = *reinterpret_cast<const u16x8_t*>(&Ul[r * UP + j0 + 8 * q]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) bfr.v[e] = Ul[r * UP + j0 + Mfma<ET>::k32(q, e)];
        }
        // dz^T: rows = r, so use U as A and g as B: C[r][n] = sum_j U[r][j] g[n][j]
        acc[rt] = Mfma<ET>::mma32(bfr, afr, acc[rt]);
      }
    }
    __syncthreads();
  }
  // lane holds dz[token n = lane % 16][r = rt*16 + 4q + ii]
  ET* dz = static_cast<ET*>(p.dz) + b * p.dzs0;
  const int t = t0 + nw;
  if (t < p.T) {
#pragma unroll
    for (int rt = 0; rt < RP / 16; ++rt)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int r = rt * 16 + 4 * q + ii;
        if (r < p.R) {
          const int64_t o = int64_t(t) * p.dzs1 + r;
          if constexpr (sizeof(ET) == 2) {
            reinterpret_cast<uint16_t*>(dz)[o] = to_bf16_bits(acc[rt][ii]);
          } else {
            dz[o] = acc[rt][ii];
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
  constexpr int DC = (KS * W <= 8) ? 64 : 32;
  hipLaunchKernelGGL((k_lowrank_bwd<ET, W, KS, DC>), dim3(unsigned(pl.blocks)), dim3(kBlockThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t zblocks = int64_t(p.B) * ((p.T + 63) / 64);
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
  const int DC = (!bwd || ks * W <= 8) ? 64 : 32;
  pl.nCs = int((D + DC - 1) / DC);
  // about 2048 workgroups (8 per CU), tiles of 16 tokens, ranges in whole tiles
  int64_t per_seq = (2048 + B * pl.nCs - 1) / (B * pl.nCs);
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
