// The dynamic short convolution in the epilogue of the producing projection (gfx950):
//   X = A W_p^T  (never written to memory),  y = X + sum_{k<W} w_k(t) X_{t-k}
// with per-token filters read from memory, or low-rank filters w = z U + b made on the
// matrix cores in the same epilogue.
//
// From "Dynamic Short Convolutions Improve Transformers" (reading note): section
// "Parameterization" (the convolution acts on the outputs of the QKV projection, eq. 2 and
// eq. 3, and the low-rank generator) and the closing analysis of the end-to-end throughput
// section (fusing the dynamic convolution into the matmul epilogue removes the projection
// output's write and read).
//
// Tile. A workgroup of 8 waves (4 along the rows x 2 along the columns, 64 x 64 each)
// computes 256 consecutive token rows x 128 columns of X. Rows are the flattened tokens
// m = b T + t; the first 16 rows of a tile are the previous tile's last ones, computed
// again only as the causal halo of the tile's 240 output rows (W - 1 <= 4 rows are read).
// A tile may straddle two sequences: tap k of token t is present only when t >= k.
//
// Main loop. K advances 64 at a time through a ring of 3 LDS stages (A: 256 rows x 128 B,
// W_p: 128 rows x 128 B), filled two steps ahead by LDS DMA (global_load_lds_dwordx4, 16
// bytes per lane). A row's eight 16-byte chunks sit at chunk ^ (row & 7), so the 16 lanes
// of a fragment read (16 rows, one chunk) touch distinct banks. Each wave runs 16
// v_mfma_f32_16x16x32 per 32 of K; lane (n, q) then holds X rows 4q .. 4q+3 of column n
// of each 16 x 16 tile.
//
// Epilogue. The rows before a lane's rows are the previous lane group's (ds_bpermute by 16
// lanes), the previous row tile's, or, for a wave's first rows, the previous wave's last
// rows (a small LDS exchange). Per-token filters are read from memory per (row, column);
// low-rank filters come from W MFMA chains per 16 x 16 tile with z rows as A, a copy of
// the tile's columns of U in LDS as B (one row of R ranks per (tap, column), so a lane's
// 8 ranks are one 16-byte read) and the bias as the initial accumulator: they land in the
// same lane layout as X. y is rounded to the storage type and stored.
#include <type_traits>

#include "dynconv_common.hpp"
#include "dynconv_gemm_internal.hpp"

namespace dynconv {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
using lds_void = __attribute__((address_space(3))) void;

constexpr int GBM = kGemmRows, GHALO = kGemmHalo, GBMO = kGemmOutRows, GBN = kGemmCols, GKT = kGemmK;
constexpr int GNS = 3;                       // LDS stages
constexpr int GNT = 512;                     // threads
constexpr int AST = GBM * GKT * 2;           // bytes of a stage's A rows (32 KiB)
constexpr int BST = GBN * GKT * 2;           // bytes of a stage's W_p rows (16 KiB)
constexpr int STAGE = AST + BST;
constexpr int AI = AST / 16 / GNT;           // A transfers per thread and stage
constexpr int BI = BST / 16 / GNT;           // W_p transfers per thread and stage
constexpr int XCH = 6 * 4 * 4 * 16 * 4;      // halo exchange: 6 writer waves x 4 tiles x 4 rows x 16 lanes

// LDS copy of U for the low-rank epilogue: [tap][column][rank], a (tap, column) row of
// 32 KS ranks padded by 8 (16 bytes), so the 16 lanes of a read hit distinct banks.
constexpr int ut_pitch(int KS) { return 32 * KS + 8; }
constexpr int ut_bytes(int W, int KS) { return W * GBN * ut_pitch(KS) * 2; }
constexpr int smem_bytes(int EPI, int W, int KS) {
  const int main_loop = GNS * STAGE;
  const int epi = (EPI == 2 ? ut_bytes(W, KS) : 0) + XCH;
  return main_loop > epi ? main_loop : epi;
}
constexpr bool lowrank_fits(int W, int KS) { return ut_bytes(W, KS) + XCH <= GNS * STAGE; }

__device__ __forceinline__ void dma16(const void* g, unsigned char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)(lds_wave_base), 16, 0, 0);
}

// Waits until at most N of this wave's vector memory operations are outstanding and its
// LDS operations are done, then joins the workgroup barrier.
template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  asm volatile("s_barrier" ::: "memory");
}

template <typename ET>
__device__ __forceinline__ f32x4_t mma32(const u16x8_t& a, const u16x8_t& b, f32x4_t c) {
  if constexpr (std::is_same<ET, bf16_t>::value) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0,
                                                  0, 0);
  }
}

// Value of lane (lane - 16) mod 64.
__device__ __forceinline__ float from_lane_minus16(float v, int addr) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(v)));
}

// EPI 1: filters from memory (WVEC: the 4 taps of a (token, group) as one 8-byte load);
// EPI 2: low-rank filters, R <= 32 KS.
template <typename ET, int W, int EPI, int KS, bool WVEC>
__global__ __launch_bounds__(GNT) void k_gemm_conv(const GemmParams p) {
  static_assert(W >= 1 && W <= 5, "the halo is the previous lane group's 4 rows");
  static_assert(!WVEC || W == 4, "vector taps");
  constexpr int SMEM = smem_bytes(EPI, W, KS);
  static_assert(SMEM <= 160 * 1024, "LDS");
  __shared__ __align__(16) unsigned char smem[SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int q = lane >> 4;
  const int l16 = lane & 15;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv & 3;   // 64-row slice of the tile
  const int wn = wv >> 2;  // 64-column half of the tile

  // Tile order: consecutive logical ids on one XCD; groups of 8 row tiles are walked
  // column tile by column tile, so the workgroups running together share A and W_p rows
  // in that XCD's L2.
  const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const uint32_t per_group = 8u * uint32_t(p.nTn);
  const int grp = int(lb / per_group);
  const int rem = int(lb % per_group);
  const int rows_in_grp = min(8, p.nTm - 8 * grp);
  const int tm = 8 * grp + rem % rows_in_grp;
  const int tn = rem / rows_in_grp;
  const int m0 = tm * GBMO - GHALO;  // first computed row (negative for the first tile)
  const int n0 = tn * GBN;
  const int nk = p.K / GKT;

  // ---- LDS DMA sources: transfer i of wave wv fills 1 KiB of a stage (slot wv + 8 i);
  // its lane's 16-byte chunk is chunk (slot position ^ row & 7) of its row ----
  const char* ag[AI];
  const char* bg[BI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int pidx = (wv + 8 * i) * 64 + lane;
    const int row = pidx >> 3, c = (pidx & 7) ^ (row & 7);
    const int m = min(max(m0 + row, 0), p.M - 1);  // rows outside 0 .. M-1 are never stored
    const int b = m / p.T, t = m - b * p.T;
    ag[i] = reinterpret_cast<const char*>(p.A) + (int64_t(b) * p.as0 + int64_t(t) * p.as1 + 8 * c) * 2;
  }
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int pidx = (wv + 8 * i) * 64 + lane;
    const int row = pidx >> 3, c = (pidx & 7) ^ (row & 7);
    bg[i] = reinterpret_cast<const char*>(p.Wp) + (int64_t(n0 + row) * p.ldw + 8 * c) * 2;
  }
  auto issue = [&](int s) {
    unsigned char* st = smem + (s % GNS) * STAGE;
    const int64_t ko = int64_t(s) * GKT * 2;
#pragma unroll
    for (int i = 0; i < AI; ++i) dma16(ag[i] + ko, st + (wv + 8 * i) * 1024);
#pragma unroll
    for (int i = 0; i < BI; ++i) dma16(bg[i] + ko, st + AST + (wv + 8 * i) * 1024);
  };

  // ---- main loop ----
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  issue(0);
  if (nk > 1) issue(1);
  int aoff[4], boff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) aoff[i] = (64 * wm + 16 * i + l16) * 128;
#pragma unroll
  for (int j = 0; j < 4; ++j) boff[j] = AST + (64 * wn + 16 * j + l16) * 128;
  const int pos[2] = {(q ^ (l16 & 7)) * 16, ((4 + q) ^ (l16 & 7)) * 16};
  for (int s = 0; s < nk; ++s) {
    if (s + 1 < nk) {
      vm_wait_barrier<AI + BI>();
    } else {
      vm_wait_barrier<0>();
    }
    if (s + 2 < nk) issue(s + 2);
    const unsigned char* st = smem + (s % GNS) * STAGE;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u16x8_t a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const u16x8_t*>(st + aoff[i] + pos[kk]);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const u16x8_t*>(st + boff[j] + pos[kk]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mma32<ET>(a[i], b[j], acc[i][j]);
    }
  }
  __syncthreads();  // every wave is done with the stages: the epilogue reuses the LDS

  // ---- halo exchange: a wave's last 4 rows go to the next wave along the rows ----
  float* xch = reinterpret_cast<float*>(smem + (EPI == 2 ? ut_bytes(W, KS) : 0));
  if (wm < 3 && q == 3) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) xch[(((wm * 2 + wn) * 4 + j) * 4 + e) * 16 + l16] = acc[3][j][e];
  }

  const int G0 = n0 / p.H;  // first filter group of the tile (H divides 128)
  const int hsh = __builtin_ctz(unsigned(p.H));
  // ---- low-rank: the tile's columns of U in LDS, [tap][column][rank], ranks >= R zero ----
  if constexpr (EPI == 2) {
    constexpr int UP = ut_pitch(KS);
    uint16_t* ut = reinterpret_cast<uint16_t*>(smem);
    const int nG = GBN >> hsh;
    const int ncol = nG * W;  // U columns of the tile: groups G0 .. G0 + nG - 1, all taps
    const int total = 32 * KS * ncol;
    const uint16_t* Ug = static_cast<const uint16_t*>(p.U) + int64_t(G0) * W;
    for (int idx0 = tid; idx0 < total; idx0 += 8 * GNT) {
      uint16_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int idx = idx0 + u * GNT;
        const int r = idx / ncol, jj = idx - r * ncol;
        v[u] = (idx < total && r < p.R) ? Ug[int64_t(r) * p.ldu + jj] : uint16_t(0);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int idx = idx0 + u * GNT;
        if (idx < total) {
          const int r = idx / ncol, jj = idx - r * ncol;
          const int gl = jj / W, k = jj - gl * W;
          for (int h = 0; h < p.H; ++h) ut[(k * GBN + (gl << hsh) + h) * UP + r] = v[u];
        }
      }
    }
  }
  __syncthreads();

  // (b, t) of the lane's output rows of row tile i, element e: row 64 wm + 16 i + 4 q + e
  const int bp_addr = ((lane - 16) & 63) * 4;
  // the rows before the lane's first row, per column tile: 4 values (rows 4q - 4 .. 4q - 1)
  float prv[4][4];
  float rprev[4][4];  // the previous row tile's values passed from lane group q - 1 (mod 4)
  if (wm > 0 && q == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) rprev[j][e] = xch[((((wm - 1) * 2 + wn) * 4 + j) * 4 + e) * 16 + l16];
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) rprev[j][e] = 0.f;
  }

  ET* yb = static_cast<ET*>(p.y);
  const int colbase = n0 + 64 * wn + l16;  // + 16 j
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // rows of this lane in row tile i
    int tok[4];
    int64_t yrow[4], frow[4];
    bool out[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 64 * wm + 16 * i + 4 * q + e;
      const int m = m0 + r;
      const int mc = min(max(m, 0), p.M - 1);
      const int b = mc / p.T, t = mc - b * p.T;
      tok[e] = t;
      out[e] = r >= GHALO && m < p.M;
      yrow[e] = int64_t(b) * p.ys0 + int64_t(t) * p.ys1;
      frow[e] = EPI == 1 ? int64_t(b) * p.ws0 + int64_t(t) * p.ws1 : int64_t(b) * p.zs0 + int64_t(t) * p.zs1;
    }
    // previous rows: lane group q - 1 of this tile, or (q == 0) the previous tile's last
    // group / the previous wave's last rows
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float recv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) recv[e] = e > 4 - W ? from_lane_minus16(acc[i][j][e], bp_addr) : 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        prv[j][e] = q == 0 ? rprev[j][e] : recv[e];
        rprev[j][e] = recv[e];
      }
    }
    // filters of row 4q + e, column 16 j + l16, tap k: wk[j][k][e] (EPI 1: loaded for every
    // column tile before the first is used; EPI 2: formed per column tile just before use)
    float wk[EPI == 1 ? 4 : 1][W][4];
    if constexpr (EPI == 1) {
      const ET* wb = static_cast<const ET*>(p.w);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t gcol = int64_t((colbase + 16 * j) >> hsh) * W;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const ET* src = wb + frow[e] + gcol;
          if constexpr (WVEC) {
            const u32x2 v = *reinterpret_cast<const u32x2*>(src);
            wk[j][0][e] = Cvt<ET>::lo(v[0]);
            wk[j][1][e] = Cvt<ET>::hi(v[0]);
            wk[j][2][e] = Cvt<ET>::lo(v[1]);
            wk[j][3][e] = Cvt<ET>::hi(v[1]);
          } else {
#pragma unroll
            for (int k = 0; k < W; ++k) wk[j][k][e] = Cvt<ET>::of_bits(reinterpret_cast<const uint16_t*>(src)[k]);
          }
        }
      }
    }
    // EPI 2, A operand: z rows of this row tile (row l16), ranks 32 ks + 8 q .. + 7 (zero >= R)
    u16x8_t za[EPI == 2 ? KS : 1];
    if constexpr (EPI == 2) {
      const int rz = 64 * wm + 16 * i + l16;
      const int mz = min(max(m0 + rz, 0), p.M - 1);
      const int bz = mz / p.T, tz = mz - bz * p.T;
      const uint16_t* zrow = static_cast<const uint16_t*>(p.z) + int64_t(bz) * p.zs0 + int64_t(tz) * p.zs1;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 32 * ks + 8 * q + e;
          za[ks][e] = r < p.R ? zrow[r] : uint16_t(0);
        }
    }
    // y = X + sum_k w_k X_{t-k}, rounded and stored
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = colbase + 16 * j;
      float(&f)[W][4] = wk[EPI == 1 ? j : 0];
      if constexpr (EPI == 2) {
        constexpr int UP = ut_pitch(KS);
        const uint16_t* ut = reinterpret_cast<const uint16_t*>(smem);
        const uint16_t* bsrc = static_cast<const uint16_t*>(p.bias);
        const int cl = 64 * wn + 16 * j + l16;  // column of the tile
        const int64_t gcol = int64_t((n0 + cl) >> hsh) * W;
#pragma unroll
        for (int k = 0; k < W; ++k) {
          const float b0 = bsrc != nullptr ? Cvt<ET>::of_bits(bsrc[gcol + k]) : 0.f;
          f32x4_t c = {b0, b0, b0, b0};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const u16x8_t ub = *reinterpret_cast<const u16x8_t*>(ut + (k * GBN + cl) * UP + 32 * ks + 8 * q);
            c = mma32<ET>(za[ks], ub, c);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) f[k][e] = c[e];
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = acc[i][j][e];
        float y = fmaf(f[0][e], x0, x0);
#pragma unroll
        for (int k = 1; k < W; ++k) {
          const float xv = e >= k ? acc[i][j][e - k] : prv[j][4 + e - k];
          const float wkk = tok[e] >= k ? f[k][e] : 0.f;
          y = fmaf(wkk, xv, y);
        }
        if (out[e]) reinterpret_cast<uint16_t*>(yb)[yrow[e] + col] = Cvt<ET>::bits(y);
      }
    }
  }
}

template <typename ET, int W>
hipError_t conv_inst(const GemmParams& p, bool wvec, hipStream_t s) {
  const dim3 grid(unsigned(int64_t(p.nTm) * p.nTn));
  if constexpr (W == 4) {
    if (wvec) {
      hipLaunchKernelGGL((k_gemm_conv<ET, 4, 1, 1, true>), grid, dim3(GNT), 0, s, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((k_gemm_conv<ET, W, 1, 1, false>), grid, dim3(GNT), 0, s, p);
  return hipGetLastError();
}

template <typename ET, int W, int KS>
hipError_t lowrank_inst(const GemmParams& p, hipStream_t s) {
  if constexpr (lowrank_fits(W, KS)) {
    hipLaunchKernelGGL((k_gemm_conv<ET, W, 2, KS, false>), dim3(unsigned(int64_t(p.nTm) * p.nTn)), dim3(GNT), 0, s,
                       p);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

template <typename ET, int W>
hipError_t lowrank_ks(const GemmParams& p, hipStream_t s) {
  switch ((p.R + 31) / 32) {
    case 1: return lowrank_inst<ET, W, 1>(p, s);
    case 2: return lowrank_inst<ET, W, 2>(p, s);
    case 3: return lowrank_inst<ET, W, 3>(p, s);
    case 4: return lowrank_inst<ET, W, 4>(p, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename ET>
hipError_t conv_w(const GemmParams& p, int W, bool wvec, hipStream_t s) {
  switch (W) {
    case 1: return conv_inst<ET, 1>(p, wvec, s);
    case 2: return conv_inst<ET, 2>(p, wvec, s);
    case 3: return conv_inst<ET, 3>(p, wvec, s);
    case 4: return conv_inst<ET, 4>(p, wvec, s);
    case 5: return conv_inst<ET, 5>(p, wvec, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename ET>
hipError_t lowrank_w(const GemmParams& p, int W, hipStream_t s) {
  switch (W) {
    case 1: return lowrank_ks<ET, 1>(p, s);
    case 2: return lowrank_ks<ET, 2>(p, s);
    case 3: return lowrank_ks<ET, 3>(p, s);
    case 4: return lowrank_ks<ET, 4>(p, s);
    case 5: return lowrank_ks<ET, 5>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool gemm_lowrank_fits(int W, int R) {
  const int ks = (R + 31) / 32;
  return W >= 1 && W <= 5 && ks >= 1 && ks <= 4 && lowrank_fits(W, ks);
}

hipError_t launch_gemm_conv(const GemmParams& p, int W, bool wvec, dynconv_dtype dt, hipStream_t s) {
  return dt == DYNCONV_F16 ? conv_w<f16_t>(p, W, wvec, s) : conv_w<bf16_t>(p, W, wvec, s);
}

hipError_t launch_gemm_lowrank(const GemmParams& p, int W, dynconv_dtype dt, hipStream_t s) {
  return dt == DYNCONV_F16 ? lowrank_w<f16_t>(p, W, s) : lowrank_w<bf16_t>(p, W, s);
}

}  // namespace dynconv
