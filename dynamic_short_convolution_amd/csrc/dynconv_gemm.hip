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

constexpr int GBM = kGemmRows, GHALO = kGemmHalo, GBMO = kGemmOutRows, GBN = kGemmCols;
#ifndef GEMM_KT
#define GEMM_KT 64
#endif
constexpr int GKT = GEMM_KT;                 // K per pipeline stage (the host requires K % 64 == 0)
constexpr int GNS = GKT == 64 ? 3 : 6;        // LDS stages (144 KiB)
constexpr int GNT = 512;                     // threads
constexpr int AST = GBM * GKT * 2;           // bytes of a stage's A rows (32 KiB)
constexpr int BST = GBN * GKT * 2;           // bytes of a stage's W_p rows (16 KiB)
constexpr int STAGE = AST + BST;
constexpr int CPR = GKT / 8;                 // 16-byte chunks per stage row
// Chunk c of stage row r sits at chunk c ^ swz(r): the 16 rows of a fragment read then
// touch 16 distinct 16-byte bank groups (rows of 128 bytes: r & 7; of 64 bytes: r / 4).
__device__ __forceinline__ int swz(int r) { return GKT == 64 ? (r & 7) : ((r >> 2) & 3); }
constexpr int AI = AST / 16 / GNT;           // A transfers per thread and stage
constexpr int BI = BST / 16 / GNT;           // W_p transfers per thread and stage
constexpr int XCH = 6 * 4 * 4 * 16 * 4;      // halo exchange: 6 writer waves x 4 tiles x 4 rows x 16 lanes

// LDS copy of U for the low-rank epilogue: [tap][column][rank], a (tap, column) row of
// 32 KS ranks padded by 8 (16 bytes), so the 16 lanes of a fragment read (16 columns, 8
// ranks each) hit distinct banks; lanes staging consecutive rank pairs of one column
// write consecutive words.
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

// vm_wait_barrier<n> for a count known only at run time (n <= 2 * 5 * 3 here).
__device__ __forceinline__ void vm_wait_stage_ops(int n) {
  switch (n) {
    case 0: vm_wait_barrier<0>(); break;
    case 3: vm_wait_barrier<3>(); break;
    case 6: vm_wait_barrier<6>(); break;
    case 9: vm_wait_barrier<9>(); break;
    case 12: vm_wait_barrier<12>(); break;
    case 15: vm_wait_barrier<15>(); break;
    default: vm_wait_barrier<0>(); break;
  }
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
    const int row = pidx / CPR, c = (pidx % CPR) ^ swz(row);
    const int m = min(max(m0 + row, 0), p.M - 1);  // rows outside 0 .. M-1 are never stored
    const int b = m / p.T, t = m - b * p.T;
    ag[i] = reinterpret_cast<const char*>(p.A) + (int64_t(b) * p.as0 + int64_t(t) * p.as1 + 8 * c) * 2;
  }
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int pidx = (wv + 8 * i) * 64 + lane;
    const int row = pidx / CPR, c = (pidx % CPR) ^ swz(row);
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

  const int G0 = n0 / p.H;  // first filter group of the tile (H divides 128)
  const int hsh = __builtin_ctz(unsigned(p.H));
  // ---- low-rank: the tile's columns of U (groups G0 .. G0 + 128/H - 1, all taps; ranks
  // >= R zero), fetched as 16-byte pieces into registers before the main loop, so their
  // latency hides behind it; written to LDS after it ----
  // A piece is two consecutive ranks (2 rp, 2 rp + 1) x 8 consecutive U columns; piece v
  // is rank pair v % (16 KS), column chunk v / (16 KS), so the lanes of a wave take
  // consecutive rank pairs of one chunk.
  constexpr int UPAIRS = 16 * KS;
  constexpr int UVN = EPI == 2 ? (KS * W + 1) / 2 : 1;  // pieces per thread at H = 1
  // Up to 4 pieces (32 registers) are held through the main loop; larger ranks fetch theirs
  // after it, 4 at a time (the registers would otherwise spill).
  constexpr bool UPRE = EPI == 2 && UVN <= 4;
  u32x4 upre[UPRE ? UVN : 1][2];
  const int ucols = (GBN >> hsh) * W;  // U columns of the tile (a multiple of 8)
  const int nchunk = ucols >> 3;       // 16-byte column chunks per U row
  const uint16_t* Ug = static_cast<const uint16_t*>(p.U) + int64_t(G0) * W;
  auto fetch_piece = [&](int v, u32x4(&pc)[2]) {
    const int rp = v % UPAIRS, ch = v / UPAIRS;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 2 * rp + h;
      pc[h] = u32x4{0u, 0u, 0u, 0u};
      if (ch < nchunk && r < p.R) pc[h] = *reinterpret_cast<const u32x4*>(Ug + int64_t(r) * p.ldu + 8 * ch);
    }
  };
  if constexpr (UPRE) {
    if (p.uvec) {
#pragma unroll
      for (int u = 0; u < UVN; ++u) fetch_piece(tid + GNT * u, upre[u]);
    }
  }

  // ---- main loop ----
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  int aoff[4], boff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) aoff[i] = (64 * wm + 16 * i + l16) * (2 * GKT);
#pragma unroll
  for (int j = 0; j < 4; ++j) boff[j] = AST + (64 * wn + 16 * j + l16) * (2 * GKT);
  // chunk 4 kk + q of the fragment rows (row % 16 == l16, so swz(row) == swz(l16))
  const int pos[2] = {(q ^ swz(l16)) * 16, ((4 + q) ^ swz(l16)) * 16};
  // fragments of one 32-wide K sub-step: rows of A (row tile i) and of W_p (column tile j)
  auto load_frags = [&](int s, int kk, u16x8_t(&a)[4], u16x8_t(&b)[4]) {
    const unsigned char* st = smem + (s % GNS) * STAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const u16x8_t*>(st + aoff[i] + pos[kk]);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const u16x8_t*>(st + boff[j] + pos[kk]);
  };
  auto mma_all = [&](const u16x8_t(&a)[4], const u16x8_t(&b)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mma32<ET>(a[i], b[j], acc[i][j]);
  };
  // GNS stages, transfers GNS - 1 steps ahead: the wait at step s covers stage s, and
  // the stage that step s + GNS - 1 fills was last read at step s - 1 (every wave has
  // passed the barrier of step s, so those reads are complete).
#pragma unroll
  for (int i = 0; i < GNS - 1; ++i)
    if (i < nk) issue(i);
  for (int s = 0; s < nk; ++s) {
    // operations issued after stage s: those of the stages up to s + GNS - 2 that exist
    const int after = min(nk - 1 - s, GNS - 2);
    vm_wait_stage_ops(after * (AI + BI));
    if (s + GNS - 1 < nk) issue(s + GNS - 1);
#pragma unroll
    for (int kk = 0; kk < GKT / 32; ++kk) {
      u16x8_t a[4], b[4];
      load_frags(s, kk, a, b);
      mma_all(a, b);
    }
  }
  __syncthreads();  // every wave is done with the stages: the epilogue reuses the LDS

  // ---- epilogue ----
  // Rows of the lane in row tile i: r = 64 wm + 16 i + 4 q + e (e = 0..3), token m0 + r.
  struct Rows {
    int tok[4];       // t of the row (taps k > t are absent)
    bool out[4];      // an output row of this tile inside 0 .. M-1
    int64_t yrow[4];  // element offset of the row in y
    int64_t frow[4];  // element offset of the row in w (EPI 1)
  };
  auto rows_of = [&](int i) {
    Rows rw;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 64 * wm + 16 * i + 4 * q + e;
      const int m = m0 + r;
      const int mc = min(max(m, 0), p.M - 1);
      const int b = mc / p.T, t = mc - b * p.T;
      rw.tok[e] = t;
      rw.out[e] = r >= GHALO && m < p.M;
      rw.yrow[e] = int64_t(b) * p.ys0 + int64_t(t) * p.ys1;
      rw.frow[e] = int64_t(b) * p.ws0 + int64_t(t) * p.ws1;
    }
    return rw;
  };
  const int colbase = n0 + 64 * wn + l16;  // + 16 j
  // EPI 1: raw filter taps of a row tile, [j][e] (WVEC: 4 taps in one 8-byte load)
  constexpr int WR = EPI == 1 ? (WVEC ? 1 : W) : 1;
  struct WRaw {
    uint32_t v[4][4][WVEC ? 2 : WR];
  };
  auto load_w = [&](const Rows& rw, WRaw& raw) {
    if constexpr (EPI == 1) {
      const uint16_t* wb = static_cast<const uint16_t*>(p.w);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t gcol = int64_t((colbase + 16 * j) >> hsh) * W;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint16_t* src = wb + rw.frow[e] + gcol;
          if constexpr (WVEC) {
            const u32x2 v = *reinterpret_cast<const u32x2*>(src);
            raw.v[j][e][0] = v[0];
            raw.v[j][e][1] = v[1];
          } else {
#pragma unroll
            for (int k = 0; k < W; ++k) raw.v[j][e][k] = src[k];
          }
        }
      }
    }
  };
  Rows cur = rows_of(0);
  WRaw wcur;
  load_w(cur, wcur);  // in flight while the halo rows are exchanged

  // ---- halo exchange: a wave's last 4 rows go to the next wave along the rows ----
  float* xch = reinterpret_cast<float*>(smem + (EPI == 2 ? ut_bytes(W, KS) : 0));
  if (wm < 3 && q == 3) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) xch[(((wm * 2 + wn) * 4 + j) * 4 + e) * 16 + l16] = acc[3][j][e];
  }

  // ---- low-rank, A operands of every row tile: z row 64 wm + 16 i + l16, ranks
  // 32 ks + 8 q .. + 7 (zero >= R), all issued here so that one latency covers them ----
  u16x8_t za[EPI == 2 ? 4 : 1][EPI == 2 ? KS : 1];
  if constexpr (EPI == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int mz = min(max(m0 + 64 * wm + 16 * i + l16, 0), p.M - 1);
      const int bz = mz / p.T, tz = mz - bz * p.T;
      const uint16_t* zrow = static_cast<const uint16_t*>(p.z) + int64_t(bz) * p.zs0 + int64_t(tz) * p.zs1;
      if (p.zvec) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int r = 32 * ks + 8 * q;
          za[i][ks] = r < p.R ? *reinterpret_cast<const u16x8_t*>(zrow + r) : u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int r = 32 * ks + 8 * q + e;
            za[i][ks][e] = r < p.R ? zrow[r] : uint16_t(0);
          }
      }
    }
  }
  // ---- low-rank: the tile's columns of U in LDS, [tap][column][rank], ranks >= R zero ----
  if constexpr (EPI == 2) {
    constexpr int UP = ut_pitch(KS);
    uint16_t* ut = reinterpret_cast<uint16_t*>(smem);
    // piece v -> the (tap, column) rows of its 8 U columns, ranks 2 rp, 2 rp + 1 as one word
    auto put = [&](int v, const u32x4(&pc)[2]) {
      const int rp = v % UPAIRS, ch = v / UPAIRS;
      if (ch < nchunk) {
        const u16x8_t lo = __builtin_bit_cast(u16x8_t, pc[0]);
        const u16x8_t hi = __builtin_bit_cast(u16x8_t, pc[1]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int jj = 8 * ch + e;
          const int gl = jj / W, k = jj - gl * W;
          const uint32_t word = uint32_t(lo[e]) | (uint32_t(hi[e]) << 16);
          for (int h = 0; h < p.H; ++h)
            *reinterpret_cast<uint32_t*>(ut + (k * GBN + (gl << hsh) + h) * UP + 2 * rp) = word;
        }
      }
    };
    if (p.uvec) {
      if constexpr (UPRE) {
#pragma unroll
        for (int u = 0; u < UVN; ++u) put(tid + GNT * u, upre[u]);
      } else {
#pragma unroll
        for (int u0 = 0; u0 < UVN; u0 += 2) {
          u32x4 pc[2][2];
#pragma unroll
          for (int u = 0; u < 2; ++u)
            if (u0 + u < UVN) fetch_piece(tid + GNT * (u0 + u), pc[u]);
#pragma unroll
          for (int u = 0; u < 2; ++u)
            if (u0 + u < UVN) put(tid + GNT * (u0 + u), pc[u]);
        }
      }
    } else {
      // unaligned U: element loads here, 8 in flight per thread
      const int total = 32 * KS * ucols;
      for (int idx0 = tid; idx0 < total; idx0 += 8 * GNT) {
        uint16_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int idx = idx0 + u * GNT;
          const int r = idx / ucols, jj = idx - r * ucols;
          v[u] = (idx < total && r < p.R) ? Ug[int64_t(r) * p.ldu + jj] : uint16_t(0);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int idx = idx0 + u * GNT;
          if (idx < total) {
            const int r = idx / ucols, jj = idx - r * ucols;
            const int gl = jj / W, k = jj - gl * W;
            for (int h = 0; h < p.H; ++h) ut[(k * GBN + (gl << hsh) + h) * UP + r] = v[u];
          }
        }
      }
    }
  }
  __syncthreads();

  const int bp_addr = ((lane - 16) & 63) * 4;  // ds_bpermute from lane - 16 (mod 64)
  // rprev: the previous row tile's last 4 rows as passed from lane group q - 1 (mod 4);
  // before row tile 0 of waves 1..3, the previous wave's last rows
  float rprev[4][4];
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

  uint16_t* yb = static_cast<uint16_t*>(p.y);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // the next row tile's rows and filters, in flight during this one
    Rows nxt;
    WRaw wnxt;
    if (i + 1 < 4) {
      nxt = rows_of(i + 1);
      load_w(nxt, wnxt);
    }
    // rows before the lane's first row: lane group q - 1 of this tile, or (q == 0) the
    // previous tile's last group / the previous wave's last rows
    float prv[4][4];
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
    // y = X + sum_k w_k X_{t-k}, rounded and stored, one column tile at a time
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = colbase + 16 * j;
      float f[W][4];  // filters of tap k, row 4q + e
      if constexpr (EPI == 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (WVEC) {
            f[0][e] = Cvt<ET>::lo(wcur.v[j][e][0]);
            f[1][e] = Cvt<ET>::hi(wcur.v[j][e][0]);
            f[2][e] = Cvt<ET>::lo(wcur.v[j][e][1]);
            f[3][e] = Cvt<ET>::hi(wcur.v[j][e][1]);
          } else {
#pragma unroll
            for (int k = 0; k < W; ++k) f[k][e] = Cvt<ET>::of_bits(wcur.v[j][e][k]);
          }
        }
      } else {
        // low-rank: W matrix-core chains over the ranks, bias as the initial value
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
            // B operand: ranks 32 ks + 8 q .. + 7 of column 64 wn + 16 j + l16
            const u16x8_t ub = *reinterpret_cast<const u16x8_t*>(ut + (k * GBN + cl) * UP + 32 * ks + 8 * q);
            c = mma32<ET>(za[i][ks], ub, c);
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
          const float wkk = cur.tok[e] >= k ? f[k][e] : 0.f;
          y = fmaf(wkk, xv, y);
        }
        if (cur.out[e]) yb[cur.yrow[e] + col] = Cvt<ET>::bits(y);
      }
    }
    if (i + 1 < 4) {
      cur = nxt;
      wcur = wnxt;
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
