// Low-rank dynamic short convolution, bf16 fast path for gfx950: the filters w = z U + b
// are formed on the matrix cores and consumed in registers; they never reach HBM.
//
// From "Dynamic Short Convolutions Improve Transformers" (reading note): section
// "Parameterization" (low-rank generator D -> R -> W*D with a bias; eq. 2 and eq. 3) and
// section "Efficient training (Triton kernels)" (the fused kernel reads z and U, generates
// z U on-chip and applies the convolution at once).
//
// Forward, k_lowrank_fwd_fast. One workgroup (4 waves) owns 64 channels of one sequence
// over a range of tokens and walks it in steps of 64 tokens.
//  * Staging: the step's x rows (64 x 128 B) and z rows (64 x 2R B) are copied to LDS by
//    LDS DMA (global_load_lds_dwordx4) ahead of the step that uses them. x sits in a ring
//    of steps, so the W-1 rows before a step are the previous step's last rows. The
//    16-byte chunks of a row are rotated by (row / 4) to spread the reads over the banks.
//  * Filter generation: for token group j (0..3) the MFMA B operand column n is token
//    4n + j of the step, and A holds U^T with rows (channel, tap) ordered so that lane
//    (n, q = lane / 16) receives the W taps of channels 4q .. 4q+3 of the wave's 16
//    (one per 16-row tile mt). The bias enters as the accumulator's initial value.
//    A lane thus holds the filters of 4 consecutive tokens 4n .. 4n+3 for 4 channels.
//  * Convolution: the lane reads x rows 4n-3 .. 4n+3 of its 4 channels (8 bytes each),
//    converts each once, and forms y = x_t + sum_k w_k(t) x_{t-k} in float32.
//  * Stores: the step's y goes to an LDS tile and is written one step later by the same
//    waves as whole 128-byte rows (16 bytes per lane), through a buffer resource whose
//    extent is the sequence: rows at or past T (the last partial step) are dropped by the
//    hardware, so every wave issues the same number of memory operations and the vmcnt
//    waits are exact. (Writing y straight from the MFMA layout, 8 bytes per lane spread
//    over 16 rows, measured 82 us instead of 64 us.)
#include <type_traits>

#include "dynconv_common.hpp"
#include "dynconv_internal.hpp"
#include "dynconv_lowrank_internal.hpp"

namespace dynconv {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
using lds_void = __attribute__((address_space(3))) void;

constexpr int kStep = 64;    // tokens per pipeline step
constexpr uint32_t kBufWord3 = 0x00020000u;  // raw buffer resource, 32-bit elements

// Pipeline shape: waves per workgroup (16 channels each), x ring stages and how many
// steps ahead x is fetched, z stages and how many steps ahead z is fetched. Measured on
// MI355X at B8 T4096 D2048 W4 R64 (bf16): 4 waves, x and z one step ahead (56 KiB of
// LDS, two workgroups per CU) ran at 62.6 us; fetching 2-4 steps ahead, or 8 waves per
// workgroup, gave 61-68 us. The kernel is bound by latency inside the waves (two per
// SIMD), not by the distance of the fetches. Overridable at build time for a sweep.
#ifndef LRF_NWV
#define LRF_NWV 4
#endif
#ifndef LRF_XN
#define LRF_XN 3
#endif
#ifndef LRF_XD
#define LRF_XD 1
#endif
#ifndef LRF_ZN
#define LRF_ZN 2
#endif
#ifndef LRF_ZD
#define LRF_ZD 1
#endif

__device__ __forceinline__ void dma16(const void* g, unsigned char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)(lds_wave_base), 16, 0, 0);
}

// Waits until at most N of this wave's vector memory operations are outstanding (they
// complete in issue order) and its LDS operations are done, then joins the workgroup
// barrier.
template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  asm volatile("s_barrier" ::: "memory");
}

__device__ __forceinline__ f32x4_t mma32(const u16x8_t& a, const u16x8_t& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

template <int KS, int NWV_, int XN_, int XD_, int ZN_, int ZD_>
struct FwdFast {
  static constexpr int NWV = NWV_, XN = XN_, XD = XD_, ZN = ZN_, ZD = ZD_;
  static constexpr int NT = 64 * NWV;                // threads
  static constexpr int CPB = 16 * NWV;               // channels per workgroup
  static constexpr int XCPR = CPB / 8;               // 16-byte chunks of an x (or y) row
  static constexpr int XROW = CPB * 2;               // bytes of an x row
  static constexpr int XSTAGE = kStep * XROW;
  static constexpr int ZCPR = 4 * KS;                // 16-byte chunks of a z row (R = 32 KS)
  static constexpr int ZROW = 16 * ZCPR;
  static constexpr int ZSTAGE = kStep * ZROW;
  static constexpr int Z_OFF = XN * XSTAGE;
  static constexpr int Y_OFF = Z_OFF + ZN * ZSTAGE;
  static constexpr int BYTES = Y_OFF + 2 * XSTAGE;  // two y tiles
  static constexpr int XI = kStep * XCPR / 64 / NWV;  // x transfers per wave per step (2)
  static constexpr int ZI = kStep * ZCPR / 64 / NWV;  // z transfers per wave per step
  static constexpr int NS = kStep * XCPR / 64 / NWV;  // y stores per wave per step (2)
  static_assert((kStep * ZCPR) % (64 * NWV) == 0, "z transfers split evenly over the waves");
  static_assert(XD >= 1 && XD <= XN - 2 && ZD >= 1 && ZD <= ZN - 1 && ZD <= XD, "pipeline depths");
  static_assert((XCPR & (XCPR - 1)) == 0 && 16 % XCPR == 0, "x row rotation");

  // Issue order of one wave's vector memory operations: a prologue x(0), z(0), x(1),
  // z(1), ... (z only below ZD, x below XD); then step k issues x(k + XD), z(k + ZD) and,
  // from k = 1 on, the stores of step k - 1. Returns how many operations follow the later
  // of x(s) and z(s) when step s waits for them.
  static constexpr int step_ops(int k) { return XI + ZI + (k >= 1 ? NS : 0); }
  static constexpr int prologue_end_x(int i) {
    int pos = 0;
    for (int a = 0; a < i; ++a) pos += XI + (a < ZD ? ZI : 0);
    return pos + XI;
  }
  static constexpr int prologue_ops() { return prologue_end_x(XD - 1) + (XD - 1 < ZD ? ZI : 0); }
  static constexpr int steps_before(int k) {
    int pos = prologue_ops();
    for (int a = 0; a < k; ++a) pos += step_ops(a);
    return pos;
  }
  static constexpr int wait_after(int s) {
    const int end_x = s < XD ? prologue_end_x(s) : steps_before(s - XD) + XI;
    const int end_z = s < ZD ? prologue_end_x(s) + ZI : steps_before(s - ZD) + XI + ZI;
    const int last = end_x > end_z ? end_x : end_z;
    return steps_before(s) - last;
  }
  static constexpr int kSteady = XD + 1;  // from this step on the count no longer changes
};

template <class F, int S>
__device__ __forceinline__ void step_wait(int s) {
  if constexpr (S >= F::kSteady) {
    vm_wait_barrier<F::wait_after(F::kSteady)>();
  } else {
    if (s == S) {
      vm_wait_barrier<F::wait_after(S)>();
    } else {
      step_wait<F, S + 1>(s);
    }
  }
}

template <int W, int KS>
__global__ __launch_bounds__(64 * LRF_NWV) void k_lowrank_fwd_fast(const LowRankParams p) {
  using F = FwdFast<KS, LRF_NWV, LRF_XN, LRF_XD, LRF_ZN, LRF_ZD>;
  constexpr int NWV = F::NWV, XN = F::XN, XD = F::XD, ZN = F::ZN, ZD = F::ZD, CPB = F::CPB;
  constexpr int XCPR = F::XCPR, XROW = F::XROW, XSTAGE = F::XSTAGE;
  constexpr int ZCPR = F::ZCPR, ZROW = F::ZROW, ZSTAGE = F::ZSTAGE, Z_OFF = F::Z_OFF, Y_OFF = F::Y_OFF;
  constexpr int XI = F::XI, ZI = F::ZI;
  constexpr int HR = W - 1;       // rows before a token that its filter reaches
  constexpr int MLO = -HR;        // x rows 4n + m, m = MLO .. 3, feed the lane's 4 tokens
  constexpr int NM = 4 - MLO;
  __shared__ __align__(16) unsigned char smem[F::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int q = lane >> 4;
  const int n = lane & 15;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int cs = p.cs0 + int(lb % uint32_t(p.nCsL));
  lb /= uint32_t(p.nCsL);
  const int tr = int(lb % uint32_t(p.nTr));
  const int b = int(lb / uint32_t(p.nTr));
  const int c_base = cs * CPB;
  const int t_first = tr * p.Ltok;
  const int t_end = min(p.T, t_first + p.Ltok);
  const int nsteps = (t_end - t_first + kStep - 1) / kStep;
  const bf16_t* xb = static_cast<const bf16_t*>(p.x) + b * p.xs0 + c_base;
  const bf16_t* zb = static_cast<const bf16_t*>(p.z) + b * p.zs0;
  const int cw = c_base + 16 * wv;  // the wave's first channel

  // ---- LDS DMA of one step: rows t0 .. t0 + 63 (clamped to T - 1) ----
  // Transfer i of a wave fills 1 KiB of a stage (slot wv + NWV i); per lane the byte offset
  // of its 16-byte source chunk from the step's first row. The chunks of a row are rotated
  // by (row / 4) within the row.
  uint32_t xoff[XI], zoff[ZI];
  int xrl[XI], zrl[ZI];
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int idx = (wv + NWV * i) * 64 + lane;
    const int rl = idx / XCPR, pc = idx % XCPR;
    const int c = (pc - (rl >> 2)) & (XCPR - 1);
    xrl[i] = rl;
    xoff[i] = uint32_t(rl * int(p.xs1) + 8 * c) * 2u;
  }
#pragma unroll
  for (int i = 0; i < ZI; ++i) {
    const int idx = (wv + NWV * i) * 64 + lane;
    const int rl = idx / ZCPR, pc = idx % ZCPR;
    const int c = ((pc - (rl >> 2)) % ZCPR + ZCPR) % ZCPR;
    zrl[i] = rl;
    zoff[i] = uint32_t(rl * int(p.zs1) + 8 * c) * 2u;
  }
  const char* xbc = reinterpret_cast<const char*>(xb);
  const char* zbc = reinterpret_cast<const char*>(zb);
  auto issue_x = [&](int st, int t0) {
    unsigned char* xs = smem + st * XSTAGE;
    if (t0 + kStep <= p.T) {
      const char* xg = xbc + int64_t(t0) * p.xs1 * 2;
#pragma unroll
      for (int i = 0; i < XI; ++i) dma16(xg + xoff[i], xs + (wv + NWV * i) * 1024);
    } else {
      // rows past T - 1 (the last, partial step, or steps past the range) read row T - 1;
      // their results are never stored
#pragma unroll
      for (int i = 0; i < XI; ++i) {
        const int t = min(t0 + xrl[i], p.T - 1);
        dma16(xbc + (int64_t(t) - xrl[i]) * p.xs1 * 2 + xoff[i], xs + (wv + NWV * i) * 1024);
      }
    }
  };
  auto issue_z = [&](int st, int t0) {
    unsigned char* zs = smem + Z_OFF + st * ZSTAGE;
    if (t0 + kStep <= p.T) {
      const char* zg = zbc + int64_t(t0) * p.zs1 * 2;
#pragma unroll
      for (int i = 0; i < ZI; ++i) dma16(zg + zoff[i], zs + (wv + NWV * i) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < ZI; ++i) {
        const int t = min(t0 + zrl[i], p.T - 1);
        dma16(zbc + (int64_t(t) - zrl[i]) * p.zs1 * 2 + zoff[i], zs + (wv + NWV * i) * 1024);
      }
    }
  };

  // ---- A operands (U^T rows in the lane order above) and the bias, once ----
  // Loads are unconditional (a clamped tap, U standing in for a missing bias) and the
  // unused values are zeroed afterwards, so nothing waits on a branch here.
  u16x8_t afr[4][KS];
  f32x4_t binit[4];
  {
    const uint16_t* U = static_cast<const uint16_t*>(p.U);
    const bool has_bias = p.bias != nullptr;
    const uint16_t* bsrc = has_bias ? static_cast<const uint16_t*>(p.bias) : U;
    const uint32_t bmask = has_bias ? ~0u : 0u;
    const int tap = n & 3;
    const int ltap = tap < W ? tap : W - 1;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int ch = cw + 4 * (n >> 2) + mt;
      const int64_t col = int64_t(ch) * W + ltap;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint16_t v = U[int64_t(32 * ks + 8 * q + e) * p.ldu + col];
          afr[mt][ks][e] = tap < W ? v : uint16_t(0);
        }
      const int chq = cw + 4 * q + mt;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint16_t v = bsrc[(has_bias ? int64_t(chq) * W : 0) + (i < W ? i : W - 1)];
        binit[mt][i] = __uint_as_float((uint32_t(v) << 16) & (i < W ? bmask : 0u));
      }
    }
  }

  // ---- the W-1 rows before the range: the last rows of ring stage XN - 1 ----
  if constexpr (HR > 0) {
    unsigned char* hbase = smem + XN * XSTAGE - HR * XROW;
    if (t_first > 0) {
      if (wv == 0 && lane < HR * XCPR) {
        const int rl = kStep - HR + lane / XCPR, pc = lane % XCPR;
        const int c = (pc - (rl >> 2)) & (XCPR - 1);
        dma16(xbc + (int64_t(t_first - HR + lane / XCPR) * p.xs1 + 8 * c) * 2, hbase);
      }
    } else {
      for (int i = tid; i < HR * XROW / 4; i += F::NT) reinterpret_cast<uint32_t*>(hbase)[i] = 0u;
    }
  }
#pragma unroll
  for (int i = 0; i < XD; ++i) {
    issue_x(i, t_first + i * kStep);
    if (i < ZD) issue_z(i, t_first + i * kStep);
  }

  // ---- per-lane LDS offsets ----
  // x row 4n + m of ring stage u sits at u * XSTAGE + (4n + m) * XROW (rows before the
  // stage, m < 0, are the previous stage's last rows; from stage 0 they wrap to the ring's
  // end), chunk rotated by (row / 4): n - 1 for m < 0, n for m >= 0.
  const int xc = 2 * wv + (q >> 1);  // logical 16-byte chunk of the lane's 4 channels
  const int xlo = 4 * n * XROW + ((xc + n - 1) & (XCPR - 1)) * 16 + 8 * (q & 1);  // + m * XROW, m < 0
  const int xhi = 4 * n * XROW + ((xc + n) & (XCPR - 1)) * 16 + 8 * (q & 1);      // + m * XROW, m >= 0
  const int xwrap = n == 0 ? XN * XSTAGE : 0;
  int zr[KS];  // + j * ZROW for token group j
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) zr[ks] = 4 * n * ZROW + ((4 * ks + q + n) % ZCPR) * 16;
  const int ytw = xhi;  // y tile: the lane writes row 4n + j (+ j * XROW), same rotation as x

  // y: buffer resource spanning this sequence's rows 0 .. T-1 (stores past it are dropped)
  __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
      static_cast<bf16_t*>(p.out) + b * p.os0, 0, int((int64_t(p.T - 1) * p.os1 + p.D) * 2), kBufWord3);
  const int ystep = int(p.os1 * 2);
  // a step's y tile is stored by the same waves one step later, 16 bytes per lane, whole
  // rows: store i of wave wv covers tile slot wv + NWV i
  int ytr[F::NS], ygo[F::NS];
#pragma unroll
  for (int i = 0; i < F::NS; ++i) {
    const int idx = (wv + NWV * i) * 64 + lane;
    const int r = idx / XCPR, pc = idx % XCPR;
    const int c = (pc - (r >> 2)) & (XCPR - 1);
    ytr[i] = idx * 16;
    ygo[i] = int((r * p.os1 + c_base + 8 * c) * 2);
  }
  auto yflush = [&](int buf, int t0) {
    const unsigned char* yt = smem + Y_OFF + buf * XSTAGE;
#pragma unroll
    for (int i = 0; i < F::NS; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(yt + ytr[i]);
      __builtin_amdgcn_raw_buffer_store_b128(v, yr, ygo[i] + t0 * ystep, 0, 0);
    }
  };

  for (int s = 0; s < nsteps; ++s) {
    const int t0 = t_first + s * kStep;
    const int ux = s % XN, uz = s % ZN;
    step_wait<F, 0>(s);
    issue_x((s + XD) % XN, t0 + XD * kStep);
    issue_z((s + ZD) % ZN, t0 + ZD * kStep);
    if (s > 0) yflush((s - 1) & 1, t0 - kStep);
    // x rows 4n + MLO .. 4n + 3 of the lane's channels, as float32
    const unsigned char* xst = smem + ux * XSTAGE;
    const int lo = xlo + (ux == 0 ? xwrap : 0);
    float xv[NM][4];
#pragma unroll
    for (int mi = 0; mi < NM; ++mi) {
      const int m = MLO + mi;
      const u32x2 v = *reinterpret_cast<const u32x2*>(xst + (m < 0 ? lo : xhi) + m * XROW);
      xv[mi][0] = bf16_lo(v[0]);
      xv[mi][1] = bf16_hi(v[0]);
      xv[mi][2] = bf16_lo(v[1]);
      xv[mi][3] = bf16_hi(v[1]);
    }
    const unsigned char* zs = smem + Z_OFF + uz * ZSTAGE;
    unsigned char* yt = smem + Y_OFF + (s & 1) * XSTAGE + ytw;
    // filters of token group j (MFMA), issued one group ahead of the convolution
    auto gen = [&](int j, f32x4_t (&acc)[4]) {
      u16x8_t bfr[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) bfr[ks] = *reinterpret_cast<const u16x8_t*>(zs + zr[ks] + j * ZROW);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        acc[mt] = mma32(afr[mt][0], bfr[0], binit[mt]);
#pragma unroll
        for (int ks = 1; ks < KS; ++ks) acc[mt] = mma32(afr[mt][ks], bfr[ks], acc[mt]);
      }
    };
    f32x4_t acc[2][4];
    gen(0, acc[0]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j + 1 < 4) gen(j + 1, acc[(j + 1) & 1]);
      const f32x4_t(&a)[4] = acc[j & 1];
      float yv[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const float xt = xv[j - MLO][mt];
        float y = fmaf(a[mt][0], xt, xt);
#pragma unroll
        for (int k = 1; k < W; ++k) y = fmaf(a[mt][k], xv[j - k - MLO][mt], y);
        yv[mt] = y;
      }
      *reinterpret_cast<u32x2*>(yt + j * XROW) = u32x2{pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3])};
    }
  }
  __syncthreads();
  yflush((nsteps - 1) & 1, t_first + (nsteps - 1) * kStep);
  // the transfers still in flight land in stages nobody reads; drain them (and the last
  // stores) before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
}

template <int W, int KS>
hipError_t fwd_fast_inst(const LowRankParams& p, int64_t blocks, hipStream_t s) {
  hipLaunchKernelGGL((k_lowrank_fwd_fast<W, KS>), dim3(unsigned(blocks)), dim3(64 * LRF_NWV), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Backward dx, k_lowrank_bwd_dx_fast:
//   dx_s = dy_s + sum_k w_k(s + k) dy_{s+k}    (the adjoint of eq. 2 + eq. 3)
// Same workgroup shape, staging and filter generation as the forward, with dy in place
// of x (dx needs no x). Lane (n, q) holds the filters of tokens 4n .. 4n+3 of the step
// and forms P_k(t) = w_k(t) dy_t for them. A term P_k(t) belongs to dx_{t-k}: to the
// lane's own tokens when t - k >= 4n, else to the previous lane's tokens 4n-3 .. 4n-1
// (three "outgoing" sums, O_1..O_3). Each lane receives the O sums of lane n + 1 by a
// DPP rotate within its 16-lane row (row_ror:15). Lane 15 receives lane 0's sums, which
// complete its tokens 61 .. 63 of the previous step: lane 15 keeps those three partial
// sums from one step to the next and writes them then. A step's dx tile therefore holds
// tokens t0 - 3 .. t0 + 60; the step after the range (tail) only completes its first
// three rows, and the first step's first three rows belong to the previous range.
// dy rows at or past T are zeroed, so the tail contributes nothing past the sequence.
// ---------------------------------------------------------------------------------
template <int KS>
struct BwdDxFast {
  static constexpr int NWV = 4;
  static constexpr int CPB = 64;
  static constexpr int XCPR = 8, XROW = 128;
  static constexpr int XSTAGE = kStep * XROW;        // dy stage, dx tile
  static constexpr int ZCPR = 4 * KS;
  static constexpr int ZROW = 16 * ZCPR;
  static constexpr int ZSTAGE = kStep * ZROW;
  static constexpr int Z_OFF = 2 * XSTAGE;            // two dy stages
  static constexpr int T_OFF = Z_OFF + 2 * ZSTAGE;    // two z stages, then two dx tiles
  static constexpr int BYTES = T_OFF + 2 * XSTAGE;
  static constexpr int DI = 2, ZI = KS, ND = DI + ZI, NS = 2;
};

template <int W, int KS>
__global__ __launch_bounds__(256) void k_lowrank_bwd_dx_fast(const LowRankParams p) {
  using F = BwdDxFast<KS>;
  constexpr int XCPR = F::XCPR, XROW = F::XROW, XSTAGE = F::XSTAGE;
  constexpr int ZCPR = F::ZCPR, ZROW = F::ZROW, ZSTAGE = F::ZSTAGE, Z_OFF = F::Z_OFF, T_OFF = F::T_OFF;
  __shared__ __align__(16) unsigned char smem[F::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int q = lane >> 4;
  const int n = lane & 15;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int cs = p.cs0 + int(lb % uint32_t(p.nCsL));
  lb /= uint32_t(p.nCsL);
  const int tr = int(lb % uint32_t(p.nTr));
  const int b = int(lb / uint32_t(p.nTr));
  const int c_base = cs * F::CPB;
  const int t_first = tr * p.Ltok;
  const int t_end = min(p.T, t_first + p.Ltok);
  const int nsteps = (t_end - t_first + kStep - 1) / kStep;
  const char* dyc = reinterpret_cast<const char*>(static_cast<const bf16_t*>(p.dy) + b * p.dys0 + c_base);
  const char* zc = reinterpret_cast<const char*>(static_cast<const bf16_t*>(p.z) + b * p.zs0);
  const int cw = c_base + 16 * wv;

  // ---- LDS DMA of a step's dy and z rows (rows past T - 1 read row T - 1) ----
  uint32_t doff[F::DI], zoff[F::ZI];
  int drl[F::DI], zrl[F::ZI];
#pragma unroll
  for (int i = 0; i < F::DI; ++i) {
    const int idx = (wv + 4 * i) * 64 + lane;
    const int rl = idx / XCPR, pc = idx % XCPR;
    const int c = (pc - (rl >> 2)) & (XCPR - 1);
    drl[i] = rl;
    doff[i] = uint32_t(rl * int(p.dys1) + 8 * c) * 2u;
  }
#pragma unroll
  for (int i = 0; i < F::ZI; ++i) {
    const int idx = (wv + 4 * i) * 64 + lane;
    const int rl = idx / ZCPR, pc = idx % ZCPR;
    const int c = ((pc - (rl >> 2)) % ZCPR + ZCPR) % ZCPR;
    zrl[i] = rl;
    zoff[i] = uint32_t(rl * int(p.zs1) + 8 * c) * 2u;
  }
  auto issue = [&](int st, int t0) {
    unsigned char* ds = smem + st * XSTAGE;
    unsigned char* zs = smem + Z_OFF + st * ZSTAGE;
    if (t0 + kStep <= p.T) {
      const char* dg = dyc + int64_t(t0) * p.dys1 * 2;
      const char* zg = zc + int64_t(t0) * p.zs1 * 2;
#pragma unroll
      for (int i = 0; i < F::DI; ++i) dma16(dg + doff[i], ds + (wv + 4 * i) * 1024);
#pragma unroll
      for (int i = 0; i < F::ZI; ++i) dma16(zg + zoff[i], zs + (wv + 4 * i) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < F::DI; ++i) {
        const int t = min(t0 + drl[i], p.T - 1);
        dma16(dyc + (int64_t(t) - drl[i]) * p.dys1 * 2 + doff[i], ds + (wv + 4 * i) * 1024);
      }
#pragma unroll
      for (int i = 0; i < F::ZI; ++i) {
        const int t = min(t0 + zrl[i], p.T - 1);
        dma16(zc + (int64_t(t) - zrl[i]) * p.zs1 * 2 + zoff[i], zs + (wv + 4 * i) * 1024);
      }
    }
  };

  // ---- A operands and bias, as in the forward ----
  u16x8_t afr[4][KS];
  f32x4_t binit[4];
  {
    const uint16_t* U = static_cast<const uint16_t*>(p.U);
    const bool has_bias = p.bias != nullptr;
    const uint16_t* bsrc = has_bias ? static_cast<const uint16_t*>(p.bias) : U;
    const uint32_t bmask = has_bias ? ~0u : 0u;
    const int tap = n & 3;
    const int ltap = tap < W ? tap : W - 1;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int ch = cw + 4 * (n >> 2) + mt;
      const int64_t col = int64_t(ch) * W + ltap;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint16_t v = U[int64_t(32 * ks + 8 * q + e) * p.ldu + col];
          afr[mt][ks][e] = tap < W ? v : uint16_t(0);
        }
      const int chq = cw + 4 * q + mt;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint16_t v = bsrc[(has_bias ? int64_t(chq) * W : 0) + (i < W ? i : W - 1)];
        binit[mt][i] = __uint_as_float((uint32_t(v) << 16) & (i < W ? bmask : 0u));
      }
    }
  }
  issue(0, t_first);

  // ---- per-lane LDS offsets ----
  const int xc = 2 * wv + (q >> 1);  // logical 16-byte chunk of the lane's 4 channels
  const int drd = 4 * n * XROW + ((xc + n) & (XCPR - 1)) * 16 + 8 * (q & 1);  // dy row 4n (+ j * XROW)
  int zr[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) zr[ks] = 4 * n * ZROW + ((4 * ks + q + n) % ZCPR) * 16;
  // dx tile row of the lane's output j: token 4n + j sits in row 4n + j + 3; lane 15's
  // outputs 1..3 are the previous step's tokens 61..63, rows 0..2
  int trow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = (n == 15 && j > 0) ? j - 1 : 4 * n + j + 3;
    trow[j] = r * XROW + ((xc + (r >> 2)) & (XCPR - 1)) * 16 + 8 * (q & 1);
  }
  __amdgpu_buffer_rsrc_t dxr = __builtin_amdgcn_make_buffer_rsrc(
      static_cast<bf16_t*>(p.out) + b * p.os0, 0, int((int64_t(p.T - 1) * p.os1 + p.D) * 2), kBufWord3);
  const int dstep = int(p.os1 * 2);
  int ttr[F::NS], tgo[F::NS], trr[F::NS];
#pragma unroll
  for (int i = 0; i < F::NS; ++i) {
    const int idx = (wv + 4 * i) * 64 + lane;
    const int r = idx / XCPR, pc = idx % XCPR;
    const int c = (pc - (r >> 2)) & (XCPR - 1);
    ttr[i] = idx * 16;
    trr[i] = r;
    tgo[i] = int(((r - 3) * p.os1 + c_base + 8 * c) * 2);  // tile row r is token t0 - 3 + r
  }
  // Stores tile `buf` of step s (tokens t0 - 3 ..): the first step's rows 0..2 belong to
  // the previous range and the tail's rows 3.. to the next; their offsets are pushed out
  // of the buffer so the hardware drops them.
  auto tflush = [&](int buf, int s, int t0) {
    const unsigned char* tt = smem + T_OFF + buf * XSTAGE;
#pragma unroll
    for (int i = 0; i < F::NS; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(tt + ttr[i]);
      const bool keep = (s > 0 || trr[i] >= 3) && (s < nsteps || trr[i] < 3);
      __builtin_amdgcn_raw_buffer_store_b128(v, dxr, keep ? tgo[i] + t0 * dstep : int(0x80000000u), 0, 0);
    }
  };

  float pend[3][4];  // lane 15: tokens 61..63 of the previous step, without lane 0's terms
#pragma unroll
  for (int m = 0; m < 3; ++m)
#pragma unroll
    for (int c = 0; c < 4; ++c) pend[m][c] = 0.f;

  for (int s = 0; s <= nsteps; ++s) {
    const int t0 = t_first + s * kStep;
    const int u = s & 1;
    if (s >= 2) {
      vm_wait_barrier<F::NS>();
    } else {
      vm_wait_barrier<0>();
    }
    if (s < nsteps) issue(u ^ 1, t0 + kStep);
    if (s > 0) tflush(u ^ 1, s - 1, t0 - kStep);
    // dy of the lane's tokens 4n .. 4n+3, 4 channels; zero at or past T
    float dyv[4][4];
    {
      const unsigned char* ds = smem + u * XSTAGE + drd;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(ds + j * XROW);
        dyv[j][0] = bf16_lo(v[0]);
        dyv[j][1] = bf16_hi(v[0]);
        dyv[j][2] = bf16_lo(v[1]);
        dyv[j][3] = bf16_hi(v[1]);
      }
      if (t0 + kStep > p.T) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool ok = t0 + 4 * n + j < p.T;
#pragma unroll
          for (int c = 0; c < 4; ++c) dyv[j][c] = ok ? dyv[j][c] : 0.f;
        }
      }
    }
    const unsigned char* zs = smem + Z_OFF + u * ZSTAGE;
    auto gen = [&](int j, f32x4_t (&acc)[4]) {
      u16x8_t bfr[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) bfr[ks] = *reinterpret_cast<const u16x8_t*>(zs + zr[ks] + j * ZROW);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        acc[mt] = mma32(afr[mt][0], bfr[0], binit[mt]);
#pragma unroll
        for (int ks = 1; ks < KS; ++ks) acc[mt] = mma32(afr[mt][ks], bfr[ks], acc[mt]);
      }
    };
    // own[j]: dx of the lane's token j from its own terms; out[m]: terms for the previous
    // lane's token m (1..3)
    float own[4][4], out[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        own[j][c] = dyv[j][c];
        out[j][c] = 0.f;
      }
    f32x4_t acc[2][4];
    gen(0, acc[0]);
#pragma unroll
    for (int jp = 0; jp < 4; ++jp) {
      if (jp + 1 < 4) gen(jp + 1, acc[(jp + 1) & 1]);
      const f32x4_t(&a)[4] = acc[jp & 1];
#pragma unroll
      for (int k = 0; k < W; ++k) {
        const int j = jp - k;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (j >= 0) {
            own[j][c] = fmaf(a[c][k], dyv[jp][c], own[j][c]);
          } else {
            out[4 + j][c] = fmaf(a[c][k], dyv[jp][c], out[4 + j][c]);
          }
        }
      }
    }
    // the next lane's outgoing sums (lane 15: lane 0's, for the previous step's tokens)
    float dxv[4][4];
#pragma unroll
    for (int c = 0; c < 4; ++c) dxv[0][c] = own[0][c];
#pragma unroll
    for (int m = 1; m < 4; ++m)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float in = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(out[m][c]), 0x12F, 0xf, 0xf, false));
        const float base = n == 15 ? pend[m - 1][c] : own[m][c];
        dxv[m][c] = base + in;
        pend[m - 1][c] = own[m][c];
      }
    unsigned char* tt = smem + T_OFF + u * XSTAGE;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<u32x2*>(tt + trow[j]) = u32x2{pack_bf16x2(dxv[j][0], dxv[j][1]), pack_bf16x2(dxv[j][2], dxv[j][3])};
  }
  __syncthreads();
  tflush(nsteps & 1, nsteps, t_first + nsteps * kStep);
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
}

template <int KS>
using FwdCfg = FwdFast<KS, LRF_NWV, LRF_XN, LRF_XD, LRF_ZN, LRF_ZD>;

// A rank of 32 KS is served when its z transfers split evenly over the waves.
constexpr bool fwd_fast_rank_ok(int ks) {
  return (ks == 1 || ks == 2 || ks == 4) && (kStep * 4 * ks) % (64 * LRF_NWV) == 0;
}

// Workgroups resident per CU: 160 KiB of LDS and 8 waves (about 190 VGPRs each).
constexpr int fwd_fast_resident(int lds_bytes) {
  const int by_lds = 160 * 1024 / lds_bytes;
  const int by_waves = 8 / LRF_NWV;
  return by_lds < by_waves ? by_lds : by_waves;
}

template <int W, int KS>
hipError_t fwd_fast_try(const LowRankParams& p, int64_t blocks, hipStream_t s) {
  if constexpr (fwd_fast_rank_ok(KS)) {
    return fwd_fast_inst<W, KS>(p, blocks, s);
  } else {
    return hipErrorInvalidValue;
  }
}

template <int W>
hipError_t fwd_fast_ks(const LowRankParams& p, int64_t blocks, hipStream_t s) {
  switch (p.R / 32) {
    case 1: return fwd_fast_try<W, 1>(p, blocks, s);
    case 2: return fwd_fast_try<W, 2>(p, blocks, s);
    case 4: return fwd_fast_try<W, 4>(p, blocks, s);
    default: return hipErrorInvalidValue;
  }
}

template <int KS>
constexpr int fwd_fast_lds_ks() {
  if constexpr (fwd_fast_rank_ok(KS)) {
    return FwdCfg<KS>::BYTES;
  } else {
    return 160 * 1024;
  }
}

int fwd_fast_lds(int ks) {
  return ks == 1 ? fwd_fast_lds_ks<1>() : ks == 2 ? fwd_fast_lds_ks<2>() : fwd_fast_lds_ks<4>();
}

}  // namespace

bool lowrank_fwd_fast_ok(const LowRankParams& p, int W, dynconv_dtype dt) {
  const int ks = p.R / 32;
  return dt == DYNCONV_BF16 && p.H == 1 && W >= 1 && W <= 4 && p.R % 32 == 0 && fwd_fast_rank_ok(ks) &&
         p.D % (16 * LRF_NWV) == 0 && p.act16 != 0 && p.z16 != 0 &&
         (int64_t(p.T) + kStep) * p.os1 * 2 < (int64_t(1) << 31) && int64_t(kStep) * p.xs1 < (int64_t(1) << 30) &&
         int64_t(kStep) * p.zs1 < (int64_t(1) << 30);
}

LowRankPlan plan_lowrank_fwd_fast(int64_t B, int64_t T, int64_t D, int ks) {
  // one round of resident workgroups when the shape allows it, token ranges in whole steps
  LowRankPlan pl{};
  pl.nCs = int(D / (16 * LRF_NWV));
  const int64_t target = 256 * int64_t(fwd_fast_resident(fwd_fast_lds(ks)));
  int64_t per_seq = (target + B * pl.nCs - 1) / (B * pl.nCs);
  const int64_t max_ranges = (T + kStep - 1) / kStep;
  if (per_seq > max_ranges) per_seq = max_ranges;
  if (per_seq < 1) per_seq = 1;
  int64_t L = (T + per_seq - 1) / per_seq;
  L = (L + kStep - 1) / kStep * kStep;
  pl.Ltok = int(L);
  pl.nTr = int((T + L - 1) / L);
  pl.blocks = B * int64_t(pl.nTr) * pl.nCs;
  return pl;
}

hipError_t launch_lowrank_fwd_fast(const LowRankParams& p, int W, hipStream_t s) {
  const LowRankPlan pl = plan_lowrank_fwd_fast(p.B, p.T, p.D, p.R / 32);
  LowRankParams q = p;
  q.cs0 = 0;
  q.nCsL = pl.nCs;
  q.nCs = pl.nCs;
  q.Ltok = pl.Ltok;
  q.nTr = pl.nTr;
  switch (W) {
    case 1: return fwd_fast_ks<1>(q, pl.blocks, s);
    case 2: return fwd_fast_ks<2>(q, pl.blocks, s);
    case 3: return fwd_fast_ks<3>(q, pl.blocks, s);
    case 4: return fwd_fast_ks<4>(q, pl.blocks, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dynconv

namespace dynconv {

namespace {

template <int W, int KS>
hipError_t bwd_dx_inst(const LowRankParams& p, int64_t blocks, hipStream_t s) {
  hipLaunchKernelGGL((k_lowrank_bwd_dx_fast<W, KS>), dim3(unsigned(blocks)), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int W>
hipError_t bwd_dx_ks(const LowRankParams& p, int64_t blocks, hipStream_t s) {
  switch (p.R / 32) {
    case 1: return bwd_dx_inst<W, 1>(p, blocks, s);
    case 2: return bwd_dx_inst<W, 2>(p, blocks, s);
    case 4: return bwd_dx_inst<W, 4>(p, blocks, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool lowrank_bwd_dx_fast_ok(const LowRankParams& p, int W, dynconv_dtype dt) {
  const int ks = p.R / 32;
  return dt == DYNCONV_BF16 && p.H == 1 && W >= 1 && W <= 4 && p.R % 32 == 0 && (ks == 1 || ks == 2 || ks == 4) &&
         p.D % 64 == 0 && p.act16 != 0 && p.z16 != 0 && (int64_t(p.T) + kStep) * p.os1 * 2 < (int64_t(1) << 31) &&
         int64_t(kStep) * p.dys1 < (int64_t(1) << 30) && int64_t(kStep) * p.zs1 < (int64_t(1) << 30);
}

hipError_t launch_lowrank_bwd_dx_fast(const LowRankParams& p, int W, hipStream_t s) {
  // two or three workgroups per CU (48 KiB of LDS at R = 64): about 512 of them
  LowRankPlan pl{};
  pl.nCs = p.D / 64;
  const int64_t target = 512;
  int64_t per_seq = (target + int64_t(p.B) * pl.nCs - 1) / (int64_t(p.B) * pl.nCs);
  const int64_t max_ranges = (p.T + kStep - 1) / kStep;
  if (per_seq > max_ranges) per_seq = max_ranges;
  if (per_seq < 1) per_seq = 1;
  int64_t L = (p.T + per_seq - 1) / per_seq;
  L = (L + kStep - 1) / kStep * kStep;
  LowRankParams q = p;
  q.cs0 = 0;
  q.nCsL = pl.nCs;
  q.nCs = pl.nCs;
  q.Ltok = int(L);
  q.nTr = int((p.T + L - 1) / L);
  const int64_t blocks = int64_t(p.B) * q.nTr * pl.nCs;
  switch (W) {
    case 1: return bwd_dx_ks<1>(q, blocks, s);
    case 2: return bwd_dx_ks<2>(q, blocks, s);
    case 3: return bwd_dx_ks<3>(q, blocks, s);
    case 4: return bwd_dx_ks<4>(q, blocks, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dynconv
