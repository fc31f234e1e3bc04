// Low-rank dynamic short convolution, 16-bit (bf16, float16) fast path for gfx950: the filters w = z U + b
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
//    Head-wise generation (H consecutive channels share a group's filter, H <= 16): each
//    channel's rows of A are its group's columns of U, so the matrix work repeats per
//    channel while the x / y traffic is that of H = 1.
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
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
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

// z rows go to LDS in ZB-byte pieces per lane: 16 when the rows are 16-byte aligned and
// R % 8 == 0, else 4 (rows 4-byte aligned, R even). Ranks from R up to 32 KS (the padding
// of the matrix-core K extent) are read from this zero word instead.
__device__ __align__(16) uint32_t g_lr_zero16[4];

template <int ZB>
__device__ __forceinline__ void dmaz(const void* g, unsigned char* lds_wave_base) {
  static_assert(ZB == 16 || ZB == 4, "z piece");
  if constexpr (ZB == 16) {
    __builtin_amdgcn_global_load_lds(g, (lds_void*)(lds_wave_base), 16, 0, 0);
  } else {
    __builtin_amdgcn_global_load_lds(g, (lds_void*)(lds_wave_base), 4, 0, 0);
  }
}

// Source of z piece `idx` (ZB bytes each) of a stage whose rows are ZROW bytes with their
// 16-byte chunks rotated by rot (logical chunk c sits at position (c + rot) % (ZROW / 16)):
// the row, the byte offset inside the row, and whether the piece holds ranks below R.
struct ZPiece {
  int row;
  int byte;
  bool valid;
};
template <int ZB, int ZROW>
__device__ __forceinline__ ZPiece z_piece(int idx, int R, int (*rot)(int)) {
  constexpr int ZCPR = ZROW / 16;
  const int o = idx * ZB;
  const int row = o / ZROW, ob = o % ZROW;
  const int c = ((ob / 16 - rot(row)) % ZCPR + ZCPR) % ZCPR;
  const int gb = 16 * c + (ob & 15);
  return ZPiece{row, gb, gb / 2 < R};
}
__device__ __forceinline__ int rot_quarter(int row) { return row >> 2; }
__device__ __forceinline__ int rot_double(int row) { return 2 * row; }
// Stages shared by both roles of the fused backward: the four rows of a transposing read
// (8q + e, e = 0..3) land on distinct chunk positions as with 2 row, and the 16 rows
// 4n + j that the dx role reads at once spread over 8 positions.
__device__ __forceinline__ int rot_fused(int row) { return 2 * row + (row >> 2); }

// Waits until at most N of this wave's vector memory operations are outstanding (they
// complete in issue order) and its LDS operations are done, then joins the workgroup
// barrier.
template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  asm volatile("s_barrier" ::: "memory");
}

// 16x16x32 matrix-core product of 16-bit operands (bf16 or float16 storage)
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

template <int KS, int NWV_, int XN_, int XD_, int ZN_, int ZD_, int SG_ = 0, int ZB_ = 16, int IH_ = 4>
struct FwdFast {
  static constexpr int NWV = NWV_, XN = XN_, XD = XD_, ZN = ZN_, ZD = ZD_;
  static constexpr int ZB = ZB_;  // bytes of a z piece per lane and transfer
  // SG: packed sequences. Each step also stages the segment ids of tokens t0 - IH .. t0 + 63
  // (IH = 4, or 8 for filters of more than 5 taps: 17 or 18 chunks of 16 bytes, 5 per wave:
  // every wave issues exactly one more transfer, right before its x transfers, so it is
  // complete whenever x is).
  static constexpr int SG = SG_;
  static constexpr int IH = IH_;
  static_assert(IH == 4 || IH == 8, "id rows before the step: one or two row groups");
  static constexpr int SCH = (kStep + IH) / 4, SPW = 5, SSTAGE = NWV_ * SPW * 16;
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
  static constexpr int S_OFF = Y_OFF + 2 * XSTAGE;   // two y tiles, then the id stages
  static constexpr int BYTES = S_OFF + (SG ? XN * SSTAGE : 0);
  static constexpr int XI = kStep * XCPR / 64 / NWV;  // x transfers per wave per step (2)
  static constexpr int ZI = kStep * ZROW / (64 * ZB) / NWV;  // z transfers per wave per step
  static constexpr int NS = kStep * XCPR / 64 / NWV;  // y stores per wave per step (2)
  static_assert((kStep * ZROW) % (64 * ZB * NWV) == 0, "z transfers split evenly over the waves");
  static_assert(XD >= 1 && XD <= XN - 2 && ZD >= 1 && ZD <= ZN - 1 && ZD <= XD, "pipeline depths");
  static_assert((XCPR & (XCPR - 1)) == 0 && 16 % XCPR == 0, "x row rotation");
  static_assert(!SG || (NWV * SPW >= SCH && (NWV - 1) * SPW < SCH), "id chunks: at least one in every wave");
  static constexpr int XG = XI + SG;  // operations of the x group (ids first)

  // Issue order of one wave's vector memory operations: a prologue x(0), z(0), x(1),
  // z(1), ... (z only below ZD, x below XD); then step k issues x(k + XD), z(k + ZD) and,
  // from k = 1 on, the stores of step k - 1. Returns how many operations follow the later
  // of x(s) and z(s) when step s waits for them.
  static constexpr int step_ops(int k) { return XG + ZI + (k >= 1 ? NS : 0); }
  static constexpr int prologue_end_x(int i) {
    int pos = 0;
    for (int a = 0; a < i; ++a) pos += XG + (a < ZD ? ZI : 0);
    return pos + XG;
  }
  static constexpr int prologue_ops() { return prologue_end_x(XD - 1) + (XD - 1 < ZD ? ZI : 0); }
  static constexpr int steps_before(int k) {
    int pos = prologue_ops();
    for (int a = 0; a < k; ++a) pos += step_ops(a);
    return pos;
  }
  static constexpr int wait_after(int s) {
    const int end_x = s < XD ? prologue_end_x(s) : steps_before(s - XD) + XG;
    const int end_z = s < ZD ? prologue_end_x(s) + ZI : steps_before(s - ZD) + XG + ZI;
    const int last = end_x > end_z ? end_x : end_z;
    return steps_before(s) - last;
  }
  static constexpr int kSteady = XD + 1;  // from this step on the count no longer changes
};

// Matrix-core tiles that generate a wave's filters: tile c4 (0..3) holds taps 0..3 of the
// lane's channel c4 and, for W > 4, tile 4 + c4 its taps 4..7, so a lane receives every
// tap of its 4 channels.
template <int W>
constexpr int gen_tiles() {
  return W > 4 ? 8 : 4;
}

// A operands of the generation (U^T rows: the MFMA row n of tile mt is channel
// cw + 4 (n / 4) + mt % 4, tap 4 (mt / 4) + n % 4; ranks 32 ks + 8 q + e) and the bias as
// the accumulators' initial values (lane (n, q): channel cw + 4 q + mt % 4, taps
// 4 (mt / 4) + i). Loads are unconditional (a clamped tap and rank, U standing in for a
// missing bias) and the unused values are zeroed afterwards, so nothing waits on a branch.
template <typename ET, int W, int KS>
__device__ __forceinline__ void generation_operands(const LowRankParams& p, int cw, int n, int q,
                                                    u16x8_t (&afr)[gen_tiles<W>()][KS],
                                                    f32x4_t (&binit)[gen_tiles<W>()]) {
  const uint16_t* U = static_cast<const uint16_t*>(p.U);
  const bool has_bias = p.bias != nullptr;
  const uint16_t* bsrc = has_bias ? static_cast<const uint16_t*>(p.bias) : U;
  const int hsh = __builtin_ctz(unsigned(p.H));  // channel c takes group c / H's columns
#pragma unroll
  for (int mt = 0; mt < gen_tiles<W>(); ++mt) {
    const int c4 = mt & 3, half = mt >> 2;
    const int tap = 4 * half + (n & 3);
    const int ltap = tap < W ? tap : W - 1;
    const int ch = cw + 4 * (n >> 2) + c4;
    const int64_t col = int64_t(ch >> hsh) * W + ltap;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // ranks from R up to 32 KS are zero (the row read is clamped inside U)
        const int r = 32 * ks + 8 * q + e;
        const uint16_t v = U[int64_t(min(r, p.R - 1)) * p.ldu + col];
        afr[mt][ks][e] = (tap < W && r < p.R) ? v : uint16_t(0);
      }
    const int chq = cw + 4 * q + c4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tq = 4 * half + i;
      const uint16_t v = bsrc[(has_bias ? int64_t(chq >> hsh) * W : 0) + (tq < W ? tq : W - 1)];
      binit[mt][i] = (tq < W && has_bias) ? Cvt<ET>::of_bits(v) : 0.f;
    }
  }
}

// Filter tap k of the lane's channel c4 from the generation results of one token group.
template <int W>
__device__ __forceinline__ float tap_of(const f32x4_t (&a)[gen_tiles<W>()], int c4, int k) {
  return k < 4 ? a[c4][k] : a[4 + c4][k - 4];
}

// Rank tiles of the filter-gradient role's partial sums staged in LDS at a time (two LDS
// barriers each): up to 4, 2 when W > 4 (rows of 64 W + 1 floats).
constexpr int gdu_tiles_per_chunk(int W, int KS) {
  return (2 * KS < 4 ? 2 * KS : 4) / (W > 4 && 2 * KS >= 4 ? 2 : 1);
}

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

template <typename ET, int W, int KS, int SG, int ZB>
__global__ __launch_bounds__(64 * LRF_NWV) void k_lowrank_fwd_fast(const LowRankParams p) {
  using F = FwdFast<KS, LRF_NWV, LRF_XN, LRF_XD, LRF_ZN, LRF_ZD, SG, ZB, (W > 5 ? 8 : 4)>;
  constexpr int NWV = F::NWV, XN = F::XN, XD = F::XD, ZN = F::ZN, ZD = F::ZD, CPB = F::CPB;
  constexpr int XCPR = F::XCPR, XROW = F::XROW, XSTAGE = F::XSTAGE;
  constexpr int ZCPR = F::ZCPR, ZROW = F::ZROW, ZSTAGE = F::ZSTAGE, Z_OFF = F::Z_OFF, Y_OFF = F::Y_OFF;
  constexpr int XI = F::XI, ZI = F::ZI;
  constexpr int HR = W - 1;       // rows before a token that its filter reaches
  constexpr int MLO = -HR;        // x rows 4n + m, m = MLO .. 3, feed the lane's 4 tokens
  constexpr int NM = 4 - MLO;
  constexpr int NGT = gen_tiles<W>();
  constexpr int IH = F::IH;       // id rows before the lane's first token
  static_assert(HR <= 7 && HR <= IH, "x rows 4n + m with m >= -8: the lane's row group or one of the two before");
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
  const ET* xb = static_cast<const ET*>(p.x) + b * p.xs0 + c_base;
  const ET* zb = static_cast<const ET*>(p.z) + b * p.zs0;
  const int cw = c_base + 16 * wv;  // the wave's first channel

  // ---- LDS DMA of one step: rows t0 .. t0 + 63 (clamped to T - 1) ----
  // Transfer i of a wave fills 1 KiB of a stage (slot wv + NWV i); per lane the byte offset
  // of its 16-byte source chunk from the step's first row. The chunks of a row are rotated
  // by (row / 4) within the row.
  uint32_t xoff[XI], zoff[ZI];
  int xrl[XI], zrl[ZI];
  bool zval[ZI];
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
    const ZPiece zp = z_piece<ZB, ZROW>((wv + NWV * i) * 64 + lane, p.R, rot_quarter);
    zrl[i] = zp.row;
    zval[i] = zp.valid;
    zoff[i] = uint32_t(zp.row * int(p.zs1)) * 2u + uint32_t(zp.byte);
  }
  const char* xbc = reinterpret_cast<const char*>(xb);
  const char* zbc = reinterpret_cast<const char*>(zb);
  const char* zero = reinterpret_cast<const char*>(g_lr_zero16);
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
  // segment ids (SG): chunk sc = 5 wv + lane holds the ids of tokens t0 - IH + 4 sc .. + 3
  // (clamped into 0 .. T - 1: before t = 0 the x rows are zero, past T nothing is stored)
  const int sc = F::SPW * wv + lane;
  const bool sact = SG && lane < F::SPW && sc < F::SCH;
  const char* sgc = SG ? reinterpret_cast<const char*>(p.seg + b * p.ss0) : nullptr;
  auto issue_s = [&](int st, int t0) {
    if constexpr (SG) {
      if (sact) {
        const int tk = min(max(t0 - IH + 4 * sc, 0), p.T - 4);
        dma16(sgc + int64_t(tk) * 4, smem + F::S_OFF + st * F::SSTAGE + wv * F::SPW * 16);
      }
    }
  };
  auto issue_z = [&](int st, int t0) {
    unsigned char* zs = smem + Z_OFF + st * ZSTAGE;
    if (t0 + kStep <= p.T) {
      const char* zg = zbc + int64_t(t0) * p.zs1 * 2;
#pragma unroll
      for (int i = 0; i < ZI; ++i) dmaz<ZB>(zval[i] ? zg + zoff[i] : zero, zs + (wv + NWV * i) * (64 * ZB));
    } else {
#pragma unroll
      for (int i = 0; i < ZI; ++i) {
        const int t = min(t0 + zrl[i], p.T - 1);
        dmaz<ZB>(zval[i] ? zbc + (int64_t(t) - zrl[i]) * p.zs1 * 2 + zoff[i] : zero,
                 zs + (wv + NWV * i) * (64 * ZB));
      }
    }
  };

  // ---- A operands (U^T rows in the lane order above) and the bias, once ----
  u16x8_t afr[NGT][KS];
  f32x4_t binit[NGT];
  generation_operands<ET, W, KS>(p, cw, n, q, afr, binit);

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
    issue_s(i, t_first + i * kStep);
    issue_x(i, t_first + i * kStep);
    if (i < ZD) issue_z(i, t_first + i * kStep);
  }

  // ---- per-lane LDS offsets ----
  // x row 4n + m of ring stage u sits at u * XSTAGE + (4n + m) * XROW (rows before the
  // stage, 4n + m < 0, are the previous stage's last rows; from stage 0 they wrap to the
  // ring's end), chunk rotated by (row / 4): n - 2 for m < -4, n - 1 for m < 0, n for m >= 0
  // (the rotation is taken modulo XCPR, which divides the 16 row groups of a stage, so a
  // wrapped row keeps it).
  const int xc = 2 * wv + (q >> 1);  // logical 16-byte chunk of the lane's 4 channels
  const int xlo2 = 4 * n * XROW + ((xc + n - 2) & (XCPR - 1)) * 16 + 8 * (q & 1);  // + m * XROW, m < -4
  const int xlo = 4 * n * XROW + ((xc + n - 1) & (XCPR - 1)) * 16 + 8 * (q & 1);   // + m * XROW, -4 <= m < 0
  const int xhi = 4 * n * XROW + ((xc + n) & (XCPR - 1)) * 16 + 8 * (q & 1);       // + m * XROW, m >= 0
  const int xwrap = n == 0 ? XN * XSTAGE : 0;
  const int xwrap2 = n <= 1 ? XN * XSTAGE : 0;
  int zr[KS];  // + j * ZROW for token group j
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) zr[ks] = 4 * n * ZROW + ((4 * ks + q + n) % ZCPR) * 16;
  const int ytw = xhi;  // y tile: the lane writes row 4n + j (+ j * XROW), same rotation as x
  // optional convolution bias of the lane's 4 channels c_base + 8 xc + 4 (q & 1) + mt
  float cb[4] = {0.f, 0.f, 0.f, 0.f};
  if (p.cbias != nullptr) {  // 4-byte aligned (C ABI)
    const uint32_t* v =
        reinterpret_cast<const uint32_t*>(static_cast<const ET*>(p.cbias) + c_base + 8 * xc + 4 * (q & 1));
    const uint32_t v0 = v[0], v1 = v[1];
    cb[0] = Cvt<ET>::lo(v0);
    cb[1] = Cvt<ET>::hi(v0);
    cb[2] = Cvt<ET>::lo(v1);
    cb[3] = Cvt<ET>::hi(v1);
  }

  // y: buffer resource spanning this sequence's rows 0 .. T-1 (stores past it are dropped)
  __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
      static_cast<ET*>(p.out) + b * p.os0, 0, int((int64_t(p.T - 1) * p.os1 + p.D) * 2), kBufWord3);
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
    issue_s((s + XD) % XN, t0 + XD * kStep);
    issue_x((s + XD) % XN, t0 + XD * kStep);
    issue_z((s + ZD) % ZN, t0 + ZD * kStep);
    if (s > 0) yflush((s - 1) & 1, t0 - kStep);
    // ids of rows 4n - IH .. 4n + 3 (tap k of the lane's token 4n + j: kept when the id of
    // row 4n + j - k equals that of row 4n + j)
    int idv[IH + 4] = {};
    if constexpr (SG) {
      const int* ids = reinterpret_cast<const int*>(smem + F::S_OFF + ux * F::SSTAGE) + 4 * n;
#pragma unroll
      for (int i = 0; i < IH + 4; ++i) idv[i] = ids[i];
    }
    // x rows 4n + MLO .. 4n + 3 of the lane's channels, as float32
    const unsigned char* xst = smem + ux * XSTAGE;
    const int lo = xlo + (ux == 0 ? xwrap : 0);
    const int lo2 = xlo2 + (ux == 0 ? xwrap2 : 0);
    float xv[NM][4];
#pragma unroll
    for (int mi = 0; mi < NM; ++mi) {
      const int m = MLO + mi;
      const u32x2 v = *reinterpret_cast<const u32x2*>(xst + (m < -4 ? lo2 : m < 0 ? lo : xhi) + m * XROW);
      xv[mi][0] = Cvt<ET>::lo(v[0]);
      xv[mi][1] = Cvt<ET>::hi(v[0]);
      xv[mi][2] = Cvt<ET>::lo(v[1]);
      xv[mi][3] = Cvt<ET>::hi(v[1]);
    }
    const unsigned char* zs = smem + Z_OFF + uz * ZSTAGE;
    unsigned char* yt = smem + Y_OFF + (s & 1) * XSTAGE + ytw;
    // filters of token group j (MFMA), issued one group ahead of the convolution
    auto gen = [&](int j, f32x4_t (&acc)[NGT]) {
      u16x8_t bfr[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) bfr[ks] = *reinterpret_cast<const u16x8_t*>(zs + zr[ks] + j * ZROW);
#pragma unroll
      for (int mt = 0; mt < NGT; ++mt) {
        acc[mt] = mma32<ET>(afr[mt][0], bfr[0], binit[mt]);
#pragma unroll
        for (int ks = 1; ks < KS; ++ks) acc[mt] = mma32<ET>(afr[mt][ks], bfr[ks], acc[mt]);
      }
    };
    // the filters of group j + 1 are generated while group j's are applied, except where
    // the second accumulator set would not fit next to the rest (more than 5 taps at 64
    // ranks: one set, two workgroups per CU instead of one)
    constexpr bool AHEAD = W <= 5 || KS == 1;
    f32x4_t acc[AHEAD ? 2 : 1][NGT];
    if constexpr (AHEAD) gen(0, acc[0]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (AHEAD) {
        if (j + 1 < 4) gen(j + 1, acc[(j + 1) & 1]);
      } else {
        gen(j, acc[0]);
      }
      const f32x4_t(&a)[NGT] = acc[AHEAD ? (j & 1) : 0];
      float yv[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const float xt = xv[j - MLO][mt];
        float y = fmaf(a[mt][0], xt, xt + cb[mt]);
#pragma unroll
        for (int k = 1; k < W; ++k) {
          const float ak = (!SG || idv[j + IH - k] == idv[j + IH]) ? tap_of<W>(a, mt, k) : 0.f;
          y = fmaf(ak, xv[j - k - MLO][mt], y);
        }
        yv[mt] = y;
      }
      *reinterpret_cast<u32x2*>(yt + j * XROW) = u32x2{Cvt<ET>::pack2(yv[0], yv[1]), Cvt<ET>::pack2(yv[2], yv[3])};
    }
  }
  __syncthreads();
  yflush((nsteps - 1) & 1, t_first + (nsteps - 1) * kStep);
  // the transfers still in flight land in stages nobody reads; drain them (and the last
  // stores) before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
}

// z pieces of 16 bytes where the rows allow them and R % 8 == 0, else 4 bytes.
bool z_pieces16(const LowRankParams& p) { return p.z16 != 0 && p.R % 8 == 0; }

template <typename ET, int W, int KS, int ZB>
hipError_t fwd_fast_zb(const LowRankParams& p, int64_t blocks, hipStream_t s) {
  if (p.seg != nullptr) {
    hipLaunchKernelGGL((k_lowrank_fwd_fast<ET, W, KS, 1, ZB>), dim3(unsigned(blocks)), dim3(64 * LRF_NWV), 0, s, p);
  } else {
    hipLaunchKernelGGL((k_lowrank_fwd_fast<ET, W, KS, 0, ZB>), dim3(unsigned(blocks)), dim3(64 * LRF_NWV), 0, s, p);
  }
  return hipGetLastError();
}

template <typename ET, int W, int KS>
hipError_t fwd_fast_inst(const LowRankParams& p, int64_t blocks, hipStream_t s) {
  return z_pieces16(p) ? fwd_fast_zb<ET, W, KS, 16>(p, blocks, s) : fwd_fast_zb<ET, W, KS, 4>(p, blocks, s);
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
template <int KS, int SG = 0, int ZB = 16>
struct BwdDxFast {
  static constexpr int NWV = 4;
  // SG: packed sequences; the ids of tokens t0 - 4 .. t0 + 63 ride with each step's dy
  // (one more transfer per wave, issued first)
  static constexpr int SCH = 17, SPW = 5, SSTAGE = NWV * SPW * 16;
  static constexpr int CPB = 64;
  static constexpr int XCPR = 8, XROW = 128;
  static constexpr int XSTAGE = kStep * XROW;        // dy stage, dx tile
  static constexpr int ZCPR = 4 * KS;
  static constexpr int ZROW = 16 * ZCPR;
  static constexpr int ZSTAGE = kStep * ZROW;
  static constexpr int Z_OFF = 2 * XSTAGE;            // two dy stages
  static constexpr int T_OFF = Z_OFF + 2 * ZSTAGE;    // two z stages, then two dx tiles
  static constexpr int S_OFF = T_OFF + 2 * XSTAGE;    // then two id stages (SG)
  static constexpr int BYTES = S_OFF + (SG ? 2 * SSTAGE : 0);
  static constexpr int DI = 2, ZI = kStep * ZROW / (64 * ZB) / NWV, ND = DI + ZI, NS = 2;
};

// Layout of the fused backward (k_lowrank_bwd_fast, 8 waves): x in a ring of 4 steps, dy,
// z (and the ids of packed sequences) in 3 stages each, loaded two steps ahead by the
// filter-gradient role, then the dx role's two output tiles.
template <int KS, int SG_, int ZB>
struct BwdFused {
  static constexpr int SG = SG_;
  static constexpr int CPR = 8, ROW = 128, STAGE = kStep * ROW;  // x, dy: 64 channels
  static constexpr int ZCPR = 4 * KS, ZROW = 16 * ZCPR, ZSTAGE = kStep * ZROW;
  static constexpr int DIST = 2, XN = 4, SN = 3;
  static constexpr int SCH = 17, SPW = 5, SSTAGE = 4 * SPW * 16;
  static constexpr int D_OFF = XN * STAGE;
  static constexpr int Z_OFF = D_OFF + SN * STAGE;
  static constexpr int S_OFF = Z_OFF + SN * ZSTAGE;
  static constexpr int T_OFF = S_OFF + (SG ? SN * SSTAGE : 0);
  static constexpr int BYTES = T_OFF + 2 * STAGE;
  static constexpr int XI = 2, DI = 2, ZI = kStep * ZROW / (64 * ZB) / 4, ND = XI + DI + ZI + SG;
};

// The dx computation. Standalone (FUSED false): its own kernel, staging dy and z itself.
// FUSED: waves 0..3 of the fused backward, reading dy, z and ids from the stages of layout
// FL that the other role fills, writing its tiles at FL::T_OFF, and running one barrier per
// step (the range's steps and the tail step) plus the epilogue's.
template <typename ET, int W, int KS, int SG, int ZB, bool FUSED, class FL>
__device__ __forceinline__ void lowrank_dx_role(const LowRankParams& p, unsigned char* smem, int tid,
                                                uint32_t lb) {
  using F = BwdDxFast<KS, SG, ZB>;
  constexpr int XCPR = F::XCPR, XROW = F::XROW, XSTAGE = F::XSTAGE;
  constexpr int ZCPR = F::ZCPR, ZROW = F::ZROW, ZSTAGE = F::ZSTAGE, Z_OFF = F::Z_OFF;
  constexpr int T_OFF = FUSED ? FL::T_OFF : F::T_OFF;
  constexpr int NGT = gen_tiles<W>();
  // Rows of delay: a token's dx needs the terms of the next W - 1 tokens, so a lane's first
  // E tokens are complete from its own terms, the others wait for the next lane's (lane 15:
  // for the next step's lane 0). The step's tile holds tokens t0 - DXH .. t0 + 63 - DXH.
  constexpr int DXH = W > 4 ? 4 : 3;
  constexpr int E = 4 - DXH;
  static_assert(W <= 5, "terms reach the previous lane's tokens only");

  const int lane = tid & 63;
  const int q = lane >> 4;
  const int n = lane & 15;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cs = p.cs0 + int(lb % uint32_t(p.nCsL));
  lb /= uint32_t(p.nCsL);
  const int tr = int(lb % uint32_t(p.nTr));
  const int b = int(lb / uint32_t(p.nTr));
  const int c_base = cs * F::CPB;
  const int t_first = tr * p.Ltok;
  const int t_end = min(p.T, t_first + p.Ltok);
  const int nsteps = (t_end - t_first + kStep - 1) / kStep;
  const char* dyc = reinterpret_cast<const char*>(static_cast<const ET*>(p.dy) + b * p.dys0 + c_base);
  const char* zc = reinterpret_cast<const char*>(static_cast<const ET*>(p.z) + b * p.zs0);
  const int cw = c_base + 16 * wv;

  // ---- LDS DMA of a step's dy and z rows (rows past T - 1 read row T - 1) ----
  uint32_t doff[F::DI], zoff[F::ZI];
  int drl[F::DI], zrl[F::ZI];
  bool zval[F::ZI];
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
    const ZPiece zp = z_piece<ZB, ZROW>((wv + 4 * i) * 64 + lane, p.R, rot_quarter);
    zrl[i] = zp.row;
    zval[i] = zp.valid;
    zoff[i] = uint32_t(zp.row * int(p.zs1)) * 2u + uint32_t(zp.byte);
  }
  const char* zero = reinterpret_cast<const char*>(g_lr_zero16);
  // segment ids (SG): chunk sc = 5 wv + lane holds the ids of tokens t0 - 4 + 4 sc .. + 3
  const int sc = F::SPW * wv + lane;
  const bool sact = SG && lane < F::SPW && sc < F::SCH;
  const char* sgc = SG ? reinterpret_cast<const char*>(p.seg + b * p.ss0) : nullptr;
  auto issue = [&](int st, int t0) {
    unsigned char* ds = smem + st * XSTAGE;
    unsigned char* zs = smem + Z_OFF + st * ZSTAGE;
    if constexpr (SG) {
      if (sact) {
        const int tk = min(max(t0 - 4 + 4 * sc, 0), p.T - 4);
        dma16(sgc + int64_t(tk) * 4, smem + F::S_OFF + st * F::SSTAGE + wv * F::SPW * 16);
      }
    }
    if (t0 + kStep <= p.T) {
      const char* dg = dyc + int64_t(t0) * p.dys1 * 2;
      const char* zg = zc + int64_t(t0) * p.zs1 * 2;
#pragma unroll
      for (int i = 0; i < F::DI; ++i) dma16(dg + doff[i], ds + (wv + 4 * i) * 1024);
#pragma unroll
      for (int i = 0; i < F::ZI; ++i) dmaz<ZB>(zval[i] ? zg + zoff[i] : zero, zs + (wv + 4 * i) * (64 * ZB));
    } else {
#pragma unroll
      for (int i = 0; i < F::DI; ++i) {
        const int t = min(t0 + drl[i], p.T - 1);
        dma16(dyc + (int64_t(t) - drl[i]) * p.dys1 * 2 + doff[i], ds + (wv + 4 * i) * 1024);
      }
#pragma unroll
      for (int i = 0; i < F::ZI; ++i) {
        const int t = min(t0 + zrl[i], p.T - 1);
        dmaz<ZB>(zval[i] ? zc + (int64_t(t) - zrl[i]) * p.zs1 * 2 + zoff[i] : zero, zs + (wv + 4 * i) * (64 * ZB));
      }
    }
  };

  // ---- A operands and bias, as in the forward ----
  u16x8_t afr[NGT][KS];
  f32x4_t binit[NGT];
  generation_operands<ET, W, KS>(p, cw, n, q, afr, binit);
  if constexpr (!FUSED) issue(0, t_first);

  // ---- per-lane LDS offsets ----
  const int xc = 2 * wv + (q >> 1);  // logical 16-byte chunk of the lane's 4 channels
  const int drd = 4 * n * XROW + ((xc + n) & (XCPR - 1)) * 16 + 8 * (q & 1);  // dy row 4n (+ j * XROW)
  int zr[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) zr[ks] = 4 * n * ZROW + ((4 * ks + q + n) % ZCPR) * 16;
  // dy row 4n + j and the chunk 4 ks + q of z row 4n + j inside a step's stage: rotation
  // row / 4 in the kernel's own stages, the shared one in the fused kernel's
  auto dy_at = [&](int j) -> int {
    if constexpr (FUSED) {
      const int r = 4 * n + j;
      return r * XROW + ((xc + rot_fused(r)) & (XCPR - 1)) * 16 + 8 * (q & 1);
    } else {
      return drd + j * XROW;
    }
  };
  // byte offsets of step s's dy, z and id stages
  auto dy_stage = [&](int s) -> int {
    if constexpr (FUSED) {
      return FL::D_OFF + (s % FL::SN) * FL::STAGE;
    } else {
      return (s & 1) * XSTAGE;
    }
  };
  auto z_stage = [&](int s) -> int {
    if constexpr (FUSED) {
      return FL::Z_OFF + (s % FL::SN) * FL::ZSTAGE;
    } else {
      return Z_OFF + (s & 1) * ZSTAGE;
    }
  };
  auto id_stage = [&](int s) -> int {
    if constexpr (FUSED) {
      return FL::S_OFF + (s % FL::SN) * FL::SSTAGE;
    } else {
      return F::S_OFF + (s & 1) * F::SSTAGE;
    }
  };
  auto z_at = [&](int j, int ks) -> int {
    if constexpr (FUSED) {
      const int r = 4 * n + j;
      return r * ZROW + ((4 * ks + q + rot_fused(r)) % ZCPR) * 16;
    } else {
      return zr[ks] + j * ZROW;
    }
  };
  // dx tile row of the lane's output j: token 4n + j sits in row 4n + j + 3; lane 15's
  // outputs 1..3 are the previous step's tokens 61..63, rows 0..2
  int trow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = (n == 15 && j >= E) ? j - E : 4 * n + j + DXH;
    trow[j] = r * XROW + ((xc + (r >> 2)) & (XCPR - 1)) * 16 + 8 * (q & 1);
  }
  __amdgpu_buffer_rsrc_t dxr = __builtin_amdgcn_make_buffer_rsrc(
      static_cast<ET*>(p.out) + b * p.os0, 0, int((int64_t(p.T - 1) * p.os1 + p.D) * 2), kBufWord3);
  const int dstep = int(p.os1 * 2);
  int ttr[F::NS], tgo[F::NS], trr[F::NS];
#pragma unroll
  for (int i = 0; i < F::NS; ++i) {
    const int idx = (wv + 4 * i) * 64 + lane;
    const int r = idx / XCPR, pc = idx % XCPR;
    const int c = (pc - (r >> 2)) & (XCPR - 1);
    ttr[i] = idx * 16;
    trr[i] = r;
    tgo[i] = int(((r - DXH) * p.os1 + c_base + 8 * c) * 2);  // tile row r is token t0 - DXH + r
  }
  // Stores tile `buf` of step s (tokens t0 - DXH ..): the first step's rows 0 .. DXH - 1
  // belong to the previous range and the tail's rows DXH .. to the next; their offsets are
  // pushed out of the buffer so the hardware drops them.
  auto tflush = [&](int buf, int s, int t0) {
    const unsigned char* tt = smem + T_OFF + buf * XSTAGE;
#pragma unroll
    for (int i = 0; i < F::NS; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(tt + ttr[i]);
      const bool keep = (s > 0 || trr[i] >= DXH) && (s < nsteps || trr[i] < DXH);
      __builtin_amdgcn_raw_buffer_store_b128(v, dxr, keep ? tgo[i] + t0 * dstep : int(0x80000000u), 0, 0);
    }
  };

  float pend[DXH][4];  // lane 15: tokens 64 - DXH .. 63 of the previous step, without lane 0's terms
#pragma unroll
  for (int m = 0; m < DXH; ++m)
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
    if constexpr (!FUSED) {
      if (s < nsteps) issue(u ^ 1, t0 + kStep);
    }
    if (s > 0) tflush(u ^ 1, s - 1, t0 - kStep);
    // dy of the lane's tokens 4n .. 4n+3, 4 channels; zero at or past T
    float dyv[4][4];
    {
      const unsigned char* ds = smem + dy_stage(s);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(ds + dy_at(j));
        dyv[j][0] = Cvt<ET>::lo(v[0]);
        dyv[j][1] = Cvt<ET>::hi(v[0]);
        dyv[j][2] = Cvt<ET>::lo(v[1]);
        dyv[j][3] = Cvt<ET>::hi(v[1]);
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
    const unsigned char* zs = smem + z_stage(s);
    // ids of rows 4n - 4 .. 4n + 3 (SG): the term of tap k of token 4n + jp is kept when
    // row 4n + jp - k has the id of row 4n + jp
    int idv[8] = {};
    if constexpr (SG) {
      const int* ids = reinterpret_cast<const int*>(smem + id_stage(s)) + 4 * n;
#pragma unroll
      for (int i = 0; i < 8; ++i) idv[i] = ids[i];
    }
    auto gen = [&](int j, f32x4_t (&acc)[NGT]) {
      u16x8_t bfr[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) bfr[ks] = *reinterpret_cast<const u16x8_t*>(zs + z_at(j, ks));
#pragma unroll
      for (int mt = 0; mt < NGT; ++mt) {
        acc[mt] = mma32<ET>(afr[mt][0], bfr[0], binit[mt]);
#pragma unroll
        for (int ks = 1; ks < KS; ++ks) acc[mt] = mma32<ET>(afr[mt][ks], bfr[ks], acc[mt]);
      }
    };
    // own[j]: dx of the lane's token j from its own terms; out[m]: terms for the previous
    // lane's token m (E .. 3)
    float own[4][4], out[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        own[j][c] = dyv[j][c];
        out[j][c] = 0.f;
      }
    f32x4_t acc[2][NGT];
    gen(0, acc[0]);
#pragma unroll
    for (int jp = 0; jp < 4; ++jp) {
      if (jp + 1 < 4) gen(jp + 1, acc[(jp + 1) & 1]);
      const f32x4_t(&a)[NGT] = acc[jp & 1];
#pragma unroll
      for (int k = 0; k < W; ++k) {
        const int j = jp - k;
        const bool keep = !SG || k == 0 || idv[4 + jp - k] == idv[4 + jp];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float ak = keep ? tap_of<W>(a, c, k) : 0.f;
          if (j >= 0) {
            own[j][c] = fmaf(ak, dyv[jp][c], own[j][c]);
          } else {
            out[4 + j][c] = fmaf(ak, dyv[jp][c], out[4 + j][c]);
          }
        }
      }
    }
    // the next lane's outgoing sums (lane 15: lane 0's, for the previous step's tokens)
    float dxv[4][4];
#pragma unroll
    for (int m = 0; m < E; ++m)
#pragma unroll
      for (int c = 0; c < 4; ++c) dxv[m][c] = own[m][c];
#pragma unroll
    for (int m = E; m < 4; ++m)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float in = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(out[m][c]), 0x12F, 0xf, 0xf, false));
        const float base = n == 15 ? pend[m - E][c] : own[m][c];
        dxv[m][c] = base + in;
        pend[m - E][c] = own[m][c];
      }
    unsigned char* tt = smem + T_OFF + u * XSTAGE;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<u32x2*>(tt + trow[j]) = u32x2{Cvt<ET>::pack2(dxv[j][0], dxv[j][1]), Cvt<ET>::pack2(dxv[j][2], dxv[j][3])};
  }
  __syncthreads();
  tflush(nsteps & 1, nsteps, t_first + nsteps * kStep);
  if constexpr (FUSED) {
    // the filter-gradient role's epilogue: two barriers per chunk of its partial sums
    constexpr int RT = 2 * KS, TPC = gdu_tiles_per_chunk(W, KS);
#pragma unroll
    for (int c = 0; c < 2 * (RT / TPC); ++c) __syncthreads();
  }
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
}

template <typename ET, int W, int KS, int SG, int ZB>
__global__ __launch_bounds__(256) void k_lowrank_bwd_dx_fast(const LowRankParams p) {
  using F = BwdDxFast<KS, SG, ZB>;
  __shared__ __align__(16) unsigned char smem[F::BYTES];
  lowrank_dx_role<ET, W, KS, SG, ZB, false, F>(p, smem, threadIdx.x, xcd_logical_block(blockIdx.x, gridDim.x));
}


// Transposing LDS reads (ds_read_b64_tr_b16) of N 8-byte rows at 32-bit LDS byte offsets,
// issued together and waited for inside the same asm block. They are written as asm
// because the compiler places a full vmcnt wait (for every LDS DMA in flight, including
// the next step's) in front of its own form of this read; here the DMA is waited for
// explicitly at the step barrier. Outputs are early-clobber: a result that arrives must
// not overwrite the address of a later read of the group.
__device__ __forceinline__ void tr_read8(u32x2 (&o)[8], const uint32_t (&a)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n ds_read_b64_tr_b16 %1, %9\n ds_read_b64_tr_b16 %2, %10\n"
      "ds_read_b64_tr_b16 %3, %11\n ds_read_b64_tr_b16 %4, %12\n ds_read_b64_tr_b16 %5, %13\n"
      "ds_read_b64_tr_b16 %6, %14\n ds_read_b64_tr_b16 %7, %15\n s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]));
}
__device__ __forceinline__ void tr_read9(u32x2 (&o)[9], const uint32_t (&a)[9]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %9\n ds_read_b64_tr_b16 %1, %10\n ds_read_b64_tr_b16 %2, %11\n"
      "ds_read_b64_tr_b16 %3, %12\n ds_read_b64_tr_b16 %4, %13\n ds_read_b64_tr_b16 %5, %14\n"
      "ds_read_b64_tr_b16 %6, %15\n ds_read_b64_tr_b16 %7, %16\n ds_read_b64_tr_b16 %8, %17\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7]),
        "=&v"(o[8])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "v"(a[8]));
}
__device__ __forceinline__ void tr_read13(u32x2 (&o)[13], const uint32_t (&a)[13]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %13\n ds_read_b64_tr_b16 %1, %14\n ds_read_b64_tr_b16 %2, %15\n"
      "ds_read_b64_tr_b16 %3, %16\n ds_read_b64_tr_b16 %4, %17\n ds_read_b64_tr_b16 %5, %18\n"
      "ds_read_b64_tr_b16 %6, %19\n ds_read_b64_tr_b16 %7, %20\n ds_read_b64_tr_b16 %8, %21\n"
      "ds_read_b64_tr_b16 %9, %22\n ds_read_b64_tr_b16 %10, %23\n ds_read_b64_tr_b16 %11, %24\n"
      "ds_read_b64_tr_b16 %12, %25\n s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7]),
        "=&v"(o[8]), "=&v"(o[9]), "=&v"(o[10]), "=&v"(o[11]), "=&v"(o[12])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "v"(a[8]),
        "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]));
}

// 32-bit LDS byte address of a shared-memory pointer.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) unsigned char*)(p)));
}

// ---------------------------------------------------------------------------------
// Backward filter gradient, k_lowrank_bwd_gdu_fast: per token range and 64-channel slice,
// float32 partial sums of
//   dU[r][g W + k] = sum_t z_t[r] g_t[g W + k],  db[g W + k] = sum_t g_t[g W + k],
//   g_t[c W + k] = dy_t[c] x_{t-k}[c]
// (the gradient of w = z U + b; g is the per-token filter gradient of eq. 2).
// The contraction runs over tokens on the matrix cores with M = 16 channels of one tap,
// N = 16 ranks and K = 32 tokens. Both operands come from LDS by transposing reads
// (ds_read_b64_tr_b16), which hand lane i column i of 4 consecutive rows: the dy and x
// columns of the lane's channel (x read 4 rows early and late, so each tap's shift is a
// choice of registers) give g in the A layout directly, and the z columns give B. So g
// never goes to LDS. x sits in a ring of 4 steps (its rows before a step are the previous
// step's), dy and z in 3 stages each, all filled by LDS DMA two steps ahead; a row's
// 16-byte chunks are rotated by 2 row so that the 4 rows of a transposing read hit
// distinct banks.
// ---------------------------------------------------------------------------------
template <int KS, int SG_ = 0, int ZB = 16>
struct BwdGduFast {
  static constexpr int CPR = 8, ROW = 128, STAGE = kStep * ROW;  // x, dy: 64 channels
  static constexpr int ZCPR = 4 * KS, ZROW = 16 * ZCPR, ZSTAGE = kStep * ZROW;
  // SG: packed sequences. The ids of tokens t0 - 4 .. t0 + 63 ride with each step (one
  // more transfer per wave, issued first). The stages then load one step ahead instead of
  // two (two dy / z stages, 16 KiB less), which keeps two workgroups per CU at R = 64 with
  // the id stages (80 KiB each without them).
  static constexpr int SG = SG_;
  static constexpr int DIST = SG ? 1 : 2;   // steps loaded ahead
  static constexpr int XN = 4;   // x ring: the step, the previous one, two in flight
  static constexpr int SN = DIST + 1;       // dy and z stages: the step and those in flight
  static constexpr int SCH = 17, SPW = 5, SSTAGE = 4 * SPW * 16;
  static constexpr int D_OFF = XN * STAGE;
  static constexpr int Z_OFF = D_OFF + SN * STAGE;
  static constexpr int S_OFF = Z_OFF + SN * ZSTAGE;
  static constexpr int BYTES = S_OFF + (SG ? SN * SSTAGE : 0);
  static constexpr int XI = 2, DI = 2, ZI = kStep * ZROW / (64 * ZB) / 4, ND = XI + DI + ZI + SG;
};

// The g / dU / db partial sums. Standalone (FUSED false): its own kernel with layout
// BwdGduFast. FUSED: waves 4..7 of the fused backward with layout BwdFused, which also
// stage dy and z for the tail step (s == nsteps) that the dx role needs, stay in step with
// it (one barrier per step, the tail included) and meet its epilogue barriers.
template <typename ET, int W, int KS, int SG, int ZB, bool FUSED, class F>
__device__ __forceinline__ void lowrank_gdu_role(const LowRankParams& p, unsigned char* smem, int tid,
                                                 uint32_t lb) {
  constexpr int CPR = F::CPR, ROW = F::ROW, STAGE = F::STAGE, XN = F::XN;
  constexpr int ZCPR = F::ZCPR, ZROW = F::ZROW, ZSTAGE = F::ZSTAGE, D_OFF = F::D_OFF, Z_OFF = F::Z_OFF;
  constexpr int RT = 2 * KS;  // 16-rank tiles
  constexpr int HR = W - 1;
  constexpr int TAIL = FUSED ? 1 : 0;  // the dx role's tail step
  auto rot = [](int row) { return FUSED ? rot_fused(row) : rot_double(row); };

  const int lane = tid & 63;
  const int q = lane >> 4;
  const int j = lane & 15;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cs = int(lb % uint32_t(p.nCsL));
  lb /= uint32_t(p.nCsL);
  const int tr = int(lb % uint32_t(p.nTr));
  const int b = int(lb / uint32_t(p.nTr));
  const int c_base = cs * 64;
  const int t_first = tr * p.Ltok;
  const int t_end = min(p.T, t_first + p.Ltok);
  const int nsteps = (t_end - t_first + kStep - 1) / kStep;
  const char* xc = reinterpret_cast<const char*>(static_cast<const ET*>(p.x) + b * p.xs0 + c_base);
  const char* dc = reinterpret_cast<const char*>(static_cast<const ET*>(p.dy) + b * p.dys0 + c_base);
  const char* zc = reinterpret_cast<const char*>(static_cast<const ET*>(p.z) + b * p.zs0);

  // ---- LDS DMA: per lane the byte offset of its source chunk from a step's first row ----
  uint32_t xoff[2], doff[2], zoff[F::ZI];
  int arl[2], zrl[F::ZI];
  bool zval[F::ZI];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = (wv + 4 * i) * 64 + lane;
    const int rl = idx / CPR, pc = idx % CPR;
    const int c = (pc - rot(rl)) & (CPR - 1);
    arl[i] = rl;
    xoff[i] = uint32_t(rl * int(p.xs1) + 8 * c) * 2u;
    doff[i] = uint32_t(rl * int(p.dys1) + 8 * c) * 2u;
  }
#pragma unroll
  for (int i = 0; i < F::ZI; ++i) {
    const ZPiece zp = z_piece<ZB, ZROW>((wv + 4 * i) * 64 + lane, p.R, FUSED ? rot_fused : rot_double);
    zrl[i] = zp.row;
    zval[i] = zp.valid;
    zoff[i] = uint32_t(zp.row * int(p.zs1)) * 2u + uint32_t(zp.byte);
  }
  const char* zero = reinterpret_cast<const char*>(g_lr_zero16);
  const int sc = F::SPW * wv + lane;
  const bool sact = SG && lane < F::SPW && sc < F::SCH;
  const char* sgc = SG ? reinterpret_cast<const char*>(p.seg + b * p.ss0) : nullptr;
  auto issue = [&](int s, int t0) {
    unsigned char* xs = smem + (s % XN) * STAGE;
    unsigned char* ds = smem + D_OFF + (s % F::SN) * STAGE;
    unsigned char* zs = smem + Z_OFF + (s % F::SN) * ZSTAGE;
    if constexpr (SG) {
      if (sact) {
        const int tk = min(max(t0 - 4 + 4 * sc, 0), p.T - 4);
        dma16(sgc + int64_t(tk) * 4, smem + F::S_OFF + (s % F::SN) * F::SSTAGE + wv * F::SPW * 16);
      }
    }
    if (t0 + kStep <= p.T) {
      const int64_t o1 = int64_t(t0) * 2;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        dma16(xc + o1 * p.xs1 + xoff[i], xs + (wv + 4 * i) * 1024);
        dma16(dc + o1 * p.dys1 + doff[i], ds + (wv + 4 * i) * 1024);
      }
#pragma unroll
      for (int i = 0; i < F::ZI; ++i)
        dmaz<ZB>(zval[i] ? zc + o1 * p.zs1 + zoff[i] : zero, zs + (wv + 4 * i) * (64 * ZB));
    } else {
      // rows past T - 1 read row T - 1; their dy is zeroed below
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int64_t t = min(t0 + arl[i], p.T - 1) - arl[i];
        dma16(xc + t * p.xs1 * 2 + xoff[i], xs + (wv + 4 * i) * 1024);
        dma16(dc + t * p.dys1 * 2 + doff[i], ds + (wv + 4 * i) * 1024);
      }
#pragma unroll
      for (int i = 0; i < F::ZI; ++i) {
        const int64_t t = min(t0 + zrl[i], p.T - 1) - zrl[i];
        dmaz<ZB>(zval[i] ? zc + t * p.zs1 * 2 + zoff[i] : zero, zs + (wv + 4 * i) * (64 * ZB));
      }
    }
  };

  // ---- the W-1 x rows before the range: the last rows of ring stage XN - 1 ----
  if constexpr (HR > 0) {
    unsigned char* hbase = smem + XN * STAGE - HR * ROW;
    if (t_first > 0) {
      if (wv == 0 && lane < HR * CPR) {
        const int rl = kStep - HR + lane / CPR, pc = lane % CPR;
        const int c = (pc - rot(rl)) & (CPR - 1);
        dma16(xc + (int64_t(t_first - HR + lane / CPR) * p.xs1 + 8 * c) * 2, hbase);
      }
    } else if (tid < HR * ROW / 4) {
      reinterpret_cast<uint32_t*>(hbase)[tid] = 0u;
    }
  }
  issue(0, t_first);
  if (F::DIST > 1 && nsteps + TAIL > 1) issue(1, t_first + kStep);

  // Transposing-read addresses. Lane (j, q) reads 8 bytes of row 8q + j/4 (+ 4), channel
  // columns 16 wv + 4 (j % 4) .. + 3; lane i then holds column 16 wv + i of 4 rows.
  const int trow = 8 * q + (j >> 2);
  const int tch = 2 * wv + ((j & 3) >> 1);  // logical 16-byte chunk
  const int thalf = 8 * (j & 1);
  auto arow = [&](int row) { return row * ROW + ((tch + rot(row)) & (CPR - 1)) * 16 + thalf; };
  // z: lane holds rank column 16 rt + i
  auto zaddr = [&](int row, int rt) {
    const int c = 2 * rt + ((j & 3) >> 1);
    return row * ZROW + ((c + rot(row)) % ZCPR) * 16 + thalf;
  };

  f32x4_t dU[W][RT];
#pragma unroll
  for (int k = 0; k < W; ++k)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) dU[k][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float db[W];
#pragma unroll
  for (int k = 0; k < W; ++k) db[k] = 0.f;

  const uint32_t lds0 = lds_addr(smem);
  constexpr int NR = 5 + 2 * RT;  // transposing reads per K step: dy 2, x 3, z 2 per rank tile
  auto bf = [](const u32x2& w, int e) { return (e & 1) ? Cvt<ET>::hi(w[e >> 1]) : Cvt<ET>::lo(w[e >> 1]); };

  for (int s = 0; s < nsteps + TAIL; ++s) {
    const int t0 = t_first + s * kStep;
    // this step's transfers were followed by the next step's, if there is one (loading two
    // steps ahead); loading one step ahead, nothing newer is in flight
    if (F::DIST > 1 && s + 1 < nsteps + TAIL) {
      vm_wait_barrier<F::ND>();
    } else {
      vm_wait_barrier<0>();
    }
    if (s + F::DIST < nsteps + TAIL) issue(s + F::DIST, t0 + F::DIST * kStep);
    if (FUSED && s == nsteps) continue;  // the tail step's rows are the dx role's alone
    const int ux = s % XN;
    const uint32_t dsa = lds0 + D_OFF + (s % F::SN) * STAGE;
    const uint32_t zsa = lds0 + Z_OFF + (s % F::SN) * ZSTAGE;
    const bool partial = t0 + kStep > p.T;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int r0 = 32 * kk + trow;  // the lane's first row of this K step
      // dy rows r0, r0 + 4; x rows r0 - 4, r0, r0 + 4 of the ring (rows before the stage
      // are the previous one's); z rows r0, r0 + 4 of each rank tile
      uint32_t a[NR];
      a[0] = dsa + arow(r0);
      a[1] = dsa + arow(r0 + 4);
#pragma unroll
      for (int h = 0; h < 3; ++h) {
        const int xr = ux * kStep + r0 + 4 * (h - 1);
        a[2 + h] = lds0 + arow(xr < 0 ? xr + XN * kStep : xr);
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        a[5 + 2 * rt] = zsa + zaddr(r0, rt);
        a[6 + 2 * rt] = zsa + zaddr(r0 + 4, rt);
      }
      u32x2 v[NR];
      if constexpr (NR == 9) {
        tr_read9(v, a);
      } else if constexpr (NR == 13) {
        tr_read13(v, a);
      } else {
        static_assert(NR == 21, "rank tiles");
        uint32_t a1[13], a2[8];
        u32x2 v1[13], v2[8];
#pragma unroll
        for (int i = 0; i < 13; ++i) a1[i] = a[i];
#pragma unroll
        for (int i = 0; i < 8; ++i) a2[i] = a[13 + i];
        tr_read13(v1, a1);
        tr_read8(v2, a2);
#pragma unroll
        for (int i = 0; i < 13; ++i) v[i] = v1[i];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[13 + i] = v2[i];
      }
      // lane i now holds, for its channel 16 wv + i (rank 16 rt + i for z), the rows
      // r0 - 4 + e .. of each read, 4 per read
      float dyv[8], xv[12];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dyv[e] = bf(v[0], e);
        dyv[4 + e] = bf(v[1], e);
        xv[e] = bf(v[2], e);
        xv[4 + e] = bf(v[3], e);
        xv[8 + e] = bf(v[4], e);
      }
      if (partial) {
        const int tk = t0 + 32 * kk + 8 * q;
#pragma unroll
        for (int e = 0; e < 8; ++e) dyv[e] = tk + e < p.T ? dyv[e] : 0.f;
      }
      // ids of rows rb - 4 .. rb + 7, rb = 32 kk + 8 q (SG): g_k of token rb + e is kept
      // when row rb + e - k has the id of row rb + e
      int idv[12] = {};
      if constexpr (SG) {
        const int* ids =
            reinterpret_cast<const int*>(smem + F::S_OFF + (s % F::SN) * F::SSTAGE) + 32 * kk + 8 * q;
#pragma unroll
        for (int i = 0; i < 12; ++i) idv[i] = ids[i];
      }
      u16x8_t bz[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const u32x4 w = {v[5 + 2 * rt][0], v[5 + 2 * rt][1], v[6 + 2 * rt][0], v[6 + 2 * rt][1]};
        bz[rt] = __builtin_bit_cast(u16x8_t, w);
      }
#pragma unroll
      for (int k = 0; k < W; ++k) {
        float g[8];
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const bool keep = !SG || k == 0 || idv[4 + e - k] == idv[4 + e];
          g[e] = keep ? dyv[e] * xv[4 + e - k] : 0.f;
          sum += g[e];
        }
        db[k] += sum;
        const u32x4 w = {Cvt<ET>::pack2(g[0], g[1]), Cvt<ET>::pack2(g[2], g[3]), Cvt<ET>::pack2(g[4], g[5]),
                         Cvt<ET>::pack2(g[6], g[7])};
        const u16x8_t a16 = __builtin_bit_cast(u16x8_t, w);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) dU[k][rt] = mma32<ET>(a16, bz[rt], dU[k][rt]);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));

  // ---- partial sums of this (sequence, token range). Lane (n = j, q) holds rows 4q + i
  // (channels) of rank column n for each tap and rank tile. They are staged in LDS (the
  // stages are idle now) as rank rows of the slice's 64 W columns, so that each row goes
  // to memory as one contiguous run of 64 W floats; a pitch of 64 W + 1 floats spreads
  // the lanes' scattered writes over the banks. Up to 4 rank tiles at a time. ----
  const int range = b * p.nTr + tr;
  const int cw = c_base + 16 * wv;
  constexpr int COLS = 64 * W;
  constexpr int PITCH = COLS + 1;
  constexpr int TPC = gdu_tiles_per_chunk(W, KS);  // rank tiles per chunk
  static_assert(16 * TPC * PITCH * 4 <= F::BYTES, "staging fits the stages");
  if constexpr (FUSED) {
    static_assert(16 * TPC * PITCH * 4 <= F::T_OFF, "the staging leaves the dx tiles alone");
    __syncthreads();  // the dx role's last tile is complete before its final stores
  }
  // Head-wise generation (H consecutive channels share a group's columns, H <= 16): the H
  // channels of a group are summed here, in channel order, so that one partial per
  // (sequence, token range) and group column is written.
  const int H = p.H;
  const int hsh = __builtin_ctz(unsigned(H));
  float* st = reinterpret_cast<float*>(smem);
  float* pdu = p.part_dU + int64_t(range) * p.R * p.J + int64_t(c_base >> hsh) * W;
#pragma unroll
  for (int rt0 = 0; rt0 < RT; rt0 += TPC) {
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TPC; ++t)
#pragma unroll
      for (int k = 0; k < W; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) st[(16 * t + j) * PITCH + (16 * wv + 4 * q + i) * W + k] = dU[k][rt0 + t][i];
    __syncthreads();
    // rows 16 rt0 .. 16 (rt0 + TPC) - 1, 4 floats per thread and pass
    if (H == 1) {
      constexpr int PER_ROW = COLS / 4;
#pragma unroll 4
      for (int idx = tid; idx < 16 * TPC * PER_ROW; idx += 256) {
        const int r = idx / PER_ROW, c4 = (idx % PER_ROW) * 4;
        if (16 * rt0 + r >= p.R) continue;  // padding ranks: nothing to store
        const float* src = st + r * PITCH + c4;
        const f32x4_t v = {src[0], src[1], src[2], src[3]};
        *reinterpret_cast<f32x4_t*>(pdu + int64_t(16 * rt0 + r) * p.J + c4) = v;
      }
    } else {
      const int per_row = (COLS >> hsh) / 4;  // group columns of the slice, 4 at a time
      for (int idx = tid; idx < 16 * TPC * per_row; idx += 256) {
        const int r = idx / per_row, c4 = (idx % per_row) * 4;
        if (16 * rt0 + r >= p.R) continue;  // padding ranks: nothing to store
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int g = (c4 + e) / W, k = (c4 + e) % W;
          const float* src = st + r * PITCH + (g << hsh) * W + k;
          float v = src[0];
          for (int h = 1; h < H; ++h) v += src[h * W];
          o[e] = v;
        }
        *reinterpret_cast<f32x4_t*>(pdu + int64_t(16 * rt0 + r) * p.J + c4) = f32x4_t{o[0], o[1], o[2], o[3]};
      }
    }
  }
  if (p.part_db != nullptr) {
#pragma unroll
    for (int k = 0; k < W; ++k) {
      float v = db[k];
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      for (int m = 1; m < H; m <<= 1) v += __shfl_xor(v, m, 64);  // the group's lanes j
      if (q == 0 && (j & (H - 1)) == 0) p.part_db[int64_t(range) * p.J + int64_t((cw + j) >> hsh) * W + k] = v;
    }
  }
}

template <typename ET, int W, int KS, int SG, int ZB>
__global__ __launch_bounds__(256) void k_lowrank_bwd_gdu_fast(const LowRankParams p) {
  using F = BwdGduFast<KS, SG, ZB>;
  __shared__ __align__(16) unsigned char smem[F::BYTES];
  lowrank_gdu_role<ET, W, KS, SG, ZB, false, F>(p, smem, threadIdx.x, xcd_logical_block(blockIdx.x, gridDim.x));
}

// ---------------------------------------------------------------------------------
// Fused backward, k_lowrank_bwd_fast: dx and the g / dU / db partial sums in one pass over
// x, dy and z. A workgroup of 8 waves owns one (sequence, token range, 64-channel slice):
// waves 4..7 stage x (a ring of 4 steps), dy and z (3 stages each) by LDS DMA two steps
// ahead and form the partial sums (lowrank_gdu_role); waves 0..3 form dx from the same dy
// and z stages (lowrank_dx_role). Each role runs its own loop, so the two roles' registers
// are never live together; both loops run the range's steps plus dx's tail step with one
// barrier each, and the epilogues meet at the same barriers. dy and z are read from memory
// once instead of twice.
// ---------------------------------------------------------------------------------
template <typename ET, int W, int KS, int SG, int ZB>
__global__ __launch_bounds__(512) void k_lowrank_bwd_fast(const LowRankParams p) {
  using FL = BwdFused<KS, SG, ZB>;
  __shared__ __align__(16) unsigned char smem[FL::BYTES];
  const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
  if (__builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 8) == 0) {
    lowrank_dx_role<ET, W, KS, SG, ZB, true, FL>(p, smem, int(threadIdx.x) & 255, lb);
  } else {
    lowrank_gdu_role<ET, W, KS, SG, ZB, true, FL>(p, smem, int(threadIdx.x) & 255, lb);
  }
}

// W = 5 takes a second set of generation tiles (taps 4..7), whose registers fit up to 64
// ranks: at 128 ranks the fused backward would spill hundreds of registers. The backward's
// dx terms reach one lane back (W <= 5).
constexpr bool fast_width_ok(int w, int ks) { return w >= 1 && (w <= 4 || (w == 5 && ks <= 2)); }
// The forward reaches up to two row groups back: up to eight taps.
constexpr bool fwd_fast_width_ok(int w, int ks) { return w >= 1 && (w <= 4 || (w <= 8 && ks <= 2)); }

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

template <typename ET, int W, int KS>
hipError_t fwd_fast_try(const LowRankParams& p, int64_t blocks, hipStream_t s) {
  if constexpr (fwd_fast_rank_ok(KS) && fwd_fast_width_ok(W, KS)) {
    return fwd_fast_inst<ET, W, KS>(p, blocks, s);
  } else {
    return hipErrorInvalidValue;
  }
}

template <typename ET, int W>
hipError_t fwd_fast_ks(const LowRankParams& p, int64_t blocks, hipStream_t s) {
  switch ((p.R + 31) / 32) {
    case 1: return fwd_fast_try<ET, W, 1>(p, blocks, s);
    case 2: return fwd_fast_try<ET, W, 2>(p, blocks, s);
    case 4: return fwd_fast_try<ET, W, 4>(p, blocks, s);
    default: return hipErrorInvalidValue;
  }
}

template <int KS>
constexpr int fwd_fast_lds_ks() {
  if constexpr (fwd_fast_rank_ok(KS)) {
    return FwdFast<KS, LRF_NWV, LRF_XN, LRF_XD, LRF_ZN, LRF_ZD, 1>::BYTES;  // with the id stages
  } else {
    return 160 * 1024;
  }
}

int fwd_fast_lds(int ks) {
  return ks == 1 ? fwd_fast_lds_ks<1>() : ks == 2 ? fwd_fast_lds_ks<2>() : fwd_fast_lds_ks<4>();
}

}  // namespace

bool lowrank_fast_group_ok(int H) { return H == 1 || H == 2 || H == 4 || H == 8 || H == 16; }

// Ranks served by the fast kernels: R zero-padded to 32 KS with KS in {1, 2, 4} (R <= 64 or
// 97 <= R <= 128), z rows staged in 16-byte pieces (aligned rows, R % 8 == 0) or 4-byte
// pieces (4-byte aligned rows, R even).
bool lowrank_fast_rank_ok(const LowRankParams& p) {
  const int ks = (p.R + 31) / 32;
  return (ks == 1 || ks == 2 || ks == 4) && (z_pieces16(p) || (p.z4 != 0 && p.R % 2 == 0));
}

bool lowrank_fwd_fast_ok(const LowRankParams& p, int W, dynconv_dtype dt) {
  const int ks = (p.R + 31) / 32;
  return (dt == DYNCONV_BF16 || dt == DYNCONV_F16) && lowrank_fast_group_ok(p.H) && fwd_fast_width_ok(W, ks) &&
         lowrank_fast_rank_ok(p) && fwd_fast_rank_ok(ks) &&
         p.D % (16 * LRF_NWV) == 0 && p.act16 != 0 &&
         (int64_t(p.T) + kStep) * p.os1 * 2 < (int64_t(1) << 31) && int64_t(kStep) * p.xs1 < (int64_t(1) << 30) &&
         int64_t(kStep) * p.zs1 < (int64_t(1) << 30);
}

bool lowrank_seg_fast_ok(const LowRankParams& p) {
  // id rows contiguous and 16-byte aligned, whole 16-byte chunks of ids
  return p.seg != nullptr && p.ss1 == 1 && reinterpret_cast<uintptr_t>(p.seg) % 16 == 0 && p.ss0 % 4 == 0 &&
         p.T % 4 == 0 && p.T >= 4;
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

hipError_t launch_lowrank_fwd_fast(const LowRankParams& p, int W, dynconv_dtype dt, hipStream_t s) {
  const LowRankPlan pl = plan_lowrank_fwd_fast(p.B, p.T, p.D, (p.R + 31) / 32);
  LowRankParams q = p;
  q.cs0 = 0;
  q.nCsL = pl.nCs;
  q.nCs = pl.nCs;
  q.Ltok = pl.Ltok;
  q.nTr = pl.nTr;
  auto by_w = [&](auto tag) -> hipError_t {
    using ET = decltype(tag);
    switch (W) {
      case 1: return fwd_fast_ks<ET, 1>(q, pl.blocks, s);
      case 2: return fwd_fast_ks<ET, 2>(q, pl.blocks, s);
      case 3: return fwd_fast_ks<ET, 3>(q, pl.blocks, s);
      case 4: return fwd_fast_ks<ET, 4>(q, pl.blocks, s);
      case 5: return fwd_fast_ks<ET, 5>(q, pl.blocks, s);
      case 6: return fwd_fast_ks<ET, 6>(q, pl.blocks, s);
      case 7: return fwd_fast_ks<ET, 7>(q, pl.blocks, s);
      case 8: return fwd_fast_ks<ET, 8>(q, pl.blocks, s);
      default: return hipErrorInvalidValue;
    }
  };
  return dt == DYNCONV_F16 ? by_w(f16_t{}) : by_w(bf16_t{});
}

namespace {

// The standalone dx and g / dU / db kernels serve 128 ranks (the fused kernel's 8 waves
// would spill there).
template <typename ET, int W, int KS, int ZB>
hipError_t bwd_dx_zb(const LowRankParams& p, int64_t blocks, hipStream_t s) {
  if (p.seg != nullptr) {
    hipLaunchKernelGGL((k_lowrank_bwd_dx_fast<ET, W, KS, 1, ZB>), dim3(unsigned(blocks)), dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL((k_lowrank_bwd_dx_fast<ET, W, KS, 0, ZB>), dim3(unsigned(blocks)), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

template <typename ET, int W>
hipError_t bwd_dx_ks(const LowRankParams& p, int64_t blocks, hipStream_t s) {
  if constexpr (W <= 4) {
    if ((p.R + 31) / 32 == 4)
      return z_pieces16(p) ? bwd_dx_zb<ET, W, 4, 16>(p, blocks, s) : bwd_dx_zb<ET, W, 4, 4>(p, blocks, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool lowrank_bwd_fast_shape_ok(const LowRankParams& p, int W, dynconv_dtype dt) {
  return (dt == DYNCONV_BF16 || dt == DYNCONV_F16) && lowrank_fast_group_ok(p.H) &&
         fast_width_ok(W, (p.R + 31) / 32) && lowrank_fast_rank_ok(p) && p.D % 64 == 0 && p.act16 != 0 &&
         (int64_t(p.T) + kStep) * p.os1 * 2 < (int64_t(1) << 31) &&
         int64_t(kStep) * p.dys1 < (int64_t(1) << 30) && int64_t(kStep) * p.zs1 < (int64_t(1) << 30) &&
         int64_t(kStep) * p.xs1 < (int64_t(1) << 30);
}

namespace {

template <typename ET, int W, int KS, int ZB>
hipError_t bwd_gdu_zb(const LowRankParams& p, int64_t blocks, hipStream_t s) {
  if (p.seg != nullptr) {
    hipLaunchKernelGGL((k_lowrank_bwd_gdu_fast<ET, W, KS, 1, ZB>), dim3(unsigned(blocks)), dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL((k_lowrank_bwd_gdu_fast<ET, W, KS, 0, ZB>), dim3(unsigned(blocks)), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

template <typename ET, int W>
hipError_t bwd_gdu_ks(const LowRankParams& p, int64_t blocks, hipStream_t s) {
  if constexpr (W <= 4) {
    if ((p.R + 31) / 32 == 4)
      return z_pieces16(p) ? bwd_gdu_zb<ET, W, 4, 16>(p, blocks, s) : bwd_gdu_zb<ET, W, 4, 4>(p, blocks, s);
  }
  return hipErrorInvalidValue;
}

template <typename ET, int W, int KS, int ZB>
hipError_t bwd_fused_zb(const LowRankParams& p, int64_t blocks, hipStream_t s) {
  if (p.seg != nullptr) {
    hipLaunchKernelGGL((k_lowrank_bwd_fast<ET, W, KS, 1, ZB>), dim3(unsigned(blocks)), dim3(512), 0, s, p);
  } else {
    hipLaunchKernelGGL((k_lowrank_bwd_fast<ET, W, KS, 0, ZB>), dim3(unsigned(blocks)), dim3(512), 0, s, p);
  }
  return hipGetLastError();
}

template <typename ET, int W>
hipError_t bwd_fused_ks(const LowRankParams& p, int64_t blocks, hipStream_t s) {
  const bool z16 = z_pieces16(p);
  switch ((p.R + 31) / 32) {
    case 1: return z16 ? bwd_fused_zb<ET, W, 1, 16>(p, blocks, s) : bwd_fused_zb<ET, W, 1, 4>(p, blocks, s);
    case 2: return z16 ? bwd_fused_zb<ET, W, 2, 16>(p, blocks, s) : bwd_fused_zb<ET, W, 2, 4>(p, blocks, s);
    default: return hipErrorInvalidValue;
  }
}

// dx by k_lowrank_bwd_dx_fast over its own token ranges (about 512 workgroups of 4 waves),
// then the g / dU / db partial sums by k_lowrank_bwd_gdu_fast over the planned ranges.
template <typename ET, int W>
hipError_t bwd_split(const LowRankParams& p, hipStream_t s) {
  const int nCs = p.D / 64;
  int64_t per_seq = (512 + int64_t(p.B) * nCs - 1) / (int64_t(p.B) * nCs);
  const int64_t max_ranges = (p.T + kStep - 1) / kStep;
  if (per_seq > max_ranges) per_seq = max_ranges;
  if (per_seq < 1) per_seq = 1;
  int64_t L = (p.T + per_seq - 1) / per_seq;
  L = (L + kStep - 1) / kStep * kStep;
  LowRankParams q = p;
  q.cs0 = 0;
  q.nCsL = nCs;
  q.nCs = nCs;
  q.Ltok = int(L);
  q.nTr = int((p.T + L - 1) / L);
  hipError_t e = bwd_dx_ks<ET, W>(q, int64_t(p.B) * q.nTr * nCs, s);
  if (e != hipSuccess) return e;
  LowRankParams r = p;
  r.cs0 = 0;
  r.nCsL = nCs;
  return bwd_gdu_ks<ET, W>(r, int64_t(p.B) * p.nTr * nCs, s);
}

}  // namespace

bool lowrank_bwd_fast(const LowRankParams& p, int W, dynconv_dtype dt) {
  return (p.seg == nullptr || lowrank_seg_fast_ok(p)) && lowrank_bwd_fast_shape_ok(p, W, dt);
}

hipError_t launch_lowrank_bwd_fused(const LowRankParams& p, int W, dynconv_dtype dt, hipStream_t s) {
  // up to 64 ranks: one workgroup of 8 waves per (sequence, planned token range, 64-channel
  // slice) running both roles; 128 ranks: the two roles as kernels of their own (4-wave
  // workgroups, whose registers hold the g / dU / db role's 128 accumulators per lane)
  LowRankParams q = p;
  q.cs0 = 0;
  q.nCsL = p.D / 64;
  q.nCs = q.nCsL;
  const int64_t blocks = int64_t(p.B) * p.nTr * q.nCsL;
  const bool split = (p.R + 31) / 32 == 4;
  auto by_w = [&](auto tag) -> hipError_t {
    using ET = decltype(tag);
    switch (W) {
      case 1: return split ? bwd_split<ET, 1>(p, s) : bwd_fused_ks<ET, 1>(q, blocks, s);
      case 2: return split ? bwd_split<ET, 2>(p, s) : bwd_fused_ks<ET, 2>(q, blocks, s);
      case 3: return split ? bwd_split<ET, 3>(p, s) : bwd_fused_ks<ET, 3>(q, blocks, s);
      case 4: return split ? bwd_split<ET, 4>(p, s) : bwd_fused_ks<ET, 4>(q, blocks, s);
      case 5: return split ? hipErrorInvalidValue : bwd_fused_ks<ET, 5>(q, blocks, s);
      default: return hipErrorInvalidValue;
    }
  };
  return dt == DYNCONV_F16 ? by_w(f16_t{}) : by_w(bf16_t{});
}

}  // namespace dynconv
