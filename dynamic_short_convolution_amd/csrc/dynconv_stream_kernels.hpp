// Streaming kernels (materialised / static filters), instantiated once per storage type
// by dynconv_stream_{f32,bf16,f16}.hip so that the three compile in parallel.
#pragma once

// Streaming kernels of the dynamic short convolution with materialised (per-token) or
// static filters, for gfx950.
//
// Operation ("Dynamic Short Convolutions Improve Transformers", reading note, section
// "Parameterization", eq. 1-3, head-wise parameterisation):
//   y[b,t,d] = x[b,t,d] + sum_{k<W} w[b,t,d/H,k] * x[b,t-k,d],  x[b,t<0,d] = 0.
// The page's kernel section states the memory contract these kernels keep: every input
// is read from HBM once and every output written once; the filter tensor (W times the
// activations when H = 1) dominates the traffic.
//
// Design: one wave owns a slice of 64*VEC channels of one sequence over a run of L
// tokens and sweeps time. Each lane keeps its channels' last W-1 inputs (forward) or
// its pending dx sums (backward) in registers, so the time halo costs no LDS traffic
// and only W-1 extra rows per chunk. Every global access of a wave is a contiguous,
// coalesced run: x/y as 4 or 16 bytes per lane, the filter taps of the lane's channels
// as VEC*W contiguous elements (H = 1) or one broadcast group (H > 1). Loads of U
// consecutive tokens are issued before any of them is used, with U sized so that about
// DYNCONV_{FWD,BWD}_INFLIGHT bytes of loads per lane are in flight; the data is streamed with
// non-temporal hints.
#include <cmath>
#include <type_traits>

#include "dynconv_common.hpp"
#include "dynconv_internal.hpp"

// Tuning, measured on MI355X at the pages' model shapes (B8 T4096 D2048 and B4 T8192
// D3072, W = 4): the forward streams best with plain stores and about 128 bytes of loads
// in flight per lane (unroll 4 for the per-channel form) at 8 waves per CU; the per-channel
// backward with non-temporal stores (up to W = 5), unroll 2 and 16 waves per CU; the head-wise and
// static backward with plain stores at 12 and 8 waves per CU; the static forms prefer
// neighbouring workgroups to walk channels rather than time. Each constant can be
// overridden at build time for a sweep.
#ifndef DYNCONV_FWD_INFLIGHT
#define DYNCONV_FWD_INFLIGHT 128
#endif
#ifndef DYNCONV_BWD_INFLIGHT
#define DYNCONV_BWD_INFLIGHT 64
#endif
#ifndef DYNCONV_FWD_UNROLL  // > 0 overrides the unroll derived from the bytes in flight
#define DYNCONV_FWD_UNROLL 0
#endif
#ifndef DYNCONV_BWD_UNROLL
#define DYNCONV_BWD_UNROLL 0
#endif
// The head-wise and static backward load the next batch of tokens before using the
// current one (measured: H = 16 89.8 -> 86.9 us, static W = 3 103.7 -> 99.6 us); the
// per-channel backward, with 16 waves per CU, is faster without (271 vs 276 us).
#ifndef DYNCONV_BWD_PIPELINE
#define DYNCONV_BWD_PIPELINE 1
#endif

namespace dynconv {

namespace {

// Every streamed input is read once, so loads carry the non-temporal hint.
__device__ __forceinline__ uint32_t ld32(const uint32_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ uint16_t ld16(const uint16_t* p) { return __builtin_nontemporal_load(p); }
template <bool NT>
__device__ __forceinline__ void st32(uint32_t* p, uint32_t v) {
  if constexpr (NT) {
    __builtin_nontemporal_store(v, p);
  } else {
    *p = v;
  }
}
template <bool NT>
__device__ __forceinline__ void st16(uint16_t* p, uint16_t v) {
  if constexpr (NT) {
    __builtin_nontemporal_store(v, p);
  } else {
    *p = v;
  }
}

// N contiguous elements at a 4-byte aligned address, kept as raw 32-bit words until
// they are used (the compiler fuses the word loads into dwordx2/x3/x4).
template <typename ET, int N>
struct Words {
  static_assert((N * sizeof(ET)) % 4 == 0, "a word vector holds whole 32-bit words");
  static constexpr int ND = int(N * sizeof(ET) / 4);
  uint32_t u[ND];
  __device__ __forceinline__ void load(const ET* p) {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
    for (int i = 0; i < ND; ++i) u[i] = ld32(q + i);
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < ND; ++i) u[i] = 0u;
  }
  __device__ __forceinline__ float at(int i) const {
    if constexpr (sizeof(ET) == 2) {
      return (i & 1) ? Cvt<ET>::hi(u[i >> 1]) : Cvt<ET>::lo(u[i >> 1]);
    } else {
      return __uint_as_float(u[i]);
    }
  }
};

// N contiguous elements with only element alignment (16-bit filter groups of odd W).
template <typename ET, int N>
struct Halves {
  uint16_t h[N];
  __device__ __forceinline__ void load(const ET* p) {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(p);
#pragma unroll
    for (int i = 0; i < N; ++i) h[i] = ld16(q + i);
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < N; ++i) h[i] = 0;
  }
  __device__ __forceinline__ float at(int i) const { return Cvt<ET>::of_bits(h[i]); }
};

template <bool NT, typename ET, int N>
__device__ __forceinline__ void store_words(ET* p, const float (&v)[N]) {
  uint32_t* q = reinterpret_cast<uint32_t*>(p);
  if constexpr (sizeof(ET) == 2) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) st32<NT>(q + i, Cvt<ET>::pack2(v[2 * i], v[2 * i + 1]));
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) st32<NT>(q + i, __float_as_uint(v[i]));
  }
}

// N elements at element alignment; words when N elements fill whole 32-bit words and the
// caller guarantees 4-byte alignment (WORDS), 16-bit stores otherwise.
template <bool NT, bool WORDS, typename ET, int N>
__device__ __forceinline__ void store_elems(ET* p, const float (&v)[N]) {
  if constexpr (sizeof(ET) == 2 && !WORDS) {
    uint16_t* q = reinterpret_cast<uint16_t*>(p);
#pragma unroll
    for (int i = 0; i < N; ++i) st16<NT>(q + i, Cvt<ET>::bits(v[i]));
  } else {
    store_words<NT, ET, N>(p, v);
  }
}

// The lane's VEC channels of one activation row: 32-bit words, or one 16-bit element for
// a lane of a single channel (head-wise groups of odd H in 16-bit storage).
template <typename ET, int VEC>
using ActRaw = typename std::conditional<(VEC * sizeof(ET)) % 4 == 0, Words<ET, VEC>, Halves<ET, VEC>>::type;

template <bool NT, typename ET, int VEC>
__device__ __forceinline__ void store_act(ET* p, const float (&v)[VEC]) {
  store_elems<NT, (VEC * sizeof(ET)) % 4 == 0, ET, VEC>(p, v);
}

// Raw taps of one token for one lane: the VEC*W taps of its channels (H = 1) or the W
// taps of its group (H > 1). Groups of whole 32-bit words are 4-byte aligned (the C ABI
// checks it), odd bf16 groups are read as 16-bit halves.
template <typename ET, int W, int VEC, bool PERCH>
struct TapsRaw {
  static constexpr bool group_words = (W * sizeof(ET)) % 4 == 0;
  using type = typename std::conditional<PERCH, Words<ET, VEC * W>,
                                         typename std::conditional<group_words, Words<ET, W>,
                                                                   Halves<ET, W>>::type>::type;
  static constexpr int bytes = PERCH ? VEC * W * int(sizeof(ET)) : W * int(sizeof(ET));
};

template <typename T>
__device__ __forceinline__ float tap_of(const T& r, int v, int k, int W, bool perch) {
  return r.at(perch ? v * W + k : k);
}

constexpr int pow2_floor(int v) { return v >= 16 ? 16 : v >= 8 ? 8 : v >= 4 ? 4 : v >= 2 ? 2 : 1; }
constexpr int clamp_unroll(int v) { return v < 2 ? 2 : (v > 16 ? 16 : v); }

struct WaveTile {
  int b, c0, t0, t1, chunk;
  bool valid;
};

// CHANNEL_FASTEST: consecutive workgroups take neighbouring channel blocks of the same
// tokens (used by the static forms); otherwise consecutive time chunks of a channel block.
// XCD: consecutive logical workgroups run on the same XCD (the backward); without it the
// hardware's round-robin spreads consecutive workgroups over the 8 XCDs, which measured
// faster for the forward (per-channel 136 -> 132 us at B8 T4096 D2048 W4; the backward
// is unchanged or slightly slower without it).
template <bool CHANNEL_FASTEST, bool XCD>
__device__ __forceinline__ WaveTile wave_tile(const StreamParams& p, int vec) {
  WaveTile wt;
  const int lane = threadIdx.x & (kWaveSize - 1);
  const int wv = threadIdx.x / kWaveSize;
  uint32_t lb = XCD ? xcd_logical_block(blockIdx.x, gridDim.x) : blockIdx.x;
  int tb, db;
  if constexpr (CHANNEL_FASTEST) {
    db = lb % p.nDb;
    lb /= p.nDb;
    tb = lb % p.nTb;
    wt.b = lb / p.nTb;
  } else {
    tb = lb % p.nTb;
    lb /= p.nTb;
    db = lb % p.nDb;
    wt.b = lb / p.nDb;
  }
  const int dsl = db * p.WD + (wv % p.WD);
  const int tch = tb * p.WT + (wv / p.WD);
  // a wave's slice is lpw lanes of vec channels (lanes past lpw idle, see lanes_in_use)
  wt.c0 = (dsl * p.lpw + lane) * vec;
  wt.t0 = tch * p.L;
  wt.t1 = min(p.T, wt.t0 + p.L);
  wt.chunk = wt.b * p.nTw + tch;
  wt.valid = dsl < p.nDw && tch < p.nTw && lane < p.lpw && wt.c0 < p.D;
  return wt;
}

// Segment ids of packed sequences (several documents in one row): tap k of token t is
// present only when token t-k carries the id of token t. Every lane of a wave is at the
// same token, so the ids are wave-uniform and read through the scalar cache (the sequence
// and token indices are marked uniform here only: doing it for the wave index of every
// kernel slowed the head-wise forward, 75 -> 83 us at H = 4); before the step at token t,
// id[j] holds the id of token t-1-j, the step shifts in the id of t.
typedef const __attribute__((address_space(4))) int32_t* seg_ptr;

template <int W, bool SEG>
struct Segs {
  int id[W > 1 ? W - 1 : 1];
  seg_ptr base;
  int64_t s1;
  __device__ __forceinline__ void init(const StreamParams& p, int b, int t0) {
    if constexpr (SEG) {
      base = (seg_ptr)(p.seg + int64_t(__builtin_amdgcn_readfirstlane(b)) * p.ss0);
      s1 = p.ss1;
#pragma unroll
      for (int k = 1; k < W; ++k) id[k - 1] = t0 - k >= 0 ? load(t0 - k) : INT32_MIN;
    }
  }
  __device__ __forceinline__ int load(int t) const {
    if constexpr (SEG) return base[int64_t(__builtin_amdgcn_readfirstlane(t)) * s1];
    return 0;
  }
  // Presence of taps k = 1..W-1 of the token with id `cur` (m[0] is always true).
  __device__ __forceinline__ void mask(int cur, bool (&m)[W]) const {
    m[0] = true;
#pragma unroll
    for (int k = 1; k < W; ++k) m[k] = !SEG || id[k - 1] == cur;
  }
  __device__ __forceinline__ void push(int cur) {
    if constexpr (SEG && W > 1) {
#pragma unroll
      for (int j = W - 2; j >= 1; --j) id[j] = id[j - 1];
      id[0] = cur;
    }
  }
};

// ---------------------------------------------------------------------------------
// Forward: y_t = x_t + sum_k w_k^(t) x_{t-k}
// ---------------------------------------------------------------------------------
// The forward's grid holds about 2 waves per SIMD (8 per CU). For the per-channel form the
// compiler may spend registers on loads in flight rather than on occupancy it would never
// get: chasing 8 waves per SIMD it had serialised the filter loads (135 -> 209 us at
// B8 T4096 D2048 W4; W = 8 296 -> 262 us with the cap). The head-wise and static forms run
// faster without it (H = 4: 75 vs 83 us).
constexpr int fwd_max_waves_per_simd(bool perch, bool is_static) { return perch && !is_static ? 4 : 8; }

template <typename ET, int W, int VEC, bool PERCH, bool STATIC, bool SEG>
__global__ __launch_bounds__(kBlockThreads) __attribute__((amdgpu_waves_per_eu(
    1, fwd_max_waves_per_simd(PERCH, STATIC)))) void k_stream_fwd(const StreamParams p) {
  using XR = ActRaw<ET, VEC>;
  using TR = typename TapsRaw<ET, W, VEC, PERCH>::type;
  constexpr int NC = PERCH ? VEC : 1;
  constexpr int LB = VEC * int(sizeof(ET)) + (STATIC ? 0 : TapsRaw<ET, W, VEC, PERCH>::bytes);
  // (more than 32 bytes of loads per token, i.e. per-channel W = 8: 4 tokens, 305 -> 296 us)
  constexpr int U = DYNCONV_FWD_UNROLL > 0 ? DYNCONV_FWD_UNROLL
                    : LB > 32              ? 4
                                           : clamp_unroll(pow2_floor(DYNCONV_FWD_INFLIGHT / LB));
  constexpr bool NT = false;

  const WaveTile wt = wave_tile<STATIC, false>(p, VEC);
  if (!wt.valid) return;
  const int g = PERCH ? wt.c0 : wt.c0 / p.H;
  const ET* xb = static_cast<const ET*>(p.x) + wt.b * p.xs0 + wt.c0;
  ET* yb = static_cast<ET*>(p.out) + wt.b * p.os0 + wt.c0;
  const ET* wb = static_cast<const ET*>(p.w) + (STATIC ? 0 : wt.b * p.ws0) + int64_t(g) * W;

  // Window of inputs. Before the step at token t, xh[j] holds x_{t-1-j} (j < W-1); the
  // step shifts it by one and inserts x_t, after which xh[k] = x_{t-k}.
  float xh[W][VEC];
#pragma unroll
  for (int k = 1; k < W; ++k) {
    const int t = wt.t0 - k;
    XR r;
    if (t >= 0) {
      r.load(xb + t * p.xs1);
    } else {
      r.zero();
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) xh[k - 1][v] = r.at(v);
  }
  float wst[NC][W];
  if constexpr (STATIC) {
    TR r;
    r.load(wb);
#pragma unroll
    for (int v = 0; v < NC; ++v)
#pragma unroll
      for (int k = 0; k < W; ++k) wst[v][k] = tap_of(r, v, k, W, PERCH);
  }
  Segs<W, SEG> sg;
  sg.init(p, wt.b, wt.t0);
  // optional convolution bias of the lane's channels (zero without one)
  float cb[VEC];
  {
    XR r;
    if (p.cbias != nullptr) {
      r.load(static_cast<const ET*>(p.cbias) + wt.c0);
    } else {
      r.zero();
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) cb[v] = r.at(v);
  }

  auto step = [&](int t, const XR& xr, const TR& wr, int sid) {
    bool m[W];
    sg.mask(sid, m);
    sg.push(sid);
#pragma unroll
    for (int k = W - 1; k >= 1; --k)
#pragma unroll
      for (int v = 0; v < VEC; ++v) xh[k][v] = xh[k - 1][v];
#pragma unroll
    for (int v = 0; v < VEC; ++v) xh[0][v] = xr.at(v);
    float yv[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      float acc = xh[0][v] + cb[v];
#pragma unroll
      for (int k = 0; k < W; ++k) {
        const float f = STATIC ? wst[PERCH ? v : 0][k] : tap_of(wr, v, k, W, PERCH);
        acc = fmaf(m[k] ? f : 0.f, xh[k][v], acc);
      }
      yv[v] = acc;
    }
    store_act<NT, ET, VEC>(yb + t * p.os1, yv);
  };

  int t = wt.t0;
  for (; t + U <= wt.t1; t += U) {
    XR xr[U];
    TR wr[U];
    int sid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      xr[u].load(xb + (t + u) * p.xs1);
      if constexpr (!STATIC) wr[u].load(wb + (t + u) * p.ws1);
      sid[u] = sg.load(t + u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) step(t + u, xr[u], wr[u], sid[u]);
  }
  for (; t < wt.t1; ++t) {
    XR xr;
    TR wr;
    xr.load(xb + t * p.xs1);
    if constexpr (!STATIC) wr.load(wb + t * p.ws1);
    step(t, xr, wr, sg.load(t));
  }
}

// ---------------------------------------------------------------------------------
// Backward. A forward sweep over t scatters w_k^(t) dy_t into dx_{t-k}; dx_s is final
// once step s + W - 1 is done, so each lane keeps W-1 pending sums. The chunk's last
// W-1 dx rows need the next chunk's first W-1 rows of w and dy (the future halo).
//   dx_s = dy_s + sum_k w_k^(s+k) dy_{s+k}
//   dw_t[g,k] = sum_{d in g} dy_t[d] x_{t-k}[d]
// ---------------------------------------------------------------------------------
// Sums of the N values v[k] over the `lanes` consecutive lanes of a group; `pos` is the
// lane's place in it. A group never straddles a wave (lanes_in_use). Groups of 2^n lanes
// use a butterfly, every lane ending with the sums: after the rounds below 2^r each lane
// holds its aligned 2^r-lane sum, so any partner in the other half of the aligned 2^(r+1)
// lanes completes the next one. Within 16 lanes the partners are DPP operand modifiers
// (lane ^ 1, lane ^ 2, the mirror within 8, the mirror within 16: no LDS traffic); wider
// rounds use ds_bpermute. Other group sizes use a suffix scan whose first lane (pos 0) ends
// with the sums: after the round with offset o, lane pos holds the sum over pos ..
// min(pos + 2o, lanes) - 1 (DPP shifts of the whole wave measured slower than ds_bpermute
// there). Each round moves all N values at once, so their exchanges are in flight together
// and one-lane groups pay a single branch. Backward at B8 T4096 W4 against one value per
// call with ds_bpermute rounds: H = 128 99.9 -> 78.6 us, H = 32 87.8 -> 81.9, H = 16 86.6 ->
// 86.4 (D = 2048); H = 12 226 -> 184, H = 96 181 -> 142 (D = 3072).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuadSwap1 = 0xB1;    // quad_perm [1, 0, 3, 2]: lane ^ 1
constexpr int kDppQuadSwap2 = 0x4E;    // quad_perm [2, 3, 0, 1]: lane ^ 2
constexpr int kDppHalfMirror = 0x141;  // lane 7 - i within 8 lanes
constexpr int kDppMirror = 0x140;      // lane 15 - i within 16 lanes

template <int N>
__device__ __forceinline__ void group_sums(float (&v)[N], int lanes, int pos) {
  if (lanes == 1) return;
  if ((lanes & (lanes - 1)) == 0) {
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] += dpp_mov<kDppQuadSwap1>(v[k]);
    if (lanes > 2) {
#pragma unroll
      for (int k = 0; k < N; ++k) v[k] += dpp_mov<kDppQuadSwap2>(v[k]);
      if (lanes > 4) {
#pragma unroll
        for (int k = 0; k < N; ++k) v[k] += dpp_mov<kDppHalfMirror>(v[k]);
        if (lanes > 8) {
#pragma unroll
          for (int k = 0; k < N; ++k) v[k] += dpp_mov<kDppMirror>(v[k]);
          for (int m = 16; m < lanes; m <<= 1) {
#pragma unroll
            for (int k = 0; k < N; ++k) v[k] += __shfl_xor(v[k], m, kWaveSize);
          }
        }
      }
    }
  } else {
    for (int o = 1; o < lanes; o <<= 1) {
      const bool in = pos + o < lanes;
#pragma unroll
      for (int k = 0; k < N; ++k) {
        const float u = __shfl_down(v[k], o, kWaveSize);
        if (in) v[k] += u;
      }
    }
  }
}

// ALL: both dx and dw are wanted, known at compile time (static filters only: their
// runtime output tests had split every batch of loads into branches, 91.5 -> 79.1 us at
// B8 T4096 D2048 W3; the other forms measured no gain).
// CB: the convolution-bias gradient is wanted (sums of dy per chunk; a separate variant so
// that the sweep without it carries no extra work).
template <typename ET, int W, int VEC, bool PERCH, bool STATIC, bool ALL, bool SEG, bool CB>
__global__ __launch_bounds__(kBlockThreads) void k_stream_bwd(const StreamParams p) {
  using XR = ActRaw<ET, VEC>;
  using TR = typename TapsRaw<ET, W, VEC, PERCH>::type;
  constexpr int WM = W > 1 ? W - 1 : 1;
  constexpr int NC = PERCH ? VEC : 1;
  constexpr int LB = 2 * VEC * int(sizeof(ET)) + (STATIC ? 0 : TapsRaw<ET, W, VEC, PERCH>::bytes);
  constexpr int U = DYNCONV_BWD_UNROLL > 0 ? DYNCONV_BWD_UNROLL : clamp_unroll(pow2_floor(DYNCONV_BWD_INFLIGHT / LB));
  // Non-temporal stores up to W = 5; wider filters store plain (their taps take several
  // store instructions per lane). Measured as back-to-back forward + backward steps at B8
  // T4096 D2048 bf16 (per-launch timings after a cache flush leave a kernel's last dirty
  // lines to the untimed flush and mislead here): non-temporal vs plain 401.5 vs 424.8 us
  // at W = 4, 571.7 vs 581.2 at W = 5, 702.0 vs 678.4 at W = 6, 772.5 vs 761.1 at W = 7,
  // 832.5 vs 800.3 at W = 8.
  constexpr bool NT = PERCH && !STATIC && W <= 5;

  const WaveTile wt = wave_tile<STATIC, true>(p, VEC);
  // Group reductions need every lane of a group; a whole group is either valid or not
  // (H divides D and groups are lane-aligned), so invalid lanes can leave now.
  if (!wt.valid) return;
  const int lane = threadIdx.x & (kWaveSize - 1);
  const int lanes_per_group = PERCH ? 1 : p.lpg;
  const int group_pos = PERCH ? 0 : lane % lanes_per_group;
  const bool group_lead = group_pos == 0;
  const int g = PERCH ? wt.c0 : wt.c0 / p.H;
  const bool want_dx = ALL || p.out != nullptr;
  const bool want_dw = ALL || (STATIC ? (p.partial != nullptr) : (p.dw != nullptr));

  const ET* xb = static_cast<const ET*>(p.x) + wt.b * p.xs0 + wt.c0;
  const ET* dyb = static_cast<const ET*>(p.dy) + wt.b * p.dys0 + wt.c0;
  const ET* wb = static_cast<const ET*>(p.w) + (STATIC ? 0 : wt.b * p.ws0) + int64_t(g) * W;
  ET* dxb = want_dx ? static_cast<ET*>(p.out) + wt.b * p.os0 + wt.c0 : nullptr;
  ET* dwb = (!STATIC && want_dw) ? static_cast<ET*>(p.dw) + wt.b * p.dws0 + int64_t(g) * W : nullptr;

  float xh[WM][VEC];   // x_{t-1} .. x_{t-W+1}
  float acc[WM][VEC];  // pending dx sums for s = t-1 .. t-W+1
#pragma unroll
  for (int j = 0; j < WM; ++j)
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      acc[j][v] = 0.f;
      xh[j][v] = 0.f;
    }
  if (want_dw) {
#pragma unroll
    for (int k = 1; k < W; ++k) {
      const int t = wt.t0 - k;
      if (t >= 0) {
        XR r;
        r.load(xb + t * p.xs1);
#pragma unroll
        for (int v = 0; v < VEC; ++v) xh[k - 1][v] = r.at(v);
      }
    }
  }
  Segs<W, SEG> sg;
  sg.init(p, wt.b, wt.t0);
  float sdy[VEC];  // sums of dy over the chunk's tokens: the convolution-bias gradient
#pragma unroll
  for (int v = 0; v < VEC; ++v) sdy[v] = 0.f;
  float wst[NC][W];
  float sdw[NC][W];  // static: per-lane partial sums of dw over the chunk
  if constexpr (STATIC) {
    TR r;
    r.load(wb);
#pragma unroll
    for (int v = 0; v < NC; ++v)
#pragma unroll
      for (int k = 0; k < W; ++k) {
        wst[v][k] = tap_of(r, v, k, W, PERCH);
        sdw[v][k] = 0.f;
      }
  }

  // One step at token t. MAIN: t inside the chunk (x is read, dw produced); HAVE: t < T.
  auto step = [&](int t, bool main, bool have, const XR& dyr, const TR& wr, const XR& xr, int sid) {
    bool m[W];
    sg.mask(sid, m);
    sg.push(sid);
    float dyv[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) dyv[v] = have ? dyr.at(v) : 0.f;
    if constexpr (CB) {
      if (main) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) sdy[v] += dyv[v];
      }
    }
    if (main && want_dw) {
      float d[W][VEC];
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        d[0][v] = dyv[v] * xr.at(v);
#pragma unroll
        for (int k = 1; k < W; ++k) d[k][v] = m[k] ? dyv[v] * xh[k - 1][v] : 0.f;
      }
      if constexpr (PERCH) {
        if constexpr (STATIC) {
#pragma unroll
          for (int v = 0; v < VEC; ++v)
#pragma unroll
            for (int k = 0; k < W; ++k) sdw[v][k] += d[k][v];
        } else {
          float o[VEC * W];
#pragma unroll
          for (int v = 0; v < VEC; ++v)
#pragma unroll
            for (int k = 0; k < W; ++k) o[v * W + k] = d[k][v];
          store_words<NT, ET, VEC * W>(dwb + t * p.dws1, o);
        }
      } else {
        float s[W];
#pragma unroll
        for (int k = 0; k < W; ++k) {
          float a = 0.f;
#pragma unroll
          for (int v = 0; v < VEC; ++v) a += d[k][v];
          s[k] = a;
        }
        if constexpr (STATIC) {
#pragma unroll
          for (int k = 0; k < W; ++k) sdw[0][k] += s[k];
        } else {
          group_sums<W>(s, lanes_per_group, group_pos);
          if (group_lead) store_elems<NT, TapsRaw<ET, W, VEC, PERCH>::group_words, ET, W>(dwb + t * p.dws1, s);
        }
      }
    }
    if (want_dx) {
      float nacc[VEC];
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        const float f0 = STATIC ? wst[PERCH ? v : 0][0] : (have ? tap_of(wr, v, 0, W, PERCH) : 0.f);
        nacc[v] = fmaf(f0, dyv[v], dyv[v]);
      }
#pragma unroll
      for (int j = 1; j < W; ++j)
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          const float fj = STATIC ? wst[PERCH ? v : 0][j] : (have ? tap_of(wr, v, j, W, PERCH) : 0.f);
          acc[j - 1][v] = fmaf(m[j] ? fj : 0.f, dyv[v], acc[j - 1][v]);
        }
      const int s = t - (W - 1);
      if (s >= wt.t0 && s < wt.t1) {
        if constexpr (W == 1) {
          store_act<NT, ET, VEC>(dxb + s * p.os1, nacc);
        } else {
          store_act<NT, ET, VEC>(dxb + s * p.os1, acc[W - 2]);
        }
      }
#pragma unroll
      for (int j = WM - 1; j >= 1; --j)
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[j][v] = acc[j - 1][v];
      if constexpr (W > 1) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[0][v] = nacc[v];
      }
    }
    if (main && want_dw) {
#pragma unroll
      for (int j = WM - 1; j >= 1; --j)
#pragma unroll
        for (int v = 0; v < VEC; ++v) xh[j][v] = xh[j - 1][v];
#pragma unroll
      for (int v = 0; v < VEC; ++v) xh[0][v] = xr.at(v);
    }
  };

  // Loads of a batch of U tokens; when pipelined, the next batch is loaded before the
  // current one is used, so each wave keeps two batches in flight.
  struct Batch {
    XR x[U], dy[U];
    TR w[U];
    int sid[U];
  };
  auto load_batch = [&](Batch& bt, int tb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      bt.sid[u] = sg.load(tb + u);
      bt.dy[u].load(dyb + (tb + u) * p.dys1);
      if (want_dw) {
        bt.x[u].load(xb + (tb + u) * p.xs1);
      } else {
        bt.x[u].zero();
      }
      if constexpr (!STATIC) {
        if (want_dx) {
          bt.w[u].load(wb + (tb + u) * p.ws1);
        } else {
          bt.w[u].zero();
        }
      }
    }
  };
  auto run_batch = [&](const Batch& bt, int tb) {
#pragma unroll
    for (int u = 0; u < U; ++u) step(tb + u, true, true, bt.dy[u], bt.w[u], bt.x[u], bt.sid[u]);
  };
  // The future halo: the W-1 tokens after the chunk complete its last dx rows. Their
  // loads are issued first, so that they are in by the end of the chunk.
  XR hx[WM], hdy[WM];
  TR hw[WM];
  int hsid[WM];
  if (want_dx) {
#pragma unroll
    for (int e = 0; e < W - 1; ++e) {
      const int tt = wt.t1 + e;
      hx[e].zero();
      hsid[e] = INT32_MIN;
      if (tt < p.T) {
        hsid[e] = sg.load(tt);
        hdy[e].load(dyb + tt * p.dys1);
        if constexpr (!STATIC) hw[e].load(wb + tt * p.ws1);
      } else {
        hdy[e].zero();
        if constexpr (!STATIC) hw[e].zero();
      }
    }
  }
  int t = wt.t0;
  // (per-channel: only the widest filters gain, W = 8 713 -> 659 us; W = 4 loses 276 -> 279)
  if constexpr (DYNCONV_BWD_PIPELINE && (!PERCH || STATIC || W >= 6)) {
    Batch b0, b1;
    if (t + U <= wt.t1) load_batch(b0, t);
    while (t + U <= wt.t1) {
      if (t + 2 * U <= wt.t1) load_batch(b1, t + U);
      run_batch(b0, t);
      t += U;
      if (t + U > wt.t1) break;
      if (t + 2 * U <= wt.t1) load_batch(b0, t + U);
      run_batch(b1, t);
      t += U;
    }
  } else {
    for (; t + U <= wt.t1; t += U) {
      Batch bt;
      load_batch(bt, t);
      run_batch(bt, t);
    }
  }
  for (; t < wt.t1; ++t) {
    XR xr, dyr;
    TR wr;
    dyr.load(dyb + t * p.dys1);
    if (want_dw) {
      xr.load(xb + t * p.xs1);
    } else {
      xr.zero();
    }
    if constexpr (!STATIC) {
      if (want_dx) {
        wr.load(wb + t * p.ws1);
      } else {
        wr.zero();
      }
    }
    step(t, true, true, dyr, wr, xr, sg.load(t));
  }
  if (want_dx) {
#pragma unroll
    for (int e = 0; e < W - 1; ++e) {
      const int tt = wt.t1 + e;
      step(tt, false, tt < p.T, hdy[e], hw[e], hx[e], hsid[e]);
    }
  }
  if constexpr (CB) {
    float* part = p.cb_partial + int64_t(wt.chunk) * p.D + wt.c0;
#pragma unroll
    for (int v = 0; v < VEC; ++v) part[v] = sdy[v];
  }
  if constexpr (STATIC) {
    if (want_dw) {
      float* part = p.partial + int64_t(wt.chunk) * p.G * W;
      if constexpr (PERCH) {
#pragma unroll
        for (int v = 0; v < VEC; ++v)
#pragma unroll
          for (int k = 0; k < W; ++k) part[int64_t(wt.c0 + v) * W + k] = sdw[v][k];
      } else {
        float s[W];
#pragma unroll
        for (int k = 0; k < W; ++k) s[k] = sdw[0][k];
        group_sums<W>(s, lanes_per_group, group_pos);
        if (group_lead) {
#pragma unroll
          for (int k = 0; k < W; ++k) part[int64_t(g) * W + k] = s[k];
        }
      }
    }
  }
}


template <typename ET, int W, int VEC, bool PERCH, bool STATIC>
hipError_t launch_fwd_inst(const StreamParams& p, const StreamPlan& plan, hipStream_t s) {
  if (p.seg != nullptr) {
    hipLaunchKernelGGL((k_stream_fwd<ET, W, VEC, PERCH, STATIC, true>), dim3(unsigned(plan.blocks)),
                       dim3(kBlockThreads), 0, s, p);
  } else {
    hipLaunchKernelGGL((k_stream_fwd<ET, W, VEC, PERCH, STATIC, false>), dim3(unsigned(plan.blocks)),
                       dim3(kBlockThreads), 0, s, p);
  }
  return hipGetLastError();
}

template <typename ET, int W, int VEC, bool PERCH, bool STATIC, bool ALL, bool SEG>
void launch_bwd_cb(const StreamParams& p, const StreamPlan& plan, hipStream_t s) {
  if (p.cb_partial != nullptr) {
    hipLaunchKernelGGL((k_stream_bwd<ET, W, VEC, PERCH, STATIC, ALL, SEG, true>), dim3(unsigned(plan.blocks)),
                       dim3(kBlockThreads), 0, s, p);
  } else {
    hipLaunchKernelGGL((k_stream_bwd<ET, W, VEC, PERCH, STATIC, ALL, SEG, false>), dim3(unsigned(plan.blocks)),
                       dim3(kBlockThreads), 0, s, p);
  }
}

template <typename ET, int W, int VEC, bool PERCH, bool STATIC, bool ALL = false>
hipError_t launch_bwd_inst(const StreamParams& p, const StreamPlan& plan, hipStream_t s) {
  if (p.seg != nullptr) {
    launch_bwd_cb<ET, W, VEC, PERCH, STATIC, ALL, true>(p, plan, s);
  } else {
    launch_bwd_cb<ET, W, VEC, PERCH, STATIC, ALL, false>(p, plan, s);
  }
  return hipGetLastError();
}

template <bool BWD, typename ET, int W, int VEC, bool PERCH>
hipError_t dispatch_static(const StreamParams& p, const StreamPlan& plan, bool st, hipStream_t s) {
  if constexpr (BWD) {
    if (!st) return launch_bwd_inst<ET, W, VEC, PERCH, false>(p, plan, s);
    return (p.out != nullptr && p.partial != nullptr) ? launch_bwd_inst<ET, W, VEC, PERCH, true, true>(p, plan, s)
                                                      : launch_bwd_inst<ET, W, VEC, PERCH, true, false>(p, plan, s);
  } else {
    return st ? launch_fwd_inst<ET, W, VEC, PERCH, true>(p, plan, s) : launch_fwd_inst<ET, W, VEC, PERCH, false>(p, plan, s);
  }
}

template <bool BWD, typename ET, int W>
hipError_t dispatch_mode(const StreamParams& p, const StreamPlan& plan, bool st, hipStream_t s) {
  constexpr int k4 = 4 / int(sizeof(ET));
  if (plan.mode == StreamMode::PerChannel) return dispatch_static<BWD, ET, W, k4, true>(p, plan, st, s);
  if (plan.vec == 4 * k4) return dispatch_static<BWD, ET, W, 4 * k4, false>(p, plan, st, s);
  if (plan.vec == 2 * k4) return dispatch_static<BWD, ET, W, 2 * k4, false>(p, plan, st, s);
  if constexpr (k4 == 2) {
    // one 16-bit channel per lane: groups of odd H
    if (plan.vec == 1) return dispatch_static<BWD, ET, W, 1, false>(p, plan, st, s);
  }
  if constexpr (k4 == 2) {
    // 16-bit groups of 3 * 2^k and 5 * 2^k channels (group_vec)
    if (plan.vec == 6) return dispatch_static<BWD, ET, W, 6, false>(p, plan, st, s);
    if (plan.vec == 10) return dispatch_static<BWD, ET, W, 10, false>(p, plan, st, s);
    // odd groups of 3 or 5 channels, one group per lane
    if (plan.vec == 3) return dispatch_static<BWD, ET, W, 3, false>(p, plan, st, s);
    if (plan.vec == 5) return dispatch_static<BWD, ET, W, 5, false>(p, plan, st, s);
  }
  return dispatch_static<BWD, ET, W, k4, false>(p, plan, st, s);
}

template <bool BWD, typename ET>
hipError_t dispatch_w(const StreamParams& p, const StreamPlan& plan, int W, bool st, hipStream_t s) {
  switch (W) {
    case 1: return dispatch_mode<BWD, ET, 1>(p, plan, st, s);
    case 2: return dispatch_mode<BWD, ET, 2>(p, plan, st, s);
    case 3: return dispatch_mode<BWD, ET, 3>(p, plan, st, s);
    case 4: return dispatch_mode<BWD, ET, 4>(p, plan, st, s);
    case 5: return dispatch_mode<BWD, ET, 5>(p, plan, st, s);
    case 6: return dispatch_mode<BWD, ET, 6>(p, plan, st, s);
    case 7: return dispatch_mode<BWD, ET, 7>(p, plan, st, s);
    case 8: return dispatch_mode<BWD, ET, 8>(p, plan, st, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Launches the forward (bwd == false) or backward streaming kernel for storage type ET.
template <typename ET>
hipError_t stream_dispatch(const StreamParams& p, const StreamPlan& plan, int W, bool is_static, bool bwd,
                           hipStream_t s) {
  return bwd ? dispatch_w<true, ET>(p, plan, W, is_static, s) : dispatch_w<false, ET>(p, plan, W, is_static, s);
}

}  // namespace dynconv
