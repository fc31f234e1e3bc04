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
// as VEC*W contiguous elements (H = 1) or one broadcast group (H > 1).
#include "dynconv_common.hpp"
#include "dynconv_internal.hpp"

namespace dynconv {

namespace {

template <typename ET, int N>
__device__ __forceinline__ void load_dwords(const ET* p, float (&o)[N]) {
  // N contiguous elements at a 4-byte aligned address, as N*sizeof/4 dword loads
  // (the compiler fuses them into dwordx2/x3/x4).
  if constexpr (sizeof(ET) == 2) {
    static_assert(N % 2 == 0, "bf16 dword loads need an even element count");
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const uint32_t u = q[i];
      o[2 * i] = bf16_lo(u);
      o[2 * i + 1] = bf16_hi(u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) o[i] = reinterpret_cast<const float*>(p)[i];
  }
}

template <typename ET, int N>
__device__ __forceinline__ void store_dwords(ET* p, const float (&v)[N]) {
  if constexpr (sizeof(ET) == 2) {
    uint32_t* q = reinterpret_cast<uint32_t*>(p);
#pragma unroll
    for (int i = 0; i < N / 2; ++i) q[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) reinterpret_cast<float*>(p)[i] = v[i];
  }
}

// Filters held by one lane for one token: NC rows of W taps (NC = VEC per channel when
// H == 1, a single shared row when H > 1).
template <typename ET, int W, int VEC, bool PERCH>
struct Taps {
  static constexpr int NC = PERCH ? VEC : 1;
  float f[NC][W];

  __device__ __forceinline__ void load(const ET* p) {
    if constexpr (PERCH) {
      float tmp[VEC * W];
      load_dwords<ET, VEC * W>(p, tmp);
#pragma unroll
      for (int v = 0; v < VEC; ++v)
#pragma unroll
        for (int k = 0; k < W; ++k) f[v][k] = tmp[v * W + k];
    } else {
      float tmp[W];
      load_unaligned<ET, W>(p, tmp);
#pragma unroll
      for (int k = 0; k < W; ++k) f[0][k] = tmp[k];
    }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int v = 0; v < NC; ++v)
#pragma unroll
      for (int k = 0; k < W; ++k) f[v][k] = 0.f;
  }
  __device__ __forceinline__ float tap(int v, int k) const { return f[PERCH ? v : 0][k]; }
};

struct WaveTile {
  int b, c0, t0, t1, chunk;
  bool valid;
};

__device__ __forceinline__ WaveTile wave_tile(const StreamParams& p, int vec) {
  WaveTile wt;
  const int lane = threadIdx.x & (kWaveSize - 1);
  const int wv = threadIdx.x / kWaveSize;
  uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int tb = lb % p.nTb;
  lb /= p.nTb;
  const int db = lb % p.nDb;
  wt.b = lb / p.nDb;
  const int dsl = db * p.WD + (wv % p.WD);
  const int tch = tb * p.WT + (wv / p.WD);
  wt.c0 = (dsl * kWaveSize + lane) * vec;
  wt.t0 = tch * p.L;
  wt.t1 = min(p.T, wt.t0 + p.L);
  wt.chunk = wt.b * p.nTw + tch;
  wt.valid = dsl < p.nDw && tch < p.nTw && wt.c0 < p.D;
  return wt;
}

constexpr int kUnroll = 4;

// ---------------------------------------------------------------------------------
// Forward: y_t = x_t + sum_k w_k^(t) x_{t-k}
// ---------------------------------------------------------------------------------
template <typename ET, int W, int VEC, bool PERCH, bool STATIC>
__global__ __launch_bounds__(kBlockThreads) void k_stream_fwd(const StreamParams p) {
  const WaveTile wt = wave_tile(p, VEC);
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
    if (t >= 0) {
      Vec<ET, VEC>::load(xb + t * p.xs1, xh[k - 1]);
    } else {
#pragma unroll
      for (int v = 0; v < VEC; ++v) xh[k - 1][v] = 0.f;
    }
  }
  Taps<ET, W, VEC, PERCH> wst;
  if constexpr (STATIC) wst.load(wb);

  auto compute_store = [&](int t, const float (&xv)[VEC], const Taps<ET, W, VEC, PERCH>& f) {
#pragma unroll
    for (int k = W - 1; k >= 1; --k)
#pragma unroll
      for (int v = 0; v < VEC; ++v) xh[k][v] = xh[k - 1][v];
#pragma unroll
    for (int v = 0; v < VEC; ++v) xh[0][v] = xv[v];
    float yv[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      float acc = xh[0][v];
#pragma unroll
      for (int k = 0; k < W; ++k) acc = fmaf(f.tap(v, k), xh[k][v], acc);
      yv[v] = acc;
    }
    Vec<ET, VEC>::store(yb + t * p.os1, yv);
  };

  int t = wt.t0;
  for (; t + kUnroll <= wt.t1; t += kUnroll) {
    float xin[kUnroll][VEC];
    Taps<ET, W, VEC, PERCH> win[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      Vec<ET, VEC>::load(xb + (t + u) * p.xs1, xin[u]);
      if constexpr (STATIC) {
        win[u] = wst;
      } else {
        win[u].load(wb + (t + u) * p.ws1);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) compute_store(t + u, xin[u], win[u]);
  }
  for (; t < wt.t1; ++t) {
    float xin[VEC];
    Taps<ET, W, VEC, PERCH> win;
    Vec<ET, VEC>::load(xb + t * p.xs1, xin);
    if constexpr (STATIC) {
      win = wst;
    } else {
      win.load(wb + t * p.ws1);
    }
    compute_store(t, xin, win);
  }
}

// ---------------------------------------------------------------------------------
// Backward. A forward sweep over t scatters w_k^(t) dy_t into dx_{t-k}; dx_s is final
// once step s + W - 1 is done, so each lane keeps W-1 pending sums. The chunk's last
// W-1 dx rows need the next chunk's first W-1 rows of w and dy (the future halo).
//   dx_s = dy_s + sum_k w_k^(s+k) dy_{s+k}
//   dw_t[g,k] = sum_{d in g} dy_t[d] x_{t-k}[d]
// ---------------------------------------------------------------------------------
template <int VEC>
__device__ __forceinline__ float group_sum(float v, int lanes) {
  for (int m = 1; m < lanes; m <<= 1) v += __shfl_xor(v, m, kWaveSize);
  return v;
}

template <typename ET, int W, int VEC, bool PERCH, bool STATIC>
__global__ __launch_bounds__(kBlockThreads) void k_stream_bwd(const StreamParams p) {
  const WaveTile wt = wave_tile(p, VEC);
  // Group reductions need every lane of a group; a whole group is either valid or not
  // (H divides D and groups are lane-aligned), so invalid lanes can leave now.
  if (!wt.valid) return;
  constexpr int WM = W > 1 ? W - 1 : 1;
  constexpr int NC = PERCH ? VEC : 1;
  const int lane = threadIdx.x & (kWaveSize - 1);
  const int lanes_per_group = PERCH ? 1 : p.H / VEC;
  const bool group_lead = PERCH || (lane % lanes_per_group) == 0;
  const int g = PERCH ? wt.c0 : wt.c0 / p.H;
  const bool want_dx = p.out != nullptr;
  const bool want_dw = STATIC ? (p.partial != nullptr) : (p.dw != nullptr);

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
      if (t >= 0) Vec<ET, VEC>::load(xb + t * p.xs1, xh[k - 1]);
    }
  }
  Taps<ET, W, VEC, PERCH> wst;
  float sdw[NC][W];  // static: per-lane partial sums of dw over the chunk
  if constexpr (STATIC) {
    wst.load(wb);
#pragma unroll
    for (int v = 0; v < NC; ++v)
#pragma unroll
      for (int k = 0; k < W; ++k) sdw[v][k] = 0.f;
  }

  // One step at token t. MAIN: t inside the chunk (x is read, dw produced).
  auto step = [&](int t, bool main, const float (&dyv)[VEC], const Taps<ET, W, VEC, PERCH>& f,
                  const float (&xv)[VEC]) {
    if (main && want_dw) {
      float d[W][VEC];
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        d[0][v] = dyv[v] * xv[v];
#pragma unroll
        for (int k = 1; k < W; ++k) d[k][v] = dyv[v] * xh[k - 1][v];
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
          store_dwords<ET, VEC * W>(dwb + t * p.dws1, o);
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
#pragma unroll
          for (int k = 0; k < W; ++k) s[k] = group_sum<VEC>(s[k], lanes_per_group);
          if (group_lead) store_unaligned<ET, W>(dwb + t * p.dws1, s);
        }
      }
    }
    if (want_dx) {
      float nacc[VEC];
#pragma unroll
      for (int v = 0; v < VEC; ++v) nacc[v] = fmaf(f.tap(v, 0), dyv[v], dyv[v]);
#pragma unroll
      for (int j = 1; j < W; ++j)
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[j - 1][v] = fmaf(f.tap(v, j), dyv[v], acc[j - 1][v]);
      const int s = t - (W - 1);
      if (s >= wt.t0 && s < wt.t1) {
        if constexpr (W == 1) {
          Vec<ET, VEC>::store(dxb + s * p.os1, nacc);
        } else {
          Vec<ET, VEC>::store(dxb + s * p.os1, acc[W - 2]);
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
      for (int v = 0; v < VEC; ++v) xh[0][v] = xv[v];
    }
  };

  int t = wt.t0;
  for (; t + kUnroll <= wt.t1; t += kUnroll) {
    float xin[kUnroll][VEC], dyin[kUnroll][VEC];
    Taps<ET, W, VEC, PERCH> win[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      Vec<ET, VEC>::load(dyb + (t + u) * p.dys1, dyin[u]);
      if (want_dw) {
        Vec<ET, VEC>::load(xb + (t + u) * p.xs1, xin[u]);
      } else {
#pragma unroll
        for (int v = 0; v < VEC; ++v) xin[u][v] = 0.f;
      }
      if constexpr (STATIC) {
        win[u] = wst;
      } else {
        if (want_dx) {
          win[u].load(wb + (t + u) * p.ws1);
        } else {
          win[u].zero();
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) step(t + u, true, dyin[u], win[u], xin[u]);
  }
  for (; t < wt.t1; ++t) {
    float xin[VEC], dyin[VEC];
    Taps<ET, W, VEC, PERCH> win;
    Vec<ET, VEC>::load(dyb + t * p.dys1, dyin);
    if (want_dw) {
      Vec<ET, VEC>::load(xb + t * p.xs1, xin);
    } else {
#pragma unroll
      for (int v = 0; v < VEC; ++v) xin[v] = 0.f;
    }
    if constexpr (STATIC) {
      win = wst;
    } else {
      if (want_dx) {
        win.load(wb + t * p.ws1);
      } else {
        win.zero();
      }
    }
    step(t, true, dyin, win, xin);
  }
  // Future halo: the W-1 tokens after the chunk complete its last dx rows.
  if (want_dx) {
#pragma unroll
    for (int e = 0; e < W - 1; ++e) {
      const int tt = wt.t1 + e;
      float dyin[VEC], xin[VEC];
      Taps<ET, W, VEC, PERCH> win;
#pragma unroll
      for (int v = 0; v < VEC; ++v) xin[v] = 0.f;
      if (tt < p.T) {
        Vec<ET, VEC>::load(dyb + tt * p.dys1, dyin);
        if constexpr (STATIC) {
          win = wst;
        } else {
          win.load(wb + tt * p.ws1);
        }
      } else {
#pragma unroll
        for (int v = 0; v < VEC; ++v) dyin[v] = 0.f;
        win.zero();
      }
      step(tt, false, dyin, win, xin);
    }
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
        for (int k = 0; k < W; ++k) s[k] = group_sum<VEC>(sdw[0][k], lanes_per_group);
        if (group_lead) {
#pragma unroll
          for (int k = 0; k < W; ++k) part[int64_t(g) * W + k] = s[k];
        }
      }
    }
  }
}

// Fixed-order (chunk 0, 1, 2, ...) sum of partials, accumulated in float64.
__global__ __launch_bounds__(kBlockThreads) void k_reduce_partials(const float* __restrict__ part, int64_t nchunk,
                                                                   int64_t n, float* __restrict__ out) {
  const int64_t i = int64_t(blockIdx.x) * kBlockThreads + threadIdx.x;
  if (i >= n) return;
  double s = 0.0;
  for (int64_t c = 0; c < nchunk; ++c) s += double(part[c * n + i]);
  out[i] = float(s);
}

template <typename ET, int W, int VEC, bool PERCH, bool STATIC>
hipError_t launch_fwd_inst(const StreamParams& p, const StreamPlan& plan, hipStream_t s) {
  hipLaunchKernelGGL((k_stream_fwd<ET, W, VEC, PERCH, STATIC>), dim3(unsigned(plan.blocks)), dim3(kBlockThreads), 0,
                     s, p);
  return hipGetLastError();
}

template <typename ET, int W, int VEC, bool PERCH, bool STATIC>
hipError_t launch_bwd_inst(const StreamParams& p, const StreamPlan& plan, hipStream_t s) {
  hipLaunchKernelGGL((k_stream_bwd<ET, W, VEC, PERCH, STATIC>), dim3(unsigned(plan.blocks)), dim3(kBlockThreads), 0,
                     s, p);
  return hipGetLastError();
}

template <bool BWD, typename ET, int W, int VEC, bool PERCH>
hipError_t dispatch_static(const StreamParams& p, const StreamPlan& plan, bool st, hipStream_t s) {
  if constexpr (BWD) {
    return st ? launch_bwd_inst<ET, W, VEC, PERCH, true>(p, plan, s) : launch_bwd_inst<ET, W, VEC, PERCH, false>(p, plan, s);
  } else {
    return st ? launch_fwd_inst<ET, W, VEC, PERCH, true>(p, plan, s) : launch_fwd_inst<ET, W, VEC, PERCH, false>(p, plan, s);
  }
}

template <bool BWD, typename ET, int W>
hipError_t dispatch_mode(const StreamParams& p, const StreamPlan& plan, bool st, hipStream_t s) {
  constexpr int kSmall = 4 / int(sizeof(ET));
  constexpr int kWide = 16 / int(sizeof(ET));
  if (plan.mode == StreamMode::PerChannel) return dispatch_static<BWD, ET, W, kSmall, true>(p, plan, st, s);
  if (plan.vec == kWide) return dispatch_static<BWD, ET, W, kWide, false>(p, plan, st, s);
  return dispatch_static<BWD, ET, W, kSmall, false>(p, plan, st, s);
}

template <bool BWD, typename ET>
hipError_t dispatch_w(const StreamParams& p, const StreamPlan& plan, int W, bool st, hipStream_t s) {
  switch (W) {
    case 1: return dispatch_mode<BWD, ET, 1>(p, plan, st, s);
    case 2: return dispatch_mode<BWD, ET, 2>(p, plan, st, s);
    case 3: return dispatch_mode<BWD, ET, 3>(p, plan, st, s);
    case 4: return dispatch_mode<BWD, ET, 4>(p, plan, st, s);
    case 5: return dispatch_mode<BWD, ET, 5>(p, plan, st, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

StreamPlan plan_stream(int64_t B, int64_t T, int64_t D, int H, int elem_bytes, bool wide_ok, bool bwd,
                       bool is_static) {
  StreamPlan pl{};
  const int small = 4 / elem_bytes;
  const int wide = 16 / elem_bytes;
  if (H == 1) {
    pl.mode = StreamMode::PerChannel;
    pl.vec = small;
  } else {
    pl.mode = StreamMode::Group;
    pl.vec = (wide_ok && H % wide == 0 && D % wide == 0) ? wide : small;
  }
  const int64_t span = int64_t(kWaveSize) * pl.vec;
  pl.nDw = int((D + span - 1) / span);
  // Aim at about 16 waves per CU over the 256 CUs, with chunks of at least 16 tokens.
  const int64_t target_waves = 256 * 16;
  int64_t per_seq = (target_waves + B * pl.nDw - 1) / (B * pl.nDw);
  const int64_t max_chunks = (T + 15) / 16;
  if (per_seq > max_chunks) per_seq = max_chunks;
  if (per_seq < 1) per_seq = 1;
  int64_t L = (T + per_seq - 1) / per_seq;
  L = (L + 3) / 4 * 4;
  if (bwd && is_static && L < 64) L = T < 64 ? L : 64;  // fewer partials to reduce
  pl.L = int(L);
  pl.nTw = int((T + L - 1) / L);
  pl.WD = pl.nDw >= 4 ? 4 : (pl.nDw >= 2 ? 2 : 1);
  pl.WT = 4 / pl.WD;
  pl.nDb = (pl.nDw + pl.WD - 1) / pl.WD;
  pl.nTb = (pl.nTw + pl.WT - 1) / pl.WT;
  pl.blocks = B * int64_t(pl.nDb) * pl.nTb;
  return pl;
}

dynconv_status launch_stream_fwd(const StreamParams& p, const StreamPlan& plan, int W, dynconv_dtype dt,
                                 bool is_static, hipStream_t stream) {
  const hipError_t e = dt == DYNCONV_BF16 ? dispatch_w<false, bf16_t>(p, plan, W, is_static, stream)
                                          : dispatch_w<false, float>(p, plan, W, is_static, stream);
  return e == hipSuccess ? DYNCONV_OK : record_hip_error(e);
}

dynconv_status launch_stream_bwd(const StreamParams& p, const StreamPlan& plan, int W, dynconv_dtype dt,
                                 bool is_static, float* dw_static_out, hipStream_t stream) {
  hipError_t e = dt == DYNCONV_BF16 ? dispatch_w<true, bf16_t>(p, plan, W, is_static, stream)
                                    : dispatch_w<true, float>(p, plan, W, is_static, stream);
  if (e != hipSuccess) return record_hip_error(e);
  if (is_static && p.partial != nullptr) {
    return launch_reduce_partials(p.partial, int64_t(p.B) * plan.nTw, int64_t(p.G) * W, dw_static_out, stream);
  }
  return DYNCONV_OK;
}

dynconv_status launch_reduce_partials(const float* partial, int64_t nchunk, int64_t n, float* out,
                                      hipStream_t stream) {
  const int64_t blocks = (n + kBlockThreads - 1) / kBlockThreads;
  hipLaunchKernelGGL(k_reduce_partials, dim3(unsigned(blocks)), dim3(kBlockThreads), 0, stream, partial, nchunk, n,
                     out);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? DYNCONV_OK : record_hip_error(e);
}

}  // namespace dynconv
