// Streaming kernels of the dynamic short convolution: planning, launch and the fixed-order
// reduce of partial sums. The kernels themselves are in dynconv_stream_kernels.hpp,
// compiled once per storage type (dynconv_stream_{f32,bf16,f16}.hip).
#include <cmath>

#include "dynconv_common.hpp"
#include "dynconv_internal.hpp"

#ifndef DYNCONV_FWD_WAVES_PER_CU
#define DYNCONV_FWD_WAVES_PER_CU 8
#endif
// head-wise forward (group filters): 12 waves per CU measured best (H = 4: 77.3 -> 75.2 us,
// H = 16: 55.7 -> 53.3 us at B8 T4096 D2048 W4; the static forward is slower there)
#ifndef DYNCONV_FWD_GROUP_WAVES_PER_CU
#define DYNCONV_FWD_GROUP_WAVES_PER_CU 12
#endif
#ifndef DYNCONV_BWD_WAVES_PER_CU
#define DYNCONV_BWD_WAVES_PER_CU 16
#endif
#ifndef DYNCONV_BWD_GROUP_WAVES_PER_CU
#define DYNCONV_BWD_GROUP_WAVES_PER_CU 12
#endif
#ifndef DYNCONV_BWD_STATIC_WAVES_PER_CU
#define DYNCONV_BWD_STATIC_WAVES_PER_CU 8
#endif
// Per-channel dynamic filters with W >= 7 stream twice the filter bytes per lane and token,
// so fewer, longer streams keep as many bytes in flight. Backward: its registers (about 150
// VGPRs) hold 3 waves per SIMD, not the 4 the target above assumes, and whole rounds of 2
// per SIMD measured fastest (W = 8 at B8 T4096 D2048: 653 us at 16 waves per CU, 683 at 12,
// 594 at 8, 591 at 6). Forward: 259 us at 8 waves per CU, 235 at 4.
#ifndef DYNCONV_BWD_WIDE_WAVES_PER_CU
#define DYNCONV_BWD_WIDE_WAVES_PER_CU 8
#endif
#ifndef DYNCONV_FWD_WIDE_WAVES_PER_CU
#define DYNCONV_FWD_WIDE_WAVES_PER_CU 4
#endif

namespace dynconv {

namespace {

// Fixed-order sum of partials: out[i] = sum_c part[c * n + i]. A workgroup owns 32
// consecutive columns; its 8 thread groups take chunks c = grp, grp + 8, ... in order
// (float64), and the 8 group sums are added in order grp = 0..7. The order depends only
// on (nchunk, n), so results are run-to-run identical.
constexpr int kRedCols = 32;
constexpr int kRedGroups = kBlockThreads / kRedCols;

__global__ __launch_bounds__(kBlockThreads) void k_reduce_partials(const float* __restrict__ part, int64_t nchunk,
                                                                   int64_t n, float* __restrict__ out) {
  __shared__ double red[kRedGroups][kRedCols];
  const int col = threadIdx.x % kRedCols;
  const int grp = threadIdx.x / kRedCols;
  const int64_t i = int64_t(blockIdx.x) * kRedCols + col;
  double s = 0.0;
  if (i < n) {
    for (int64_t c = grp; c < nchunk; c += kRedGroups) s += double(part[c * n + i]);
  }
  red[grp][col] = s;
  __syncthreads();
  if (grp == 0 && i < n) {
    double tot = 0.0;
#pragma unroll
    for (int r = 0; r < kRedGroups; ++r) tot += red[r][col];
    out[i] = float(tot);
  }
}

// The same sums, 4 consecutive columns per thread (16-byte loads and stores): n % 4 == 0
// and 16-byte aligned pointers. G thread groups split the chunks (group g takes chunks
// g, g + G, ... in order, float64) and the G group sums are added in order g = 0 .. G-1.
// G = 8 gives exactly the order of k_reduce_partials (bit-identical results); G = 32 serves
// many chunks (short dependent chains, 4x the workgroups for the same columns). Either
// order depends only on (nchunk, n): results are run-to-run identical.
constexpr int kRedTallChunks = 64;  // from this many chunks on, G = 32
constexpr int red_groups(int64_t nchunk) { return nchunk >= kRedTallChunks ? 32 : kRedGroups; }

template <int G>
__device__ __forceinline__ void reduce4_block(const float* __restrict__ part, int64_t nchunk, int64_t n,
                                              float* __restrict__ out, int64_t blk) {
  constexpr int C = kBlockThreads / G;  // float4 columns of a workgroup
  __shared__ double red[G][C][4];
  const int col = threadIdx.x % C;
  const int grp = threadIdx.x / C;
  const int64_t i = blk * (4 * C) + 4 * col;
  double s[4] = {0.0, 0.0, 0.0, 0.0};
  if (i < n) {
    for (int64_t c = grp; c < nchunk; c += G) {
      const float4 v = *reinterpret_cast<const float4*>(part + c * n + i);
      s[0] += double(v.x);
      s[1] += double(v.y);
      s[2] += double(v.z);
      s[3] += double(v.w);
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) red[grp][col][e] = s[e];
  __syncthreads();
  if (grp == 0 && i < n) {
    double tot[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 8
    for (int r = 0; r < G; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) tot[e] += red[r][col][e];
    *reinterpret_cast<float4*>(out + i) = float4{float(tot[0]), float(tot[1]), float(tot[2]), float(tot[3])};
  }
}

template <int G>
__global__ __launch_bounds__(kBlockThreads) void k_reduce_partials4(const float* __restrict__ part, int64_t nchunk,
                                                                    int64_t n, float* __restrict__ out) {
  reduce4_block<G>(part, nchunk, n, out, blockIdx.x);
}

// Two independent sums with the same number of chunks in one launch (one dispatch gap
// fewer): workgroups below nblk0 take the first, the others the second.
template <int G>
__global__ __launch_bounds__(kBlockThreads) void k_reduce_partials4x2(const float* __restrict__ part0, int64_t n0,
                                                                      float* __restrict__ out0, int64_t nblk0,
                                                                      const float* __restrict__ part1, int64_t n1,
                                                                      float* __restrict__ out1, int64_t nchunk) {
  if (int64_t(blockIdx.x) < nblk0) {
    reduce4_block<G>(part0, nchunk, n0, out0, blockIdx.x);
  } else {
    reduce4_block<G>(part1, nchunk, n1, out1, int64_t(blockIdx.x) - nblk0);
  }
}

// Partial column sums: workgroup (chunk, db) sums 256 lanes x one 32-bit word of channels
// over the chunk's tokens (8 rows of loads in flight per lane).
template <typename ET>
__global__ __launch_bounds__(kBlockThreads) void k_column_partials(const ET* __restrict__ a, int64_t s0, int64_t s1,
                                                                   int T, int D, int L, int nchunk, int nDb,
                                                                   float* __restrict__ part) {
  constexpr int V = 4 / int(sizeof(ET));  // channels per lane
  const int db = int(blockIdx.x % unsigned(nDb));
  const int chunk = int(blockIdx.x / unsigned(nDb));  // b * nchunk + token chunk
  const int b = chunk / nchunk, tc = chunk % nchunk;
  const int c = (db * kBlockThreads + int(threadIdx.x)) * V;
  if (c >= D) return;
  const int t0 = tc * L, t1 = min(T, t0 + L);
  const uint32_t* p = reinterpret_cast<const uint32_t*>(a + b * s0 + c);
  const int64_t row = s1 * int64_t(sizeof(ET)) / 4;  // words per row
  float s[V];
#pragma unroll
  for (int v = 0; v < V; ++v) s[v] = 0.f;
  auto add = [&](uint32_t w) {
    if constexpr (V == 2) {
      s[0] += Cvt<ET>::lo(w);
      s[1] += Cvt<ET>::hi(w);
    } else {
      s[0] += __uint_as_float(w);
    }
  };
  int t = t0;
  for (; t + 8 <= t1; t += 8) {
    uint32_t w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) w[u] = p[(t + u) * row];
#pragma unroll
    for (int u = 0; u < 8; ++u) add(w[u]);
  }
  for (; t < t1; ++t) add(p[t * row]);
  float* o = part + int64_t(chunk) * D + c;
#pragma unroll
  for (int v = 0; v < V; ++v) o[v] = s[v];
}

bool reduce4_ok(const float* part, int64_t n, const float* out) {
  return n % 4 == 0 && reinterpret_cast<uintptr_t>(part) % 16 == 0 && reinterpret_cast<uintptr_t>(out) % 16 == 0;
}

}  // namespace


StreamPlan plan_stream(int64_t B, int64_t T, int64_t D, int W, int H, int elem_bytes, int act_align, bool bwd,
                       bool is_static) {
  StreamPlan pl{};
  if (H == 1) {
    // a channel pair per lane, so that the lane's W taps of both are one contiguous run
    // (static filters with 16 bytes of channels per lane measured slower: 47.7 vs 46.4 us
    // forward, 100.5 vs 91.6 us backward at B8 T4096 D2048 W3)
    pl.mode = StreamMode::PerChannel;
    pl.vec = 4 / elem_bytes;
    pl.lpg = 1;
  } else {
    pl.mode = StreamMode::Group;
    pl.vec = group_vec(H, elem_bytes, act_align, bwd);
    pl.lpg = H / pl.vec;
  }
  // The forward reduces nothing over a group: every lane in use, slices of whole cache lines
  // (H = 12 at B8 T4096 D3072: 111.9 -> 87.9 us). The backward keeps each group inside a wave
  // (aligning its slices to 128 or 64 bytes at the cost of more idle lanes measured no gain).
  pl.lpw = bwd ? lanes_in_use(pl.lpg) : kWaveSize;
  const int64_t span = int64_t(pl.lpw) * pl.vec;
  pl.nDw = int((D + span - 1) / span);
  pl.WD = pl.nDw >= 4 ? 4 : (pl.nDw >= 2 ? 2 : 1);
  pl.WT = 4 / pl.WD;
  pl.nDb = (pl.nDw + pl.WD - 1) / pl.WD;
  // Time chunking: aim at a number of waves per CU, but prefer grids that spread evenly
  // over the 256 CUs (a grid of 4.03 workgroups per CU runs as long as one of 5). Chunks
  // hold a multiple of 4 tokens and at least 16 (64 for the static backward, which writes
  // one partial sum per chunk).
  const bool wide = H == 1 && !is_static && W >= 7;
  const int waves_per_cu = !bwd ? (wide                   ? DYNCONV_FWD_WIDE_WAVES_PER_CU
                                   : H > 1 && !is_static ? DYNCONV_FWD_GROUP_WAVES_PER_CU
                                                         : DYNCONV_FWD_WAVES_PER_CU)
                           : is_static ? DYNCONV_BWD_STATIC_WAVES_PER_CU
                           : H > 1     ? DYNCONV_BWD_GROUP_WAVES_PER_CU
                           : wide      ? DYNCONV_BWD_WIDE_WAVES_PER_CU
                                       : DYNCONV_BWD_WAVES_PER_CU;
  const double target_blocks = 256.0 * waves_per_cu / (kBlockThreads / kWaveSize);
  const int64_t min_len = (bwd && is_static) ? 64 : 16;
  const int64_t max_chunks = T <= min_len ? 1 : (T + min_len - 1) / min_len;
  const double per_seq_target = target_blocks * pl.WT / double(B * pl.nDb);
  int64_t lo = int64_t(per_seq_target / 4), hi = int64_t(per_seq_target * 4) + 1;
  if (lo < 1) lo = 1;
  if (hi > max_chunks) hi = max_chunks;
  if (lo > hi) lo = hi;
  double best = -1e30;
  int64_t bestL = T;
  for (int64_t c = lo; c <= hi; ++c) {
    int64_t L = (T + c - 1) / c;
    L = (L + 3) / 4 * 4;
    const int64_t nTw = (T + L - 1) / L;
    const int64_t blocks = B * pl.nDb * ((nTw + pl.WT - 1) / pl.WT);
    const int64_t per_cu = (blocks + 255) / 256;
    const double eff = double(blocks) / double(256 * per_cu);
    const double dist = std::fabs(std::log(double(blocks) / target_blocks));
    const double score = eff - 0.25 * dist;
    if (score > best + 1e-12) {
      best = score;
      bestL = L;
    }
  }
  pl.L = int(bestL);
  pl.nTw = int((T + bestL - 1) / bestL);
  pl.nTb = (pl.nTw + pl.WT - 1) / pl.WT;
  pl.blocks = B * int64_t(pl.nDb) * pl.nTb;
  return pl;
}

dynconv_status launch_stream_fwd(const StreamParams& p, const StreamPlan& plan, int W, dynconv_dtype dt,
                                 bool is_static, hipStream_t stream) {
  const hipError_t e = dt == DYNCONV_BF16   ? stream_dispatch_bf16(p, plan, W, is_static, false, stream)
                       : dt == DYNCONV_F16 ? stream_dispatch_f16(p, plan, W, is_static, false, stream)
                                           : stream_dispatch_f32(p, plan, W, is_static, false, stream);
  return e == hipSuccess ? DYNCONV_OK : record_hip_error(e);
}

dynconv_status launch_stream_bwd(const StreamParams& p, const StreamPlan& plan, int W, dynconv_dtype dt,
                                 bool is_static, float* dw_static_out, float* dcbias_out, hipStream_t stream) {
  hipError_t e = dt == DYNCONV_BF16   ? stream_dispatch_bf16(p, plan, W, is_static, true, stream)
                 : dt == DYNCONV_F16 ? stream_dispatch_f16(p, plan, W, is_static, true, stream)
                                     : stream_dispatch_f32(p, plan, W, is_static, true, stream);
  if (e != hipSuccess) return record_hip_error(e);
  const int64_t nchunk = int64_t(p.B) * plan.nTw;
  const bool sdw = is_static && p.partial != nullptr;
  if (sdw && p.cb_partial != nullptr) {
    return launch_reduce_partials2(p.partial, int64_t(p.G) * W, dw_static_out, p.cb_partial, p.D, dcbias_out, nchunk,
                                   stream);
  }
  if (sdw) return launch_reduce_partials(p.partial, nchunk, int64_t(p.G) * W, dw_static_out, stream);
  if (p.cb_partial != nullptr) return launch_reduce_partials(p.cb_partial, nchunk, p.D, dcbias_out, stream);
  return DYNCONV_OK;
}

dynconv_status launch_reduce_partials(const float* partial, int64_t nchunk, int64_t n, float* out,
                                      hipStream_t stream) {
  if (reduce4_ok(partial, n, out)) {
    const int G = red_groups(nchunk);
    const int64_t cols = 4 * (kBlockThreads / G);
    const int64_t blocks = (n + cols - 1) / cols;
    if (G == 32) {
      hipLaunchKernelGGL(k_reduce_partials4<32>, dim3(unsigned(blocks)), dim3(kBlockThreads), 0, stream, partial,
                         nchunk, n, out);
    } else {
      hipLaunchKernelGGL(k_reduce_partials4<kRedGroups>, dim3(unsigned(blocks)), dim3(kBlockThreads), 0, stream,
                         partial, nchunk, n, out);
    }
  } else {
    const int64_t blocks = (n + kRedCols - 1) / kRedCols;
    hipLaunchKernelGGL(k_reduce_partials, dim3(unsigned(blocks)), dim3(kBlockThreads), 0, stream, partial, nchunk, n,
                       out);
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? DYNCONV_OK : record_hip_error(e);
}

dynconv_status launch_reduce_partials2(const float* part0, int64_t n0, float* out0, const float* part1, int64_t n1,
                                       float* out1, int64_t nchunk, hipStream_t stream) {
  if (!reduce4_ok(part0, n0, out0) || !reduce4_ok(part1, n1, out1)) {
    const dynconv_status st = launch_reduce_partials(part0, nchunk, n0, out0, stream);
    if (st != DYNCONV_OK) return st;
    return launch_reduce_partials(part1, nchunk, n1, out1, stream);
  }
  const int G = red_groups(nchunk);
  const int64_t cols = 4 * (kBlockThreads / G);
  const int64_t nblk0 = (n0 + cols - 1) / cols;
  const int64_t nblk1 = (n1 + cols - 1) / cols;
  if (G == 32) {
    hipLaunchKernelGGL(k_reduce_partials4x2<32>, dim3(unsigned(nblk0 + nblk1)), dim3(kBlockThreads), 0, stream, part0,
                       n0, out0, nblk0, part1, n1, out1, nchunk);
  } else {
    hipLaunchKernelGGL(k_reduce_partials4x2<kRedGroups>, dim3(unsigned(nblk0 + nblk1)), dim3(kBlockThreads), 0,
                       stream, part0, n0, out0, nblk0, part1, n1, out1, nchunk);
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? DYNCONV_OK : record_hip_error(e);
}

// About 2048 workgroups (of 256 channels each at one channel per lane), chunks of at least
// 64 tokens.
int64_t colsum_chunks(int64_t B, int64_t T, int64_t D) {
  const int64_t per_seq = (2048 + B * ((D + 255) / 256) - 1) / (B * ((D + 255) / 256));
  const int64_t most = (T + 63) / 64;
  return per_seq < 1 ? 1 : (per_seq > most ? (most < 1 ? 1 : most) : per_seq);
}

dynconv_status launch_column_sums(const void* a, int64_t s0, int64_t s1, int64_t B, int64_t T, int64_t D,
                                  dynconv_dtype dt, float* part, float* out, hipStream_t stream) {
  const int64_t nchunk = colsum_chunks(B, T, D);
  const int64_t L = (T + nchunk - 1) / nchunk;
  const int V = dt == DYNCONV_F32 ? 1 : 2;
  const int64_t nDb = (D + int64_t(kBlockThreads) * V - 1) / (int64_t(kBlockThreads) * V);
  const dim3 grid(unsigned(B * nchunk * nDb));
  if (dt == DYNCONV_BF16) {
    hipLaunchKernelGGL(k_column_partials<bf16_t>, grid, dim3(kBlockThreads), 0, stream, static_cast<const bf16_t*>(a),
                       s0, s1, int(T), int(D), int(L), int(nchunk), int(nDb), part);
  } else if (dt == DYNCONV_F16) {
    hipLaunchKernelGGL(k_column_partials<f16_t>, grid, dim3(kBlockThreads), 0, stream, static_cast<const f16_t*>(a),
                       s0, s1, int(T), int(D), int(L), int(nchunk), int(nDb), part);
  } else {
    hipLaunchKernelGGL(k_column_partials<float>, grid, dim3(kBlockThreads), 0, stream, static_cast<const float*>(a),
                       s0, s1, int(T), int(D), int(L), int(nchunk), int(nDb), part);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return record_hip_error(e);
  return launch_reduce_partials(part, B * nchunk, D, out, stream);
}

}  // namespace dynconv
