// Internal interface between the C ABI layer (argument checks) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/dynconv.h"

namespace dynconv {

constexpr int kWaveSize = 64;
constexpr int kMaxW = 8;         // widest filter (materialised, static and head-wise forms, decoding)
constexpr int kMaxLowrankW = 8;  // widest filter of the low-rank form (W > 5: the general kernels)
// Row strides (x, z, dy, y / dx) and U's row stride of the low-rank form stay below this many
// elements: its kernels form the offsets of up to 128 rows (a step of 64 tokens with its halo,
// or the rank rows of U) in 32-bit arithmetic.
constexpr int64_t kLowrankMaxRowStride = int64_t(1) << 24;
constexpr int kBlockThreads = 256;  // 4 waves per workgroup

// Lane mapping of the streaming kernels: each lane owns VEC consecutive channels and
// sweeps a run of tokens, keeping the W-1 token halo in registers.
enum class StreamMode {
  PerChannel,  // H == 1: lane loads the VEC*W contiguous taps of its channels
  Group,       // H > 1: the lane's VEC channels share one filter (group_vec below)
};

// Channels per lane of the head-wise (H > 1) streaming kernels, so that a lane never
// straddles two groups and a group spans H / VEC consecutive lanes: the largest power of
// two that divides H and fits the widest lane vector the activations allow (`act_align`
// bytes), except for groups of m * 2^k channels with m = 3 or 5 (k >= 1) in 16-bit storage,
// which take 2m channels (12 or 20 bytes) per lane in the backward, so that H / VEC is a
// power of two and the group's dw sums take the butterfly; the forward, which sums
// nothing, takes 6 channels for m = 3 where the power of two is narrower. Measured at B8
// T4096 W4 bf16 against the power-of-two layout (groups of 3 or 5 lanes and the scan):
// backward H = 6 260 -> 149 us, H = 12 184 -> 129, H = 24 139 -> 122, H = 96 142 -> 117
// (D = 3072), H = 10 234 -> 136 (D = 2560); forward H = 6 100 -> 92, H = 12 88 -> 81. Lanes of
// 20 or 24 bytes (5 or 6 words: two load instructions per row, each spanning the wave's
// row with gaps) were slower in the forward than the power of two, even 4-byte lanes.
// Groups of exactly 3 or 5 channels in 16-bit storage take one whole group per lane (16-bit
// loads) instead of one channel per lane and the scan: H = 3 forward / backward 169 / 430
// -> 144 / 271 us (D = 3072), H = 5 152 / 420 -> 105 / 163 us (D = 2560).
constexpr int group_vec(int H, int elem_bytes, int act_align, bool bwd) {
  int v = act_align / elem_bytes;
  while (v > 1 && H % v != 0) v /= 2;
  int m = H;  // the odd part of H
  while (m % 2 == 0) m /= 2;
  if (elem_bytes == 2 && (m == 3 || m == 5) && H % (2 * m) == 0) {
    if (bwd) return 2 * m;
    if (m == 3 && v < 6) return 6;
  }
  if (elem_bytes == 2 && (m == 3 || m == 5) && H == m) return m;  // one group per lane (16-bit loads)
  return v;
}

// Lanes of a wave in use: whole groups only, so that no group straddles two waves (all 64
// when the group's lanes divide 64, e.g. 63 for groups of 3 lanes, 60 for groups of 12).
constexpr int lanes_in_use(int lanes_per_group) { return (kWaveSize / lanes_per_group) * lanes_per_group; }

// Parameters of the streaming (materialised / static filter) kernels, passed by value.
struct StreamParams {
  const void* x;
  const void* w;
  const void* dy;
  void* out;        // y (forward) or dx (backward, may be null)
  void* dw;         // per-token dw (backward, may be null)
  float* partial;   // static dw: per (b, time chunk) partial sums [B*nTw][G][W]
  const void* cbias;   // forward: optional convolution bias [D] (dtype), or null
  float* cb_partial;   // backward: per (b, time chunk) sums of dy [B*nTw][D] for the bias gradient, or null
  const int32_t* seg;  // packed sequences: segment id per token [B,T] (strides ss0, ss1), or null
  int64_t ss0, ss1;
  int64_t xs0, xs1;
  int64_t ws0, ws1;
  int64_t dys0, dys1;
  int64_t os0, os1;
  int64_t dws0, dws1;
  int32_t B, T, D, H, G;
  int32_t lpg;       // lanes per group (1 for the per-channel form)
  int32_t lpw;       // lanes of a wave in use (backward: a multiple of lpg; forward: 64)
  int32_t L;         // tokens per wave time chunk
  int32_t nTw;       // time chunks per sequence
  int32_t nDw;       // channel slices (one wave wide) across D
  int32_t WD, WT;    // waves per workgroup along D and along T (WD * WT == 4)
  int32_t nDb, nTb;  // workgroups along D and along T
};

struct StreamPlan {
  int vec;      // channels per lane
  int lpg;      // lanes per group
  int lpw;      // lanes of a wave in use
  StreamMode mode;
  int L, nTw, nDw, WD, WT, nDb, nTb;
  int64_t blocks;
};

// Chooses the lane vector width and the time chunking. `act_align` (4, 8 or 16) is the
// widest lane vector, in bytes, that every activation-shaped tensor allows; the layout must
// be one the C ABI admits (a group of at most a wave's lanes).
StreamPlan plan_stream(int64_t B, int64_t T, int64_t D, int W, int H, int elem_bytes, int act_align, bool bwd,
                       bool is_static);

// The streaming kernels for one storage type (one translation unit each).
hipError_t stream_dispatch_f32(const StreamParams& p, const StreamPlan& plan, int W, bool is_static, bool bwd,
                               hipStream_t s);
hipError_t stream_dispatch_bf16(const StreamParams& p, const StreamPlan& plan, int W, bool is_static, bool bwd,
                                hipStream_t s);
hipError_t stream_dispatch_f16(const StreamParams& p, const StreamPlan& plan, int W, bool is_static, bool bwd,
                               hipStream_t s);

dynconv_status launch_stream_fwd(const StreamParams& p, const StreamPlan& plan, int W, dynconv_dtype dt,
                                 bool is_static, hipStream_t stream);
dynconv_status launch_stream_bwd(const StreamParams& p, const StreamPlan& plan, int W, dynconv_dtype dt,
                                 bool is_static, float* dw_static_out, float* dcbias_out, hipStream_t stream);

// Fixed-order sum of [nchunk][n] float32 partials into out[n].
dynconv_status launch_reduce_partials(const float* partial, int64_t nchunk, int64_t n, float* out,
                                      hipStream_t stream);
// The same for two sums over the same number of chunks, in one launch where both allow
// 16-byte loads (else two launches). Each result is bit-identical to its own reduce.
dynconv_status launch_reduce_partials2(const float* part0, int64_t n0, float* out0, const float* part1, int64_t n1,
                                       float* out1, int64_t nchunk, hipStream_t stream);

// Column sums of an activation-shaped tensor a [B,T,D] (strides s0, s1; 4-byte aligned rows):
// out[d] = sum over (b, t) of a[b,t,d], the gradient of a convolution bias. Float32 partial
// sums per (sequence, chunk of tokens) go to part [B * colsum_chunks(B, T, D)][D], then the
// fixed-order reduce, so results are run-to-run identical.
int64_t colsum_chunks(int64_t B, int64_t T, int64_t D);
dynconv_status launch_column_sums(const void* a, int64_t s0, int64_t s1, int64_t B, int64_t T, int64_t D,
                                  dynconv_dtype dt, float* part, float* out, hipStream_t stream);

// Records a HIP failure for dynconv_last_hip_error(); returns DYNCONV_ERR_HIP.
dynconv_status record_hip_error(hipError_t e);

}  // namespace dynconv
