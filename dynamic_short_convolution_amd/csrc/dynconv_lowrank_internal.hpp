// Internal interface of the low-rank kernels: parameters, planning and launchers.
#pragma once

#include "dynconv_internal.hpp"

namespace dynconv {

// ---------------------------------------------------------------------------------
// Low-rank form
// ---------------------------------------------------------------------------------
constexpr int kLowrankTT = 16;  // tokens per tile of the general kernels (one MFMA's N or K extent)

struct LowRankParams {
  const void* x;
  const void* z;
  const void* U;
  const void* bias;  // may be null
  const void* cbias; // forward: optional convolution bias [D] (dtype), added to y; may be null
  const void* dy;
  void* out;   // y (forward) or dx (backward)
  void* dz;
  float* part_dU;  // [nTr][R][J]   partial dU per token range
  float* part_db;  // [nTr][J]      partial db per token range
  int64_t xs0, xs1;
  int64_t zs0, zs1;
  int64_t ldu;
  int64_t dys0, dys1;
  int64_t os0, os1;
  int64_t dzs0, dzs1;
  int32_t B, T, D, H, G, R, J;
  int32_t nCs;     // channel slices
  int32_t cs0, nCsL;   // channel slices of one launch: cs0 .. cs0 + nCsL - 1
  int32_t tbb0, nTbL;  // dz token blocks of one launch (per sequence): tbb0 .. + nTbL - 1
  int32_t Ltok;    // tokens per token range
  int32_t nTr;     // token ranges per sequence
  int32_t act16;   // every activation-shaped tensor allows 16-byte vectors
  int32_t z16;     // z rows allow 16-byte vectors
  int32_t z4;      // z rows allow 4-byte pieces (base and row strides)
  int32_t u16;     // U rows allow 16-byte vectors
  const int32_t* seg;  // packed sequences: segment id per token [B,T] (strides ss0, ss1), or null
  int64_t ss0, ss1;
};

// Low-rank forward tiling, shared by the planner and the kernel: each wave generates MT
// 16-row MFMA tiles of filter columns; a filter of W <= 4 taps takes 4 rows (one lane
// group), W = 5..8 take 8 rows (two lane groups). A workgroup of 4 waves covers
// 4 * MT * 16 / rows_per_channel channels.
#ifndef LOWRANK_FWD_MT
#define LOWRANK_FWD_MT 8
#endif
constexpr int lowrank_fwd_mt(int KS) { return KS <= 2 ? LOWRANK_FWD_MT : 4; }
constexpr int lowrank_rows_per_channel(int W) { return W > 4 ? 8 : 4; }
constexpr int lowrank_fwd_dc(int W, int KS) { return 4 * lowrank_fwd_mt(KS) * 16 / lowrank_rows_per_channel(W); }
// Backward: fewer filter tiles per wave (its registers also hold dU accumulators); the
// pipeline advances kLowrankBwdStep tokens per step.
constexpr int lowrank_bwd_mt(int) { return 2; }
constexpr int lowrank_bwd_dc(int W, int KS) { return 4 * lowrank_bwd_mt(KS) * 16 / lowrank_rows_per_channel(W); }
constexpr int kLowrankBwdStep = 64;
// dz kernel: tokens per workgroup (16 per wave) and channels per staged chunk.
constexpr int kLowrankDzTokens = 64;
constexpr int kLowrankDzChunk = 32;

struct LowRankPlan {
  int nCs, Ltok, nTr;
  int64_t blocks;
  size_t ws_dU, ws_db;  // byte offsets inside the workspace
  size_t ws_total;
};

// The general low-rank kernels for one storage type (one translation unit each).
hipError_t lowrank_dispatch_f32(const LowRankParams& p, const LowRankPlan& pl, int W, bool bwd, hipStream_t s);
hipError_t lowrank_dispatch_bf16(const LowRankParams& p, const LowRankPlan& pl, int W, bool bwd, hipStream_t s);
hipError_t lowrank_dispatch_f16(const LowRankParams& p, const LowRankPlan& pl, int W, bool bwd, hipStream_t s);

LowRankPlan plan_lowrank(int64_t B, int64_t T, int64_t D, int W, int H, int R, bool bwd, dynconv_dtype dt);

dynconv_status launch_lowrank_fwd(const LowRankParams& p, const LowRankPlan& plan, int W, dynconv_dtype dt,
                                  hipStream_t stream);
// Group sizes the fast bf16 kernels serve: H in {1, 2, 4, 8, 16}, so that a 64-channel
// slice holds whole groups (each channel loads its group's columns of U and of the bias).
bool lowrank_fast_group_ok(int H);
// 16-bit (bf16, float16) fast forward (LDS DMA pipeline; W <= 4, or W = 5..8 up to 64 ranks;
// R zero-padded to 32, 64 or 128 ranks (R <= 64 or R > 96) with 16-byte z pieces (aligned
// rows, R % 8 == 0) or 4-byte ones (R even), those H, 16-byte aligned activation rows, D a
// multiple of 64). It plans its own token ranges.
// Packed sequences on the fast forward: contiguous, 16-byte aligned id rows, T % 4 == 0.
bool lowrank_seg_fast_ok(const LowRankParams& p);
bool lowrank_fwd_fast_ok(const LowRankParams& p, int W, dynconv_dtype dt);
hipError_t launch_lowrank_fwd_fast(const LowRankParams& p, int W, dynconv_dtype dt, hipStream_t stream);
// Shapes and layouts the 16-bit fast backward serves (the forward's conditions, on x, dy,
// z and dx).
bool lowrank_bwd_fast_shape_ok(const LowRankParams& p, int W, dynconv_dtype dt);
// The 16-bit fast backward's dx and g / dU / db partial sums over the planned token ranges
// (Ltok, nTr) and 64-channel slices; one partial per token range and group column (a
// group's H channels summed inside the workgroup). Up to 64 ranks one kernel of 8 waves
// runs both (the roles share the staged dy and z); at 128 ranks two kernels of 4 waves.
hipError_t launch_lowrank_bwd_fused(const LowRankParams& p, int W, dynconv_dtype dt, hipStream_t stream);
// Whether the backward runs on the fast kernels (dx, then g / dU / db): they write
// B * nTr partials per filter column, the general kernel B * nTr * H.
bool lowrank_bwd_fast(const LowRankParams& p, int W, dynconv_dtype dt);

dynconv_status launch_lowrank_bwd(const LowRankParams& p, const LowRankPlan& plan, int W, dynconv_dtype dt,
                                  float* dU, float* db, hipStream_t stream);

}  // namespace dynconv
