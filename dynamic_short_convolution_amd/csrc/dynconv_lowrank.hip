// Low-rank form: planning and launch. The general kernels are in
// dynconv_lowrank_kernels.hpp (compiled once per storage type), the bf16 fast ones in
// dynconv_lowrank_fast.hip.
#include "dynconv_common.hpp"
#include "dynconv_internal.hpp"
#include "dynconv_lowrank_internal.hpp"

namespace dynconv {

LowRankPlan plan_lowrank(int64_t B, int64_t T, int64_t D, int W, int H, int R, bool bwd, dynconv_dtype dt) {
  LowRankPlan pl{};
  const int ks = (R + 31) / 32;
  const int DC = !bwd ? lowrank_fwd_dc(W, ks) : lowrank_bwd_dc(W, ks);
  pl.nCs = int((D + DC - 1) / DC);
  // About 1024 (forward) or 2048 (backward) workgroups, ranges in whole 16-token tiles.
  // Where the bf16 fast kernels can serve the backward, its partial sums of dU and db come
  // from a kernel over 64-channel slices: about 512 workgroups then, so that fewer float32
  // partial sums are written and reduced (two per sequence at the pages' model shapes).
  // The choice uses only what the workspace query knows; if alignment then rules the fast
  // kernels out, the main kernel runs with these token ranges instead.
  const int ksr = (R + 31) / 32;
  const bool lean = bwd && (dt == DYNCONV_BF16 || dt == DYNCONV_F16) && lowrank_fast_group_ok(H) &&
                    (W <= 4 || (W == 5 && ksr <= 2)) &&
                    R % 2 == 0 && ksr != 3 && D % 64 == 0;
  const int64_t target = !bwd ? 1024 : lean ? 512 : 2048;
  const int64_t slices = lean ? D / 64 : pl.nCs;  // the fast kernel's 64-channel slices
  int64_t per_seq = (target + B * slices - 1) / (B * slices);
  const int64_t max_ranges = (T + kLowrankTT - 1) / kLowrankTT;
  if (per_seq > max_ranges) per_seq = max_ranges;
  if (per_seq < 1) per_seq = 1;
  int64_t L = (T + per_seq - 1) / per_seq;
  const int64_t step = bwd ? kLowrankBwdStep : kLowrankTT;
  L = (L + step - 1) / step * step;
  pl.Ltok = int(L);
  pl.nTr = int((T + L - 1) / L);
  pl.blocks = B * int64_t(pl.nTr) * pl.nCs;
  const int64_t J = (D / H) * W;
  const int64_t nR = B * int64_t(pl.nTr);
  // one partial per (token range, channel of a group): H of them per group column
  pl.ws_dU = 0;
  pl.ws_db = size_t(nR) * size_t(H) * size_t(R) * size_t(J) * sizeof(float);
  pl.ws_total = bwd ? pl.ws_db + size_t(nR) * size_t(H) * size_t(J) * sizeof(float) : 0;
  return pl;
}

dynconv_status launch_lowrank_fwd(const LowRankParams& p, const LowRankPlan& plan, int W, dynconv_dtype dt,
                                  hipStream_t stream) {
  if (lowrank_fwd_fast_ok(p, W, dt) && (p.seg == nullptr || lowrank_seg_fast_ok(p))) {
    const hipError_t e = launch_lowrank_fwd_fast(p, W, dt, stream);
    return e == hipSuccess ? DYNCONV_OK : record_hip_error(e);
  }
  const hipError_t e = dt == DYNCONV_BF16   ? lowrank_dispatch_bf16(p, plan, W, false, stream)
                       : dt == DYNCONV_F16 ? lowrank_dispatch_f16(p, plan, W, false, stream)
                                           : lowrank_dispatch_f32(p, plan, W, false, stream);
  return e == hipSuccess ? DYNCONV_OK : record_hip_error(e);
}

dynconv_status launch_lowrank_bwd(const LowRankParams& p, const LowRankPlan& plan, int W, dynconv_dtype dt,
                                  float* dU, float* db, hipStream_t stream) {
  const hipError_t e = dt == DYNCONV_BF16   ? lowrank_dispatch_bf16(p, plan, W, true, stream)
                       : dt == DYNCONV_F16 ? lowrank_dispatch_f16(p, plan, W, true, stream)
                                           : lowrank_dispatch_f32(p, plan, W, true, stream);
  if (e != hipSuccess) return record_hip_error(e);
  // partials per filter column: one per token range on the fast kernels, one per (token
  // range, channel of the group) on the general kernel
  const int64_t nR = int64_t(p.B) * plan.nTr * (lowrank_bwd_fast(p, W, dt) ? 1 : p.H);
  if (db == nullptr) return launch_reduce_partials(p.part_dU, nR, int64_t(p.R) * p.J, dU, stream);
  return launch_reduce_partials2(p.part_dU, int64_t(p.R) * p.J, dU, p.part_db, p.J, db, nR, stream);
}

}  // namespace dynconv
