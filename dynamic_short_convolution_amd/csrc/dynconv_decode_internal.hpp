// Internal interface of the inference kernels: the rolling cache of the last W-1 inputs
// and the single-token decoding step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dynconv.h"

namespace dynconv {

struct DecodeParams {
  const void* x;    // cache fill: [B,T,D] (xs0, xs1); decoding step: [B,D] (xs0)
  const void* w;    // [B,D/H,W] (ws0; taps of a group contiguous), static: ws0 == 0
  const void* z;    // low-rank: [B,R] (zs0)
  const void* U;    // low-rank: [R,(D/H)*W] (ldu)
  const void* bias; // low-rank: [(D/H)*W] or null
  void* cache;      // [B,W-1,D] (cs0, cs1); token s in slot s mod (W-1)
  void* y;          // [B,D] (ys0)
  int64_t xs0, xs1, ws0, zs0, ldu, cs0, cs1, ys0;
  int64_t t;        // decoding step: index of the new token; cache fill: prompt length T
  int32_t B, D, H, R;
  const void* cbias;   // decoding step (materialised filters): optional convolution bias [D], or null
  const int32_t* seg;  // cache fill of packed prompts: segment id per token [B,T] (ss0, ss1), or null
  int64_t ss0, ss1;
};

dynconv_status launch_cache_fill(const DecodeParams& p, int W, dynconv_dtype dt, hipStream_t s);
dynconv_status launch_decode_step(const DecodeParams& p, int W, dynconv_dtype dt, hipStream_t s);
dynconv_status launch_lowrank_decode_step(const DecodeParams& p, int W, dynconv_dtype dt, hipStream_t s);

}  // namespace dynconv
