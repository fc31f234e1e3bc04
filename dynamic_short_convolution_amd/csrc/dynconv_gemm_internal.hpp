// Internal interface of the projection + convolution kernel (dynconv_gemm.hip).
#pragma once

#include "dynconv_internal.hpp"

namespace dynconv {

// Tile of the fused kernel: 256 computed token rows (the first 16 only as the causal halo
// of the next 240) x 128 output columns, K in steps of 64.
constexpr int kGemmRows = 256;
constexpr int kGemmHalo = 16;
constexpr int kGemmOutRows = kGemmRows - kGemmHalo;
constexpr int kGemmCols = 128;
constexpr int kGemmK = 64;

struct GemmParams {
  const void* A;     // [B,T,K] activations, strides as0, as1 (elements), unit inner stride
  const void* Wp;    // [N,K] projection weight (a linear layer's out x in), rows ldw apart
  const void* w;     // per-token filters [B,T,N/H,W] (strides ws0, ws1; static: both 0)
  const void* z;     // low-rank: z [B,T,R] (strides zs0, zs1)
  const void* U;     // low-rank: U [R,(N/H)*W], rows ldu apart, column g*W + k
  const void* bias;  // low-rank: [(N/H)*W] or null
  void* y;           // [B,T,N] output, strides ys0, ys1
  int64_t as0, as1, ldw, ws0, ws1, zs0, zs1, ldu, ys0, ys1;
  int32_t B, T, N, K, H, R;
  int32_t M;         // B * T
  int32_t nTm, nTn;  // tiles along the rows and the columns
  int32_t uvec;      // low-rank: U rows allow 16-byte loads (base and ldu)
  int32_t zvec;      // low-rank: z rows allow 16-byte loads and R % 8 == 0
};

// Whether the kernels serve these sizes (the C ABI has checked everything else).
bool gemm_lowrank_fits(int W, int R);

// Per-token (or static) filters read from memory; `wvec` selects 8-byte tap loads (W == 4
// with 8-byte aligned filter rows).
hipError_t launch_gemm_conv(const GemmParams& p, int W, bool wvec, dynconv_dtype dt, hipStream_t s);
// Low-rank filters made on the matrix cores from z, U and the bias.
hipError_t launch_gemm_lowrank(const GemmParams& p, int W, dynconv_dtype dt, hipStream_t s);

}  // namespace dynconv
