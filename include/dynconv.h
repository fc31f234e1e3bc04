/*
 * dynconv.h: C ABI of the dynamic short convolution library (libdynconv.so), gfx950.
 *
 * The operation, from "Dynamic Short Convolutions Improve Transformers" (reading note),
 * section "Parameterization":
 *
 *   eq. 2 + eq. 3:   y[b,t,d] = x[b,t,d] + sum_{k=0}^{W-1} w[b,t,g(d),k] * x[b,t-k,d]
 *
 * with x[b,t,d] = 0 for t < 0 in every sequence b, g(d) = d / H (one filter shared by H
 * consecutive channels: H = 1 is the per-channel form, H > 1 the head-wise form), and a
 * static filter (eq. 1) as the case where w does not depend on (b, t). In the low-rank
 * form (same section, and "Efficient training (Triton kernels)") the filters are
 * generated on the GPU from z (B x T x R) and the second projection U (R x (D/H)*W)
 * plus a bias b: w[b,t,g,k] = sum_r z[b,t,r] U[r, g*W+k] + b[g*W+k], and are never
 * written to memory.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers. The caller owns every buffer, including
 *   the workspace; the library never allocates or frees device memory, never
 *   synchronises, and keeps no mutable global state (thread-safe) apart from the
 *   per-device address of dynconv_bwd_ex_noalloc's scratch array (set once, under a lock).
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and the call
 *   returns without waiting.
 * - Strides are in ELEMENTS, int64, in PyTorch .stride() order. Activation-shaped tensors
 *   (x, y, dy, dx) are [B, T, D] with strides s[0..2], s[2] == 1. Filter-shaped tensors
 *   (w, dw) are [B, T, D/H, W] with strides s[0..3], s[3] == 1 and s[2] == W (the W taps
 *   of one group are contiguous). w with s[0] == s[1] == 0 is a static filter [D/H, W].
 *   z and dz are [B, T, R] with strides s[0..2], s[2] == 1.
 * - Element types: x, w, z, U, bias, y, dy, dx, dw (per token) and dz all have `dtype`
 *   (float32, bfloat16 or float16). Reduced parameter gradients (static dw, dU, db) are
 *   always float32 and contiguous.
 * - Arithmetic is float32 (products and sums), 16-bit results are rounded to nearest even.
 *   The fast low-rank kernels serve bfloat16 and float16; float32 takes the general ones.
 * - Validation happens before any HIP call; invalid input returns a status, never aborts.
 *   B == 0 or T == 0 or D == 0 is a no-op returning DYNCONV_OK.
 * - Supported parameters: 1 <= W <= 8; H any divisor of D, with
 *   H / VEC <= 64 for the materialised and static forms, where VEC (channels per lane) is,
 *   in 16-bit storage, 2m when H = m * 2^k with m = 3 or 5 and k >= 1 and H itself when H is
 *   3 or 5, and otherwise the largest power of two that divides H and is at most the widest
 *   lane vector allowed by the alignment below / element size (so with 16-byte aligned
 *   activations: powers of two up to 512 in 16-bit storage and 256 in float32; H = 3 * 2^k up
 *   to 384 and H = 5 * 2^k up to 640 in 16-bit storage, 192 and 160 in float32; other odd H
 *   up to 63); low-rank form: 1 <= R <= 128.
 * - Alignment: base pointers of activation-shaped tensors and their s[0], s[1] (in bytes)
 *   must be multiples of 4 bytes (bf16: D even); wider lane vectors (8 or 16 bytes) are
 *   used when every activation-shaped tensor of the call allows them. Filters: base and
 *   s[0], s[1] multiples of 4 bytes for H == 1, and for H > 1 when the W taps of a group
 *   fill whole 32-bit words (float32, or bf16 with W even); element alignment otherwise.
 *   Violations return DYNCONV_ERR_UNSUPPORTED.
 * - An output pointer equal to any input pointer returns DYNCONV_ERR_INVALID_ARG
 *   (in-place use would corrupt the time halo); partial overlap is undefined behaviour.
 * - A failed kernel launch returns DYNCONV_ERR_HIP; dynconv_last_hip_error() then gives
 *   the hipError_t of the calling thread's last failure.
 */
#ifndef DYNCONV_H
#define DYNCONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type codes and status codes are plain 32-bit integers, so that any value a caller
 * passes is well defined (an unknown dtype code is refused with DYNCONV_ERR_INVALID_ARG). */
typedef int32_t dynconv_dtype;
enum { DYNCONV_F32 = 0, DYNCONV_BF16 = 1, DYNCONV_F16 = 2 };

typedef int32_t dynconv_status;
enum {
  DYNCONV_OK = 0,
  DYNCONV_ERR_INVALID_ARG = 1, /* null / negative / inconsistent argument, aliasing */
  DYNCONV_ERR_UNSUPPORTED = 2, /* valid per the equations but outside this library's limits */
  DYNCONV_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the size query */
  DYNCONV_ERR_HIP = 4          /* a HIP launch failed */
};

/* Human-readable name of a status code (static storage). */
const char* dynconv_status_string(dynconv_status s);

/* hipError_t (as int) of the calling thread's last DYNCONV_ERR_HIP, 0 if none. */
int dynconv_last_hip_error(void);

/*
 * Forward, eq. 2 + eq. 3 (eq. 1 when w is static).
 *   x  [B,T,D]      input activations (read once)
 *   w  [B,T,D/H,W]  per-token filters, or static [D/H,W] given by ws[0] == ws[1] == 0
 *   y  [B,T,D]      output, y = x + conv(x) (written once)
 */
dynconv_status dynconv_fwd(const void* x, const int64_t* xs, const void* w, const int64_t* ws,
                           void* y, const int64_t* ys, int64_t B, int64_t T, int64_t D, int32_t W,
                           int32_t H, dynconv_dtype dtype, void* stream);

/*
 * Backward of dynconv_fwd given dy = dL/dy (the exact adjoint of eq. 2 + eq. 3):
 *   dx[b,s,d]   = dy[b,s,d] + sum_k w[b,s+k,g(d),k] * dy[b,s+k,d]        (s + k < T)
 *   dw[b,t,g,k] = sum_{d : g(d) = g} dy[b,t,d] * x[b,t-k,d]              (0 for t < k)
 * x and w are independent inputs (the filters are generated from another tensor), so dx
 * has no term through w.
 *   dx  [B,T,D] or NULL to skip.
 *   dw  per-token filters: [B,T,D/H,W] with strides dws, dtype `dtype`, or NULL to skip.
 *       static w: float32 [D/H, W] contiguous, the sum over all (b, t); dws is ignored.
 * At least one of dx, dw must be non-NULL. A static w needs a workspace of
 * dynconv_bwd_workspace_size(...) bytes when dw is requested (per-tile partial sums,
 * reduced in a fixed order, so results are run-to-run deterministic).
 */
dynconv_status dynconv_bwd(const void* x, const int64_t* xs, const void* w, const int64_t* ws,
                           const void* dy, const int64_t* dys, void* dx, const int64_t* dxs, void* dw,
                           const int64_t* dws, int64_t B, int64_t T, int64_t D, int32_t W, int32_t H,
                           dynconv_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes needed by dynconv_bwd (0 unless the filter is static). */
size_t dynconv_bwd_workspace_size(int64_t B, int64_t T, int64_t D, int32_t W, int32_t H, int is_static,
                                  dynconv_dtype dtype);

/*
 * Low-rank forward: filters w[b,t,g,k] = sum_r z[b,t,r] U[r, g*W+k] + bias[g*W+k] are
 * formed on the GPU (matrix cores, float32 accumulation) and applied at once; they are
 * never written to memory. Then y = x + conv(x) as in dynconv_fwd.
 *   z     [B,T,R] with strides zs
 *   U     [R, (D/H)*W] with row stride ldu (elements), column j = g*W + k
 *   bias  [(D/H)*W] or NULL (zero bias)
 * Row strides (xs[1], zs[1], ys[1], ldu; and dys[1], dxs[1] of the backward) must be below
 * 2^24 elements (DYNCONV_ERR_UNSUPPORTED otherwise).
 */
dynconv_status dynconv_lowrank_fwd(const void* x, const int64_t* xs, const void* z, const int64_t* zs,
                                   const void* U, int64_t ldu, const void* bias, void* y, const int64_t* ys,
                                   int64_t B, int64_t T, int64_t D, int32_t W, int32_t H, int32_t R,
                                   dynconv_dtype dtype, void* stream);

/*
 * Low-rank backward. With g[b,t,j] = dw[b,t,g,k] (j = g*W + k) the per-token filter
 * gradient of dynconv_bwd (never written to memory):
 *   dx = as in dynconv_bwd with the generated filters,
 *   dz[b,t,r] = sum_j g[b,t,j] U[r,j],
 *   dU[r,j]   = sum_{b,t} z[b,t,r] g[b,t,j]   (float32 [R, (D/H)*W] contiguous, overwritten),
 *   db[j]     = sum_{b,t} g[b,t,j]            (float32 [(D/H)*W], overwritten; NULL to skip).
 * dx, dz and dU are required. Needs dynconv_lowrank_bwd_workspace_size(...) bytes of
 * workspace for fixed-order partial sums (run-to-run deterministic, no float atomics).
 */
dynconv_status dynconv_lowrank_bwd(const void* x, const int64_t* xs, const void* z, const int64_t* zs,
                                   const void* U, int64_t ldu, const void* bias, const void* dy,
                                   const int64_t* dys, void* dx, const int64_t* dxs, void* dz,
                                   const int64_t* dzs, float* dU, float* db, int64_t B, int64_t T, int64_t D,
                                   int32_t W, int32_t H, int32_t R, dynconv_dtype dtype, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Workspace bytes needed by dynconv_lowrank_bwd. */
size_t dynconv_lowrank_bwd_workspace_size(int64_t B, int64_t T, int64_t D, int32_t W, int32_t H, int32_t R,
                                          dynconv_dtype dtype);

/*
 * Inference: decoding one token at a time (the reading note lists inference among the
 * things it left unoptimised). A sequence keeps its last W-1 inputs in a rolling cache
 *   cache [B, W-1, D] with strides cs[0..2] (cs[2] == 1), dtype `dtype`,
 * where token s sits in slot s mod (W-1) and the slots of positions before 0 hold zeros
 * (the zero padding before t = 0). The cache is read and written in place. W == 1 needs
 * no cache (it may be NULL).
 */

/*
 * After a prompt of T tokens (y from dynconv_fwd or dynconv_lowrank_fwd on x [B,T,D]):
 * slot s mod (W-1) of each sequence receives x[b, s] for s = T-W+1 .. T-1, and zero for
 * s < 0 (so T == 0 empties the cache). Decoding then continues at t = T.
 */
dynconv_status dynconv_cache_fill(const void* x, const int64_t* xs, void* cache, const int64_t* cs, int64_t B,
                                  int64_t T, int64_t D, int32_t W, dynconv_dtype dtype, void* stream);

/*
 * One decoding step at token index t >= 0 (the same for every sequence of the batch):
 *   y[b,d] = x[b,d] + sum_{k<W} w[b,g(d),k] * x_{t-k}[b,d],   x_{t-k} from the cache for k >= 1,
 * after which x[b, :] is stored in slot t mod (W-1). Equal to row t of dynconv_fwd over the
 * whole sequence.
 *   x  [B, D] with strides xs[0..1] (xs[1] == 1)
 *   w  [B, D/H, W] with strides ws[0..2] (ws[2] == 1, ws[1] == W), or a static filter
 *      [D/H, W] given by ws[0] == 0
 *   y  [B, D] with strides ys[0..1] (ys[1] == 1); y may not be x, w or the cache.
 */
dynconv_status dynconv_decode_step(const void* x, const int64_t* xs, const void* w, const int64_t* ws,
                                   void* cache, const int64_t* cs, void* y, const int64_t* ys, int64_t t,
                                   int64_t B, int64_t D, int32_t W, int32_t H, dynconv_dtype dtype, void* stream);

/*
 * Low-rank decoding step: the filters of the new token, w[b,g,k] = sum_r z[b,r] U[r, g*W+k]
 * + bias[g*W+k], are formed on the GPU (float32) and applied as in dynconv_decode_step.
 *   z  [B, R] with strides zs[0..1] (zs[1] == 1); U, ldu, bias as in dynconv_lowrank_fwd.
 * 1 <= R <= 128, W <= 8.
 */
dynconv_status dynconv_lowrank_decode_step(const void* x, const int64_t* xs, const void* z, const int64_t* zs,
                                           const void* U, int64_t ldu, const void* bias, void* cache,
                                           const int64_t* cs, void* y, const int64_t* ys, int64_t t, int64_t B,
                                           int64_t D, int32_t W, int32_t H, int32_t R, dynconv_dtype dtype,
                                           void* stream);

/*
 * Packed sequences (several documents in one row of x): the same calls with a segment id
 * per token,
 *   seq_idx  int32 [B,T] with strides ss[0..1] >= 0 (elements), 4-byte aligned,
 * after which tap k of token t is present only when seq_idx[b,t-k] == seq_idx[b,t]: a
 * document never reads the inputs of the one before it (the RubiConv page's point that
 * a convolution over packed sequences must not cross a document start). Documents are
 * normally contiguous runs of equal ids; any ids work, the test is equality. Gradients
 * are those of the masked forward. The bf16 fast low-rank kernels take packed calls whose
 * id rows are contiguous, 16-byte aligned and T % 4 == 0; others take the general kernels.
 * seq_idx == NULL returns DYNCONV_ERR_INVALID_ARG; every other argument is as in the call
 * without the suffix.
 */
dynconv_status dynconv_fwd_varlen(const void* x, const int64_t* xs, const void* w, const int64_t* ws,
                                  const int32_t* seq_idx, const int64_t* ss, void* y, const int64_t* ys, int64_t B,
                                  int64_t T, int64_t D, int32_t W, int32_t H, dynconv_dtype dtype, void* stream);

dynconv_status dynconv_bwd_varlen(const void* x, const int64_t* xs, const void* w, const int64_t* ws,
                                  const int32_t* seq_idx, const int64_t* ss, const void* dy, const int64_t* dys,
                                  void* dx, const int64_t* dxs, void* dw, const int64_t* dws, int64_t B, int64_t T,
                                  int64_t D, int32_t W, int32_t H, dynconv_dtype dtype, void* workspace,
                                  size_t workspace_bytes, void* stream);

dynconv_status dynconv_lowrank_fwd_varlen(const void* x, const int64_t* xs, const void* z, const int64_t* zs,
                                          const void* U, int64_t ldu, const void* bias, const int32_t* seq_idx,
                                          const int64_t* ss, void* y, const int64_t* ys, int64_t B, int64_t T,
                                          int64_t D, int32_t W, int32_t H, int32_t R, dynconv_dtype dtype,
                                          void* stream);

dynconv_status dynconv_lowrank_bwd_varlen(const void* x, const int64_t* xs, const void* z, const int64_t* zs,
                                          const void* U, int64_t ldu, const void* bias, const int32_t* seq_idx,
                                          const int64_t* ss, const void* dy, const int64_t* dys, void* dx,
                                          const int64_t* dxs, void* dz, const int64_t* dzs, float* dU, float* db,
                                          int64_t B, int64_t T, int64_t D, int32_t W, int32_t H, int32_t R,
                                          dynconv_dtype dtype, void* workspace, size_t workspace_bytes,
                                          void* stream);

/*
 * Optional convolution bias (the Conv1D module of the convolution technical report: a
 * per-channel bias c added to every output, y = x + conv(x) + c), together with optional
 * segment ids (seq_idx == NULL: one document per row, ss ignored):
 *   conv_bias   [D] of `dtype`, contiguous, 4-byte aligned, or NULL
 *   dconv_bias  [D] float32, overwritten with sum over (b, t) of dy (NULL to skip)
 * The backward's workspace then holds float32 partial sums of dy per (sequence, time
 * chunk) after those of a static filter: size it with dynconv_bwd_ex_workspace_size.
 * Materialised, static and head-wise forms (the low-rank form: dynconv_lowrank_*_ex below);
 * the decoding step adds c to its output.
 */
dynconv_status dynconv_fwd_ex(const void* x, const int64_t* xs, const void* w, const int64_t* ws,
                              const int32_t* seq_idx, const int64_t* ss, const void* conv_bias, void* y,
                              const int64_t* ys, int64_t B, int64_t T, int64_t D, int32_t W, int32_t H,
                              dynconv_dtype dtype, void* stream);

size_t dynconv_bwd_ex_workspace_size(int64_t B, int64_t T, int64_t D, int32_t W, int32_t H, int is_static,
                                     int want_dconv_bias, dynconv_dtype dtype);

dynconv_status dynconv_bwd_ex(const void* x, const int64_t* xs, const void* w, const int64_t* ws,
                              const int32_t* seq_idx, const int64_t* ss, const void* dy, const int64_t* dys, void* dx,
                              const int64_t* dxs, void* dw, const int64_t* dws, float* dconv_bias, int64_t B,
                              int64_t T, int64_t D, int32_t W, int32_t H, dynconv_dtype dtype, void* workspace,
                              size_t workspace_bytes, void* stream);

dynconv_status dynconv_decode_step_ex(const void* x, const int64_t* xs, const void* w, const int64_t* ws,
                                      const void* conv_bias, void* cache, const int64_t* cs, void* y,
                                      const int64_t* ys, int64_t t, int64_t B, int64_t D, int32_t W, int32_t H,
                                      dynconv_dtype dtype, void* stream);

/*
 * The same optional convolution bias on the low-rank form (y = x + conv(x) + c with the
 * generated filters), together with optional segment ids (seq_idx == NULL: one document
 * per row, ss ignored); every other argument is as in dynconv_lowrank_{fwd,bwd} and
 * dynconv_lowrank_decode_step.
 *   conv_bias   [D] of `dtype`, contiguous, 4-byte aligned (decoding step: element
 *               aligned), or NULL
 *   dconv_bias  [D] float32, 4-byte aligned, overwritten with sum over (b, t) of dy (NULL
 *               to skip); its float32 partial sums per (sequence, chunk of tokens) take
 *               workspace after those of dU and db: size the workspace with
 *               dynconv_lowrank_bwd_ex_workspace_size(..., want_dconv_bias = 1, ...).
 * The bias gradient reads dy once more (one extra pass over B*T*D elements).
 */
dynconv_status dynconv_lowrank_fwd_ex(const void* x, const int64_t* xs, const void* z, const int64_t* zs,
                                      const void* U, int64_t ldu, const void* bias, const int32_t* seq_idx,
                                      const int64_t* ss, const void* conv_bias, void* y, const int64_t* ys, int64_t B,
                                      int64_t T, int64_t D, int32_t W, int32_t H, int32_t R, dynconv_dtype dtype,
                                      void* stream);

size_t dynconv_lowrank_bwd_ex_workspace_size(int64_t B, int64_t T, int64_t D, int32_t W, int32_t H, int32_t R,
                                             int want_dconv_bias, dynconv_dtype dtype);

dynconv_status dynconv_lowrank_bwd_ex(const void* x, const int64_t* xs, const void* z, const int64_t* zs,
                                      const void* U, int64_t ldu, const void* bias, const int32_t* seq_idx,
                                      const int64_t* ss, const void* dy, const int64_t* dys, void* dx,
                                      const int64_t* dxs, void* dz, const int64_t* dzs, float* dU, float* db,
                                      float* dconv_bias, int64_t B, int64_t T, int64_t D, int32_t W, int32_t H,
                                      int32_t R, dynconv_dtype dtype, void* workspace, size_t workspace_bytes,
                                      void* stream);

dynconv_status dynconv_lowrank_decode_step_ex(const void* x, const int64_t* xs, const void* z, const int64_t* zs,
                                              const void* U, int64_t ldu, const void* bias, const void* conv_bias,
                                              void* cache, const int64_t* cs, void* y, const int64_t* ys, int64_t t,
                                              int64_t B, int64_t D, int32_t W, int32_t H, int32_t R,
                                              dynconv_dtype dtype, void* stream);

/*
 * The convolution in the epilogue of the producing projection (the reading note's
 * end-to-end throughput section, closing analysis: fusing the dynamic convolution into
 * the matmul epilogue removes memory traffic; its "Parameterization" section puts the
 * convolution on the QKV projection's outputs). One kernel computes
 *   X = A W_p^T          (the projection; X is never written to memory)
 *   y = X + conv(X)      (eq. 2 + eq. 3 on X, zeros before t = 0 of every sequence)
 * with float32 accumulation (X is not rounded before the convolution).
 *   A   [B,T,K] activations with strides as[0..2], as[2] == 1
 *   Wp  [N,K] projection weight (a linear layer's out x in layout), rows ldw apart
 *   y   [B,T,N] with strides ys[0..2], ys[2] == 1
 * dynconv_gemm_fwd takes per-token filters w [B,T,N/H,W] (strides ws, ws[3] == 1,
 * ws[2] == W; ws[0] == ws[1] == 0: a static [N/H,W] filter); dynconv_gemm_lowrank_fwd
 * forms them as w = z U + bias on the matrix cores (z [B,T,R] strides zs, zs[2] == 1;
 * U [R,(N/H)*W] rows ldu apart, column g*W + k; bias [(N/H)*W] or NULL).
 * Limits (DYNCONV_ERR_UNSUPPORTED otherwise): bfloat16 or float16; 1 <= W <= 5;
 * H in {1, 2, 4, 8, 16}; K a positive multiple of 64; N a multiple of 128; B*T < 2^31;
 * A and W_p rows 16-byte aligned (base, as[0], as[1], ldw); low-rank: R <= 128 with
 * W * (32 ceil(R/32) + 8) <= 552 (R <= 128 at W <= 4, R <= 96 at W = 5).
 * y may not be any input (DYNCONV_ERR_INVALID_ARG). Forward only.
 */
dynconv_status dynconv_gemm_fwd(const void* A, const int64_t* as, const void* Wp, int64_t ldw, const void* w,
                                const int64_t* ws, void* y, const int64_t* ys, int64_t B, int64_t T, int64_t N,
                                int64_t K, int32_t W, int32_t H, dynconv_dtype dtype, void* stream);

dynconv_status dynconv_gemm_lowrank_fwd(const void* A, const int64_t* as, const void* Wp, int64_t ldw, const void* z,
                                        const int64_t* zs, const void* U, int64_t ldu, const void* bias, void* y,
                                        const int64_t* ys, int64_t B, int64_t T, int64_t N, int64_t K, int32_t W,
                                        int32_t H, int32_t R, dynconv_dtype dtype, void* stream);

/*
 * Allocation-free backward, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). The same
 * operation and arguments as dynconv_bwd_ex, without a workspace: the float32 partial
 * sums of a static filter's dw and of dconv_bias go to a scratch array that the library
 * holds in device memory, DYNCONV_NOALLOC_SCRATCH_BYTES per GPU, kept from the library's
 * load until the process ends. Calls that need no partial sums (per-token filters without
 * dconv_bias) do not touch it.
 *   - A call whose partial sums need more than DYNCONV_NOALLOC_SCRATCH_BYTES (the bytes
 *     dynconv_bwd_ex_workspace_size reports) returns DYNCONV_ERR_WORKSPACE.
 *   - The scratch array of the CURRENT device is used: `stream` must belong to it. Its
 *     device address is resolved on the first call on each device (hipGetSymbolAddress),
 *     so that first call must not be made during a graph capture.
 *   - Every call on a GPU shares that GPU's array: calls that overlap in time on one GPU
 *     (on different streams, or from different threads without ordering) race and give
 *     wrong sums. Calls ordered on one stream are safe; each call overwrites every
 *     partial it later reads, so nothing has to start at zero.
 *   - No hipMalloc, hipFree or allocating library routine is called.
 */
#define DYNCONV_NOALLOC_SCRATCH_BYTES (16u << 20)

dynconv_status dynconv_bwd_ex_noalloc(const void* x, const int64_t* xs, const void* w, const int64_t* ws,
                                      const int32_t* seq_idx, const int64_t* ss, const void* dy, const int64_t* dys,
                                      void* dx, const int64_t* dxs, void* dw, const int64_t* dws, float* dconv_bias,
                                      int64_t B, int64_t T, int64_t D, int32_t W, int32_t H, dynconv_dtype dtype,
                                      void* stream);

/*
 * Cache fill after a packed prompt: decoding continues the document of token T-1, so the
 * slots of tokens with another segment id than token T-1 are zero (the start of that
 * document). T == 0 empties the cache as in dynconv_cache_fill.
 */
dynconv_status dynconv_cache_fill_varlen(const void* x, const int64_t* xs, const int32_t* seq_idx, const int64_t* ss,
                                         void* cache, const int64_t* cs, int64_t B, int64_t T, int64_t D, int32_t W,
                                         dynconv_dtype dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DYNCONV_H */
