// C ABI of libdynconv: argument checks (before any HIP call) and dispatch to the
// kernel launchers. See include/dynconv.h for the contract of every entry point.
#include <hip/hip_runtime.h>

#include <mutex>

#include "dynconv_decode_internal.hpp"
#include "dynconv_gemm_internal.hpp"
#include "dynconv_internal.hpp"
#include "dynconv_lowrank_internal.hpp"

namespace dynconv {

namespace {

thread_local int g_last_hip_error = 0;

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int elem_bytes(dynconv_dtype dt) { return dt == DYNCONV_F32 ? 4 : 2; }

bool aligned(const void* p, int64_t a) { return (reinterpret_cast<uintptr_t>(p) % uint64_t(a)) == 0; }

// Activation-shaped tensor [B,T,D] with strides s[0..2].
struct Act {
  const void* p;
  const int64_t* s;
};

dynconv_status check_act(const void* p, const int64_t* s, bool required) {
  if (p == nullptr) return required ? DYNCONV_ERR_INVALID_ARG : DYNCONV_OK;
  if (s == nullptr) return DYNCONV_ERR_INVALID_ARG;
  if (s[2] != 1) return DYNCONV_ERR_UNSUPPORTED;
  if (s[0] < 0 || s[1] < 0) return DYNCONV_ERR_UNSUPPORTED;
  return DYNCONV_OK;
}

// Every activation-shaped tensor must allow 4-byte lane vectors; `wide` reports whether
// all of them also allow 16-byte vectors.
bool act_align_ok(const Act* a, int n, int eb, int64_t align_bytes) {
  for (int i = 0; i < n; ++i) {
    if (a[i].p == nullptr) continue;
    if (!aligned(a[i].p, align_bytes)) return false;
    if ((a[i].s[0] * eb) % align_bytes != 0 || (a[i].s[1] * eb) % align_bytes != 0) return false;
  }
  return true;
}

dynconv_status check_common(int64_t B, int64_t T, int64_t D, int32_t W, int32_t H, dynconv_dtype dt) {
  if (dt != DYNCONV_F32 && dt != DYNCONV_BF16 && dt != DYNCONV_F16) return DYNCONV_ERR_INVALID_ARG;
  if (B < 0 || T < 0 || D < 0) return DYNCONV_ERR_INVALID_ARG;
  if (W < 1 || H < 1) return DYNCONV_ERR_INVALID_ARG;
  if (W > kMaxW) return DYNCONV_ERR_UNSUPPORTED;
  if (D > 0 && D % H != 0) return DYNCONV_ERR_INVALID_ARG;
  if (B > INT32_MAX || T > INT32_MAX || D > INT32_MAX) return DYNCONV_ERR_UNSUPPORTED;
  // Token indices, and a token plus a step of lookahead, stay in int; so do the filter
  // column counts (D/H)*W.
  if (T > INT32_MAX - 65536 || D * W > INT32_MAX) return DYNCONV_ERR_UNSUPPORTED;
  // Every kernel's workgroup covers at least 16 tokens (or all of T) and 16 channels (or
  // all of D), so this bounds every grid by INT32_MAX workgroups.
  const int64_t bt = B * ((T + 15) / 16);
  if (bt > 0 && (D + 15) / 16 > INT32_MAX / bt) return DYNCONV_ERR_UNSUPPORTED;
  return DYNCONV_OK;
}

// Widest lane vector (16, 8 or 4 bytes) that every activation-shaped tensor allows, or 0.
int act_alignment(const Act* a, int n, int eb) {
  for (int al : {16, 8, 4})
    if (act_align_ok(a, n, eb, al)) return al;
  return 0;
}

// The lane layout of the streaming kernels puts VEC channels on a lane and H / VEC lanes
// on a group (group_vec), at most a wave; activation rows are whole 32-bit words, so with
// 16-bit elements D must be even.
dynconv_status check_stream_layout(int64_t D, int32_t H, int eb, int act_align) {
  if (act_align == 0 || D % (4 / eb) != 0) return DYNCONV_ERR_UNSUPPORTED;
  // the backward's layout has the most lanes per group
  if (H > 1 && H / group_vec(H, eb, act_align, true) > kWaveSize) return DYNCONV_ERR_UNSUPPORTED;
  return DYNCONV_OK;
}

// Filter groups (H > 1) of whole 32-bit words are read as words: 4-byte alignment.
bool group_words_aligned(const void* w, const int64_t* ws, int32_t W, int eb) {
  if ((int64_t(W) * eb) % 4 != 0) return true;
  return aligned(w, 4) && (ws[0] * eb) % 4 == 0 && (ws[1] * eb) % 4 == 0;
}

struct FilterInfo {
  bool is_static;
};

dynconv_status check_filter(const void* w, const int64_t* ws, int32_t W, int32_t H, int eb, bool bwd,
                            FilterInfo* fi) {
  if (w == nullptr || ws == nullptr) return DYNCONV_ERR_INVALID_ARG;
  if (ws[3] != 1 || ws[2] != W) return DYNCONV_ERR_UNSUPPORTED;
  if (ws[0] < 0 || ws[1] < 0) return DYNCONV_ERR_UNSUPPORTED;
  fi->is_static = ws[0] == 0 && ws[1] == 0;
  if (bwd && !fi->is_static && (ws[0] == 0 || ws[1] == 0)) return DYNCONV_ERR_UNSUPPORTED;
  if (H == 1) {
    if (!aligned(w, 4) || (ws[0] * eb) % 4 != 0 || (ws[1] * eb) % 4 != 0) return DYNCONV_ERR_UNSUPPORTED;
  } else if (!aligned(w, eb) || !group_words_aligned(w, ws, W, eb)) {
    return DYNCONV_ERR_UNSUPPORTED;
  }
  return DYNCONV_OK;
}

// Segment ids of packed sequences: int32 [B,T] with strides ss[0..1] >= 0 (any strides,
// read one id per token), 4-byte aligned.
dynconv_status check_seg(const int32_t* seg, const int64_t* ss) {
  if (seg == nullptr || ss == nullptr) return DYNCONV_ERR_INVALID_ARG;
  if (ss[0] < 0 || ss[1] < 0) return DYNCONV_ERR_UNSUPPORTED;
  if (!aligned(seg, 4)) return DYNCONV_ERR_UNSUPPORTED;
  return DYNCONV_OK;
}

}  // namespace

dynconv_status record_hip_error(hipError_t e) {
  g_last_hip_error = int(e);
  return DYNCONV_ERR_HIP;
}

int last_hip_error() { return g_last_hip_error; }

}  // namespace dynconv

using namespace dynconv;

extern "C" {

const char* dynconv_status_string(dynconv_status s) {
  switch (s) {
    case DYNCONV_OK: return "DYNCONV_OK";
    case DYNCONV_ERR_INVALID_ARG: return "DYNCONV_ERR_INVALID_ARG";
    case DYNCONV_ERR_UNSUPPORTED: return "DYNCONV_ERR_UNSUPPORTED";
    case DYNCONV_ERR_WORKSPACE: return "DYNCONV_ERR_WORKSPACE";
    case DYNCONV_ERR_HIP: return "DYNCONV_ERR_HIP";
  }
  return "DYNCONV_UNKNOWN_STATUS";
}

int dynconv_last_hip_error(void) { return dynconv::last_hip_error(); }

}  // extern "C"

namespace {

dynconv_status fwd_impl(const void* x, const int64_t* xs, const void* w, const int64_t* ws, const int32_t* seg,
                        const int64_t* ss, const void* cbias, void* y, const int64_t* ys, int64_t B, int64_t T,
                        int64_t D, int32_t W, int32_t H, dynconv_dtype dtype, void* stream) {
  dynconv_status st = check_common(B, T, D, W, H, dtype);
  if (st != DYNCONV_OK) return st;
  if ((st = check_act(x, xs, true)) != DYNCONV_OK) return st;
  if ((st = check_act(y, ys, true)) != DYNCONV_OK) return st;
  const int eb = elem_bytes(dtype);
  FilterInfo fi{};
  if ((st = check_filter(w, ws, W, H, eb, false, &fi)) != DYNCONV_OK) return st;
  if (y == x || y == w || (cbias != nullptr && y == cbias)) return DYNCONV_ERR_INVALID_ARG;
  if (cbias != nullptr && !aligned(cbias, 4)) return DYNCONV_ERR_UNSUPPORTED;
  if (B == 0 || T == 0 || D == 0) return DYNCONV_OK;
  const Act acts[2] = {{x, xs}, {y, ys}};
  const int align = act_alignment(acts, 2, eb);
  if ((st = check_stream_layout(D, H, eb, align)) != DYNCONV_OK) return st;

  const StreamPlan plan = plan_stream(B, T, D, W, H, eb, align, false, fi.is_static);
  StreamParams p{};
  p.x = x;
  p.w = w;
  p.out = y;
  p.cbias = cbias;
  if (seg != nullptr) {
    p.seg = seg;
    p.ss0 = ss[0];
    p.ss1 = ss[1];
  }
  p.xs0 = xs[0];
  p.xs1 = xs[1];
  p.ws0 = ws[0];
  p.ws1 = ws[1];
  p.os0 = ys[0];
  p.os1 = ys[1];
  p.B = int32_t(B);
  p.T = int32_t(T);
  p.D = int32_t(D);
  p.H = H;
  p.G = int32_t(D / H);
  p.lpg = plan.lpg;
  p.lpw = plan.lpw;
  p.L = plan.L;
  p.nTw = plan.nTw;
  p.nDw = plan.nDw;
  p.WD = plan.WD;
  p.WT = plan.WT;
  p.nDb = plan.nDb;
  p.nTb = plan.nTb;
  return launch_stream_fwd(p, plan, W, dtype, fi.is_static, static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

dynconv_status dynconv_fwd(const void* x, const int64_t* xs, const void* w, const int64_t* ws, void* y,
                           const int64_t* ys, int64_t B, int64_t T, int64_t D, int32_t W, int32_t H,
                           dynconv_dtype dtype, void* stream) {
  return fwd_impl(x, xs, w, ws, nullptr, nullptr, nullptr, y, ys, B, T, D, W, H, dtype, stream);
}

dynconv_status dynconv_fwd_varlen(const void* x, const int64_t* xs, const void* w, const int64_t* ws,
                                  const int32_t* seq_idx, const int64_t* ss, void* y, const int64_t* ys, int64_t B,
                                  int64_t T, int64_t D, int32_t W, int32_t H, dynconv_dtype dtype, void* stream) {
  const dynconv_status st = check_seg(seq_idx, ss);
  if (st != DYNCONV_OK) return st;
  return fwd_impl(x, xs, w, ws, seq_idx, ss, nullptr, y, ys, B, T, D, W, H, dtype, stream);
}

dynconv_status dynconv_fwd_ex(const void* x, const int64_t* xs, const void* w, const int64_t* ws,
                              const int32_t* seq_idx, const int64_t* ss, const void* conv_bias, void* y,
                              const int64_t* ys, int64_t B, int64_t T, int64_t D, int32_t W, int32_t H,
                              dynconv_dtype dtype, void* stream) {
  if (seq_idx != nullptr) {
    const dynconv_status st = check_seg(seq_idx, ss);
    if (st != DYNCONV_OK) return st;
  }
  return fwd_impl(x, xs, w, ws, seq_idx, ss, conv_bias, y, ys, B, T, D, W, H, dtype, stream);
}

}  // extern "C"

namespace {

// Workspace of the backward: float32 partial sums per (sequence, time chunk), of the
// static filter gradient [D/H][W] and/or of the convolution-bias gradient [D] (in that
// order). The chunking depends on the lane vector width only through nDw; take the
// largest over the possible widths.
size_t bwd_partial_floats(const StreamPlan& pl, int64_t B, int64_t D, int32_t W, int32_t H, bool static_dw,
                          bool dcbias) {
  return size_t(B) * size_t(pl.nTw) * ((static_dw ? size_t(D / H) * size_t(W) : 0) + (dcbias ? size_t(D) : 0));
}

size_t bwd_workspace(int64_t B, int64_t T, int64_t D, int32_t W, int32_t H, bool is_static, bool dcbias,
                     dynconv_dtype dtype) {
  if (check_common(B, T, D, W, H, dtype) != DYNCONV_OK) return 0;
  if ((!is_static && !dcbias) || B == 0 || T == 0 || D == 0) return 0;
  const int eb = elem_bytes(dtype);
  size_t best = 0;
  for (int align : {4, 8, 16}) {
    // only the lane layouts a call can take (a group wider than a wave has no plan)
    if (check_stream_layout(D, H, eb, align) != DYNCONV_OK) continue;
    const StreamPlan pl = plan_stream(B, T, D, W, H, eb, align, true, is_static);
    const size_t need = bwd_partial_floats(pl, B, D, W, H, is_static, dcbias) * sizeof(float);
    if (need > best) best = need;
  }
  return best;
}

}  // namespace

extern "C" {

size_t dynconv_bwd_workspace_size(int64_t B, int64_t T, int64_t D, int32_t W, int32_t H, int is_static,
                                  dynconv_dtype dtype) {
  return bwd_workspace(B, T, D, W, H, is_static != 0, false, dtype);
}

size_t dynconv_bwd_ex_workspace_size(int64_t B, int64_t T, int64_t D, int32_t W, int32_t H, int is_static,
                                     int want_dconv_bias, dynconv_dtype dtype) {
  return bwd_workspace(B, T, D, W, H, is_static != 0, want_dconv_bias != 0, dtype);
}

}  // extern "C"

// ---------------------------------------------------------------------------------
// Scratch memory of the allocation-free backward (dynconv_bwd_ex_noalloc): a file-scope
// device array, one copy per GPU, resolved to a device address once per device with
// hipGetSymbolAddress. Host code never passes the array's own name to a kernel or a copy
// (in host code that name is a host-side stand-in, not a device address); it uses the
// resolved pointer.
// ---------------------------------------------------------------------------------
constexpr size_t kScratchBytes = DYNCONV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of the current device's scratch array (resolved on the first call on
// that device; the call must not be inside a graph capture then).
dynconv_status current_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return record_hip_error(e);
  if (dev < 0 || dev >= kMaxScratchDevices) return DYNCONV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return record_hip_error(e);
    if (ptr == nullptr) return record_hip_error(hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DYNCONV_OK;
}

}  // namespace

namespace {

// use_scratch: the partial sums go to the current device's scratch array instead of a
// caller's workspace (workspace / workspace_bytes are then ignored); a call that needs
// more than kScratchBytes returns DYNCONV_ERR_WORKSPACE.
dynconv_status bwd_impl(const void* x, const int64_t* xs, const void* w, const int64_t* ws, const int32_t* seg,
                        const int64_t* ss, const void* dy, const int64_t* dys, void* dx, const int64_t* dxs, void* dw,
                        const int64_t* dws, float* dcb, int64_t B, int64_t T, int64_t D, int32_t W, int32_t H,
                        dynconv_dtype dtype, void* workspace, size_t workspace_bytes, void* stream,
                        bool use_scratch = false) {
  dynconv_status st = check_common(B, T, D, W, H, dtype);
  if (st != DYNCONV_OK) return st;
  if (dx == nullptr && dw == nullptr) return DYNCONV_ERR_INVALID_ARG;
  if (dcb != nullptr && !aligned(dcb, 4)) return DYNCONV_ERR_UNSUPPORTED;
  if ((st = check_act(x, xs, true)) != DYNCONV_OK) return st;
  if ((st = check_act(dy, dys, true)) != DYNCONV_OK) return st;
  if ((st = check_act(dx, dxs, false)) != DYNCONV_OK) return st;
  const int eb = elem_bytes(dtype);
  FilterInfo fi{};
  if ((st = check_filter(w, ws, W, H, eb, true, &fi)) != DYNCONV_OK) return st;
  if (dw != nullptr && !fi.is_static) {
    if (dws == nullptr) return DYNCONV_ERR_INVALID_ARG;
    if (dws[3] != 1 || dws[2] != W || dws[0] <= 0 || dws[1] <= 0) return DYNCONV_ERR_UNSUPPORTED;
    if (H == 1) {
      if (!aligned(dw, 4) || (dws[0] * eb) % 4 != 0 || (dws[1] * eb) % 4 != 0) return DYNCONV_ERR_UNSUPPORTED;
    } else if (!aligned(dw, eb) || !group_words_aligned(dw, dws, W, eb)) {
      return DYNCONV_ERR_UNSUPPORTED;
    }
  }
  if (dw != nullptr && fi.is_static && !aligned(dw, 4)) return DYNCONV_ERR_UNSUPPORTED;
  const void* ins[3] = {x, w, dy};
  for (const void* in : ins) {
    if (dx != nullptr && dx == in) return DYNCONV_ERR_INVALID_ARG;
    if (dw != nullptr && dw == in) return DYNCONV_ERR_INVALID_ARG;
  }
  if (dx != nullptr && dx == dw) return DYNCONV_ERR_INVALID_ARG;
  if (dcb != nullptr) {
    const void* others[5] = {x, w, dy, dx, dw};
    for (const void* o : others)
      if (o != nullptr && o == dcb) return DYNCONV_ERR_INVALID_ARG;
  }
  if (B == 0 || T == 0 || D == 0) {
    return DYNCONV_OK;
  }
  const Act acts[3] = {{x, xs}, {dy, dys}, {dx, dxs}};
  const int align = act_alignment(acts, 3, eb);
  if ((st = check_stream_layout(D, H, eb, align)) != DYNCONV_OK) return st;

  const StreamPlan plan = plan_stream(B, T, D, W, H, eb, align, true, fi.is_static);
  float* partial = nullptr;
  float* cb_partial = nullptr;
  const bool static_dw = fi.is_static && dw != nullptr;
  if (static_dw || dcb != nullptr) {
    const size_t need = bwd_partial_floats(plan, B, D, W, H, static_dw, dcb != nullptr) * sizeof(float);
    if (use_scratch) {
      if (need > kScratchBytes) return DYNCONV_ERR_WORKSPACE;
      if ((st = current_scratch(&workspace)) != DYNCONV_OK) return st;
      workspace_bytes = kScratchBytes;
    }
    if (workspace == nullptr || workspace_bytes < need) return DYNCONV_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return DYNCONV_ERR_UNSUPPORTED;
    float* wsf = static_cast<float*>(workspace);
    if (static_dw) partial = wsf;
    if (dcb != nullptr) cb_partial = wsf + bwd_partial_floats(plan, B, D, W, H, static_dw, false);
  }
  StreamParams p{};
  p.x = x;
  p.w = w;
  p.dy = dy;
  p.out = dx;
  p.dw = fi.is_static ? nullptr : dw;
  p.partial = partial;
  p.cb_partial = cb_partial;
  if (seg != nullptr) {
    p.seg = seg;
    p.ss0 = ss[0];
    p.ss1 = ss[1];
  }
  p.xs0 = xs[0];
  p.xs1 = xs[1];
  p.ws0 = ws[0];
  p.ws1 = ws[1];
  p.dys0 = dys[0];
  p.dys1 = dys[1];
  if (dx != nullptr) {
    p.os0 = dxs[0];
    p.os1 = dxs[1];
  }
  if (dw != nullptr && !fi.is_static) {
    p.dws0 = dws[0];
    p.dws1 = dws[1];
  }
  p.B = int32_t(B);
  p.T = int32_t(T);
  p.D = int32_t(D);
  p.H = H;
  p.G = int32_t(D / H);
  p.lpg = plan.lpg;
  p.lpw = plan.lpw;
  p.L = plan.L;
  p.nTw = plan.nTw;
  p.nDw = plan.nDw;
  p.WD = plan.WD;
  p.WT = plan.WT;
  p.nDb = plan.nDb;
  p.nTb = plan.nTb;
  return launch_stream_bwd(p, plan, W, dtype, fi.is_static, fi.is_static ? static_cast<float*>(dw) : nullptr, dcb,
                           static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

dynconv_status dynconv_bwd(const void* x, const int64_t* xs, const void* w, const int64_t* ws, const void* dy,
                           const int64_t* dys, void* dx, const int64_t* dxs, void* dw, const int64_t* dws, int64_t B,
                           int64_t T, int64_t D, int32_t W, int32_t H, dynconv_dtype dtype, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return bwd_impl(x, xs, w, ws, nullptr, nullptr, dy, dys, dx, dxs, dw, dws, nullptr, B, T, D, W, H, dtype, workspace,
                  workspace_bytes, stream);
}

dynconv_status dynconv_bwd_varlen(const void* x, const int64_t* xs, const void* w, const int64_t* ws,
                                  const int32_t* seq_idx, const int64_t* ss, const void* dy, const int64_t* dys,
                                  void* dx, const int64_t* dxs, void* dw, const int64_t* dws, int64_t B, int64_t T,
                                  int64_t D, int32_t W, int32_t H, dynconv_dtype dtype, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  const dynconv_status st = check_seg(seq_idx, ss);
  if (st != DYNCONV_OK) return st;
  return bwd_impl(x, xs, w, ws, seq_idx, ss, dy, dys, dx, dxs, dw, dws, nullptr, B, T, D, W, H, dtype, workspace,
                  workspace_bytes, stream);
}

dynconv_status dynconv_bwd_ex(const void* x, const int64_t* xs, const void* w, const int64_t* ws,
                              const int32_t* seq_idx, const int64_t* ss, const void* dy, const int64_t* dys, void* dx,
                              const int64_t* dxs, void* dw, const int64_t* dws, float* dconv_bias, int64_t B,
                              int64_t T, int64_t D, int32_t W, int32_t H, dynconv_dtype dtype, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (seq_idx != nullptr) {
    const dynconv_status st = check_seg(seq_idx, ss);
    if (st != DYNCONV_OK) return st;
  }
  return bwd_impl(x, xs, w, ws, seq_idx, ss, dy, dys, dx, dxs, dw, dws, dconv_bias, B, T, D, W, H, dtype, workspace,
                  workspace_bytes, stream);
}

dynconv_status dynconv_bwd_ex_noalloc(const void* x, const int64_t* xs, const void* w, const int64_t* ws,
                                      const int32_t* seq_idx, const int64_t* ss, const void* dy, const int64_t* dys,
                                      void* dx, const int64_t* dxs, void* dw, const int64_t* dws, float* dconv_bias,
                                      int64_t B, int64_t T, int64_t D, int32_t W, int32_t H, dynconv_dtype dtype,
                                      void* stream) {
  if (seq_idx != nullptr) {
    const dynconv_status st = check_seg(seq_idx, ss);
    if (st != DYNCONV_OK) return st;
  }
  return bwd_impl(x, xs, w, ws, seq_idx, ss, dy, dys, dx, dxs, dw, dws, dconv_bias, B, T, D, W, H, dtype, nullptr, 0,
                  stream, true);
}

}  // extern "C"

// ---------------------------------------------------------------------------------
// Low-rank form
// ---------------------------------------------------------------------------------
namespace {

dynconv_status check_lowrank(const void* x, const int64_t* xs, const void* z, const int64_t* zs, const void* U,
                             int64_t ldu, int64_t B, int64_t T, int64_t D, int32_t W, int32_t H, int32_t R,
                             dynconv_dtype dtype) {
  dynconv_status st = check_common(B, T, D, W, H, dtype);
  if (st != DYNCONV_OK) return st;
  if (R < 1) return DYNCONV_ERR_INVALID_ARG;
  if (R > 128) return DYNCONV_ERR_UNSUPPORTED;
  if (W > kMaxLowrankW) return DYNCONV_ERR_UNSUPPORTED;
  if ((st = check_act(x, xs, true)) != DYNCONV_OK) return st;
  if (z == nullptr || zs == nullptr) return DYNCONV_ERR_INVALID_ARG;
  if (zs[2] != 1) return DYNCONV_ERR_UNSUPPORTED;
  if (zs[0] < 0 || zs[1] < 0) return DYNCONV_ERR_UNSUPPORTED;
  if (U == nullptr) return DYNCONV_ERR_INVALID_ARG;
  if (ldu < (D / H) * W) return DYNCONV_ERR_INVALID_ARG;
  if (xs[1] >= kLowrankMaxRowStride || zs[1] >= kLowrankMaxRowStride || ldu >= kLowrankMaxRowStride)
    return DYNCONV_ERR_UNSUPPORTED;
  return DYNCONV_OK;
}

LowRankParams lowrank_params(const void* x, const int64_t* xs, const void* z, const int64_t* zs, const void* U,
                             int64_t ldu, const void* bias, int64_t B, int64_t T, int64_t D, int32_t W, int32_t H,
                             int32_t R, const LowRankPlan& plan) {
  LowRankParams p{};
  p.x = x;
  p.z = z;
  p.U = U;
  p.bias = bias;
  p.xs0 = xs[0];
  p.xs1 = xs[1];
  p.zs0 = zs[0];
  p.zs1 = zs[1];
  p.ldu = ldu;
  p.B = int32_t(B);
  p.T = int32_t(T);
  p.D = int32_t(D);
  p.H = H;
  p.G = int32_t(D / H);
  p.R = R;
  p.J = int32_t((D / H) * W);
  p.nCs = plan.nCs;
  p.Ltok = plan.Ltok;
  p.nTr = plan.nTr;
  return p;
}

}  // namespace

extern "C" {

}  // extern "C"

namespace {

// Workspace of the low-rank backward: the partial sums of dU and db, then (with a
// convolution-bias gradient) the column-sum partials of dy, 256-byte aligned.
constexpr size_t kCbAlign = 256;
size_t lowrank_cb_offset(const LowRankPlan& plan) { return (plan.ws_total + kCbAlign - 1) / kCbAlign * kCbAlign; }
size_t lowrank_bwd_workspace(const LowRankPlan& plan, int64_t B, int64_t T, int64_t D, bool dcbias) {
  if (!dcbias) return plan.ws_total;
  return lowrank_cb_offset(plan) + size_t(B) * size_t(colsum_chunks(B, T, D)) * size_t(D) * sizeof(float);
}

dynconv_status lowrank_fwd_impl(const void* x, const int64_t* xs, const void* z, const int64_t* zs, const void* U,
                                int64_t ldu, const void* bias, const int32_t* seg, const int64_t* ss,
                                const void* conv_bias, void* y, const int64_t* ys, int64_t B, int64_t T, int64_t D,
                                int32_t W, int32_t H, int32_t R, dynconv_dtype dtype, void* stream) {
  dynconv_status st = check_lowrank(x, xs, z, zs, U, ldu, B, T, D, W, H, R, dtype);
  if (st != DYNCONV_OK) return st;
  if ((st = check_act(y, ys, true)) != DYNCONV_OK) return st;
  if (ys[1] >= kLowrankMaxRowStride) return DYNCONV_ERR_UNSUPPORTED;
  if (y == x || y == z || y == U || (bias != nullptr && y == bias)) return DYNCONV_ERR_INVALID_ARG;
  if (conv_bias != nullptr) {
    if (conv_bias == y) return DYNCONV_ERR_INVALID_ARG;
    if (!aligned(conv_bias, 4)) return DYNCONV_ERR_UNSUPPORTED;
  }
  if (B == 0 || T == 0 || D == 0) return DYNCONV_OK;
  const int eb = elem_bytes(dtype);
  const Act acts[2] = {{x, xs}, {y, ys}};
  if (!act_align_ok(acts, 2, eb, 4)) return DYNCONV_ERR_UNSUPPORTED;
  const LowRankPlan plan = plan_lowrank(B, T, D, W, H, R, false, dtype);
  LowRankParams p = lowrank_params(x, xs, z, zs, U, ldu, bias, B, T, D, W, H, R, plan);
  p.act16 = act_align_ok(acts, 2, eb, 16) ? 1 : 0;
  p.z16 = (aligned(z, 16) && (zs[0] * eb) % 16 == 0 && (zs[1] * eb) % 16 == 0) ? 1 : 0;
  p.z4 = (aligned(z, 4) && (zs[0] * eb) % 4 == 0 && (zs[1] * eb) % 4 == 0) ? 1 : 0;
  p.out = y;
  p.os0 = ys[0];
  p.os1 = ys[1];
  p.cbias = conv_bias;
  if (seg != nullptr) {
    p.seg = seg;
    p.ss0 = ss[0];
    p.ss1 = ss[1];
  }
  return launch_lowrank_fwd(p, plan, W, dtype, static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

dynconv_status dynconv_lowrank_fwd(const void* x, const int64_t* xs, const void* z, const int64_t* zs, const void* U,
                                   int64_t ldu, const void* bias, void* y, const int64_t* ys, int64_t B, int64_t T,
                                   int64_t D, int32_t W, int32_t H, int32_t R, dynconv_dtype dtype, void* stream) {
  return lowrank_fwd_impl(x, xs, z, zs, U, ldu, bias, nullptr, nullptr, nullptr, y, ys, B, T, D, W, H, R, dtype,
                          stream);
}

dynconv_status dynconv_lowrank_fwd_varlen(const void* x, const int64_t* xs, const void* z, const int64_t* zs,
                                          const void* U, int64_t ldu, const void* bias, const int32_t* seq_idx,
                                          const int64_t* ss, void* y, const int64_t* ys, int64_t B, int64_t T,
                                          int64_t D, int32_t W, int32_t H, int32_t R, dynconv_dtype dtype,
                                          void* stream) {
  const dynconv_status st = check_seg(seq_idx, ss);
  if (st != DYNCONV_OK) return st;
  return lowrank_fwd_impl(x, xs, z, zs, U, ldu, bias, seq_idx, ss, nullptr, y, ys, B, T, D, W, H, R, dtype, stream);
}

dynconv_status dynconv_lowrank_fwd_ex(const void* x, const int64_t* xs, const void* z, const int64_t* zs,
                                      const void* U, int64_t ldu, const void* bias, const int32_t* seq_idx,
                                      const int64_t* ss, const void* conv_bias, void* y, const int64_t* ys, int64_t B,
                                      int64_t T, int64_t D, int32_t W, int32_t H, int32_t R, dynconv_dtype dtype,
                                      void* stream) {
  if (seq_idx != nullptr) {
    const dynconv_status st = check_seg(seq_idx, ss);
    if (st != DYNCONV_OK) return st;
  }
  return lowrank_fwd_impl(x, xs, z, zs, U, ldu, bias, seq_idx, ss, conv_bias, y, ys, B, T, D, W, H, R, dtype,
                          stream);
}

size_t dynconv_lowrank_bwd_workspace_size(int64_t B, int64_t T, int64_t D, int32_t W, int32_t H, int32_t R,
                                          dynconv_dtype dtype) {
  return dynconv_lowrank_bwd_ex_workspace_size(B, T, D, W, H, R, 0, dtype);
}

size_t dynconv_lowrank_bwd_ex_workspace_size(int64_t B, int64_t T, int64_t D, int32_t W, int32_t H, int32_t R,
                                             int want_dconv_bias, dynconv_dtype dtype) {
  if (check_common(B, T, D, W, H, dtype) != DYNCONV_OK || R < 1 || R > 128 || W > kMaxLowrankW) return 0;
  if (B == 0 || T == 0 || D == 0) return 0;
  return lowrank_bwd_workspace(plan_lowrank(B, T, D, W, H, R, true, dtype), B, T, D, want_dconv_bias != 0);
}

}  // extern "C"

namespace {

dynconv_status lowrank_bwd_impl(const void* x, const int64_t* xs, const void* z, const int64_t* zs, const void* U,
                                int64_t ldu, const void* bias, const int32_t* seg, const int64_t* ss, const void* dy,
                                const int64_t* dys, void* dx, const int64_t* dxs, void* dz, const int64_t* dzs,
                                float* dU, float* db, float* dcb, int64_t B, int64_t T, int64_t D, int32_t W,
                                int32_t H, int32_t R, dynconv_dtype dtype, void* workspace, size_t workspace_bytes,
                                void* stream) {
  dynconv_status st = check_lowrank(x, xs, z, zs, U, ldu, B, T, D, W, H, R, dtype);
  if (st != DYNCONV_OK) return st;
  if ((st = check_act(dy, dys, true)) != DYNCONV_OK) return st;
  if ((st = check_act(dx, dxs, true)) != DYNCONV_OK) return st;
  if (dz == nullptr || dzs == nullptr || dU == nullptr) return DYNCONV_ERR_INVALID_ARG;
  if (dzs[2] != 1 || dzs[0] < 0 || dzs[1] < 0) return DYNCONV_ERR_UNSUPPORTED;
  if (dys[1] >= kLowrankMaxRowStride || dxs[1] >= kLowrankMaxRowStride) return DYNCONV_ERR_UNSUPPORTED;
  const void* ins[5] = {x, z, U, bias, dy};
  const void* outs[5] = {dx, dz, dU, db, dcb};
  for (const void* o : outs) {
    if (o == nullptr) continue;
    for (const void* in : ins)
      if (in != nullptr && o == in) return DYNCONV_ERR_INVALID_ARG;
  }
  for (int i = 0; i < 5; ++i)
    for (int j = i + 1; j < 5; ++j)
      if (outs[i] != nullptr && outs[i] == outs[j]) return DYNCONV_ERR_INVALID_ARG;
  if (!aligned(dU, 4) || (db != nullptr && !aligned(db, 4)) || (dcb != nullptr && !aligned(dcb, 4)))
    return DYNCONV_ERR_UNSUPPORTED;
  if (B == 0 || T == 0 || D == 0) return DYNCONV_OK;
  const int eb = elem_bytes(dtype);
  const Act acts[3] = {{x, xs}, {dy, dys}, {dx, dxs}};
  if (!act_align_ok(acts, 3, eb, 4)) return DYNCONV_ERR_UNSUPPORTED;
  const LowRankPlan plan = plan_lowrank(B, T, D, W, H, R, true, dtype);
  if (workspace == nullptr || workspace_bytes < lowrank_bwd_workspace(plan, B, T, D, dcb != nullptr))
    return DYNCONV_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return DYNCONV_ERR_UNSUPPORTED;
  LowRankParams p = lowrank_params(x, xs, z, zs, U, ldu, bias, B, T, D, W, H, R, plan);
  p.act16 = act_align_ok(acts, 3, eb, 16) ? 1 : 0;
  p.z16 = (aligned(z, 16) && (zs[0] * eb) % 16 == 0 && (zs[1] * eb) % 16 == 0) ? 1 : 0;
  p.z4 = (aligned(z, 4) && (zs[0] * eb) % 4 == 0 && (zs[1] * eb) % 4 == 0) ? 1 : 0;
  p.u16 = (aligned(U, 16) && (ldu * eb) % 16 == 0) ? 1 : 0;
  p.dy = dy;
  p.dys0 = dys[0];
  p.dys1 = dys[1];
  p.out = dx;
  p.os0 = dxs[0];
  p.os1 = dxs[1];
  p.dz = dz;
  p.dzs0 = dzs[0];
  p.dzs1 = dzs[1];
  char* wsb = static_cast<char*>(workspace);
  p.part_dU = reinterpret_cast<float*>(wsb + plan.ws_dU);
  p.part_db = db != nullptr ? reinterpret_cast<float*>(wsb + plan.ws_db) : nullptr;
  if (seg != nullptr) {
    p.seg = seg;
    p.ss0 = ss[0];
    p.ss1 = ss[1];
  }
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (dcb != nullptr) {
    // the bias gradient, sum of dy over every token (packed sequences included)
    float* part = reinterpret_cast<float*>(wsb + lowrank_cb_offset(plan));
    if ((st = launch_column_sums(dy, dys[0], dys[1], B, T, D, dtype, part, dcb, hs)) != DYNCONV_OK) return st;
  }
  return launch_lowrank_bwd(p, plan, W, dtype, dU, db, hs);
}

}  // namespace

extern "C" {

dynconv_status dynconv_lowrank_bwd(const void* x, const int64_t* xs, const void* z, const int64_t* zs, const void* U,
                                   int64_t ldu, const void* bias, const void* dy, const int64_t* dys, void* dx,
                                   const int64_t* dxs, void* dz, const int64_t* dzs, float* dU, float* db, int64_t B,
                                   int64_t T, int64_t D, int32_t W, int32_t H, int32_t R, dynconv_dtype dtype,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return lowrank_bwd_impl(x, xs, z, zs, U, ldu, bias, nullptr, nullptr, dy, dys, dx, dxs, dz, dzs, dU, db, nullptr, B,
                          T, D, W, H, R, dtype, workspace, workspace_bytes, stream);
}

dynconv_status dynconv_lowrank_bwd_varlen(const void* x, const int64_t* xs, const void* z, const int64_t* zs,
                                          const void* U, int64_t ldu, const void* bias, const int32_t* seq_idx,
                                          const int64_t* ss, const void* dy, const int64_t* dys, void* dx,
                                          const int64_t* dxs, void* dz, const int64_t* dzs, float* dU, float* db,
                                          int64_t B, int64_t T, int64_t D, int32_t W, int32_t H, int32_t R,
                                          dynconv_dtype dtype, void* workspace, size_t workspace_bytes,
                                          void* stream) {
  const dynconv_status st = check_seg(seq_idx, ss);
  if (st != DYNCONV_OK) return st;
  return lowrank_bwd_impl(x, xs, z, zs, U, ldu, bias, seq_idx, ss, dy, dys, dx, dxs, dz, dzs, dU, db, nullptr, B, T,
                          D, W, H, R, dtype, workspace, workspace_bytes, stream);
}

dynconv_status dynconv_lowrank_bwd_ex(const void* x, const int64_t* xs, const void* z, const int64_t* zs,
                                      const void* U, int64_t ldu, const void* bias, const int32_t* seq_idx,
                                      const int64_t* ss, const void* dy, const int64_t* dys, void* dx,
                                      const int64_t* dxs, void* dz, const int64_t* dzs, float* dU, float* db,
                                      float* dconv_bias, int64_t B, int64_t T, int64_t D, int32_t W, int32_t H,
                                      int32_t R, dynconv_dtype dtype, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  if (seq_idx != nullptr) {
    const dynconv_status st = check_seg(seq_idx, ss);
    if (st != DYNCONV_OK) return st;
  }
  return lowrank_bwd_impl(x, xs, z, zs, U, ldu, bias, seq_idx, ss, dy, dys, dx, dxs, dz, dzs, dU, db, dconv_bias, B, T,
                          D, W, H, R, dtype, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------------------------
// Inference: rolling cache of the last W-1 inputs, single-token decoding steps
// ---------------------------------------------------------------------------------
}  // extern "C"

namespace {

// A [B, W-1, D] cache (required when W > 1) and element alignment of every pointer.
dynconv_status check_cache(const void* cache, const int64_t* cs, int32_t W, int eb) {
  if (W == 1) return DYNCONV_OK;
  if (cache == nullptr || cs == nullptr) return DYNCONV_ERR_INVALID_ARG;
  if (cs[2] != 1) return DYNCONV_ERR_UNSUPPORTED;
  if (cs[0] < 0 || cs[1] < 0) return DYNCONV_ERR_UNSUPPORTED;
  if (!aligned(cache, eb)) return DYNCONV_ERR_UNSUPPORTED;
  return DYNCONV_OK;
}

// A [B, D] row tensor with strides s[0..1].
dynconv_status check_row(const void* p, const int64_t* s, int eb) {
  if (p == nullptr || s == nullptr) return DYNCONV_ERR_INVALID_ARG;
  if (s[1] != 1) return DYNCONV_ERR_UNSUPPORTED;
  if (s[0] < 0) return DYNCONV_ERR_UNSUPPORTED;
  if (!aligned(p, eb)) return DYNCONV_ERR_UNSUPPORTED;
  return DYNCONV_OK;
}

DecodeParams decode_params(const void* x, const int64_t* xs, void* cache, const int64_t* cs, void* y,
                           const int64_t* ys, int64_t t, int64_t B, int64_t D, int32_t W, int32_t H) {
  DecodeParams p{};
  p.x = x;
  p.xs0 = xs[0];
  p.cache = cache;
  p.cs0 = W > 1 ? cs[0] : 0;
  p.cs1 = W > 1 ? cs[1] : 0;
  p.y = y;
  p.ys0 = ys != nullptr ? ys[0] : 0;
  p.t = t;
  p.B = int32_t(B);
  p.D = int32_t(D);
  p.H = H;
  return p;
}

}  // namespace

extern "C" {

}  // extern "C"

namespace {

dynconv_status cache_fill_impl(const void* x, const int64_t* xs, const int32_t* seg, const int64_t* ss, void* cache,
                               const int64_t* cs, int64_t B, int64_t T, int64_t D, int32_t W, dynconv_dtype dtype,
                               void* stream) {
  dynconv_status st = check_common(B, T, D, W, 1, dtype);
  if (st != DYNCONV_OK) return st;
  const int eb = elem_bytes(dtype);
  if ((st = check_cache(cache, cs, W, eb)) != DYNCONV_OK) return st;
  if (T > 0) {
    if ((st = check_act(x, xs, true)) != DYNCONV_OK) return st;
    if (!aligned(x, eb)) return DYNCONV_ERR_UNSUPPORTED;
    if (x == cache) return DYNCONV_ERR_INVALID_ARG;
  }
  if (W == 1 || B == 0 || D == 0) return DYNCONV_OK;
  DecodeParams p = decode_params(x, xs != nullptr ? xs : cs, cache, cs, nullptr, nullptr, T, B, D, W, 1);
  p.xs1 = (T > 0) ? xs[1] : 0;
  if (seg != nullptr && T > 0) {
    p.seg = seg;
    p.ss0 = ss[0];
    p.ss1 = ss[1];
  }
  return launch_cache_fill(p, W, dtype, static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

dynconv_status dynconv_cache_fill(const void* x, const int64_t* xs, void* cache, const int64_t* cs, int64_t B,
                                  int64_t T, int64_t D, int32_t W, dynconv_dtype dtype, void* stream) {
  return cache_fill_impl(x, xs, nullptr, nullptr, cache, cs, B, T, D, W, dtype, stream);
}

dynconv_status dynconv_cache_fill_varlen(const void* x, const int64_t* xs, const int32_t* seq_idx, const int64_t* ss,
                                         void* cache, const int64_t* cs, int64_t B, int64_t T, int64_t D, int32_t W,
                                         dynconv_dtype dtype, void* stream) {
  const dynconv_status st = check_seg(seq_idx, ss);
  if (st != DYNCONV_OK) return st;
  return cache_fill_impl(x, xs, seq_idx, ss, cache, cs, B, T, D, W, dtype, stream);
}

dynconv_status dynconv_decode_step(const void* x, const int64_t* xs, const void* w, const int64_t* ws,
                                   void* cache, const int64_t* cs, void* y, const int64_t* ys, int64_t t,
                                   int64_t B, int64_t D, int32_t W, int32_t H, dynconv_dtype dtype, void* stream) {
  return dynconv_decode_step_ex(x, xs, w, ws, nullptr, cache, cs, y, ys, t, B, D, W, H, dtype, stream);
}

dynconv_status dynconv_decode_step_ex(const void* x, const int64_t* xs, const void* w, const int64_t* ws,
                                      const void* conv_bias, void* cache, const int64_t* cs, void* y,
                                      const int64_t* ys, int64_t t, int64_t B, int64_t D, int32_t W, int32_t H,
                                      dynconv_dtype dtype, void* stream) {
  dynconv_status st = check_common(B, 1, D, W, H, dtype);
  if (st != DYNCONV_OK) return st;
  const int eb = elem_bytes(dtype);
  if (t < 0) return DYNCONV_ERR_INVALID_ARG;
  if ((st = check_row(x, xs, eb)) != DYNCONV_OK) return st;
  if ((st = check_row(y, ys, eb)) != DYNCONV_OK) return st;
  if ((st = check_cache(cache, cs, W, eb)) != DYNCONV_OK) return st;
  if (w == nullptr || ws == nullptr) return DYNCONV_ERR_INVALID_ARG;
  if (ws[2] != 1 || ws[1] != W || ws[0] < 0) return DYNCONV_ERR_UNSUPPORTED;
  if (!aligned(w, eb)) return DYNCONV_ERR_UNSUPPORTED;
  if (y == x || y == w || (W > 1 && (y == cache || cache == x || cache == w))) return DYNCONV_ERR_INVALID_ARG;
  if (conv_bias != nullptr) {
    if (conv_bias == y || conv_bias == cache) return DYNCONV_ERR_INVALID_ARG;
    if (!aligned(conv_bias, eb)) return DYNCONV_ERR_UNSUPPORTED;
  }
  if (B == 0 || D == 0) return DYNCONV_OK;
  DecodeParams p = decode_params(x, xs, cache, cs, y, ys, t, B, D, W, H);
  p.w = w;
  p.ws0 = ws[0];
  p.cbias = conv_bias;
  return launch_decode_step(p, W, dtype, static_cast<hipStream_t>(stream));
}

dynconv_status dynconv_lowrank_decode_step(const void* x, const int64_t* xs, const void* z, const int64_t* zs,
                                           const void* U, int64_t ldu, const void* bias, void* cache,
                                           const int64_t* cs, void* y, const int64_t* ys, int64_t t, int64_t B,
                                           int64_t D, int32_t W, int32_t H, int32_t R, dynconv_dtype dtype,
                                           void* stream) {
  return dynconv_lowrank_decode_step_ex(x, xs, z, zs, U, ldu, bias, nullptr, cache, cs, y, ys, t, B, D, W, H, R, dtype,
                                        stream);
}

dynconv_status dynconv_lowrank_decode_step_ex(const void* x, const int64_t* xs, const void* z, const int64_t* zs,
                                              const void* U, int64_t ldu, const void* bias, const void* conv_bias,
                                              void* cache, const int64_t* cs, void* y, const int64_t* ys, int64_t t,
                                              int64_t B, int64_t D, int32_t W, int32_t H, int32_t R,
                                              dynconv_dtype dtype, void* stream) {
  dynconv_status st = check_common(B, 1, D, W, H, dtype);
  if (st != DYNCONV_OK) return st;
  const int eb = elem_bytes(dtype);
  if (t < 0 || R < 1) return DYNCONV_ERR_INVALID_ARG;
  if (R > 128 || W > kMaxLowrankW) return DYNCONV_ERR_UNSUPPORTED;
  if ((st = check_row(x, xs, eb)) != DYNCONV_OK) return st;
  if ((st = check_row(y, ys, eb)) != DYNCONV_OK) return st;
  if ((st = check_row(z, zs, eb)) != DYNCONV_OK) return st;
  if ((st = check_cache(cache, cs, W, eb)) != DYNCONV_OK) return st;
  if (U == nullptr) return DYNCONV_ERR_INVALID_ARG;
  if (ldu < (D / H) * W) return DYNCONV_ERR_INVALID_ARG;
  if (!aligned(U, eb) || (bias != nullptr && !aligned(bias, eb))) return DYNCONV_ERR_UNSUPPORTED;
  if (y == x || y == z || y == U || (bias != nullptr && y == bias) ||
      (W > 1 && (y == cache || cache == x || cache == z || cache == U)))
    return DYNCONV_ERR_INVALID_ARG;
  if (conv_bias != nullptr) {
    if (conv_bias == y || conv_bias == cache) return DYNCONV_ERR_INVALID_ARG;
    if (!aligned(conv_bias, eb)) return DYNCONV_ERR_UNSUPPORTED;
  }
  if (B == 0 || D == 0) return DYNCONV_OK;
  DecodeParams p = decode_params(x, xs, cache, cs, y, ys, t, B, D, W, H);
  p.cbias = conv_bias;
  p.z = z;
  p.zs0 = zs[0];
  p.U = U;
  p.ldu = ldu;
  p.bias = bias;
  p.R = R;
  return launch_lowrank_decode_step(p, W, dtype, static_cast<hipStream_t>(stream));
}

}  // extern "C"

// ---------------------------------------------------------------------------------
// The convolution in the epilogue of the producing projection
// ---------------------------------------------------------------------------------
namespace {

dynconv_status check_gemm(const void* A, const int64_t* as, const void* Wp, int64_t ldw, const void* y,
                          const int64_t* ys, int64_t B, int64_t T, int64_t N, int64_t K, int32_t W, int32_t H,
                          dynconv_dtype dtype) {
  dynconv_status st = check_common(B, T, N, W, H, dtype);
  if (st != DYNCONV_OK) return st;
  if (K < 0) return DYNCONV_ERR_INVALID_ARG;
  if (A == nullptr || as == nullptr || Wp == nullptr || y == nullptr || ys == nullptr) return DYNCONV_ERR_INVALID_ARG;
  if (ldw < K) return DYNCONV_ERR_INVALID_ARG;
  if (dtype == DYNCONV_F32) return DYNCONV_ERR_UNSUPPORTED;  // matrix cores on 16-bit operands
  if (W > 5 || H > 16 || !is_pow2(H)) return DYNCONV_ERR_UNSUPPORTED;  // whole groups in a 128-column tile
  if (as[2] != 1 || ys[2] != 1) return DYNCONV_ERR_UNSUPPORTED;
  if (as[0] < 0 || as[1] < 0 || ys[0] < 0 || ys[1] < 0) return DYNCONV_ERR_UNSUPPORTED;
  if (K == 0 || K % kGemmK != 0) return DYNCONV_ERR_UNSUPPORTED;
  if (N % kGemmCols != 0) return DYNCONV_ERR_UNSUPPORTED;
  if (B * T > INT32_MAX) return DYNCONV_ERR_UNSUPPORTED;
  // 16-byte rows of A and W_p (LDS DMA of 16-byte chunks), 16-bit elements of y
  if (!aligned(A, 16) || (as[0] * 2) % 16 != 0 || (as[1] * 2) % 16 != 0) return DYNCONV_ERR_UNSUPPORTED;
  if (!aligned(Wp, 16) || (ldw * 2) % 16 != 0) return DYNCONV_ERR_UNSUPPORTED;
  if (!aligned(y, 2)) return DYNCONV_ERR_UNSUPPORTED;
  if (y == A || y == Wp) return DYNCONV_ERR_INVALID_ARG;
  return DYNCONV_OK;
}

GemmParams gemm_params(const void* A, const int64_t* as, const void* Wp, int64_t ldw, void* y, const int64_t* ys,
                       int64_t B, int64_t T, int64_t N, int64_t K, int32_t H) {
  GemmParams p{};
  p.A = A;
  p.Wp = Wp;
  p.y = y;
  p.as0 = as[0];
  p.as1 = as[1];
  p.ldw = ldw;
  p.ys0 = ys[0];
  p.ys1 = ys[1];
  p.B = int32_t(B);
  p.T = int32_t(T);
  p.N = int32_t(N);
  p.K = int32_t(K);
  p.H = H;
  p.M = int32_t(B * T);
  p.nTm = int32_t((B * T + kGemmOutRows - 1) / kGemmOutRows);
  p.nTn = int32_t(N / kGemmCols);
  return p;
}

}  // namespace

extern "C" {

dynconv_status dynconv_gemm_fwd(const void* A, const int64_t* as, const void* Wp, int64_t ldw, const void* w,
                                const int64_t* ws, void* y, const int64_t* ys, int64_t B, int64_t T, int64_t N,
                                int64_t K, int32_t W, int32_t H, dynconv_dtype dtype, void* stream) {
  dynconv_status st = check_gemm(A, as, Wp, ldw, y, ys, B, T, N, K, W, H, dtype);
  if (st != DYNCONV_OK) return st;
  if (w == nullptr || ws == nullptr) return DYNCONV_ERR_INVALID_ARG;
  if (ws[3] != 1 || ws[2] != W || ws[0] < 0 || ws[1] < 0) return DYNCONV_ERR_UNSUPPORTED;
  if (!aligned(w, 2)) return DYNCONV_ERR_UNSUPPORTED;
  if (y == w) return DYNCONV_ERR_INVALID_ARG;
  if (B == 0 || T == 0 || N == 0) return DYNCONV_OK;
  GemmParams p = gemm_params(A, as, Wp, ldw, y, ys, B, T, N, K, H);
  p.w = w;
  p.ws0 = ws[0];
  p.ws1 = ws[1];
  const bool wvec = W == 4 && aligned(w, 8) && (ws[0] * 2) % 8 == 0 && (ws[1] * 2) % 8 == 0;
  const hipError_t e = launch_gemm_conv(p, W, wvec, dtype, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DYNCONV_OK : record_hip_error(e);
}

dynconv_status dynconv_gemm_lowrank_fwd(const void* A, const int64_t* as, const void* Wp, int64_t ldw, const void* z,
                                        const int64_t* zs, const void* U, int64_t ldu, const void* bias, void* y,
                                        const int64_t* ys, int64_t B, int64_t T, int64_t N, int64_t K, int32_t W,
                                        int32_t H, int32_t R, dynconv_dtype dtype, void* stream) {
  dynconv_status st = check_gemm(A, as, Wp, ldw, y, ys, B, T, N, K, W, H, dtype);
  if (st != DYNCONV_OK) return st;
  if (R < 1) return DYNCONV_ERR_INVALID_ARG;
  if (R > 128) return DYNCONV_ERR_UNSUPPORTED;
  if (z == nullptr || zs == nullptr || U == nullptr) return DYNCONV_ERR_INVALID_ARG;
  if (zs[2] != 1 || zs[0] < 0 || zs[1] < 0) return DYNCONV_ERR_UNSUPPORTED;
  if (ldu < (N / H) * W) return DYNCONV_ERR_INVALID_ARG;
  if (!aligned(z, 2) || !aligned(U, 2) || (bias != nullptr && !aligned(bias, 2))) return DYNCONV_ERR_UNSUPPORTED;
  if (!gemm_lowrank_fits(W, R)) return DYNCONV_ERR_UNSUPPORTED;
  if (y == z || y == U || (bias != nullptr && y == bias)) return DYNCONV_ERR_INVALID_ARG;
  if (B == 0 || T == 0 || N == 0) return DYNCONV_OK;
  GemmParams p = gemm_params(A, as, Wp, ldw, y, ys, B, T, N, K, H);
  p.z = z;
  p.zs0 = zs[0];
  p.zs1 = zs[1];
  p.U = U;
  p.ldu = ldu;
  p.bias = bias;
  p.R = R;
  p.uvec = aligned(U, 16) && ldu % 8 == 0;
  p.zvec = aligned(z, 16) && zs[0] % 8 == 0 && zs[1] % 8 == 0 && R % 8 == 0;
  const hipError_t e = launch_gemm_lowrank(p, W, dtype, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DYNCONV_OK : record_hip_error(e);
}

}  // extern "C"
