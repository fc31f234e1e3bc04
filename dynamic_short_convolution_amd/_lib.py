"""ctypes declarations of libdynconv's C ABI (include/dynconv.h).

Loading fails loudly when the library has not been built: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdynconv.so")

DYNCONV_F32 = 0
DYNCONV_BF16 = 1
DYNCONV_F16 = 2

STATUS = {
    0: "DYNCONV_OK",
    1: "DYNCONV_ERR_INVALID_ARG",
    2: "DYNCONV_ERR_UNSUPPORTED",
    3: "DYNCONV_ERR_WORKSPACE",
    4: "DYNCONV_ERR_HIP",
}

# Every exported symbol of include/dynconv.h.
EXPORTS = (
    "dynconv_status_string",
    "dynconv_last_hip_error",
    "dynconv_fwd",
    "dynconv_bwd",
    "dynconv_bwd_workspace_size",
    "dynconv_lowrank_fwd",
    "dynconv_lowrank_bwd",
    "dynconv_lowrank_bwd_workspace_size",
    "dynconv_cache_fill",
    "dynconv_decode_step",
    "dynconv_lowrank_decode_step",
    "dynconv_fwd_varlen",
    "dynconv_bwd_varlen",
    "dynconv_lowrank_fwd_varlen",
    "dynconv_lowrank_bwd_varlen",
    "dynconv_cache_fill_varlen",
    "dynconv_fwd_ex",
    "dynconv_bwd_ex",
    "dynconv_bwd_ex_workspace_size",
    "dynconv_decode_step_ex",
    "dynconv_bwd_ex_noalloc",
    "dynconv_gemm_fwd",
    "dynconv_gemm_lowrank_fwd",
    "dynconv_lowrank_fwd_ex",
    "dynconv_lowrank_bwd_ex",
    "dynconv_lowrank_bwd_ex_workspace_size",
    "dynconv_lowrank_decode_step_ex",
)

# Bytes of the per-GPU scratch array of dynconv_bwd_ex_noalloc (DYNCONV_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 16 << 20

_i64p = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t

_SIGNATURES = {
    "dynconv_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "dynconv_last_hip_error": ([], ctypes.c_int),
    "dynconv_fwd": ([_vp, _i64p, _vp, _i64p, _vp, _i64p, _i64, _i64, _i64, _i32, _i32, ctypes.c_int, _vp], ctypes.c_int),
    "dynconv_bwd": (
        [_vp, _i64p, _vp, _i64p, _vp, _i64p, _vp, _i64p, _vp, _i64p, _i64, _i64, _i64, _i32, _i32, ctypes.c_int, _vp,
         _sz, _vp],
        ctypes.c_int,
    ),
    "dynconv_bwd_workspace_size": ([_i64, _i64, _i64, _i32, _i32, ctypes.c_int, ctypes.c_int], _sz),
    "dynconv_lowrank_fwd": (
        [_vp, _i64p, _vp, _i64p, _vp, _i64, _vp, _vp, _i64p, _i64, _i64, _i64, _i32, _i32, _i32, ctypes.c_int, _vp],
        ctypes.c_int,
    ),
    "dynconv_lowrank_bwd": (
        [_vp, _i64p, _vp, _i64p, _vp, _i64, _vp, _vp, _i64p, _vp, _i64p, _vp, _i64p, _vp, _vp, _i64, _i64, _i64, _i32,
         _i32, _i32, ctypes.c_int, _vp, _sz, _vp],
        ctypes.c_int,
    ),
    "dynconv_lowrank_bwd_workspace_size": ([_i64, _i64, _i64, _i32, _i32, _i32, ctypes.c_int], _sz),
    "dynconv_cache_fill": ([_vp, _i64p, _vp, _i64p, _i64, _i64, _i64, _i32, ctypes.c_int, _vp], ctypes.c_int),
    "dynconv_decode_step": (
        [_vp, _i64p, _vp, _i64p, _vp, _i64p, _vp, _i64p, _i64, _i64, _i64, _i32, _i32, ctypes.c_int, _vp],
        ctypes.c_int,
    ),
    "dynconv_lowrank_decode_step": (
        [_vp, _i64p, _vp, _i64p, _vp, _i64, _vp, _vp, _i64p, _vp, _i64p, _i64, _i64, _i64, _i32, _i32, _i32,
         ctypes.c_int, _vp],
        ctypes.c_int,
    ),
}
# The packed-sequence variants take (seq_idx, ss) after the filter (w, ws), after the
# bias (low-rank), or after x (cache fill).
_SIGNATURES["dynconv_fwd_varlen"] = (
    _SIGNATURES["dynconv_fwd"][0][:4] + [_vp, _i64p] + _SIGNATURES["dynconv_fwd"][0][4:], ctypes.c_int)
_SIGNATURES["dynconv_bwd_varlen"] = (
    _SIGNATURES["dynconv_bwd"][0][:4] + [_vp, _i64p] + _SIGNATURES["dynconv_bwd"][0][4:], ctypes.c_int)
_SIGNATURES["dynconv_lowrank_fwd_varlen"] = (
    _SIGNATURES["dynconv_lowrank_fwd"][0][:7] + [_vp, _i64p] + _SIGNATURES["dynconv_lowrank_fwd"][0][7:], ctypes.c_int)
_SIGNATURES["dynconv_lowrank_bwd_varlen"] = (
    _SIGNATURES["dynconv_lowrank_bwd"][0][:7] + [_vp, _i64p] + _SIGNATURES["dynconv_lowrank_bwd"][0][7:], ctypes.c_int)
# (seq_idx, ss, conv_bias) after the filter; bwd: (seq_idx, ss) after the filter and
# dconv_bias after dw; decoding: conv_bias after the filter.
_SIGNATURES["dynconv_fwd_ex"] = (
    _SIGNATURES["dynconv_fwd"][0][:4] + [_vp, _i64p, _vp] + _SIGNATURES["dynconv_fwd"][0][4:], ctypes.c_int)
_SIGNATURES["dynconv_bwd_ex"] = (
    _SIGNATURES["dynconv_bwd"][0][:4] + [_vp, _i64p] + _SIGNATURES["dynconv_bwd"][0][4:10] + [_vp]
    + _SIGNATURES["dynconv_bwd"][0][10:], ctypes.c_int)
_SIGNATURES["dynconv_bwd_ex_workspace_size"] = ([_i64, _i64, _i64, _i32, _i32, ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_int], _sz)
_SIGNATURES["dynconv_decode_step_ex"] = (
    _SIGNATURES["dynconv_decode_step"][0][:4] + [_vp] + _SIGNATURES["dynconv_decode_step"][0][4:], ctypes.c_int)
_SIGNATURES["dynconv_gemm_fwd"] = (
    [_vp, _i64p, _vp, _i64, _vp, _i64p, _vp, _i64p, _i64, _i64, _i64, _i64, _i32, _i32, ctypes.c_int, _vp],
    ctypes.c_int)
_SIGNATURES["dynconv_gemm_lowrank_fwd"] = (
    [_vp, _i64p, _vp, _i64, _vp, _i64p, _vp, _i64, _vp, _vp, _i64p, _i64, _i64, _i64, _i64, _i32, _i32, _i32,
     ctypes.c_int, _vp],
    ctypes.c_int)
# the workspace pointer and size of dynconv_bwd_ex dropped
_SIGNATURES["dynconv_bwd_ex_noalloc"] = (
    _SIGNATURES["dynconv_bwd_ex"][0][:-3] + [_vp], ctypes.c_int)
# low-rank with a convolution bias: (seq_idx, ss, conv_bias) after the bias; bwd: (seq_idx, ss)
# after the bias and dconv_bias after db; decoding: conv_bias after the bias
_SIGNATURES["dynconv_lowrank_fwd_ex"] = (
    _SIGNATURES["dynconv_lowrank_fwd"][0][:7] + [_vp, _i64p, _vp] + _SIGNATURES["dynconv_lowrank_fwd"][0][7:],
    ctypes.c_int)
_SIGNATURES["dynconv_lowrank_bwd_ex"] = (
    _SIGNATURES["dynconv_lowrank_bwd"][0][:7] + [_vp, _i64p] + _SIGNATURES["dynconv_lowrank_bwd"][0][7:15] + [_vp]
    + _SIGNATURES["dynconv_lowrank_bwd"][0][15:], ctypes.c_int)
_SIGNATURES["dynconv_lowrank_bwd_ex_workspace_size"] = ([_i64, _i64, _i64, _i32, _i32, _i32, ctypes.c_int,
                                                         ctypes.c_int], _sz)
_SIGNATURES["dynconv_lowrank_decode_step_ex"] = (
    _SIGNATURES["dynconv_lowrank_decode_step"][0][:7] + [_vp] + _SIGNATURES["dynconv_lowrank_decode_step"][0][7:],
    ctypes.c_int)
_SIGNATURES["dynconv_cache_fill_varlen"] = (
    _SIGNATURES["dynconv_cache_fill"][0][:2] + [_vp, _i64p] + _SIGNATURES["dynconv_cache_fill"][0][2:], ctypes.c_int)

_lib = None


class DynconvError(RuntimeError):
    """A libdynconv entry point returned a status other than DYNCONV_OK."""

    def __init__(self, fn: str, status: int, hip_error: int = 0):
        self.status = status
        self.status_name = STATUS.get(status, f"status {status}")
        self.hip_error = hip_error
        msg = f"{fn} returned {self.status_name}"
        if hip_error:
            msg += f" (hipError {hip_error})"
        super().__init__(msg)


def load(path: str | None = None) -> ctypes.CDLL:
    """Loads libdynconv.so once (or the file DYNCONV_LIBRARY names, such as the host-only
    sanitized build); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("DYNCONV_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run `python -m dynamic_short_convolution_amd.build` "
            "(or __graft_entry__.build()) first. There is no fallback implementation."
        )
    lib = ctypes.CDLL(path)
    for name, (argtypes, restype) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = restype
    _lib = lib
    return lib


def strides(vals) -> ctypes.Array:
    arr = (ctypes.c_int64 * len(vals))(*[int(v) for v in vals])
    return arr


def check(fn: str, status: int) -> None:
    if status != 0:
        hip = load().dynconv_last_hip_error() if status == 4 else 0
        raise DynconvError(fn, status, hip)
