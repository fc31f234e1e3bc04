"""Python binding of libdynconv over torch tensors (argument marshalling only).

Every function has the name of the C entry point it calls; all compute runs in the HIP
kernels. Tensors must live on a ROCm device; PyTorch provides device memory and the
current stream, nothing else.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib

_DTYPE = {torch.float32: _lib.DYNCONV_F32, torch.bfloat16: _lib.DYNCONV_BF16, torch.float16: _lib.DYNCONV_F16}


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPE:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32, bfloat16 or float16")
    return _DTYPE[t.dtype]


def _require_device(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise RuntimeError("libdynconv runs on the GPU only: got a CPU tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise RuntimeError("all tensors must be on the same device")
    return dev


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def filter_strides(w: torch.Tensor):
    """Strides of a filter tensor: [B,T,G,W] as is; a static [G,W] filter gets zero b,t strides."""
    if w.dim() == 2:
        return [0, 0, w.stride(0), w.stride(1)]
    if w.dim() != 4:
        raise ValueError("filters are [B, T, D/H, W] or a static [D/H, W]")
    return list(w.stride())


def _seg_args(seq_idx, B: int, T: int):
    """(pointer, strides) of packed-sequence segment ids: int32 [B, T] (any strides)."""
    if seq_idx.dtype != torch.int32 or tuple(seq_idx.shape) != (B, T):
        raise ValueError(f"seq_idx must be int32 [B, T] = [{B}, {T}]; got {seq_idx.dtype} {tuple(seq_idx.shape)}")
    return _ptr(seq_idx), _lib.strides(seq_idx.stride())


def _conv_bias_arg(conv_bias, x):
    if conv_bias is None:
        return None
    D = x.shape[-1]
    if conv_bias.dim() != 1 or conv_bias.numel() != D or conv_bias.stride(0) != 1 or conv_bias.dtype != x.dtype:
        raise ValueError(f"conv_bias must be a contiguous [{D}] vector of dtype {x.dtype}")
    return conv_bias


def _expect(name: str, t, shape, dtype) -> None:
    """Raises unless t (if given) has exactly this shape and dtype: the C ABI receives
    strides, not extents, so a tensor of the wrong size would be read or written out of
    bounds instead of being refused."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {list(shape)}; got {list(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} is {t.dtype} but must be {dtype}")


def _groups(D: int, H: int) -> int:
    if H < 1 or D % H != 0:
        raise ValueError(f"H = {H} must be a positive divisor of D = {D}")
    return D // H


def _check_act3(x: torch.Tensor) -> tuple:
    if x.dim() != 3:
        raise ValueError(f"x must be [B, T, D]; got shape {list(x.shape)}")
    return tuple(x.shape)


def _check_filter(w: torch.Tensor, x: torch.Tensor, H: int) -> int:
    """w is per-token [B, T, D/H, W] or static [D/H, W], of x's dtype; returns W."""
    B, T, D = x.shape
    G = _groups(D, H)
    W = w.shape[-1]
    _expect("w", w, (G, W) if w.dim() == 2 else (B, T, G, W), x.dtype)
    return W


def dynconv_fwd(x: torch.Tensor, w: torch.Tensor, H: int = 1, out: torch.Tensor | None = None,
                seq_idx: torch.Tensor | None = None, conv_bias: torch.Tensor | None = None) -> torch.Tensor:
    """y = x + causal depthwise conv of x with per-token (or static) filters w (+ conv_bias
    [D] on every token). With seq_idx (int32 [B, T] segment ids of packed sequences) no tap
    crosses into another segment."""
    B, T, D = _check_act3(x)
    W = _check_filter(w, x, H)
    conv_bias = _conv_bias_arg(conv_bias, x)
    _expect("out", out, (B, T, D), x.dtype)
    y = torch.empty_like(x) if out is None else out
    dev = _require_device(x, w, y, seq_idx, conv_bias)
    lib = _lib.load()
    head = (_ptr(x), _lib.strides(x.stride()), _ptr(w), _lib.strides(filter_strides(w)))
    tail = (_ptr(y), _lib.strides(y.stride()), B, T, D, W, H, _dtype_code(x), _stream(dev))
    if conv_bias is not None:
        seg = _seg_args(seq_idx, B, T) if seq_idx is not None else (None, None)
        st = lib.dynconv_fwd_ex(*head, *seg, _ptr(conv_bias), *tail)
    elif seq_idx is None:
        st = lib.dynconv_fwd(*head, *tail)
    else:
        st = lib.dynconv_fwd_varlen(*head, *_seg_args(seq_idx, B, T), *tail)
    _lib.check("dynconv_fwd", st)
    return y


def dynconv_bwd_workspace_size(B, T, D, W, H, is_static, dtype) -> int:
    return int(_lib.load().dynconv_bwd_workspace_size(B, T, D, W, H, int(bool(is_static)), _DTYPE[dtype]))


def dynconv_bwd(x, w, dy, H: int = 1, need_dx: bool = True, need_dw: bool = True, dx=None, dw=None, seq_idx=None,
                want_dconv_bias: bool = False):
    """(dx, dw) of <dy, dynconv_fwd(x, w, H, seq_idx=seq_idx)>; dw of a static filter is
    float32 [D/H, W]. With want_dconv_bias, (dx, dw, dconv_bias) where dconv_bias is the
    float32 [D] gradient of a convolution bias (the sum of dy over every token)."""
    B, T, D = _check_act3(x)
    W = _check_filter(w, x, H)
    is_static = w.dim() == 2
    _expect("dy", dy, (B, T, D), x.dtype)
    _expect("dx", dx, (B, T, D), x.dtype)
    _expect("dw", dw, (D // H, W) if is_static else (B, T, D // H, W), torch.float32 if is_static else x.dtype)
    if need_dx and dx is None:
        dx = torch.empty_like(x)
    if need_dw and dw is None:
        dw = (torch.empty((D // H, W), dtype=torch.float32, device=x.device) if is_static
              else torch.empty((B, T, D // H, W), dtype=x.dtype, device=x.device))
    dev = _require_device(x, w, dy, dx, dw, seq_idx)
    lib = _lib.load()
    if want_dconv_bias:
        dcb = torch.empty((D,), dtype=torch.float32, device=x.device)
        ws_bytes = int(lib.dynconv_bwd_ex_workspace_size(B, T, D, W, H, int(is_static and need_dw), 1,
                                                         _DTYPE[x.dtype]))
    else:
        ws_bytes = dynconv_bwd_workspace_size(B, T, D, W, H, is_static and need_dw, x.dtype)
    work = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device) if ws_bytes else None
    head = (_ptr(x), _lib.strides(x.stride()), _ptr(w), _lib.strides(filter_strides(w)))
    tail = (
        _ptr(dy), _lib.strides(dy.stride()),
        _ptr(dx if need_dx else None), _lib.strides(dx.stride()) if need_dx else None,
        _ptr(dw if need_dw else None), _lib.strides(dw.stride()) if (need_dw and not is_static) else None,
        B, T, D, W, H, _dtype_code(x), _ptr(work), ws_bytes, _stream(dev),
    )
    if want_dconv_bias:
        seg = _seg_args(seq_idx, B, T) if seq_idx is not None else (None, None)
        st = lib.dynconv_bwd_ex(*head, *seg, *tail[:6], _ptr(dcb), *tail[6:])
        _lib.check("dynconv_bwd", st)
        return (dx if need_dx else None), (dw if need_dw else None), dcb
    if seq_idx is None:
        st = lib.dynconv_bwd(*head, *tail)
    else:
        st = lib.dynconv_bwd_varlen(*head, *_seg_args(seq_idx, B, T), *tail)
    _lib.check("dynconv_bwd", st)
    return (dx if need_dx else None), (dw if need_dw else None)


def dynconv_bwd_ex_noalloc(x, w, dy, H: int = 1, dx=None, dw=None, dconv_bias=None, seq_idx=None):
    """The allocation-free backward: (dx, dw, dconv_bias) as dynconv_bwd(..., want_dconv_bias=
    dconv_bias is not None) computes them, with the partial sums in the library's per-GPU
    scratch array instead of a workspace. The caller passes every output it wants (dx
    [B,T,D], dw per-token [B,T,D/H,W] or float32 [D/H,W] for a static w, dconv_bias float32
    [D]); this binding allocates nothing either. Calls that overlap on one GPU race."""
    B, T, D = _check_act3(x)
    W = _check_filter(w, x, H)
    is_static = w.dim() == 2
    _expect("dy", dy, (B, T, D), x.dtype)
    _expect("dx", dx, (B, T, D), x.dtype)
    _expect("dw", dw, (D // H, W) if is_static else (B, T, D // H, W), torch.float32 if is_static else x.dtype)
    _expect("dconv_bias", dconv_bias, (D,), torch.float32)
    dev = _require_device(x, w, dy, dx, dw, dconv_bias, seq_idx)
    seg = _seg_args(seq_idx, B, T) if seq_idx is not None else (None, None)
    st = _lib.load().dynconv_bwd_ex_noalloc(
        _ptr(x), _lib.strides(x.stride()), _ptr(w), _lib.strides(filter_strides(w)), *seg,
        _ptr(dy), _lib.strides(dy.stride()), _ptr(dx), _lib.strides(dx.stride()) if dx is not None else None,
        _ptr(dw), _lib.strides(dw.stride()) if (dw is not None and not is_static) else None, _ptr(dconv_bias),
        B, T, D, W, H, _dtype_code(x), _stream(dev))
    _lib.check("dynconv_bwd_ex_noalloc", st)
    return dx, dw, dconv_bias


def _check_lowrank_operands(x, z, U, bias, J: int):
    """z is [B, T, R] (or [B, R] for a decoding step, x [B, D]), U is [R, J] with unit
    column stride (rows ldu = U.stride(0) apart), bias a contiguous [J] vector or None, and
    every operand has the dtype of x."""
    R = z.shape[-1]
    if z.dim() != x.dim() or tuple(z.shape[:-1]) != tuple(x.shape[:-1]):
        raise ValueError(f"z must be {list(x.shape[:-1]) + ['R']}; got shape {list(z.shape)}")
    if U.dim() != 2 or tuple(U.shape) != (R, J) or (J > 1 and U.stride(1) != 1):
        raise ValueError(f"U must be [R, J] = [{R}, {J}] with unit column stride; got shape "
                         f"{tuple(U.shape)} strides {tuple(U.stride())}")
    if bias is not None and (bias.dim() != 1 or bias.numel() != J or (J > 1 and bias.stride(0) != 1)):
        raise ValueError(f"bias must be a contiguous [{J}] vector")
    for name, t in (("z", z), ("U", U), ("bias", bias)):
        if t is not None and t.dtype != x.dtype:
            raise TypeError(f"{name} is {t.dtype} but x is {x.dtype}")


def dynconv_lowrank_fwd(x, z, U, bias, W: int, H: int = 1, out=None, seq_idx=None, conv_bias=None):
    """y = x + conv(x) with filters z U + bias generated on the GPU (never stored), plus
    conv_bias [D] on every token if given; with seq_idx (int32 [B, T]) no tap crosses into
    another segment."""
    B, T, D = _check_act3(x)
    R = z.shape[-1]
    _check_lowrank_operands(x, z, U, bias, _groups(D, H) * W)
    conv_bias = _conv_bias_arg(conv_bias, x)
    _expect("out", out, (B, T, D), x.dtype)
    y = torch.empty_like(x) if out is None else out
    dev = _require_device(x, z, U, bias, y, seq_idx, conv_bias)
    lib = _lib.load()
    head = (_ptr(x), _lib.strides(x.stride()), _ptr(z), _lib.strides(z.stride()), _ptr(U), U.stride(0), _ptr(bias))
    tail = (_ptr(y), _lib.strides(y.stride()), B, T, D, W, H, R, _dtype_code(x), _stream(dev))
    if conv_bias is not None:
        seg = _seg_args(seq_idx, B, T) if seq_idx is not None else (None, None)
        st = lib.dynconv_lowrank_fwd_ex(*head, *seg, _ptr(conv_bias), *tail)
    elif seq_idx is None:
        st = lib.dynconv_lowrank_fwd(*head, *tail)
    else:
        st = lib.dynconv_lowrank_fwd_varlen(*head, *_seg_args(seq_idx, B, T), *tail)
    _lib.check("dynconv_lowrank_fwd", st)
    return y


def dynconv_lowrank_bwd_workspace_size(B, T, D, W, H, R, dtype, want_dconv_bias: bool = False) -> int:
    return int(_lib.load().dynconv_lowrank_bwd_ex_workspace_size(B, T, D, W, H, R, int(bool(want_dconv_bias)),
                                                                 _DTYPE[dtype]))


def dynconv_lowrank_bwd(x, z, U, bias, dy, W: int, H: int = 1, need_db: bool = True, workspace=None,
                        seq_idx=None, want_dconv_bias: bool = False):
    """(dx, dz, dU, db) of <dy, dynconv_lowrank_fwd(...)>; dU and db are float32. With
    want_dconv_bias, (dx, dz, dU, db, dconv_bias): the float32 [D] gradient of a convolution
    bias (the sum of dy over every token). A caller's workspace must be a contiguous tensor
    on x's device of at least dynconv_lowrank_bwd_workspace_size(..., want_dconv_bias)
    bytes (the library checks the size)."""
    B, T, D = _check_act3(x)
    R = z.shape[-1]
    J = _groups(D, H) * W
    _check_lowrank_operands(x, z, U, bias, J)
    _expect("dy", dy, (B, T, D), x.dtype)
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    dev = _require_device(x, z, U, bias, dy, seq_idx, workspace)
    dx = torch.empty_like(x)
    dz = torch.empty_like(z)
    dU = torch.empty((R, J), dtype=torch.float32, device=x.device)
    db = torch.empty((J,), dtype=torch.float32, device=x.device) if need_db else None
    dcb = torch.empty((D,), dtype=torch.float32, device=x.device) if want_dconv_bias else None
    lib = _lib.load()
    if workspace is None:
        ws_bytes = dynconv_lowrank_bwd_workspace_size(B, T, D, W, H, R, x.dtype, want_dconv_bias)
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    else:
        ws_bytes = workspace.numel() * workspace.element_size()
    head = (_ptr(x), _lib.strides(x.stride()), _ptr(z), _lib.strides(z.stride()), _ptr(U), U.stride(0), _ptr(bias))
    tail = (
        _ptr(dy), _lib.strides(dy.stride()), _ptr(dx), _lib.strides(dx.stride()), _ptr(dz), _lib.strides(dz.stride()),
        _ptr(dU), _ptr(db), B, T, D, W, H, R, _dtype_code(x), _ptr(workspace), ws_bytes, _stream(dev),
    )
    if want_dconv_bias:
        seg = _seg_args(seq_idx, B, T) if seq_idx is not None else (None, None)
        st = lib.dynconv_lowrank_bwd_ex(*head, *seg, *tail[:8], _ptr(dcb), *tail[8:])
        _lib.check("dynconv_lowrank_bwd", st)
        return dx, dz, dU, db, dcb
    if seq_idx is None:
        st = lib.dynconv_lowrank_bwd(*head, *tail)
    else:
        st = lib.dynconv_lowrank_bwd_varlen(*head, *_seg_args(seq_idx, B, T), *tail)
    _lib.check("dynconv_lowrank_bwd", st)
    return dx, dz, dU, db


# ----------------------------------------------------------------------------------
# The convolution in the epilogue of the producing projection: X = A Wp^T is formed in
# the same kernel and never stored
# ----------------------------------------------------------------------------------


def _check_projection(A, Wp, H: int):
    B, T, K = _check_act3(A)
    if Wp.dim() != 2 or Wp.shape[1] != K or (K > 1 and Wp.stride(1) != 1):
        raise ValueError(f"Wp must be [N, K={K}] with unit column stride; got shape {list(Wp.shape)} "
                         f"strides {list(Wp.stride())}")
    if Wp.dtype != A.dtype:
        raise TypeError(f"Wp is {Wp.dtype} but A is {A.dtype}")
    N = Wp.shape[0]
    return B, T, K, N, _groups(N, H)


def dynconv_gemm_fwd(A, Wp, w, H: int = 1, out=None):
    """y = X + conv(X) with X = A Wp^T (A [B,T,K], Wp [N,K]) computed in the same kernel;
    w: per-token filters [B,T,N/H,W] or a static [N/H,W]."""
    B, T, K, N, G = _check_projection(A, Wp, H)
    W = w.shape[-1]
    _expect("w", w, (G, W) if w.dim() == 2 else (B, T, G, W), A.dtype)
    _expect("out", out, (B, T, N), A.dtype)
    dev = _require_device(A, Wp, w, out)
    y = torch.empty((B, T, N), dtype=A.dtype, device=A.device) if out is None else out
    st = _lib.load().dynconv_gemm_fwd(_ptr(A), _lib.strides(A.stride()), _ptr(Wp), Wp.stride(0), _ptr(w),
                                      _lib.strides(filter_strides(w)), _ptr(y), _lib.strides(y.stride()), B, T, N, K,
                                      W, H, _dtype_code(A), _stream(dev))
    _lib.check("dynconv_gemm_fwd", st)
    return y


def dynconv_gemm_lowrank_fwd(A, Wp, z, U, bias, W: int, H: int = 1, out=None):
    """y = X + conv(X) with X = A Wp^T and filters z U + bias, both formed in the same kernel
    (neither X nor the filters are stored). z [B,T,R], U [R,(N/H)*W], bias [(N/H)*W] or None."""
    B, T, K, N, G = _check_projection(A, Wp, H)
    R = z.shape[-1]
    _check_lowrank_operands(A, z, U, bias, G * W)  # z [B, T, R] like A's leading dims, A's dtype
    _expect("out", out, (B, T, N), A.dtype)
    dev = _require_device(A, Wp, z, U, bias, out)
    y = torch.empty((B, T, N), dtype=A.dtype, device=A.device) if out is None else out
    st = _lib.load().dynconv_gemm_lowrank_fwd(
        _ptr(A), _lib.strides(A.stride()), _ptr(Wp), Wp.stride(0), _ptr(z), _lib.strides(z.stride()), _ptr(U),
        U.stride(0), _ptr(bias), _ptr(y), _lib.strides(y.stride()), B, T, N, K, W, H, R, _dtype_code(A), _stream(dev))
    _lib.check("dynconv_gemm_lowrank_fwd", st)
    return y


# ----------------------------------------------------------------------------------
# Inference: rolling cache of the last W-1 inputs, single-token decoding steps
# ----------------------------------------------------------------------------------


def new_cache(B: int, D: int, W: int, dtype, device) -> torch.Tensor | None:
    """A zeroed [B, W-1, D] cache (None for W == 1)."""
    if W == 1:
        return None
    return torch.zeros((B, W - 1, D), dtype=dtype, device=device)


def dynconv_cache_fill(x, W: int, cache=None, seq_idx=None):
    """Fills the cache with the last W-1 tokens of a prompt x [B,T,D] (zeros before t = 0).
    With seq_idx (int32 [B, T]) of a packed prompt, only the tokens of the last document
    (the segment of token T-1) are kept."""
    B, T, D = _check_act3(x)
    if W < 1:
        raise ValueError(f"W = {W} must be positive")
    _expect("cache", cache, (B, W - 1, D), x.dtype)
    if cache is None:
        cache = new_cache(B, D, W, x.dtype, x.device)
    if cache is None:
        return None
    dev = _require_device(x, cache, seq_idx)
    lib = _lib.load()
    if seq_idx is None:
        st = lib.dynconv_cache_fill(_ptr(x), _lib.strides(x.stride()), _ptr(cache), _lib.strides(cache.stride()),
                                    B, T, D, W, _dtype_code(x), _stream(dev))
    else:
        st = lib.dynconv_cache_fill_varlen(_ptr(x), _lib.strides(x.stride()), *_seg_args(seq_idx, B, T), _ptr(cache),
                                           _lib.strides(cache.stride()), B, T, D, W, _dtype_code(x), _stream(dev))
    _lib.check("dynconv_cache_fill", st)
    return cache


def dynconv_decode_step(x, w, cache, t: int, H: int = 1, out=None, conv_bias=None):
    """y [B,D] of token t from x [B,D], its filters w [B,D/H,W] (or a static [D/H,W]) and
    the cache of the previous W-1 inputs, which is updated in place (+ conv_bias [D])."""
    if x.dim() != 2:
        raise ValueError(f"x must be [B, D]; got shape {list(x.shape)}")
    B, D = x.shape
    G = _groups(D, H)
    W = w.shape[-1]
    _expect("w", w, (G, W) if w.dim() == 2 else (B, G, W), x.dtype)
    _expect("cache", cache, (B, W - 1, D), x.dtype)
    if cache is None and W > 1:
        raise ValueError("a cache [B, W-1, D] is required for W > 1")
    _expect("out", out, (B, D), x.dtype)
    ws = [0, w.stride(0), w.stride(1)] if w.dim() == 2 else list(w.stride())
    y = torch.empty_like(x) if out is None else out
    conv_bias = _conv_bias_arg(conv_bias, x)
    dev = _require_device(x, w, y, cache, conv_bias)
    cs = _lib.strides(cache.stride()) if cache is not None else None
    st = _lib.load().dynconv_decode_step_ex(_ptr(x), _lib.strides(x.stride()), _ptr(w), _lib.strides(ws),
                                            _ptr(conv_bias), _ptr(cache), cs, _ptr(y), _lib.strides(y.stride()),
                                            int(t), B, D, W, H, _dtype_code(x), _stream(dev))
    _lib.check("dynconv_decode_step", st)
    return y


def dynconv_lowrank_decode_step(x, z, U, bias, cache, t: int, W: int, out=None, H: int = 1, conv_bias=None):
    """y [B,D] of token t with filters z [B,R] U + bias generated on the GPU (U: [R, (D/H)*W]),
    plus conv_bias [D] if given; the cache is updated in place."""
    if x.dim() != 2:
        raise ValueError(f"x must be [B, D]; got shape {list(x.shape)}")
    B, D = x.shape
    R = z.shape[-1]
    _check_lowrank_operands(x, z, U, bias, _groups(D, H) * W)
    _expect("cache", cache, (B, W - 1, D), x.dtype)
    if cache is None and W > 1:
        raise ValueError("a cache [B, W-1, D] is required for W > 1")
    _expect("out", out, (B, D), x.dtype)
    y = torch.empty_like(x) if out is None else out
    conv_bias = _conv_bias_arg(conv_bias, x)
    dev = _require_device(x, z, U, bias, y, cache, conv_bias)
    cs = _lib.strides(cache.stride()) if cache is not None else None
    st = _lib.load().dynconv_lowrank_decode_step_ex(
        _ptr(x), _lib.strides(x.stride()), _ptr(z), _lib.strides(z.stride()), _ptr(U), U.stride(0), _ptr(bias),
        _ptr(conv_bias), _ptr(cache), cs, _ptr(y), _lib.strides(y.stride()), int(t), B, D, W, H, R, _dtype_code(x),
        _stream(dev))
    _lib.check("dynconv_lowrank_decode_step", st)
    return y
