"""The C ABI on the host: every declared symbol is exported, and every validation path
returns its status before any HIP call (so these run without a GPU).

Pointers below are fake, non-null addresses: the calls must reject the arguments
before touching them.
"""
import ctypes
import itertools
import os
import re

import pytest

from dynamic_short_convolution_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUP, WORKSPACE = 0, 1, 2, 3
F32, BF16 = 0, 1


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from dynamic_short_convolution_amd import build

        build.build()
    return _lib.load()


def _declared_symbols():
    with open(os.path.join(ROOT, "include", "dynconv.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(dynconv_[a-z_]+)\s*\(", text)))


def test_header_symbols_are_exported(lib):
    declared = _declared_symbols()
    assert set(declared) == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code, name in _lib.STATUS.items():
        assert lib.dynconv_status_string(code).decode() == name
    assert lib.dynconv_last_hip_error() == 0


P = ctypes.c_void_p  # fake device pointers, never dereferenced
X, W_, Y, DY, DX, DW, Z, U = (P(0x10000 * (i + 1)) for i in range(8))


def S(*v):
    return _lib.strides(v)


def fwd(lib, x=X, xs=(800, 200, 1), w=W_, ws=(800 * 4, 200 * 4, 4, 1), y=Y, ys=(800, 200, 1), B=2, T=4, D=200, W=4,
        H=1, dt=BF16):
    return lib.dynconv_fwd(x, S(*xs), w, S(*ws), y, S(*ys), B, T, D, W, H, dt, None)


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(dt=7), INVALID),
        (dict(B=-1), INVALID),
        (dict(W=0), INVALID),
        (dict(W=9), UNSUP),
        (dict(H=0), INVALID),
        (dict(D=200, H=3), INVALID),  # 3 does not divide 200
        # odd H: one bf16 channel per lane, a group of 99 lanes would straddle waves
        (dict(D=198, H=99, xs=(792, 198, 1), ys=(792, 198, 1), ws=(8 * 4, 2 * 4, 4, 1)), UNSUP),
        # H = 3 * 512: 12 channels per lane, 128 lanes per group
        (dict(D=3072, H=1536, xs=(4 * 3072, 3072, 1), ys=(4 * 3072, 3072, 1), ws=(8 * 4, 2 * 4, 4, 1)), UNSUP),
        # H = 5 * 256: 10 channels per lane, 128 lanes per group
        (dict(D=2560, H=1280, xs=(4 * 2560, 2560, 1), ys=(4 * 2560, 2560, 1), ws=(8 * 4, 2 * 4, 4, 1)), UNSUP),
        # float32 H = 5 * 64 with 8-byte rows: 2 channels per lane, 160 lanes per group
        (dict(D=640, H=320, xs=(4 * 640 + 2, 640, 1), ys=(4 * 640 + 2, 640, 1), ws=(8 * 4, 2 * 4, 4, 1), dt=0),
         UNSUP),
        (dict(x=P(0)), INVALID),
        (dict(y=P(0)), INVALID),
        (dict(w=P(0)), INVALID),
        (dict(y=X), INVALID),  # in place
        (dict(xs=(800, 200, 2)), UNSUP),
        (dict(ws=(800 * 4, 200 * 4, 3, 1)), UNSUP),  # taps of a group not contiguous
        (dict(ws=(800 * 4, 200 * 4, 4, 2)), UNSUP),
        (dict(x=P(0x10002)), UNSUP),  # bf16 activations need 4-byte alignment
        (dict(D=199, xs=(796, 199, 1), ys=(796, 199, 1), ws=(796 * 4, 199 * 4, 4, 1)), UNSUP),  # odd D in bf16
        (dict(B=0), OK),  # empty: no-op
        (dict(T=0), OK),
    ],
)
def test_fwd_validation(lib, kw, status):
    assert fwd(lib, **kw) == status


def bwd(lib, dx=DX, dw=DW, ws=(800 * 4, 200 * 4, 4, 1), dws=(800 * 4, 200 * 4, 4, 1), wsp=None, wsb=0, H=1, D=200,
        dy=DY):
    return lib.dynconv_bwd(X, S(800, D, 1), W_, S(*ws), dy, S(800, D, 1), dx, S(800, D, 1), dw, S(*dws) if dws else None,
                           2, 4, D, 4, H, BF16, wsp, wsb, None)


def test_bwd_validation(lib):
    assert bwd(lib, dx=P(0), dw=P(0)) == INVALID
    assert bwd(lib, dx=DY) == INVALID  # dx aliasing dy
    assert bwd(lib, dw=W_) == INVALID  # dw aliasing w
    assert bwd(lib, dx=DW, dw=DW) == INVALID
    assert bwd(lib, dy=P(0)) == INVALID
    # batch-shared but per-token filters: dw would need a batch reduction
    assert bwd(lib, ws=(0, 200 * 4, 4, 1)) == UNSUP
    assert bwd(lib, dws=None) == INVALID
    # static filter: needs a workspace for the partial sums
    need = lib.dynconv_bwd_workspace_size(2, 4, 200, 4, 1, 1, BF16)
    assert need > 0
    assert bwd(lib, ws=(0, 0, 4, 1), dws=None, wsp=None, wsb=0) == WORKSPACE
    assert bwd(lib, ws=(0, 0, 4, 1), dws=None, wsp=P(0x900000), wsb=need - 1) == WORKSPACE
    assert lib.dynconv_bwd_workspace_size(2, 4, 200, 4, 1, 0, BF16) == 0


def test_workspace_queries(lib):
    assert lib.dynconv_bwd_workspace_size(8, 4096, 2048, 3, 1, 1, BF16) % 4 == 0
    assert lib.dynconv_bwd_workspace_size(8, 4096, 2048, 9, 1, 1, BF16) == 0  # invalid W
    assert lib.dynconv_bwd_workspace_size(8, 4096, 2048, 8, 1, 1, BF16) > 0
    # groups that only the widest lane vectors serve (512 bf16 channels: 64 lanes of 8), or
    # none (odd 99: 99 lanes), and groups whose size is not a power of two
    for H, dt in ((512, BF16), (256, F32), (384, BF16), (96, F32), (3, BF16), (63, F32), (99, BF16)):
        n = lib.dynconv_bwd_ex_workspace_size(2, 50, 16 * H, 3, H, 1, 1, dt)
        assert n > 0 or H == 99
        assert n % 4 == 0
    assert lib.dynconv_lowrank_bwd_workspace_size(8, 4096, 2048, 9, 1, 64, BF16) == 0  # low-rank: W <= 8
    assert lib.dynconv_lowrank_bwd_workspace_size(8, 4096, 2048, 8, 1, 64, BF16) > 0
    n = lib.dynconv_lowrank_bwd_workspace_size(8, 4096, 2048, 4, 1, 64, BF16)
    assert n >= 64 * 2048 * 4 * 4  # at least one float32 dU partial
    assert lib.dynconv_lowrank_bwd_workspace_size(8, 4096, 2048, 4, 1, 0, BF16) == 0


def lr_fwd(lib, R=64, z=Z, U_=U, ldu=800, H=1, x=X, y=Y, W=4, D=200):
    return lib.dynconv_lowrank_fwd(x, S(800, D, 1), z, S(4 * R, R, 1), U_, ldu, None, y, S(800, D, 1), 2, 4, D, W, H,
                                   R, BF16, None)


def test_lowrank_validation(lib):
    assert lr_fwd(lib, R=0) == INVALID
    assert lr_fwd(lib, R=129) == UNSUP
    assert lr_fwd(lib, z=P(0)) == INVALID
    assert lr_fwd(lib, U_=P(0)) == INVALID
    assert lr_fwd(lib, y=X) == INVALID
    assert lr_fwd(lib, ldu=100) == INVALID  # row shorter than (D/H)*W
    assert lr_fwd(lib, H=3) == INVALID  # 3 does not divide D = 200
    assert lr_fwd(lib, H=2, ldu=399) == INVALID  # head-wise: rows hold (D/H)*W = 400 columns
    assert lr_fwd(lib, W=9, ldu=1800) == UNSUP  # the low-rank kernels take W <= 8
    need = lib.dynconv_lowrank_bwd_workspace_size(2, 4, 200, 4, 1, 64, BF16)
    st = lib.dynconv_lowrank_bwd(X, S(800, 200, 1), Z, S(256, 64, 1), U, 800, None, DY, S(800, 200, 1), DX,
                                 S(800, 200, 1), P(0x990000), S(256, 64, 1), P(0x9a0000), None, 2, 4, 200, 4, 1, 64,
                                 BF16, P(0x9b0000), need - 1, None)
    assert st == WORKSPACE


def test_lowrank_conv_bias_validation(lib):
    """dynconv_lowrank_{fwd,bwd,decode_step}_ex: the bias may not alias the output, needs
    4-byte alignment (element alignment when decoding), and the bias gradient needs its own
    workspace (the partial sums of dy after those of dU and db) and a distinct output."""
    CB, DCB = P(0xB00000), P(0xB10000)

    def fwd_(cb=CB, y=Y, seq=None):
        return lib.dynconv_lowrank_fwd_ex(X, S(800, 200, 1), Z, S(256, 64, 1), U, 800, None, seq, S(4, 1) if seq else
                                          None, cb, y, S(800, 200, 1), 2, 4, 200, 4, 1, 64, BF16, None)

    assert fwd_(cb=Y) == INVALID
    assert fwd_(cb=P(0xB00002)) == UNSUP  # 2-byte aligned
    assert fwd_(seq=P(0xB20002)) == UNSUP  # segment ids are int32: 4-byte aligned

    base = lib.dynconv_lowrank_bwd_workspace_size(2, 4, 200, 4, 1, 64, BF16)
    need = lib.dynconv_lowrank_bwd_ex_workspace_size(2, 4, 200, 4, 1, 64, 1, BF16)
    assert lib.dynconv_lowrank_bwd_ex_workspace_size(2, 4, 200, 4, 1, 64, 0, BF16) == base
    assert need >= base + 2 * 200 * 4  # at least one float32 partial per sequence and channel
    big = lib.dynconv_lowrank_bwd_ex_workspace_size(8, 4096, 2048, 4, 1, 64, 1, BF16)
    assert big % 4 == 0 and big > lib.dynconv_lowrank_bwd_workspace_size(8, 4096, 2048, 4, 1, 64, BF16)

    def bwd_(dcb=DCB, wsb=need, db=None):
        return lib.dynconv_lowrank_bwd_ex(X, S(800, 200, 1), Z, S(256, 64, 1), U, 800, None, None, None, DY,
                                          S(800, 200, 1), DX, S(800, 200, 1), P(0x990000), S(256, 64, 1), P(0x9a0000),
                                          db, dcb, 2, 4, 200, 4, 1, 64, BF16, P(0x9b0000), wsb, None)

    assert bwd_(wsb=need - 1) == WORKSPACE
    assert bwd_(dcb=DX) == INVALID  # aliases dx
    assert bwd_(dcb=DY) == INVALID  # aliases an input
    assert bwd_(dcb=P(0x9a0000)) == INVALID  # aliases dU
    assert bwd_(dcb=P(0xB10002)) == UNSUP  # float32 output 2-byte aligned

    def dec_(cb=CB, y=P(0xC00000)):
        return lib.dynconv_lowrank_decode_step_ex(X, S(200, 1), Z, S(64, 1), U, 800, None, cb, P(0xA00000),
                                                  S(600, 200, 1), y, S(200, 1), 5, 2, 200, 4, 1, 64, BF16, None)

    assert dec_(cb=P(0xC00000)) == INVALID
    assert dec_(cb=P(0xA00000)) == INVALID  # aliases the cache
    assert dec_(cb=P(0xB00001)) == UNSUP  # not element aligned


def test_lowrank_row_stride_bound(lib):
    """Row strides of 2^24 elements or more are refused before any launch: the low-rank
    kernels form the offsets of up to 128 rows in 32-bit arithmetic."""
    big = 1 << 24

    def fwd_(xs1=200, zs1=64, ys1=200, ldu=800):
        return lib.dynconv_lowrank_fwd(X, S(4 * xs1, xs1, 1), Z, S(4 * zs1, zs1, 1), U, ldu, None, Y,
                                       S(4 * ys1, ys1, 1), 2, 4, 200, 4, 1, 64, BF16, None)

    def bwd_(dys1=200, dxs1=200):
        need = lib.dynconv_lowrank_bwd_workspace_size(2, 4, 200, 4, 1, 64, BF16)
        return lib.dynconv_lowrank_bwd(X, S(800, 200, 1), Z, S(256, 64, 1), U, 800, None, DY, S(4 * dys1, dys1, 1),
                                       DX, S(4 * dxs1, dxs1, 1), P(0x990000), S(256, 64, 1), P(0x9a0000), None, 2, 4,
                                       200, 4, 1, 64, BF16, P(0x9b0000), need, None)

    for kw in (dict(xs1=big), dict(zs1=big), dict(ys1=big), dict(ldu=big)):
        assert fwd_(**kw) == UNSUP, kw
    for kw in (dict(dys1=big), dict(dxs1=big)):
        assert bwd_(**kw) == UNSUP, kw


C = P(0xA00000)  # fake cache


def dec(lib, x=X, xs=(200, 1), w=W_, ws=(200 * 4, 4, 1), cache=C, cs=(600, 200, 1), y=Y, ys=(200, 1), t=5, B=2,
        D=200, W=4, H=1, dt=BF16):
    return lib.dynconv_decode_step(x, S(*xs), w, S(*ws), cache, S(*cs) if cs else None, y, S(*ys), t, B, D, W, H, dt,
                                   None)


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(t=-1), INVALID),
        (dict(W=9), UNSUP),
        (dict(x=P(0)), INVALID),
        (dict(y=P(0)), INVALID),
        (dict(w=P(0)), INVALID),
        (dict(cache=P(0)), INVALID),
        (dict(cs=None), INVALID),
        (dict(cs=(600, 200, 2)), UNSUP),
        (dict(xs=(200, 2)), UNSUP),
        (dict(ws=(200 * 4, 3, 1)), UNSUP),  # taps of a group not contiguous
        (dict(y=X), INVALID),
        (dict(y=C), INVALID),
        (dict(cache=X), INVALID),
        (dict(x=P(0x10001)), UNSUP),  # bf16 needs element alignment
        (dict(W=1, ws=(200, 1, 1), cache=P(0), cs=None, B=0), OK),  # no history: no cache needed
        (dict(B=0), OK),
        (dict(D=0), OK),
    ],
)
def test_decode_validation(lib, kw, status):
    assert dec(lib, **kw) == status


def test_cache_fill_and_lowrank_decode_validation(lib):
    fill = lambda **kw: lib.dynconv_cache_fill(kw.get("x", X), S(800, 200, 1), kw.get("cache", C), S(600, 200, 1), 2,
                                               kw.get("T", 4), 200, kw.get("W", 4), BF16, None)
    assert fill(W=0) == INVALID
    assert fill(T=-1) == INVALID
    assert fill(cache=P(0)) == INVALID
    assert fill(x=P(0)) == INVALID

    def lrd(**kw):
        R = kw.get("R", 64)
        return lib.dynconv_lowrank_decode_step(X, S(200, 1), kw.get("z", Z), S(R, 1), kw.get("U_", U), kw.get("ldu", 800),
                                               None, C, S(600, 200, 1), kw.get("y", Y), S(200, 1), kw.get("t", 0), 2,
                                               200, 4, kw.get("H", 1), R, BF16, None)

    assert lrd(R=0) == INVALID
    assert lrd(R=129) == UNSUP
    assert lrd(H=3) == INVALID  # 3 does not divide D = 200
    assert lrd(z=P(0)) == INVALID
    assert lrd(U_=P(0)) == INVALID
    assert lrd(ldu=100) == INVALID
    assert lrd(y=Z) == INVALID
    assert lrd(t=-3) == INVALID


def test_lowrank_bindings_reject_bad_operands():
    """The Python bindings refuse a transposed U, a strided bias and mixed dtypes before any
    device work (CPU tensors suffice: these checks come first)."""
    import torch

    from dynamic_short_convolution_amd import dynconv_lowrank_decode_step, dynconv_lowrank_fwd

    B, T, D, W, R = 2, 3, 8, 4, 16
    x = torch.zeros((B, T, D), dtype=torch.bfloat16)
    z = torch.zeros((B, T, R), dtype=torch.bfloat16)
    U = torch.zeros((R, D * W), dtype=torch.bfloat16)
    b = torch.zeros((D * W,), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="unit column stride"):
        dynconv_lowrank_fwd(x, z, torch.zeros((D * W, R), dtype=torch.bfloat16).t(), b, W)
    with pytest.raises(ValueError, match=r"\[R, J\]"):
        dynconv_lowrank_fwd(x, z, U[:, : D * W - 1], b, W)
    with pytest.raises(ValueError, match="bias"):
        dynconv_lowrank_fwd(x, z, U, torch.zeros((2 * D * W,), dtype=torch.bfloat16)[::2], W)
    with pytest.raises(TypeError, match="U is torch.float32"):
        dynconv_lowrank_fwd(x, z, U.float(), b, W)
    with pytest.raises(RuntimeError, match="GPU only"):
        dynconv_lowrank_fwd(x, z, U, b, W)
    with pytest.raises(ValueError, match="unit column stride"):
        dynconv_lowrank_decode_step(x[:, 0], z[:, 0], U.t().contiguous().t(), b, None, 0, W)


SEG = P(0x90000)


def test_varlen_validation(lib):
    """The packed-sequence calls check their segment ids first, then everything the call
    without the suffix checks (B == 0 stays a no-op)."""
    def fv(seg=SEG, ss=(4, 1), **kw):
        x, y = kw.get("x", X), kw.get("y", Y)
        return lib.dynconv_fwd_varlen(x, S(800, 200, 1), W_, S(800 * 4, 200 * 4, 4, 1), seg,
                                      S(*ss) if ss is not None else None, y, S(800, 200, 1), kw.get("B", 2), 4, 200,
                                      4, 1, BF16, None)

    assert fv(seg=P(0)) == INVALID
    assert fv(ss=None) == INVALID
    assert fv(ss=(-4, 1)) == UNSUP
    assert fv(seg=P(0x90002)) == UNSUP  # ids are 4-byte aligned
    assert fv(x=P(0)) == INVALID
    assert fv(y=X) == INVALID
    assert fv(B=0) == OK
    assert lib.dynconv_bwd_varlen(X, S(800, 200, 1), W_, S(800 * 4, 200 * 4, 4, 1), P(0), S(4, 1), DY,
                                  S(800, 200, 1), DX, S(800, 200, 1), None, None, 2, 4, 200, 4, 1, BF16, None, 0,
                                  None) == INVALID
    assert lib.dynconv_bwd_varlen(X, S(800, 200, 1), W_, S(800 * 4, 200 * 4, 4, 1), SEG, S(4, 1), DY,
                                  S(800, 200, 1), None, None, None, None, 2, 4, 200, 4, 1, BF16, None, 0,
                                  None) == INVALID  # neither output
    assert lib.dynconv_lowrank_fwd_varlen(X, S(800, 200, 1), Z, S(256, 64, 1), U, 800, None, P(0), S(4, 1), Y,
                                          S(800, 200, 1), 2, 4, 200, 4, 1, 64, BF16, None) == INVALID
    assert lib.dynconv_lowrank_fwd_varlen(X, S(800, 200, 1), Z, S(256, 64, 1), U, 800, None, SEG, S(4, -1), Y,
                                          S(800, 200, 1), 2, 4, 200, 4, 1, 64, BF16, None) == UNSUP
    assert lib.dynconv_lowrank_bwd_varlen(X, S(800, 200, 1), Z, S(256, 64, 1), U, 800, None, P(0), S(4, 1), DY,
                                          S(800, 200, 1), DX, S(800, 200, 1), P(0x70000), S(256, 64, 1),
                                          P(0x80000), None, 2, 4, 200, 4, 1, 64, BF16, None, 0, None) == INVALID
    assert lib.dynconv_cache_fill_varlen(X, S(800, 200, 1), P(0), S(4, 1), P(0xa0000), S(600, 200, 1), 2, 4, 200,
                                         4, BF16, None) == INVALID
    assert lib.dynconv_cache_fill_varlen(X, S(800, 200, 1), SEG, S(4, 1), P(0xa0000), S(600, 200, 1), 0, 4, 200,
                                         4, BF16, None) == OK


def test_float16_dtype_code(lib):
    """float16 (code 2) is a storage type like the others; codes past it are invalid."""
    assert fwd(lib, dt=2, B=0) == OK
    assert fwd(lib, dt=2, x=P(0x10002)) == UNSUP  # 16-bit activations need 4-byte alignment
    assert fwd(lib, dt=3) == INVALID
    assert lib.dynconv_bwd_workspace_size(8, 4096, 2048, 3, 1, 1, 2) > 0


def test_conv_bias_validation(lib):
    CB, DCB = P(0xb0000), P(0xc0000)

    def fx(cb=CB, y=Y, B=2):
        return lib.dynconv_fwd_ex(X, S(800, 200, 1), W_, S(800 * 4, 200 * 4, 4, 1), None, None, cb, y, S(800, 200, 1),
                                  B, 4, 200, 4, 1, BF16, None)

    assert fx(cb=P(0xb0002)) == UNSUP  # 4-byte alignment
    assert fx(cb=Y) == INVALID  # the bias may not be the output
    assert fx(B=0) == OK
    need = lib.dynconv_bwd_ex_workspace_size(2, 4, 200, 4, 1, 0, 1, BF16)
    assert need >= 200 * 4  # one float32 partial per channel and time chunk at least
    assert lib.dynconv_bwd_ex_workspace_size(2, 4, 200, 4, 1, 1, 1, BF16) > lib.dynconv_bwd_workspace_size(
        2, 4, 200, 4, 1, 1, BF16)

    def bx(dcb=DCB, wsp=P(0x900000), wsb=need, dx=DX):
        return lib.dynconv_bwd_ex(X, S(800, 200, 1), W_, S(800 * 4, 200 * 4, 4, 1), None, None, DY, S(800, 200, 1), dx,
                                  S(800, 200, 1), None, None, dcb, 2, 4, 200, 4, 1, BF16, wsp, wsb, None)

    assert bx(wsb=need - 1) == WORKSPACE
    assert bx(wsp=None, wsb=0) == WORKSPACE
    assert bx(dcb=DX) == INVALID  # aliasing dx
    assert bx(dcb=P(0xc0002)) == UNSUP
    assert bx(dx=None) == INVALID  # neither dx nor dw


def test_bindings_reject_mismatched_shapes_and_dtypes():
    """The bindings check every tensor's full shape and dtype against x and H before any
    device work: the C ABI receives strides, not extents, so a mismatch would otherwise be
    an out-of-bounds access. CPU tensors suffice, these checks come first."""
    import torch

    from dynamic_short_convolution_amd import (dynconv_bwd, dynconv_cache_fill, dynconv_decode_step, dynconv_fwd,
                                               dynconv_lowrank_bwd, dynconv_lowrank_decode_step, dynconv_lowrank_fwd)

    B, T, D, W, R = 2, 5, 32, 4, 16
    bf = torch.bfloat16
    x = torch.zeros((B, T, D), dtype=bf)
    w1 = torch.zeros((B, T, D, W), dtype=bf)
    with pytest.raises(ValueError, match="w must have shape"):
        dynconv_fwd(x, torch.zeros((B, T, D // 16, W), dtype=bf), 1)  # head-wise filters with H = 1
    with pytest.raises(ValueError, match="w must have shape"):
        dynconv_fwd(x, w1, 4)  # per-channel filters with H = 4
    with pytest.raises(ValueError, match="w must have shape"):
        dynconv_fwd(x, torch.zeros((B, T - 1, D, W), dtype=bf), 1)  # fewer tokens
    with pytest.raises(ValueError, match="w must have shape"):
        dynconv_fwd(x, torch.zeros((D // 2, W), dtype=bf), 1)  # static filter of the wrong group count
    with pytest.raises(TypeError, match="w is torch.float32"):
        dynconv_fwd(x, w1.float(), 1)
    with pytest.raises(ValueError, match="divisor"):
        dynconv_fwd(x, w1, 3)
    with pytest.raises(ValueError, match="out must have shape"):
        dynconv_fwd(x, w1, 1, out=torch.zeros((B, T, D // 2), dtype=bf))
    with pytest.raises(ValueError, match=r"x must be \[B, T, D\]"):
        dynconv_fwd(x[0], w1[0], 1)
    with pytest.raises(ValueError, match="dy must have shape"):
        dynconv_bwd(x, w1, torch.zeros((B, T - 1, D), dtype=bf), 1)
    with pytest.raises(TypeError, match="dy is torch.float16"):
        dynconv_bwd(x, w1, torch.zeros((B, T, D), dtype=torch.float16), 1)
    with pytest.raises(ValueError, match="dx must have shape"):
        dynconv_bwd(x, w1, x, 1, dx=torch.zeros((B, T, D + 2), dtype=bf))
    with pytest.raises(ValueError, match="dw must have shape"):
        dynconv_bwd(x, w1, x, 1, dw=torch.zeros((B, T, D // 2, W), dtype=bf))
    with pytest.raises(TypeError, match="dw is torch.bfloat16"):
        dynconv_bwd(x, torch.zeros((D, W), dtype=bf), x, 1, dw=torch.zeros((D, W), dtype=bf))  # static dw is fp32
    z = torch.zeros((B, T, R), dtype=bf)
    U = torch.zeros((R, D * W), dtype=bf)
    b = torch.zeros((D * W,), dtype=bf)
    with pytest.raises(ValueError, match="z must be"):
        dynconv_lowrank_fwd(x, torch.zeros((B, T - 1, R), dtype=bf), U, b, W)
    with pytest.raises(ValueError, match="z must be"):
        dynconv_lowrank_bwd(x, torch.zeros((B + 1, T, R), dtype=bf), U, b, x, W)
    with pytest.raises(ValueError, match="dy must have shape"):
        dynconv_lowrank_bwd(x, z, U, b, torch.zeros((B, T, D // 2), dtype=bf), W)
    with pytest.raises(ValueError, match="out must have shape"):
        dynconv_lowrank_fwd(x, z, U, b, W, out=torch.zeros((B, T - 1, D), dtype=bf))
    with pytest.raises(ValueError, match="workspace must be contiguous"):
        dynconv_lowrank_bwd(x, z, U, b, x, W, workspace=torch.zeros((64, 2), dtype=torch.uint8).t())
    with pytest.raises(ValueError, match="cache must have shape"):
        dynconv_cache_fill(x, W, cache=torch.zeros((B, W, D), dtype=bf))
    with pytest.raises(ValueError, match="w must have shape"):
        dynconv_decode_step(x[:, 0], torch.zeros((B, D // 2, W), dtype=bf), torch.zeros((B, W - 1, D), dtype=bf), 0)
    with pytest.raises(ValueError, match="cache must have shape"):
        dynconv_decode_step(x[:, 0], w1[:, 0], torch.zeros((B, W - 1, D // 2), dtype=bf), 0)
    with pytest.raises(ValueError, match="cache .* is required"):
        dynconv_decode_step(x[:, 0], w1[:, 0], None, 0)
    with pytest.raises(ValueError, match="z must be"):
        dynconv_lowrank_decode_step(x[:, 0], z, U, b, torch.zeros((B, W - 1, D), dtype=bf), 0, W)
    with pytest.raises(ValueError, match="conv_bias must be"):
        dynconv_lowrank_fwd(x, z, U, b, W, conv_bias=torch.zeros((D // 2,), dtype=bf))
    with pytest.raises(ValueError, match="conv_bias must be"):
        dynconv_lowrank_fwd(x, z, U, b, W, conv_bias=torch.zeros((D,), dtype=torch.float32))
    with pytest.raises(ValueError, match="conv_bias must be"):
        dynconv_lowrank_decode_step(x[:, 0], z[:, 0], U, b, torch.zeros((B, W - 1, D), dtype=bf), 0, W,
                                    conv_bias=torch.zeros((2 * D,), dtype=bf)[::2])


def test_noalloc_validation(lib):
    """dynconv_bwd_ex_noalloc validates like dynconv_bwd_ex, and refuses a call whose
    partial sums exceed its scratch array (DYNCONV_ERR_WORKSPACE) before any HIP call."""
    DCB = P(0xc0000)

    def nx(B=2, T=4, D=200, W=4, ws=(800 * 4, 200 * 4, 4, 1), dw=None, dcb=DCB, dx=DX, seg=None, ss=None):
        return lib.dynconv_bwd_ex_noalloc(X, S(T * D, D, 1), W_, S(*ws), seg, S(*ss) if ss else None, DY,
                                          S(T * D, D, 1), dx, S(T * D, D, 1), dw, None, dcb, B, T, D, W, 1, BF16, None)

    assert nx(dx=None, dcb=None) == INVALID  # neither dx nor dw
    assert nx(dcb=DX) == INVALID
    assert nx(dcb=P(0xc0002)) == UNSUP
    assert nx(seg=P(0x90002), ss=(4, 1)) == UNSUP  # ids are 4-byte aligned
    assert nx(B=0) == OK
    assert nx(W=9) == UNSUP
    B, T, D, W = 512, 64, 8192, 4
    need = lib.dynconv_bwd_ex_workspace_size(B, T, D, W, 1, 1, 1, BF16)
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    assert nx(B=B, T=T, D=D, W=W, ws=(0, 0, W, 1), dw=P(0xd0000)) == WORKSPACE
    B = 1024
    need = lib.dynconv_bwd_ex_workspace_size(B, T, D, W, 1, 0, 1, BF16)
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    assert nx(B=B, T=T, D=D, W=W, ws=(T * D * W, D * W, W, 1)) == WORKSPACE


def test_noalloc_scratch_constant_matches_header():
    with open(os.path.join(ROOT, "include", "dynconv.h")) as f:
        m = re.search(r"#define DYNCONV_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", f.read())
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.NOALLOC_SCRATCH_BYTES


def test_gemm_validation(lib):
    """The projection + convolution calls reject bad arguments before any HIP call."""
    A, WP, WF, YY, ZZ, UU = (P(0x100000 * (i + 1)) for i in range(6))
    B, T, K, N, W = 2, 10, 128, 256, 4

    def g(A_=A, as_=(T * K, K, 1), wp=WP, ldw=K, w=WF, ws=(T * N * W, N * W, W, 1), y=YY, ys=(T * N, N, 1), B_=B,
          K_=K, N_=N, W_=W, H=1, dt=BF16):
        return lib.dynconv_gemm_fwd(A_, S(*as_), wp, ldw, w, S(*ws), y, S(*ys), B_, T, N_, K_, W_, H, dt, None)

    assert g(B_=0) == OK
    assert g(A_=P(0)) == INVALID
    assert g(w=P(0)) == INVALID
    assert g(y=A) == INVALID and g(y=WF) == INVALID
    assert g(ldw=K - 8) == INVALID
    assert g(dt=F32) == UNSUP
    assert g(W_=6, ws=(T * N * 6, N * 6, 6, 1)) == UNSUP
    assert g(H=32, ws=(T * 8 * W, 8 * W, W, 1)) == UNSUP
    assert g(H=3) == INVALID  # H must divide N
    assert g(N_=384, H=6, ws=(T * 64 * W, 64 * W, W, 1), ys=(T * 384, 384, 1)) == UNSUP  # whole groups per 128 columns
    assert g(K_=96, as_=(T * 96, 96, 1), ldw=96) == UNSUP  # K % 64
    assert g(N_=192, ws=(T * 192 * W, 192 * W, W, 1)) == UNSUP  # N % 128
    assert g(A_=P(0x100008)) == UNSUP  # 16-byte rows of A
    assert g(as_=(T * (K + 4), K + 4, 1)) == UNSUP
    assert g(ldw=K + 4) == UNSUP
    assert g(ws=(T * N * W, N * W, W + 1, 1)) == UNSUP

    def gl(R=64, W_=4, z=ZZ, zs=(T * 64, 64, 1), U_=UU, ldu=N * 4, bias=None, y=YY):
        return lib.dynconv_gemm_lowrank_fwd(A, S(T * K, K, 1), WP, K, z, S(*zs), U_, ldu, bias, y, S(T * N, N, 1), B, T,
                                            N, K, W_, 1, R, BF16, None)

    assert gl(R=0) == INVALID
    assert gl(R=129) == UNSUP
    assert gl(R=128, W_=5, ldu=N * 5) == UNSUP  # the LDS copy of U would not fit
    assert gl(z=P(0)) == INVALID
    assert gl(U_=P(0)) == INVALID
    assert gl(ldu=N * 4 - 1) == INVALID
    assert gl(y=ZZ) == INVALID and gl(y=UU) == INVALID
    assert gl(zs=(T * 64, 64, 2)) == UNSUP


EXTREME = [1, 7, 1 << 20, (1 << 31) - 1]
EXTREME_T = [1, 16, 4096, (1 << 31) - 65537, (1 << 31) - 65536, (1 << 31) - 1]
EXTREME_D = [2, 2048, 1 << 20, (1 << 31) - 2]


def test_size_queries_at_extreme_sizes(lib):
    """Workspace queries over extreme B, T, D (no launch): 0 for refused sizes, otherwise a
    size that fits the partial sums and stays far from 64-bit wrap-around."""
    for B, T, D in itertools.product(EXTREME, EXTREME_T, EXTREME_D):
        for W, H, dt in itertools.product([1, 4, 5, 8], [1, 2, 16], [BF16, 7]):
            for st in (0, 1):
                n = lib.dynconv_bwd_workspace_size(B, T, D, W, H, st, dt)
                assert 0 <= n < (1 << 50), (B, T, D, W, H, st, dt, n)
                if dt == 7 or st == 0:
                    assert n == 0
            for R in (1, 64, 128):
                n = lib.dynconv_lowrank_bwd_workspace_size(B, T, D, W, H, R, dt)
                assert 0 <= n < (1 << 50), (B, T, D, W, H, R, dt, n)
                if n:
                    assert n >= R * (D // H) * W * 4


def test_sizes_past_the_grid_bound_are_refused(lib):
    """Sizes whose grids or token arithmetic would not fit 32 bits are refused before any
    launch."""
    big_t = (1 << 31) - 1
    assert fwd(lib, T=big_t) == UNSUP  # a token plus a step would pass INT32_MAX
    # B * ceil(T / 16) * ceil(D / 16) above INT32_MAX workgroups
    assert fwd(lib, B=1 << 20, T=4096, D=2048, xs=(4096 * 2048, 2048, 1), ys=(4096 * 2048, 2048, 1),
               ws=(4096 * 2048 * 4, 2048 * 4, 4, 1)) == UNSUP
    assert lib.dynconv_lowrank_bwd_workspace_size(1 << 20, 4096, 2048, 4, 1, 64, BF16) == 0
    assert lib.dynconv_lowrank_bwd_workspace_size(8, 4096, 2048, 4, 1, 64, BF16) > 0
