"""GPU parity of the convolution fused into its producing projection (dynconv_gemm_fwd,
dynconv_gemm_lowrank_fwd) against the float64 oracle (projection with a plain matmul,
then eq. 2 + eq. 3).

Tolerance. X = A Wp^T is accumulated in float32 over K products of 16-bit operands (exact
products), so |dX| <= K 2^-24 S with S = |A| |Wp|^T (elementwise absolute values); the
convolution carries it as |dy_t| <= |dX_t| + sum_k |w_k| |dX_{t-k}|, and the stored y adds
the storage type's rounding (2^-8 bf16, 2^-11 float16 relative). The test adds that
accumulation bound to the usual elementwise allowance and keeps the normwise gate. Low-rank
filters are formed from z and U in float32 on the matrix cores (exact products of 16-bit
values): their error K_r 2^-24 sum|z||U| times |X| is added the same way.
"""
import numpy as np
import pytest
import torch

import synth
from dynamic_short_convolution_amd import dynconv_gemm_fwd, dynconv_gemm_lowrank_fwd
from oracle import gemm_conv_fwd, gemm_lowrank_fwd, lowrank_filters, projection
from tests.parity import assert_close, to64

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f16": torch.float16}


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    yield
    torch.cuda.synchronize()


def _shift_sum(S, wabs):
    """S_t + sum_k |w_k(t)| S_{t-k} per (b, t, n), for filters wabs [B,T,N,W] (>= 0)."""
    out = S.copy()
    T = S.shape[1]
    for k in range(1, wabs.shape[-1]):
        if k < T:
            out[:, k:, :] += wabs[:, k:, :, k] * S[:, : T - k, :]
    return out


def _per_channel(w, N, H, B, T):
    """Filters [B,T,N,W] per channel from per-token [B,T,N/H,W] or static [N/H,W]."""
    if w.ndim == 2:
        return np.broadcast_to(np.repeat(w, H, axis=0)[None, None], (B, T, N, w.shape[-1]))
    return np.repeat(w, H, axis=2)


def _check(y, ref, A64, Wp64, wch_abs, K, dtype, extra_w=None):
    S = projection(np.abs(A64), np.abs(Wp64))
    extra = K * 2.0**-24 * _shift_sum(S, wch_abs)
    if extra_w is not None:
        extra = extra + extra_w
    assert_close("y", y, ref, DT[dtype], extra=extra)


def _inputs(B, T, K, N, seed, dtype, wscale=None):
    A = synth.draw((B, T, K), 1.0, seed, "x", dtype)
    Wp = synth.draw((N, K), (1.0 / K) ** 0.5 if wscale is None else wscale, seed, "probe", dtype)
    return A, Wp


def _lowrank_extra(A64, Wp64, z64, U64, W, H):
    """Filter error (R 2^-24 sum_r |z||U| per token and column, float32 matrix-core sums of
    exact products) times |X_{t-k}|, summed over the taps."""
    R = z64.shape[-1]
    X = np.abs(projection(A64, Wp64))
    B, T, N = X.shape
    werr = R * 2.0**-24 * _per_channel(lowrank_filters(np.abs(z64), np.abs(U64), None, W), N, H, B, T)
    ew = np.zeros_like(X)
    for k in range(W):
        if k < T:
            ew[:, k:, :] += werr[:, k:, :, k] * X[:, : T - k, :]
    return ew


CONV_CASES = []
for dtype in ("bf16", "f16"):
    for W in (1, 2, 3, 4, 5):
        for H, static in ((1, False), (4, False), (16, False), (1, True)):
            CONV_CASES.append((dtype, W, H, static))


@pytest.mark.parametrize("dtype,W,H,static", CONV_CASES)
def test_gemm_conv_small(dtype, W, H, static):
    # M = 600 rows: tiles of 240 output rows (the last one ragged), sequences straddling tiles
    B, T, K, N = 2, 300, 128, 256
    A, Wp = _inputs(B, T, K, N, 60 + W, dtype)
    w = synth.draw((N // H, W) if static else (B, T, N // H, W), (1.0 / W) ** 0.5, 60 + W, "w", dtype)
    y = dynconv_gemm_fwd(A.cuda(), Wp.cuda(), w.cuda(), H)
    A64, Wp64, w64 = to64(A), to64(Wp), to64(w)
    ref = gemm_conv_fwd(A64, Wp64, w64, H)
    _check(y, ref, A64, Wp64, np.abs(_per_channel(w64, N, H, B, T)), K, dtype)


@pytest.mark.parametrize("T", [1, 3, 5, 16, 241])
def test_gemm_conv_short_sequences(T):
    """Many sequences inside one tile (T < W, T < the 16-row halo), and T around a tile."""
    B, K, N, W, H = 37, 64, 128, 4, 1
    A, Wp = _inputs(B, T, K, N, 70 + T, "bf16")
    w = synth.draw((B, T, N, W), 0.5, 70 + T, "w", "bf16")
    y = dynconv_gemm_fwd(A.cuda(), Wp.cuda(), w.cuda(), H)
    A64, Wp64, w64 = to64(A), to64(Wp), to64(w)
    _check(y, gemm_conv_fwd(A64, Wp64, w64, H), A64, Wp64, np.abs(w64), K, "bf16")


def test_gemm_conv_strided_views():
    """A and w as views into larger buffers, y written into a slice of a larger buffer."""
    B, T, K, N, W = 3, 250, 192, 384, 4
    Abig = synth.draw((B, T, K + 64), 1.0, 80, "x", "bf16")
    A = Abig[:, :, 32:32 + K]
    Wbig = synth.draw((N, K + 128), (1.0 / K) ** 0.5, 80, "probe", "bf16")
    Wp = Wbig[:, 64:64 + K]
    wbig = synth.draw((B, T, N + 8, W), 0.5, 80, "w", "bf16")
    w = wbig[:, :, 8:, :]
    ybig = torch.zeros((B, T, N + 256), dtype=torch.bfloat16, device="cuda")
    y = ybig[:, :, 128:128 + N]
    Ag = Abig.cuda()[:, :, 32:32 + K]  # sliced on the device, so the strides are kept
    Wg = Wbig.cuda()[:, 64:64 + K]
    wg = wbig.cuda()[:, :, 8:, :]
    assert Ag.stride(1) == K + 64 and Wg.stride(0) == K + 128 and wg.stride(1) == (N + 8) * W
    dynconv_gemm_fwd(Ag, Wg, wg, 1, out=y)
    A64, Wp64, w64 = to64(A), to64(Wp), to64(w)
    _check(y, gemm_conv_fwd(A64, Wp64, w64, 1), A64, Wp64, np.abs(w64), K, "bf16")
    assert torch.count_nonzero(ybig[:, :, :128]) == 0 and torch.count_nonzero(ybig[:, :, 128 + N:]) == 0


def test_gemm_identity_projection_equals_conv():
    """Wp = I: the fused kernel's y equals the streaming forward kernel's y on A (within the
    rounding of y; X = A exactly)."""
    from dynamic_short_convolution_amd import dynconv_fwd

    B, T, N, W = 2, 500, 128, 4
    A = synth.draw((B, T, N), 1.0, 81, "x", "bf16").cuda()
    w = synth.draw((B, T, N, W), 0.5, 81, "w", "bf16").cuda()
    I = torch.eye(N, dtype=torch.bfloat16, device="cuda")
    y = dynconv_gemm_fwd(A, I, w, 1)
    ref = dynconv_fwd(A, w, 1)
    d = (y.float() - ref.float()).abs()
    assert float(d.max()) <= 2.0**-7 * float(ref.float().abs().max()), float(d.max())


LR_CASES = []
for dtype in ("bf16", "f16"):
    for W in (1, 2, 3, 4, 5):
        for R in (16, 20, 64, 96, 128):
            if W == 5 and R > 96:
                continue
            for H in (1, 8):
                LR_CASES.append((dtype, W, R, H))


@pytest.mark.parametrize("dtype,W,R,H", LR_CASES)
def test_gemm_lowrank_small(dtype, W, R, H):
    B, T, K, N = 2, 300, 128, 256
    A, Wp = _inputs(B, T, K, N, 90 + W, dtype)
    J = (N // H) * W
    z = synth.draw((B, T, R), 1.0, 90 + R, "z", dtype)
    U = synth.draw((R, J), 0.1 / R**0.5, 90 + R, "U", dtype)
    bias = synth.draw((J,), 0.1**0.5, 90 + R, "b", dtype)
    y = dynconv_gemm_lowrank_fwd(A.cuda(), Wp.cuda(), z.cuda(), U.cuda(), bias.cuda(), W, H)
    A64, Wp64, z64, U64, b64 = to64(A), to64(Wp), to64(z), to64(U), to64(bias)
    ref = gemm_lowrank_fwd(A64, Wp64, z64, U64, b64, W, H)
    wch = _per_channel(lowrank_filters(z64, U64, b64, W), N, H, B, T)
    _check(y, ref, A64, Wp64, np.abs(wch), K, dtype, extra_w=_lowrank_extra(A64, Wp64, z64, U64, W, H))


def test_gemm_lowrank_no_bias_and_strided_z():
    B, T, K, N, W, R = 2, 260, 64, 128, 4, 32
    A, Wp = _inputs(B, T, K, N, 95, "bf16")
    zbig = synth.draw((B, T, R + 8), 1.0, 95, "z", "bf16")
    z = zbig[:, :, 3:3 + R]
    U = synth.draw((R, N * W), 0.1 / R**0.5, 95, "U", "bf16")
    zg = zbig.cuda()[:, :, 3:3 + R]
    assert zg.stride(1) == R + 8
    y = dynconv_gemm_lowrank_fwd(A.cuda(), Wp.cuda(), zg, U.cuda(), None, W)
    A64, Wp64, z64, U64 = to64(A), to64(Wp), to64(z), to64(U)
    ref = gemm_lowrank_fwd(A64, Wp64, z64, U64, None, W)
    wch = lowrank_filters(z64, U64, None, W)
    _check(y, ref, A64, Wp64, np.abs(wch), K, "bf16", extra_w=_lowrank_extra(A64, Wp64, z64, U64, W, 1))


@pytest.mark.parametrize("form", ["perchannel", "lowrank"])
def test_gemm_full_qkv_shape(form):
    """The post-QKV projection shape: B4 T8192, K = 2048 -> N = 3072 (Q 2048 | K 512 | V 512)
    in one launch, every element checked against the oracle."""
    B, T, K, N, W, R = 4, 8192, 2048, 3072, 4, 64
    A, Wp = _inputs(B, T, K, N, 99, "bf16")
    Ag, Wg = A.cuda(), Wp.cuda()
    A64, Wp64 = to64(A), to64(Wp)
    if form == "perchannel":
        w = synth.draw((B, T, N, W), 0.5, 99, "w", "bf16")
        y = dynconv_gemm_fwd(Ag, Wg, w.cuda(), 1).cpu()
        w64 = to64(w)
        _check(y, gemm_conv_fwd(A64, Wp64, w64, 1), A64, Wp64, np.abs(w64), K, "bf16")
    else:
        z = synth.draw((B, T, R), 1.0, 99, "z", "bf16")
        U = synth.draw((R, N * W), 0.1 / R**0.5, 99, "U", "bf16")
        bias = synth.draw((N * W,), 0.1**0.5, 99, "b", "bf16")
        y = dynconv_gemm_lowrank_fwd(Ag, Wg, z.cuda(), U.cuda(), bias.cuda(), W).cpu()
        z64, U64, b64 = to64(z), to64(U), to64(bias)
        wch = lowrank_filters(z64, U64, b64, W)
        _check(y, gemm_lowrank_fwd(A64, Wp64, z64, U64, b64, W), A64, Wp64, np.abs(wch), K, "bf16",
               extra_w=_lowrank_extra(A64, Wp64, z64, U64, W, 1))
