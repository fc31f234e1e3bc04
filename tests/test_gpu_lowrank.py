"""GPU parity of the fused low-rank kernels against the float64 oracle, through the C ABI.

bf16 path: the generated filters stay in float32 (never rounded, never stored), but
the per-token filter gradient g is rounded to bf16 as an operand of the matrix-core
products dz = g U^T and dU = z^T g; on small shapes the elementwise bound of those two
outputs therefore adds 2^-8 * sum |terms| (2^-8 is the unit roundoff of bf16's 8-bit
significand). At full size (32768 tokens) that allowance would exceed a single token's
term, so the full-size checks compare dz and dU against the oracle's g rounded the same
way with a float32-accumulation allowance instead (check_lowrank_full_bwd).
"""
import numpy as np
import pytest
import torch

import synth
from dynamic_short_convolution_amd import dynconv_fwd, dynconv_lowrank_bwd, dynconv_lowrank_fwd
from oracle import conv_bias_grad, conv_bwd, lowrank_bwd, lowrank_filters, lowrank_fwd
from tests.parity import assert_close, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    yield
    torch.cuda.synchronize()


def _inputs(B, T, D, W, R, dtype, seed, bias=True):
    x = synth.draw((B, T, D), 1.0, seed, "x", dtype)
    dy = synth.draw((B, T, D), 1.0, seed, "dy", dtype)
    z = synth.draw((B, T, R), 1.0, seed, "z", dtype)
    U = synth.draw((R, D * W), 0.1 / R**0.5 * 3.0, seed, "U", dtype)
    b = synth.draw((D * W,), 0.1**0.5, seed, "b", dtype) if bias else None
    return x, z, U, b, dy


def _g_abs(x64, dy64, W):
    """|g| for every (b, t, j): the magnitudes of the per-token filter-gradient terms."""
    B, T, D = x64.shape
    _, dwabs = conv_bwd(np.abs(x64), np.zeros((B, T, D, W)), np.abs(dy64), 1)
    return dwabs.reshape(B * T, D * W)


def _check(B, T, D, W, R, dtype, seed, bias=True, bwd=True):
    td = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    x, z, U, b, dy = _inputs(B, T, D, W, R, dtype, seed, bias)
    xg, zg, Ug, dyg = x.cuda(), z.cuda(), U.cuda(), dy.cuda()
    bg = b.cuda() if b is not None else None
    x64, z64, U64, dy64 = to64(x), to64(z), to64(U), to64(dy)
    b64 = to64(b) if b is not None else None
    y = dynconv_lowrank_fwd(xg, zg, Ug, bg, W)
    assert_close("y", y, lowrank_fwd(x64, z64, U64, b64, W), td)
    if not bwd:
        return
    dx, dz, dU, db = dynconv_lowrank_bwd(xg, zg, Ug, bg, dyg, W)
    rdx, rdz, rdU, rdb = lowrank_bwd(x64, z64, U64, b64, dy64, W)
    assert_close("dx", dx, rdx, td)
    gabs = _g_abs(x64, dy64, W)
    u = {torch.bfloat16: 2.0**-8, torch.float16: 2.0**-11}.get(td, 2.0**-22)
    extra_dz = (u * (gabs @ np.abs(U64).T)).reshape(B, T, R)
    extra_dU = u * (np.abs(z64).reshape(B * T, R).T @ gabs)
    assert_close("dz", dz, rdz, td, extra=extra_dz)
    # dU and db are float32 outputs of sums over every token
    assert_close("dU", dU, rdU, torch.float32 if td == torch.float32 else td, rtol=1e-5, atol=1e-5, extra=extra_dU)
    assert_close("db", db, rdb, torch.float32 if td == torch.float32 else td, rtol=1e-5, atol=1e-5)


SMALL = []
for dtype in ("f32", "bf16", "f16"):
    for W in (1, 2, 3, 4, 5):
        for R in (1, 20, 33, 64, 128):
            SMALL.append((dtype, W, R))
    # the widest filters (W = 6..8, the pages' ablation reaches W = 6) take the general kernels
    for W, R in ((6, 20), (6, 64), (7, 33), (7, 128), (8, 1), (8, 64), (8, 128)):
        SMALL.append((dtype, W, R))


@pytest.mark.parametrize("dtype,W,R", SMALL)
def test_small_parity(dtype, W, R):
    _check(2, 77, 200, W, R, dtype, seed=W * 13 + R)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,D", [(1, 64), (3, 64), (5, 128), (300, 64), (1000, 96)])
def test_shapes(dtype, T, D):
    _check(2, T, D, 4, 16, dtype, seed=T + D)


def test_no_bias():
    _check(2, 50, 128, 4, 32, "bf16", seed=3, bias=False)


def test_fused_equals_materialised_path():
    """The fused kernel applied to z, U, b equals the materialised-filter kernel applied to
    the filters z U + b, up to the filter rounding the materialised path must do."""
    B, T, D, W, R = 2, 150, 256, 4, 64
    x, z, U, b, dy = _inputs(B, T, D, W, R, "f32", 21)
    wmat = torch.from_numpy(lowrank_filters(to64(z), to64(U), to64(b), W)).to(torch.float32)
    y_fused = dynconv_lowrank_fwd(x.cuda(), z.cuda(), U.cuda(), b.cuda(), W)
    y_mat = dynconv_fwd(x.cuda(), wmat.cuda(), 1)
    assert_close("fused vs materialised", y_fused, to64(y_mat), torch.float32)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("W", [6, 7, 8])
@pytest.mark.parametrize("R", [20, 64])
@pytest.mark.parametrize("packed", [False, True])
def test_wide_filters_fast_forward(dtype, W, R, packed):
    """Six to eight taps on the fast forward (16-bit, D % 64 == 0, up to 64 ranks): the taps
    reach two 4-token row groups back, across step boundaries, into the rows before a
    range, and (packed) across documents of 1 to 3 tokens at the start of each row."""
    B, T, D = 2, 388, 192
    seed = 1100 + 10 * W + R + int(packed)
    td = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    x, z, U, b, _ = _inputs(B, T, D, W, R, dtype, seed)
    seq = synth.segments(B, T, 24.0, seed, first=(1, 2, 3)) if packed else None
    y = dynconv_lowrank_fwd(x.cuda(), z.cuda(), U.cuda(), b.cuda(), W, seq_idx=seq.cuda() if packed else None)
    ref = lowrank_fwd(to64(x), to64(z), to64(U), to64(b), W, 1, seq.numpy() if packed else None)
    assert_close("y", y, ref, td)


@pytest.mark.parametrize("T", [1, 4, 7, 64, 65, 132])
@pytest.mark.parametrize("packed", [False, True])
def test_wide_filters_fast_forward_short(T, packed):
    """Eight taps on the fast forward at lengths shorter than the filter, one step, one step
    plus a token, and two steps plus four tokens (packed rows with T % 4 != 0 take the
    general kernels)."""
    B, D, W, R = 3, 128, 8, 32
    seed = 1200 + T + int(packed)
    x, z, U, b, _ = _inputs(B, T, D, W, R, "bf16", seed)
    seq = synth.segments(B, T, 3.0, seed, first=(1, 2)) if packed else None
    y = dynconv_lowrank_fwd(x.cuda(), z.cuda(), U.cuda(), b.cuda(), W, seq_idx=seq.cuda() if packed else None)
    ref = lowrank_fwd(to64(x), to64(z), to64(U), to64(b), W, 1, seq.numpy() if packed else None)
    assert_close("y", y, ref, torch.bfloat16)


def test_deterministic():
    B, T, D, W, R = 2, 400, 256, 4, 64
    x, z, U, b, dy = (t.cuda() if t is not None else None for t in _inputs(B, T, D, W, R, "bf16", 22))
    outs = [dynconv_lowrank_bwd(x, z, U, b, dy, W) for _ in range(3)]
    for o in outs[1:]:
        for a, c in zip(outs[0], o):
            assert torch.equal(a, c)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_full_lowrank_r64_fwd(dtype):
    """Every element of the B8 T4096 D2048 W4 R64 forward, one sequence at a time.
    float16: the same bf16-drawn values (exact in float16 but for a few tiny ones)."""
    wl = synth.workloads()["lowrank_r64"]
    x, z, U, b = (t.to(dtype) for t in (wl.x(), wl.z(), wl.U(), wl.b()))
    y = dynconv_lowrank_fwd(x.cuda(), z.cuda(), U.cuda(), b.cuda(), wl.W).cpu()
    U64, b64 = to64(U), to64(b)
    for s_ in range(wl.B):
        ref = lowrank_fwd(to64(x[s_ : s_ + 1]), to64(z[s_ : s_ + 1]), U64, b64, wl.W)
        assert_close(f"y[{s_}]", y[s_ : s_ + 1], ref, dtype)


def rounded(a, dtype):
    """float64 values of a rounded to the 16-bit storage type (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.float32).to(dtype).to(torch.float64).numpy()


def check_lowrank_full_bwd(x, z, U, b, dy, W, dtype, got, seq_idx=None, H=1):
    """Every element of a full-size low-rank backward, one sequence at a time.

    dx and db: against the oracle with the usual bounds. dz and dU: the normwise gate
    against the oracle, and a tight elementwise bound against the oracle's own g rounded
    to the storage type (the kernels round g = dy x_{t-k} to 16 bits as the operand of
    the matrix-core products dz = g U^T and dU = z^T g; the rounding noise of 32768 tokens
    would otherwise hide a dropped or doubled token): float32 accumulation, at most 128
    roundings of a running sum per output element, gives 2^-17 sum |terms|. Head-wise
    (H > 1): dz takes each group's g summed over its H channels in float32 and then
    rounded; dU takes every channel's g rounded, its H channels summed afterwards.
    """
    dx, dz, dU, db = (t.cpu() for t in got)
    B, T, D = x.shape
    R = z.shape[-1]
    U64 = to64(U)
    b64 = to64(b) if b is not None else None
    J = U64.shape[1]
    dU_ref = np.zeros((R, J))
    dU_rnd = np.zeros((R, J))
    dU_abs = np.zeros((R, J))
    db_ref = np.zeros((J,))
    for s_ in range(B):
        x64, z64, dy64 = to64(x[s_ : s_ + 1]), to64(z[s_ : s_ + 1]), to64(dy[s_ : s_ + 1])
        sq = seq_idx[s_ : s_ + 1] if seq_idx is not None else None
        rdx, rdz, rdU, rdb = lowrank_bwd(x64, z64, U64, b64, dy64, W, H, sq)
        assert_close(f"dx[{s_}]", dx[s_ : s_ + 1], rdx, dtype)
        # the oracle's per-token filter gradient g (independent of the filters) and its rounding
        _, g = conv_bwd(x64, np.zeros((1, T, D // H, W)), dy64, H, sq)
        g = g.reshape(T, J)
        gr = rounded(g, dtype)
        if H > 1:
            _, gc = conv_bwd(x64, np.zeros((1, T, D, W)), dy64, 1, sq)
            gr_dU = rounded(gc.reshape(T, D * W), dtype).reshape(T, D // H, H, W).sum(axis=2).reshape(T, J)
            gabs_dU = np.abs(rounded(gc.reshape(T, D * W), dtype)).reshape(T, D // H, H, W).sum(axis=2).reshape(T, J)
            del gc
        else:
            gr_dU, gabs_dU = gr, np.abs(gr)
        zf = z64.reshape(T, R)
        dz_rnd = (gr @ U64.T).reshape(1, T, R)
        err = float(np.max(np.abs(to64(dz[s_ : s_ + 1]) - rdz)) / np.max(np.abs(rdz)))
        assert err <= {torch.bfloat16: 2e-2, torch.float16: 2.5e-3}[dtype], f"dz[{s_}] normwise {err}"
        assert_close(f"dz[{s_}] vs rounded g", dz[s_ : s_ + 1], dz_rnd, dtype,
                     extra=2.0**-17 * (np.abs(gr) @ np.abs(U64).T).reshape(1, T, R))
        dU_ref += rdU
        dU_rnd += zf.T @ gr_dU
        dU_abs += np.abs(zf).T @ gabs_dU
        db_ref += rdb
    err = float(np.max(np.abs(to64(dU) - dU_ref)) / np.max(np.abs(dU_ref)))
    assert err <= {torch.bfloat16: 2e-2, torch.float16: 2.5e-3}[dtype], f"dU normwise {err}"
    assert_close("dU vs rounded g", dU, dU_rnd, torch.float32, rtol=1e-6, atol=1e-6, extra=2.0**-17 * dU_abs)
    assert_close("db", db, db_ref, torch.float32, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_full_lowrank_r64_bwd(dtype):
    """Every element of dx, dz, dU and db at B8 T4096 D2048 W4 R64."""
    wl = synth.workloads()["lowrank_r64_bwd"]
    x, z, U, b, dy = (t.to(dtype) for t in (wl.x(), wl.z(), wl.U(), wl.b(), wl.dy()))
    got = dynconv_lowrank_bwd(x.cuda(), z.cuda(), U.cuda(), b.cuda(), dy.cuda(), wl.W)
    check_lowrank_full_bwd(x, z, U, b, dy, wl.W, dtype, got)


# ---------------------------------------------------------------------------------
# The 16-bit fast paths (W <= 4 at R up to 128, W = 5 up to 64 ranks, and the forward alone
# W = 6..8 up to 64 ranks; D a multiple of 64,
# 16-byte aligned rows): token ranges of whole 64-token steps, an x ring in LDS that carries the W-1 rows
# before each step (forward), dx completed across lanes, ranges and a tail step
# (backward), buffer stores that drop rows past T.
# ---------------------------------------------------------------------------------
# Ranks that are not a multiple of 32 are zero-padded to 32, 64 or 128 on the fast kernels:
# z rows of 16-byte pieces where they are 16-byte aligned and R % 8 == 0 (8, 16, 40), of
# 4-byte pieces otherwise (2, 20, 26, 42, 52, 100: the pages' ranks among them).
FAST = []
for W in (1, 2, 3, 4, 5):
    for R in (2, 8, 16, 20, 26, 32, 40, 42, 52, 64, 100, 128):
        for (B, T, D) in ((1, 1, 64), (2, 65, 128), (3, 200, 192)):
            FAST.append((W, R, B, T, D))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("W,R,B,T,D", FAST)
def test_fast_parity(W, R, B, T, D, dtype):
    _check(B, T, D, W, R, dtype, seed=1000 + 7 * W + R + T)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("W", [1, 4])
def test_fast_no_bias(W, dtype):
    _check(2, 130, 128, W, 64, dtype, seed=77 + W, bias=False)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("W", [4, 5])
def test_fast_fwd_multistep_ranges(dtype, W):
    """Token ranges of several 64-token steps (the LDS ring wraps), a partial last step,
    and the rows before each range carried from memory; every element."""
    B, T, D, R = 2, 3000, 2048, 64
    x, z, U, b, _ = _inputs(B, T, D, W, R, dtype, 31)
    y = dynconv_lowrank_fwd(x.cuda(), z.cuda(), U.cuda(), b.cuda(), W)
    assert_close("y", y, lowrank_fwd(to64(x), to64(z), to64(U), to64(b), W), y.dtype)


def test_fast_fwd_strided_views():
    """x, z and y as column slices of wider row-major buffers (row strides above D, R)."""
    B, T, D, W, R = 2, 150, 128, 3, 64
    x, z, U, b, _ = _inputs(B, T, D, W, R, "bf16", 41)
    xw = torch.zeros(B, T, 3 * D, dtype=torch.bfloat16)
    xw[:, :, D : 2 * D] = x
    zw = torch.zeros(B, T, R + 32, dtype=torch.bfloat16)
    zw[:, :, 32:] = z
    xg, zg = xw.cuda()[:, :, D : 2 * D], zw.cuda()[:, :, 32:]
    yw = torch.zeros(B, T, 2 * D, dtype=torch.bfloat16, device="cuda")
    dynconv_lowrank_fwd(xg, zg, U.cuda(), b.cuda(), W, out=yw[:, :, D:])
    ref = lowrank_fwd(to64(x), to64(z), to64(U), to64(b), W)
    assert_close("y", yw[:, :, D:].cpu(), ref, torch.bfloat16)
    assert torch.count_nonzero(yw[:, :, :D]) == 0, "write outside the output view"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("W", [4, 5])
def test_fast_bwd_multistep_ranges(dtype, W):
    """The backward over token ranges of several steps: the rows completed by the tail step
    of one range and skipped by the first step of the next (three rows of delay up to W = 4,
    four at W = 5); every element of dx, dz, dU, db."""
    B, T, D, R = 2, 3000, 2048, 64
    x, z, U, b, dy = _inputs(B, T, D, W, R, dtype, 32)
    got = dynconv_lowrank_bwd(x.cuda(), z.cuda(), U.cuda(), b.cuda(), dy.cuda(), W)
    check_lowrank_full_bwd(x, z, U, b, dy, W, {"bf16": torch.bfloat16, "f16": torch.float16}[dtype], got)


# ------------------------------------------------------------------------------------
# head-wise generation: U is R x (D/H)*W, the H channels of a group share its filter
# ------------------------------------------------------------------------------------

HEADWISE = []
for dtype in ("f32", "bf16", "f16"):
    for H in (2, 4, 16):
        for W, R in ((1, 16), (3, 40), (4, 64), (5, 52), (5, 128)):
            HEADWISE.append((dtype, H, W, R))


# groups whose size is not a power of two take the general kernels
HEADWISE += [(dtype, H, W, R) for dtype in ("f32", "bf16", "f16") for H, W, R in ((3, 4, 64), (6, 3, 40), (12, 5, 52),
                                                                                   (24, 2, 128), (4, 6, 64),
                                                                                   (2, 8, 128), (3, 7, 40))]


@pytest.mark.parametrize("dtype,H,W,R", HEADWISE)
def test_headwise_lowrank_parity(dtype, H, W, R):
    B, T, D = 2, 150, 128 if 128 % H == 0 else 192
    seed = 80 + H + W + R
    td = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    G = D // H
    x = synth.draw((B, T, D), 1.0, seed, "x", dtype)
    dy = synth.draw((B, T, D), 1.0, seed, "dy", dtype)
    z = synth.draw((B, T, R), 1.0, seed, "z", dtype)
    U = synth.draw((R, G * W), 0.3 / R**0.5, seed, "U", dtype)
    b = synth.draw((G * W,), 0.3, seed, "b", dtype)
    x64, z64, U64, b64, dy64 = to64(x), to64(z), to64(U), to64(b), to64(dy)
    xg, zg, Ug, bg, dyg = x.cuda(), z.cuda(), U.cuda(), b.cuda(), dy.cuda()
    y = dynconv_lowrank_fwd(xg, zg, Ug, bg, W, H)
    assert_close("y", y, lowrank_fwd(x64, z64, U64, b64, W, H), td)
    dx, dz, dU, db = dynconv_lowrank_bwd(xg, zg, Ug, bg, dyg, W, H)
    rdx, rdz, rdU, rdb = lowrank_bwd(x64, z64, U64, b64, dy64, W, H)
    assert_close("dx", dx, rdx, td)
    # |g| of a group: the sum of its channels' |dy x| terms
    _, gabs = conv_bwd(np.abs(x64), np.zeros((B, T, G, W)), np.abs(dy64), H)
    gabs = gabs.reshape(B * T, G * W)
    u = {torch.bfloat16: 2.0**-8, torch.float16: 2.0**-11}.get(td, 2.0**-22)
    assert_close("dz", dz, rdz, td, extra=(u * (gabs @ np.abs(U64).T)).reshape(B, T, R))
    rt = torch.float32 if td == torch.float32 else td
    assert_close("dU", dU, rdU, rt, rtol=1e-5, atol=1e-5, extra=u * (np.abs(z64).reshape(B * T, R).T @ gabs))
    assert_close("db", db, rdb, rt, rtol=1e-5, atol=1e-5)


# head-wise generation on the bf16 fast kernels (forward, dx, g/dU/db with the group's H
# channels summed in the workgroup: H <= 16, W <= 4, R in {32, 64, 128}) and dz on the LDS
# DMA path (H = 2, 4: chunks of 32 groups, 32 * H channels); five dz chunks so that the
# three-stage ring wraps, three whole 64-token blocks and a ragged tail of 8 tokens
# (register path); the other W, R and H take the general kernels
HEADWISE_DMA = [(H, W, R) for H in (2, 4, 8, 16) for W in (1, 2, 3, 4, 5) for R in (32, 64, 96, 128)]
HEADWISE_DMA += [(H, W, R) for H in (4, 16) for W in (2, 4) for R in (20, 52)]
# the widest filters: dz on the DMA path where its stages fit (U rows of 24, 28 or 32
# 16-byte chunks per-channel), the rest of the backward and the forward on the general kernels
HEADWISE_DMA += [(H, W, R) for H in (1, 2, 4, 8, 16) for W in (6, 7, 8) for R in (32, 64, 128)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("H,W,R", HEADWISE_DMA)
def test_headwise_lowrank_fast_kernels(H, W, R, dtype):
    B, T = 2, 200
    D = 5 * 32 * H
    G = D // H
    seed = 900 + 10 * H + W + R
    td = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    x = synth.draw((B, T, D), 1.0, seed, "x", dtype)
    dy = synth.draw((B, T, D), 1.0, seed, "dy", dtype)
    z = synth.draw((B, T, R), 1.0, seed, "z", dtype)
    U = synth.draw((R, G * W), 0.3 / R**0.5, seed, "U", dtype)
    b = synth.draw((G * W,), 0.3, seed, "b", dtype)
    x64, z64, U64, b64, dy64 = to64(x), to64(z), to64(U), to64(b), to64(dy)
    y = dynconv_lowrank_fwd(x.cuda(), z.cuda(), U.cuda(), b.cuda(), W, H)
    assert_close("y", y, lowrank_fwd(x64, z64, U64, b64, W, H), td)
    dx, dz, dU, db = dynconv_lowrank_bwd(x.cuda(), z.cuda(), U.cuda(), b.cuda(), dy.cuda(), W, H)
    rdx, rdz, rdU, rdb = lowrank_bwd(x64, z64, U64, b64, dy64, W, H)
    _, gabs = conv_bwd(np.abs(x64), np.zeros((B, T, G, W)), np.abs(dy64), H)
    gabs = gabs.reshape(B * T, G * W)
    u = {torch.bfloat16: 2.0**-8, torch.float16: 2.0**-11}[td]
    assert_close("dz", dz, rdz, td, extra=(u * (gabs @ np.abs(U64).T)).reshape(B, T, R))
    assert_close("dx", dx, rdx, td)
    assert_close("dU", dU, rdU, td, rtol=1e-5, atol=1e-5, extra=u * (np.abs(z64).reshape(B * T, R).T @ gabs))
    assert_close("db", db, rdb, td, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("W", [6, 8])
def test_full_lowrank_wide_filters(W):
    """Six taps (the widest of the pages' ablation) and eight at B8 T4096 D2048 R64, the
    bench rows' launch: the fast forward (taps two row groups back), the general backward
    and the DMA dz kernel (U rows of 24 and 32 chunks); every element of y, dx, dz, dU, db."""
    B, T, D, R = 8, 4096, 2048, 64
    seed = 320 + W
    x = synth.draw((B, T, D), 1.0, seed, "x", "bf16")
    dy = synth.draw((B, T, D), 1.0, seed, "dy", "bf16")
    z = synth.draw((B, T, R), 1.0, seed, "z", "bf16")
    U = synth.draw((R, D * W), 0.1 / R**0.5, seed, "U", "bf16")
    b = synth.draw((D * W,), 0.1**0.5, seed, "b", "bf16")
    y = dynconv_lowrank_fwd(x.cuda(), z.cuda(), U.cuda(), b.cuda(), W).cpu()
    U64, b64 = to64(U), to64(b)
    for s_ in range(B):
        ref = lowrank_fwd(to64(x[s_ : s_ + 1]), to64(z[s_ : s_ + 1]), U64, b64, W)
        assert_close(f"y[{s_}]", y[s_ : s_ + 1], ref, torch.bfloat16)
    got = dynconv_lowrank_bwd(x.cuda(), z.cuda(), U.cuda(), b.cuda(), dy.cuda(), W)
    check_lowrank_full_bwd(x, z, U, b, dy, W, torch.bfloat16, got)


def _full_lowrank(W, R, H, seed, dtype=torch.bfloat16):
    """Every element of y, dx, dz, dU and db at B8 T4096 D2048 (U of R x (D/H)*W)."""
    B, T, D = 8, 4096, 2048
    dn = {torch.bfloat16: "bf16", torch.float16: "f16"}[dtype]
    x = synth.draw((B, T, D), 1.0, seed, "x", dn)
    dy = synth.draw((B, T, D), 1.0, seed, "dy", dn)
    z = synth.draw((B, T, R), 1.0, seed, "z", dn)
    U = synth.draw((R, (D // H) * W), 0.1 / R**0.5, seed, "U", dn)
    b = synth.draw(((D // H) * W,), 0.1**0.5, seed, "b", dn)
    y = dynconv_lowrank_fwd(x.cuda(), z.cuda(), U.cuda(), b.cuda(), W, H).cpu()
    U64, b64 = to64(U), to64(b)
    for s_ in range(B):
        ref = lowrank_fwd(to64(x[s_ : s_ + 1]), to64(z[s_ : s_ + 1]), U64, b64, W, H)
        assert_close(f"y[{s_}]", y[s_ : s_ + 1], ref, dtype)
    got = dynconv_lowrank_bwd(x.cuda(), z.cuda(), U.cuda(), b.cuda(), dy.cuda(), W, H)
    check_lowrank_full_bwd(x, z, U, b, dy, W, dtype, got, H=H)


def test_full_lowrank_w5_r64():
    """Five taps at 64 ranks on the fast kernels (the second generation tile set)."""
    _full_lowrank(5, 64, 1, 330)


def test_full_lowrank_h4_r64():
    """Head-wise generation, groups of 4 channels, on the fast kernels and the DMA dz."""
    _full_lowrank(4, 64, 4, 331)


def test_full_lowrank_r64_f32_fwd():
    """The float32 row (general kernels on the float32 matrix cores): every element of y."""
    B, T, D, W, R = 8, 4096, 2048, 4, 64
    seed = 332
    x = synth.draw((B, T, D), 1.0, seed, "x", "f32")
    z = synth.draw((B, T, R), 1.0, seed, "z", "f32")
    U = synth.draw((R, D * W), 0.1 / R**0.5, seed, "U", "f32")
    b = synth.draw((D * W,), 0.1**0.5, seed, "b", "f32")
    y = dynconv_lowrank_fwd(x.cuda(), z.cuda(), U.cuda(), b.cuda(), W).cpu()
    U64, b64 = to64(U), to64(b)
    for s_ in range(B):
        ref = lowrank_fwd(to64(x[s_ : s_ + 1]), to64(z[s_ : s_ + 1]), U64, b64, W)
        assert_close(f"y[{s_}]", y[s_ : s_ + 1], ref, torch.float32)


def test_full_lowrank_conv_bias():
    """The low-rank bias row at B8 T4096 D2048 W4 R64: y against the oracle with the bias,
    the bias gradient against the column sum of dy, and dx, dz, dU, db bit for bit those of
    the call without it."""
    wl = synth.workloads()["lowrank_r64_bwd"]
    x, z, U, b, dy = (t.cuda() for t in (wl.x(), wl.z(), wl.U(), wl.b(), wl.dy()))
    c = synth.draw((wl.D,), 0.5, wl.seed, "c", "bf16")
    y = dynconv_lowrank_fwd(x, z, U, b, wl.W, conv_bias=c.cuda()).cpu()
    with_cb = dynconv_lowrank_bwd(x, z, U, b, dy, wl.W, want_dconv_bias=True)
    without = dynconv_lowrank_bwd(x, z, U, b, dy, wl.W)
    for name, a_, b_ in zip(("dx", "dz", "dU", "db"), with_cb[:4], without):
        assert torch.equal(a_, b_), name
    U64, b64, c64 = to64(U.cpu()), to64(b.cpu()), to64(c)
    xc, zc, dyc = x.cpu(), z.cpu(), dy.cpu()
    for s_ in range(wl.B):
        ref = lowrank_fwd(to64(xc[s_ : s_ + 1]), to64(zc[s_ : s_ + 1]), U64, b64, wl.W, 1, None, c64)
        assert_close(f"y[{s_}]", y[s_ : s_ + 1], ref, torch.bfloat16)
    assert_close("dconv_bias", with_cb[4], conv_bias_grad(to64(dyc)), torch.float32, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("R", [16, 20, 52])
def test_full_lowrank_pages_ranks(R):
    """The pages' ranks at B8 T4096 D2048 W4 on the fast kernels (contiguous z: rows of
    40 or 104 bytes, staged in 4-byte pieces, ranks zero-padded to 32 or 64): every
    element of y, dx, dz, dU and db."""
    B, T, D, W = 8, 4096, 2048, 4
    seed = 300 + R
    x = synth.draw((B, T, D), 1.0, seed, "x", "bf16")
    dy = synth.draw((B, T, D), 1.0, seed, "dy", "bf16")
    z = synth.draw((B, T, R), 1.0, seed, "z", "bf16")
    U = synth.draw((R, D * W), 0.1 / R**0.5, seed, "U", "bf16")
    b = synth.draw((D * W,), 0.1**0.5, seed, "b", "bf16")
    y = dynconv_lowrank_fwd(x.cuda(), z.cuda(), U.cuda(), b.cuda(), W).cpu()
    U64, b64 = to64(U), to64(b)
    for s_ in range(B):
        ref = lowrank_fwd(to64(x[s_ : s_ + 1]), to64(z[s_ : s_ + 1]), U64, b64, W)
        assert_close(f"y[{s_}]", y[s_ : s_ + 1], ref, torch.bfloat16)
    got = dynconv_lowrank_bwd(x.cuda(), z.cuda(), U.cuda(), b.cuda(), dy.cuda(), W)
    check_lowrank_full_bwd(x, z, U, b, dy, W, torch.bfloat16, got)


@pytest.mark.parametrize("W", [4, 5])
def test_fast_long_sequence(W):
    """One sequence of 2^17 + 37 tokens on the fast kernels (token ranges of many steps,
    indices past 2^16, a ragged last step): every element of y, dx, dz, dU, db."""
    B, T, D, R = 1, (1 << 17) + 37, 64, 64
    x, z, U, b, dy = _inputs(B, T, D, W, R, "bf16", 91 + W)
    y = dynconv_lowrank_fwd(x.cuda(), z.cuda(), U.cuda(), b.cuda(), W).cpu()
    assert_close("y", y, lowrank_fwd(to64(x), to64(z), to64(U), to64(b), W), torch.bfloat16)
    got = dynconv_lowrank_bwd(x.cuda(), z.cuda(), U.cuda(), b.cuda(), dy.cuda(), W)
    check_lowrank_full_bwd(x, z, U, b, dy, W, torch.bfloat16, got)


def test_many_sequences_lowrank():
    """1024 sequences of 37 tokens (each shorter than one 64-token step) on the fast
    kernels."""
    _check(1024, 37, 64, 4, 64, "bf16", seed=1024)
