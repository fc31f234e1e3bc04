"""GPU parity of the optional convolution bias (dynconv_fwd_ex / dynconv_bwd_ex /
dynconv_decode_step_ex, and dynconv_lowrank_{fwd,bwd,decode_step}_ex) against the float64
oracle.

The bias is the per-channel vector of the convolution technical report's Conv1D module,
added to every output token; its gradient is the sum of dy over every token (float32,
summed per time chunk and then in a fixed order). The other outputs must be those of the
call without a bias. Tolerances as in the other parity tests; the bias gradient is a
float32 sum over all tokens like a static filter gradient (1e-5).
"""
import pytest
import torch

import synth
from dynamic_short_convolution_amd import (dynconv_bwd, dynconv_cache_fill, dynconv_decode_step, dynconv_fwd,
                                           dynconv_lowrank_bwd, dynconv_lowrank_decode_step, dynconv_lowrank_fwd)
from oracle import conv_bias_grad, conv_bwd, conv_fwd, lowrank_fwd
from tests.parity import assert_close, to64

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    yield
    torch.cuda.synchronize()


def _case(B, T, D, W, H, dtype, static, seed, packed=False, need_dx=True, need_dw=True):
    td = DT[dtype]
    x = synth.draw((B, T, D), 1.0, seed, "x", dtype)
    dy = synth.draw((B, T, D), 1.0, seed, "dy", dtype)
    w = synth.draw((D // H, W) if static else (B, T, D // H, W), (1.0 / W) ** 0.5, seed, "w", dtype)
    c = synth.draw((D,), 0.5, seed, "b", dtype)
    seq = synth.segments(B, T, 15.0, seed, first=(1, 2)) if packed else None
    s64 = seq.numpy() if packed else None
    sg = seq.cuda() if packed else None
    xg, wg, dyg, cg = x.cuda(), w.cuda(), dy.cuda(), c.cuda()
    x64, w64, dy64 = to64(x), to64(w), to64(dy)
    y = dynconv_fwd(xg, wg, H, seq_idx=sg, conv_bias=cg)
    assert_close("y", y, conv_fwd(x64, w64, H, s64, to64(c)), td)
    dx, dw, dcb = dynconv_bwd(xg, wg, dyg, H, need_dx=need_dx, need_dw=need_dw, seq_idx=sg, want_dconv_bias=True)
    assert_close("dconv_bias", dcb, conv_bias_grad(dy64), torch.float32, rtol=1e-5, atol=1e-5)
    rdx, rdw = conv_bwd(x64, w64, dy64, H, s64)
    if need_dx:
        assert_close("dx", dx, rdx, td)
    if need_dw:
        if static:
            assert_close("dw_static", dw, rdw, torch.float32, rtol=1e-5, atol=1e-5)
        else:
            assert_close("dw", dw, rdw, td)


CASES = []
for dtype in ("f32", "bf16", "f16"):
    for W in (1, 3, 4, 8):
        for H, static in ((1, False), (4, False), (16, False), (1, True), (4, True), (6, False), (3, True)):
            CASES.append((dtype, W, H, static))


@pytest.mark.parametrize("dtype,W,H,static", CASES)
def test_conv_bias_parity(dtype, W, H, static):
    D = 136 if H == 1 else (264 if H % 3 == 0 else 256)
    _case(2, 300, D, W, H, dtype, static, seed=40 + W + H + int(static))


@pytest.mark.parametrize("static", [False, True])
def test_conv_bias_packed(static):
    _case(2, 257, 200, 4, 1, "bf16", static, seed=3, packed=True)
    _case(2, 257, 256, 3, 8, "f32", static, seed=4, packed=True)


@pytest.mark.parametrize("need_dx,need_dw", [(True, False), (False, True)])
def test_conv_bias_with_one_other_output(need_dx, need_dw):
    _case(2, 190, 200, 4, 1, "bf16", False, seed=5, need_dx=need_dx, need_dw=need_dw)
    _case(2, 190, 200, 3, 1, "bf16", True, seed=6, need_dx=need_dx, need_dw=need_dw)


def test_conv_bias_many_chunks():
    """Long sequences: many time chunks per sequence, each with its own partial sum."""
    _case(4, 2048, 256, 4, 1, "bf16", False, seed=7)
    _case(4, 2048, 256, 3, 1, "bf16", True, seed=8)


def test_zero_bias_equals_no_bias():
    B, T, D, W = 2, 100, 128, 4
    x = synth.draw((B, T, D), 1.0, 9, "x", "bf16").cuda()
    w = synth.draw((B, T, D, W), 0.5, 9, "w", "bf16").cuda()
    dy = synth.draw((B, T, D), 1.0, 9, "dy", "bf16").cuda()
    z = torch.zeros(D, dtype=torch.bfloat16, device="cuda")
    assert torch.equal(dynconv_fwd(x, w, 1, conv_bias=z), dynconv_fwd(x, w, 1))
    a, b = dynconv_bwd(x, w, dy, 1, want_dconv_bias=True), dynconv_bwd(x, w, dy, 1)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("W,H,static", [(4, 1, False), (3, 4, False), (2, 1, True)])
def test_conv_bias_decode(dtype, W, H, static):
    B, Ttot, D, T0 = 3, 9, 72, 4
    x = synth.draw((B, Ttot, D), 1.0, 60 + W, "x", dtype)
    w = synth.draw((D // H, W) if static else (B, Ttot, D // H, W), 0.5, 60 + W, "w", dtype)
    c = synth.draw((D,), 0.5, 60 + W, "b", dtype)
    ref = conv_fwd(to64(x), to64(w), H, None, to64(c))
    xg, wg, cg = x.cuda(), w.cuda(), c.cuda()
    cache = dynconv_cache_fill(xg[:, :T0], W)
    for t in range(T0, Ttot):
        yt = dynconv_decode_step(xg[:, t], wg if static else wg[:, t], cache, t, H, conv_bias=cg)
        assert_close(f"y[{t}]", yt, ref[:, t], DT[dtype])


# ------------------------------------------------------------------------------------
# the low-rank form: the bias joins the generated filters' output; its gradient is one
# more pass over dy, and the other gradients are those of the call without it, bit for bit
# ------------------------------------------------------------------------------------
LOWRANK = [
    # dtype, B, T, D, W, H, R, packed: the fast kernels (bf16 / f16, D % 64, even R) and the
    # general ones (float32, W = 5 above 64 ranks, W = 6..8, odd R, groups of 6)
    ("bf16", 2, 300, 128, 4, 1, 64, False),
    ("f16", 2, 300, 128, 5, 1, 32, False),
    ("bf16", 2, 300, 256, 4, 4, 20, True),
    ("f32", 2, 300, 96, 3, 1, 16, False),
    ("bf16", 2, 150, 96, 5, 1, 100, False),
    ("bf16", 1, 77, 72, 2, 6, 7, True),
    ("bf16", 2, 150, 128, 8, 1, 64, True),
    ("f32", 2, 100, 96, 6, 2, 20, False),
]


@pytest.mark.parametrize("dtype,B,T,D,W,H,R,packed", LOWRANK)
def test_lowrank_conv_bias(dtype, B, T, D, W, H, R, packed):
    seed = 800 + W + R + H
    td = DT[dtype]
    G = D // H
    x = synth.draw((B, T, D), 1.0, seed, "x", dtype)
    dy = synth.draw((B, T, D), 1.0, seed, "dy", dtype)
    z = synth.draw((B, T, R), 1.0, seed, "z", dtype)
    U = synth.draw((R, G * W), 0.3 / R**0.5, seed, "U", dtype)
    b = synth.draw((G * W,), 0.3, seed, "b", dtype)
    c = synth.draw((D,), 0.5, seed, "c", dtype)
    seq = synth.segments(B, T, 40.0, seed) if packed else None
    xg, zg, Ug, bg, cg, dyg = x.cuda(), z.cuda(), U.cuda(), b.cuda(), c.cuda(), dy.cuda()
    sg = seq.cuda() if packed else None
    y = dynconv_lowrank_fwd(xg, zg, Ug, bg, W, H, seq_idx=sg, conv_bias=cg)
    s64 = seq.numpy() if packed else None
    assert_close("y", y, lowrank_fwd(to64(x), to64(z), to64(U), to64(b), W, H, s64, to64(c)), td)
    with_cb = dynconv_lowrank_bwd(xg, zg, Ug, bg, dyg, W, H, seq_idx=sg, want_dconv_bias=True)
    without = dynconv_lowrank_bwd(xg, zg, Ug, bg, dyg, W, H, seq_idx=sg)
    torch.cuda.synchronize()
    for name, a_, b_ in zip(("dx", "dz", "dU", "db"), with_cb[:4], without):
        assert torch.equal(a_, b_), name
    assert_close("dconv_bias", with_cb[4], conv_bias_grad(to64(dy)), torch.float32, rtol=1e-5, atol=1e-5)


def test_lowrank_conv_bias_many_chunks():
    """Long sequences: the column sums take many chunks per sequence."""
    B, T, D, W, R = 3, 3000, 192, 4, 32
    x = synth.draw((B, T, D), 1.0, 5, "x", "bf16").cuda()
    dy = synth.draw((B, T, D), 1.0, 5, "dy", "bf16")
    z = synth.draw((B, T, R), 1.0, 5, "z", "bf16").cuda()
    U = synth.draw((R, D * W), 0.05, 5, "U", "bf16").cuda()
    out = dynconv_lowrank_bwd(x, z, U, None, dy.cuda(), W, want_dconv_bias=True)
    assert_close("dconv_bias", out[4], conv_bias_grad(to64(dy)), torch.float32, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("W,H,R", [(4, 1, 64), (3, 4, 20), (5, 3, 40), (8, 2, 32), (7, 1, 100)])
def test_lowrank_conv_bias_decode(dtype, W, H, R):
    B, Ttot, D, T0 = 5, 8, 96, 3
    seed = 70 + W + R
    x = synth.draw((B, Ttot, D), 1.0, seed, "x", dtype)
    z = synth.draw((B, Ttot, R), 1.0, seed, "z", dtype)
    U = synth.draw((R, (D // H) * W), 0.3 / R**0.5, seed, "U", dtype)
    b = synth.draw(((D // H) * W,), 0.3, seed, "b", dtype)
    c = synth.draw((D,), 0.5, seed, "c", dtype)
    ref = lowrank_fwd(to64(x), to64(z), to64(U), to64(b), W, H, None, to64(c))
    xg, zg, Ug, bg, cg = x.cuda(), z.cuda(), U.cuda(), b.cuda(), c.cuda()
    cache = dynconv_cache_fill(xg[:, :T0], W)
    for t in range(T0, Ttot):
        yt = dynconv_lowrank_decode_step(xg[:, t], zg[:, t], Ug, bg, cache, t, W, H=H, conv_bias=cg)
        assert_close(f"y[{t}]", yt, ref[:, t], DT[dtype])
