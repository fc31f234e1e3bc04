"""GPU parity of the streaming kernels (materialised and static filters) against the
float64 oracle, through the C ABI.

Small cases span several time chunks and channel slices with ragged tails; the full
workloads (the pages' D = 2048, T = 4096 model shapes) are checked on every element (one
sequence at a time), in the launch configuration the benchmark uses.
"""
import numpy as np
import pytest
import torch

import synth
from dynamic_short_convolution_amd import dynconv_bwd, dynconv_fwd
from oracle import conv_bias_grad, conv_bwd, conv_fwd
from tests.parity import assert_close, to64

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    from dynamic_short_convolution_amd import _lib

    _lib.load()
    yield
    torch.cuda.synchronize()


def _inputs(B, T, D, W, H, dtype, static, seed):
    x = synth.draw((B, T, D), 1.0, seed, "x", dtype)
    dy = synth.draw((B, T, D), 1.0, seed, "dy", dtype)
    shape = (D // H, W) if static else (B, T, D // H, W)
    w = synth.draw(shape, (1.0 / W) ** 0.5, seed, "w", dtype)
    return x, w, dy


def _check_case(B, T, D, W, H, dtype, static, seed=0):
    x, w, dy = _inputs(B, T, D, W, H, dtype, static, seed)
    xg, wg, dyg = x.cuda(), w.cuda(), dy.cuda()
    y = dynconv_fwd(xg, wg, H)
    dx, dw = dynconv_bwd(xg, wg, dyg, H)
    torch.cuda.synchronize()
    x64, w64, dy64 = to64(x), to64(w), to64(dy)
    td = DT[dtype]
    assert_close("y", y, conv_fwd(x64, w64, H), td)
    rdx, rdw = conv_bwd(x64, w64, dy64, H)
    assert_close("dx", dx, rdx, td)
    if static:
        # float32 output of a sum over all (b, t): allow the float32 per-chunk sums
        assert_close("dw_static", dw, rdw, torch.float32, rtol=1e-5, atol=1e-5)
    else:
        assert_close("dw", dw, rdw, td)


SMALL = []
for dtype in ("f32", "bf16"):
    for W in (1, 2, 3, 4, 5):
        for H in (1, 2, 4, 16):
            for static in (False, True):
                D = 200 if H == 1 else 640
                for T in (3, 100, 333):
                    SMALL.append((dtype, W, H, static, D, T))


# float16 storage (the same kernels with float16 conversions)
for W in (1, 2, 3, 4, 5, 8):
    for H in (1, 4, 16):
        for static in (False, True):
            SMALL.append(("f16", W, H, static, 200 if H == 1 else 640, 333))

# the widest filters (W = 6..8; the pages' ablation reaches W = 6)
for dtype in ("f32", "bf16"):
    for W in (6, 7, 8):
        for H in (1, 2, 4, 16):
            for static in (False, True):
                for T in (5, 333):
                    SMALL.append((dtype, W, H, static, 200 if H == 1 else 640, T))


@pytest.mark.parametrize("dtype,W,H,static,D,T", SMALL)
def test_small_parity(dtype, W, H, static, D, T):
    _check_case(2, T, D, W, H, dtype, static, seed=W * 7 + H + T)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("H", [8, 32, 64, 128, 256, 512])
def test_large_head_sizes(dtype, H):
    if dtype == "f32" and H > 256:
        pytest.skip("float32 lanes hold 4 channels: at most 64 * 4 channels per group")
    _check_case(2, 77, 1024, 4, H, dtype, False, seed=H)
    _check_case(1, 50, 1024, 3, H, dtype, True, seed=H + 1)


# Head-wise groups whose size is not a power of two (the head-wise parameterisation takes
# any H that divides D): odd H other than 3 and 5 in 16-bit storage (one channel per lane),
# 63 channels and float32 groups of 3 * 2^k or 5 * 2^k channels reduce with the suffix scan
# (the lanes of a wave past the last whole group idle); 16-bit groups of 3 * 2^k and 5 * 2^k
# channels take 6 or 10 channels per lane and a power-of-two number of lanes, and the 16-bit
# backward puts a whole group of 3 or 5 channels on a lane.
ODD_H = [
    # dtype, W, H, D
    ("bf16", 4, 3, 198),
    ("f16", 3, 5, 390),
    ("f32", 4, 3, 198),
    ("f32", 2, 63, 126),
    ("bf16", 1, 6, 1152),
    ("bf16", 4, 6, 1152),
    ("f32", 5, 6, 1152),
    ("bf16", 4, 12, 1536),
    ("f16", 8, 24, 768),
    ("bf16", 3, 96, 2304),
    ("f32", 4, 96, 2304),
    ("bf16", 4, 384, 1536),
    ("bf16", 2, 10, 640),
    ("bf16", 4, 63, 126),
    # more groups of 3 * 2^k channels: wide filters, the widest group (64 lanes of 6)
    ("bf16", 8, 12, 1536),
    ("f16", 6, 96, 2304),
    ("f32", 4, 12, 1536),
    ("f32", 3, 192, 1536),
    ("bf16", 5, 384, 1536),
    # odd groups: 3 or 5 channels per lane in the 16-bit backward, 7 with the scan
    ("f16", 8, 3, 198),
    ("bf16", 5, 5, 390),
    ("bf16", 4, 7, 196),
    ("f16", 2, 7, 196),
    # 16-bit groups of 5 * 2^k channels: 10 channels per lane
    ("bf16", 4, 10, 1280),
    ("f16", 3, 20, 1280),
    ("bf16", 8, 80, 2560),
    ("bf16", 2, 640, 1280),
    ("f32", 4, 80, 1280),
]


@pytest.mark.parametrize("dtype,W,H,D", ODD_H)
@pytest.mark.parametrize("static", [False, True])
def test_non_power_of_two_groups(dtype, W, H, D, static):
    _check_case(2, 333, D, W, H, dtype, static, seed=H + W + int(static))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 2, 4, 5])
def test_short_sequences(dtype, T):
    """T < W and T = 1: every tap past the start of the sequence reads zeros."""
    for W in (4, 5):
        _check_case(3, T, 64, W, 1, dtype, False, seed=T)
        _check_case(3, T, 64, W, 1, dtype, True, seed=T)


def test_tiny_perchannel_f32_workload():
    wl = synth.workloads()["tiny_perchannel_f32"]
    x, w, dy = wl.x(), wl.w(), wl.dy()
    y = dynconv_fwd(x.cuda(), w.cuda(), wl.H)
    dx, dw = dynconv_bwd(x.cuda(), w.cuda(), dy.cuda(), wl.H)
    ry = conv_fwd(to64(x), to64(w), wl.H)
    rdx, rdw = conv_bwd(to64(x), to64(w), to64(dy), wl.H)
    assert_close("y", y, ry, torch.float32)
    assert_close("dx", dx, rdx, torch.float32)
    assert_close("dw", dw, rdw, torch.float32)


@pytest.mark.parametrize("j", [0, 1, 2, 3])
def test_one_hot_tap_rounds_to_nearest_even(j):
    """w one-hot at tap j: y_t = x_t + x_{t-j} (exact in float32), stored with RNE."""
    B, T, D, W = 2, 40, 256, 4
    x = synth.draw((B, T, D), 1.0, 5, "x", "bf16")
    w = torch.zeros((B, T, D, W), dtype=torch.bfloat16)
    w[..., j] = 1.0
    y = dynconv_fwd(x.cuda(), w.cuda(), 1).cpu()
    xs = x.float()
    ref = xs.clone()
    if j == 0:
        ref = xs + xs
    else:
        ref[:, j:, :] += xs[:, : T - j, :]
    assert torch.equal(y.view(torch.int16), ref.to(torch.bfloat16).view(torch.int16))


def test_zero_filters_identity_bitwise():
    x = synth.draw((2, 50, 300), 1.0, 6, "x", "bf16").cuda()
    dy = synth.draw((2, 50, 300), 1.0, 6, "dy", "bf16").cuda()
    w = torch.zeros((2, 50, 300, 3), dtype=torch.bfloat16, device="cuda")
    assert torch.equal(dynconv_fwd(x, w, 1), x)
    dx, dw = dynconv_bwd(x, w, dy, 1)
    assert torch.equal(dx, dy)


@pytest.mark.parametrize("H,static,D", [(1, False, 1024), (16, False, 1024), (1, True, 1024), (6, False, 1152),
                                          (3, True, 1152), (96, False, 1152)])
def test_every_output_written_and_guards_untouched(H, static, D):
    """Outputs start as NaN inside guard bands of rows and columns; afterwards every
    element is finite and the guards are still NaN (bitwise)."""
    B, T, W = 2, 130, 4
    x, w, dy = _inputs(B, T, D, W, H, "bf16", static, 9)
    xg, wg, dyg = x.cuda(), w.cuda(), dy.cuda()
    G = 3
    ybig = torch.full((B, T + 2 * G, D + 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = ybig[:, G : G + T, :D]
    dynconv_fwd(xg, wg, H, out=y)
    dxbig = torch.full_like(ybig, float("nan"))
    dx = dxbig[:, G : G + T, :D]
    dwbig = None
    dw = None
    if not static:
        dwbig = torch.full((B, T + 2 * G, D // H + 8, W), float("nan"), dtype=torch.bfloat16, device="cuda")
        dw = dwbig[:, G : G + T, : D // H, :]
    dynconv_bwd(xg, wg, dyg, H, dx=dx, dw=dw)
    torch.cuda.synchronize()
    for big, view in ((ybig, y), (dxbig, dx)):
        assert not torch.isnan(view).any()
        mask = torch.ones(big.shape, dtype=torch.bool, device="cuda")
        mask[:, G : G + T, :D] = False
        assert torch.isnan(big[mask]).all()
    if dwbig is not None:
        assert not torch.isnan(dw).any()
        mask = torch.ones(dwbig.shape, dtype=torch.bool, device="cuda")
        mask[:, G : G + T, : D // H, :] = False
        assert torch.isnan(dwbig[mask]).all()
    x64, w64, dy64 = to64(x), to64(w), to64(dy)
    assert_close("y(strided)", y, conv_fwd(x64, w64, H), torch.bfloat16)
    rdx, rdw = conv_bwd(x64, w64, dy64, H)
    assert_close("dx(strided)", dx, rdx, torch.bfloat16)
    if dw is not None:
        assert_close("dw(strided)", dw, rdw, torch.bfloat16)


@pytest.mark.parametrize("H,static", [(1, False), (4, False), (16, False), (1, True), (16, True), (12, False),
                                      (3, True)])
def test_run_to_run_deterministic(H, static):
    x, w, dy = _inputs(2, 300, 1152 if H % 3 == 0 else 1024, 4, H, "bf16", static, 11)
    xg, wg, dyg = x.cuda(), w.cuda(), dy.cuda()
    outs = []
    for _ in range(3):
        y = dynconv_fwd(xg, wg, H)
        dx, dw = dynconv_bwd(xg, wg, dyg, H)
        outs.append((y.clone(), dx.clone(), dw.clone()))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_dx_only_and_dw_only():
    x, w, dy = _inputs(2, 90, 512, 4, 1, "bf16", False, 12)
    xg, wg, dyg = x.cuda(), w.cuda(), dy.cuda()
    dx_a, dw_a = dynconv_bwd(xg, wg, dyg, 1)
    dx_b, none_b = dynconv_bwd(xg, wg, dyg, 1, need_dw=False)
    none_c, dw_c = dynconv_bwd(xg, wg, dyg, 1, need_dx=False)
    assert none_b is None and none_c is None
    assert torch.equal(dx_a, dx_b) and torch.equal(dw_a, dw_c)


def test_fused_qkv_launch_equals_separate_launches():
    """One launch over the concatenated [Q | K | V] channels equals three launches on the
    channel slices (the convolution is depthwise), and both match the oracle."""
    B, T, W = 2, 200, 4
    split = (512, 128, 128)
    D = sum(split)
    x, w, dy = _inputs(B, T, D, W, 1, "bf16", False, 13)
    xg, wg, dyg = x.cuda(), w.cuda(), dy.cuda()
    y = dynconv_fwd(xg, wg, 1)
    dx, dw = dynconv_bwd(xg, wg, dyg, 1)
    c0 = 0
    for n in split:
        ys = dynconv_fwd(xg[:, :, c0 : c0 + n], wg[:, :, c0 : c0 + n, :], 1)
        dxs, dws = dynconv_bwd(xg[:, :, c0 : c0 + n], wg[:, :, c0 : c0 + n, :], dyg[:, :, c0 : c0 + n], 1)
        assert torch.equal(ys, y[:, :, c0 : c0 + n])
        assert torch.equal(dxs, dx[:, :, c0 : c0 + n])
        assert torch.equal(dws, dw[:, :, c0 : c0 + n, :])
        c0 += n
    assert_close("y", y, conv_fwd(to64(x), to64(w)), torch.bfloat16)


# ------------------------------------------------------------------------------------
# full-size workloads, every element, one sequence at a time (each sequence's own max|ref|
# scales its bound, which is at least as strict as the whole tensor's)
# ------------------------------------------------------------------------------------


def _full_check(wl, do_fwd=True, do_bwd=True):
    x, w, dy = wl.x(), wl.w(), wl.dy() if do_bwd else None
    xg, wg = x.cuda(), w.cuda()
    H = wl.H
    y = dynconv_fwd(xg, wg, H).cpu() if do_fwd else None
    if do_bwd:
        dx, dw = dynconv_bwd(xg, wg, dy.cuda(), H)
        dx, dw = dx.cpu(), dw.cpu()
    del xg, wg
    torch.cuda.empty_cache()
    rdw_static = 0.0
    for b in range(wl.B):
        x64 = to64(x[b : b + 1])
        w64 = to64(w if wl.static else w[b : b + 1])
        if do_fwd:
            assert_close(f"{wl.name} y[{b}]", y[b : b + 1], conv_fwd(x64, w64, H), torch.bfloat16)
        if do_bwd:
            rdx, rdw = conv_bwd(x64, w64, to64(dy[b : b + 1]), H)
            assert_close(f"{wl.name} dx[{b}]", dx[b : b + 1], rdx, torch.bfloat16)
            if wl.static:
                rdw_static = rdw_static + rdw  # the static gradient sums every sequence
            else:
                assert_close(f"{wl.name} dw[{b}]", dw[b : b + 1], rdw, torch.bfloat16)
    if do_bwd and wl.static:
        assert_close(f"{wl.name} dw", dw, rdw_static, torch.float32, rtol=1e-5, atol=1e-5)


def test_full_headwise_h16_fwd():
    _full_check(synth.workloads()["headwise_h16"], do_bwd=False)


def test_full_static_w3_fwd_bwd():
    _full_check(synth.workloads()["static_w3"])


def test_full_qkv_gqa_fused_fwd_bwd():
    # every channel, the Q|K and K|V boundaries included
    _full_check(synth.workloads()["qkv_gqa_fused"])


def test_full_perchannel_h1_fwd_bwd():
    _full_check(synth.workloads()["perchannel_h1"])


def test_full_headwise_h4_bwd():
    _full_check(synth.workloads()["headwise_h4"], do_fwd=False)


def test_full_headwise_h16_bwd():
    _full_check(synth.workloads()["headwise_h16_bwd"], do_fwd=False)


def test_full_headwise_h12_fwd_bwd():
    # groups of 3 lanes (4 channels each), 63 lanes of a backward wave in use
    _full_check(synth.workloads()["headwise_h12"])


def test_full_headwise_h4_fwd():
    _full_check(synth.workloads()["headwise_h4"], do_bwd=False)


def test_full_static_w4_fwd_bwd():
    _full_check(synth.Workload("static_w4", 8, 4096, 2048, 4, 1, static=True, seed=7, w_var=0.25))


def test_full_perchannel_w8_fwd_bwd():
    # the widest filter: plain stores in the backward, 8 taps per lane window
    _full_check(synth.Workload("perchannel_w8", 8, 4096, 2048, 8, 1, seed=8))


def test_full_perchannel_conv_bias():
    """The per-channel bias row at B8 T4096 D2048 W4: y with the bias, dx and dw as without
    it, and the bias gradient (a column sum of dy over all 32768 tokens)."""
    wl = synth.Workload("convbias_perchannel_h1", 8, 4096, 2048, 4, 1, seed=9)
    x, w, dy = wl.x(), wl.w(), wl.dy()
    c = synth.draw((wl.D,), 0.5, wl.seed, "c", "bf16")
    xg, wg, dyg, cg = x.cuda(), w.cuda(), dy.cuda(), c.cuda()
    y = dynconv_fwd(xg, wg, 1, conv_bias=cg).cpu()
    dx, dw, dcb = (t.cpu() for t in dynconv_bwd(xg, wg, dyg, 1, want_dconv_bias=True))
    del xg, wg, dyg
    torch.cuda.empty_cache()
    c64 = to64(c)
    for b in range(wl.B):
        x64, w64 = to64(x[b : b + 1]), to64(w[b : b + 1])
        assert_close(f"y[{b}]", y[b : b + 1], conv_fwd(x64, w64, 1, None, c64), torch.bfloat16)
        rdx, rdw = conv_bwd(x64, w64, to64(dy[b : b + 1]), 1)
        assert_close(f"dx[{b}]", dx[b : b + 1], rdx, torch.bfloat16)
        assert_close(f"dw[{b}]", dw[b : b + 1], rdw, torch.bfloat16)
    assert_close("dconv_bias", dcb, conv_bias_grad(to64(dy)), torch.float32, rtol=1e-5, atol=1e-5)


# The fixed-order reduce of the static backward's per-chunk partials has a 16-byte path
# (row length n = D/H * W a multiple of 4, aligned pointers) and a 4-byte one; both sum
# each column in the same order. n = 594 and a dw output one float off a 16-byte boundary
# take the 4-byte path, n = 600 the 16-byte path.
@pytest.mark.parametrize("D,offset", [(198, 0), (200, 0), (200, 1)])
def test_static_dw_reduce_paths(D, offset):
    B, T, W, H = 3, 700, 3, 1
    x, w, dy = _inputs(B, T, D, W, H, "bf16", True, 31 + D + offset)
    buf = torch.full((D * W + offset,), float("nan"), dtype=torch.float32, device="cuda")
    dw = buf[offset:].view(D, W)
    dx, dw_out = dynconv_bwd(x.cuda(), w.cuda(), dy.cuda(), H, dw=dw)
    assert dw_out.data_ptr() == dw.data_ptr()
    rdx, rdw = conv_bwd(to64(x), to64(w), to64(dy), H)
    assert_close("dx", dx, rdx, torch.bfloat16)
    assert_close("dw_static", dw, rdw, torch.float32, rtol=1e-5, atol=1e-5)
    if offset:
        assert torch.isnan(buf[:offset]).all()


@pytest.mark.parametrize("H,static", [(1, False), (4, False), (1, True)])
def test_long_sequence(H, static):
    """One sequence of 2^17 + 37 tokens: token indices past 2^16, many time chunks, a
    ragged last chunk; every element."""
    _check_case(1, (1 << 17) + 37, 128, 4, H, "bf16", static, seed=171 + H)


@pytest.mark.parametrize("B,T,D", [(1024, 37, 64), (1, 17, 16384)])
def test_many_sequences_and_wide_rows(B, T, D):
    """Grids large along the batch (1024 sequences of 37 tokens) and along the channels
    (one 16384-channel row per token): per-channel, head-wise and static."""
    for H, static in ((1, False), (16, False), (1, True)):
        _check_case(B, T, D, 4, H, "bf16", static, seed=B + D + H)
