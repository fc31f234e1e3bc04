"""GPU parity of the inference path against the float64 oracle, through the C ABI.

A prompt of T0 tokens goes through the forward kernel, its last W-1 inputs into the
rolling cache (dynconv_cache_fill), and the following tokens are decoded one at a time
(dynconv_decode_step / dynconv_lowrank_decode_step). Step t must give row t of eq. 2 +
eq. 3 over the whole sequence, which the oracle computes directly; prompts shorter than
W-1 (T0 = 0, 1, 2) check the zero padding carried by the cache. Tolerances as in the
other parity tests (tests/parity.py).
"""
import numpy as np
import pytest
import torch

import synth
from dynamic_short_convolution_amd import (dynconv_cache_fill, dynconv_decode_step, dynconv_fwd,
                                           dynconv_lowrank_decode_step, dynconv_lowrank_fwd, new_cache)
from oracle import conv_fwd, lowrank_fwd
from tests.parity import assert_close, to64

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    yield
    torch.cuda.synchronize()


CASES = []
for dtype in ("f32", "bf16", "f16"):
    for W in (1, 2, 3, 4, 5, 6, 7, 8):
        for H, static in ((1, False), (4, False), (1, True)):
            for T0 in (0, 2, 7):
                CASES.append((dtype, W, H, static, T0))
    # groups whose size is not a power of two
    for W in (3, 4, 8):
        for H, static in ((6, False), (3, True), (9, False)):
            CASES.append((dtype, W, H, static, 2))


@pytest.mark.parametrize("dtype,W,H,static,T0", CASES)
def test_decode_matches_full_sequence(dtype, W, H, static, T0):
    B, Ttot, D = 3, 12, 72
    seed = 500 + 10 * W + H + 3 * T0 + int(static)
    x = synth.draw((B, Ttot, D), 1.0, seed, "x", dtype)
    w = synth.draw((D // H, W) if static else (B, Ttot, D // H, W), (1.0 / W) ** 0.5, seed, "w", dtype)
    ref = conv_fwd(to64(x), to64(w), H)
    xg, wg = x.cuda(), w.cuda()
    if T0 > 0:
        y0 = dynconv_fwd(xg[:, :T0].contiguous(), wg if static else wg[:, :T0].contiguous(), H)
        assert_close("prefill", y0, ref[:, :T0], TD[dtype])
    cache = dynconv_cache_fill(xg[:, :T0], W)
    for t in range(T0, Ttot):
        yt = dynconv_decode_step(xg[:, t], wg if static else wg[:, t], cache, t, H)
        assert_close(f"y[{t}]", yt, ref[:, t], TD[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("W,R,T0", [(1, 16, 3), (2, 40, 1), (3, 20, 0), (4, 64, 5), (4, 96, 0), (5, 128, 2), (6, 32, 2),
                                     (7, 64, 0), (8, 128, 3)])
def test_lowrank_decode_matches_full_sequence(dtype, W, R, T0):
    B, Ttot, D = 19, 10, 136  # two groups of sequences, a partial group of channels
    seed = 900 + W + R + T0
    x = synth.draw((B, Ttot, D), 1.0, seed, "x", dtype)
    z = synth.draw((B, Ttot, R), 1.0, seed, "z", dtype)
    U = synth.draw((R, D * W), 0.3 / R**0.5, seed, "U", dtype)
    b = synth.draw((D * W,), 0.3, seed, "b", dtype)
    ref = lowrank_fwd(to64(x), to64(z), to64(U), to64(b), W)
    xg, zg, Ug, bg = x.cuda(), z.cuda(), U.cuda(), b.cuda()
    if T0 > 0:
        y0 = dynconv_lowrank_fwd(xg[:, :T0].contiguous(), zg[:, :T0].contiguous(), Ug, bg, W)
        assert_close("prefill", y0, ref[:, :T0], TD[dtype])
    cache = dynconv_cache_fill(xg[:, :T0], W)
    for t in range(T0, Ttot):
        yt = dynconv_lowrank_decode_step(xg[:, t], zg[:, t], Ug, bg, cache, t, W)
        assert_close(f"y[{t}]", yt, ref[:, t], TD[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("H,W,R", [(4, 4, 64), (2, 3, 20), (16, 5, 32), (3, 4, 64), (6, 3, 20), (12, 5, 40)])
def test_headwise_lowrank_decode(dtype, H, W, R):
    """U of R x (D/H)*W: the H channels of a group share the generated filter."""
    B, Ttot, D = 5, 8, 96
    seed = 950 + H + W
    x = synth.draw((B, Ttot, D), 1.0, seed, "x", dtype)
    z = synth.draw((B, Ttot, R), 1.0, seed, "z", dtype)
    U = synth.draw((R, (D // H) * W), 0.3 / R**0.5, seed, "U", dtype)
    b = synth.draw(((D // H) * W,), 0.3, seed, "b", dtype)
    ref = lowrank_fwd(to64(x), to64(z), to64(U), to64(b), W, H)
    xg, zg, Ug, bg = x.cuda(), z.cuda(), U.cuda(), b.cuda()
    T0 = 3
    y0 = dynconv_lowrank_fwd(xg[:, :T0].contiguous(), zg[:, :T0].contiguous(), Ug, bg, W, H)
    assert_close("prefill", y0, ref[:, :T0], TD[dtype])
    cache = dynconv_cache_fill(xg[:, :T0], W)
    for t in range(T0, Ttot):
        yt = dynconv_lowrank_decode_step(xg[:, t], zg[:, t], Ug, bg, cache, t, W, H=H)
        assert_close(f"y[{t}]", yt, ref[:, t], TD[dtype])


def test_lowrank_decode_without_bias():
    B, Ttot, D, W, R = 4, 6, 64, 4, 32
    x = synth.draw((B, Ttot, D), 1.0, 77, "x", "bf16")
    z = synth.draw((B, Ttot, R), 1.0, 77, "z", "bf16")
    U = synth.draw((R, D * W), 0.1, 77, "U", "bf16")
    ref = lowrank_fwd(to64(x), to64(z), to64(U), None, W)
    cache = new_cache(B, D, W, torch.bfloat16, "cuda")
    for t in range(Ttot):
        yt = dynconv_lowrank_decode_step(x[:, t].cuda(), z[:, t].cuda(), U.cuda(), None, cache, t, W)
        assert_close(f"y[{t}]", yt, ref[:, t], torch.bfloat16)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("W", [2, 4])
def test_lowrank_decode_unaligned_operands(dtype, W):
    """z rows, U and bias starting one element past a 16-byte boundary, U rows ldu = D*W + 4
    apart: the element-wise load paths, against the same oracle."""
    B, Ttot, D, R = 5, 4, 40, 48
    x = synth.draw((B, Ttot, D), 1.0, 31 + W, "x", dtype)
    zw = synth.draw((B, Ttot, R + 1), 1.0, 31 + W, "z", dtype)
    Uw = synth.draw((R, D * W + 4), 0.3 / R**0.5, 31 + W, "U", dtype)
    bw = synth.draw((D * W + 1,), 0.3, 31 + W, "b", dtype)
    z, U, b = zw[:, :, 1:], Uw[:, 1 : 1 + D * W], bw[1:]
    ref = lowrank_fwd(to64(x), to64(z), to64(U), to64(b), W)
    zg, Ug, bg = zw.cuda()[:, :, 1:], Uw.cuda()[:, 1 : 1 + D * W], bw.cuda()[1:]
    assert Ug.stride(0) == D * W + 4 and Ug.data_ptr() % 16 != 0 and zg.data_ptr() % 16 != 0
    cache = new_cache(B, D, W, TD[dtype], "cuda")
    for t in range(Ttot):
        yt = dynconv_lowrank_decode_step(x[:, t].cuda(), zg[:, t], Ug, bg, cache, t, W)
        assert_close(f"y[{t}]", yt, ref[:, t], TD[dtype])


def test_cache_fill_contents():
    """The ring after a prompt of T tokens holds x[T-W+1 .. T-1] in slots s mod (W-1), and
    zeros for positions before 0: an exact copy."""
    B, D = 2, 40
    for W in (2, 4, 5, 8):
        for T in (0, 1, 3, 9):
            x = synth.draw((B, max(T, 1), D), 1.0, 11 + T + W, "x", "bf16")[:, :T]
            cache = dynconv_cache_fill(x.cuda(), W).cpu()
            want = torch.zeros_like(cache)
            for s in range(T - W + 1, T):
                if s >= 0:
                    want[:, s % (W - 1)] = x[:, s]
            assert torch.equal(cache, want), (W, T)


def test_decode_step_strided_rows():
    """x, w and y rows as slices of wider buffers, the cache as a slice of a larger one."""
    B, D, W, Ttot = 2, 64, 3, 5
    x = synth.draw((B, Ttot, D), 1.0, 3, "x", "bf16")
    w = synth.draw((B, Ttot, D, W), 0.5, 3, "w", "bf16")
    ref = conv_fwd(to64(x), to64(w), 1)
    big = torch.zeros((B, W + 2, 2 * D), dtype=torch.bfloat16, device="cuda")
    cache = big[:, 1:W, D:]
    yb = torch.zeros((B, 3 * D), dtype=torch.bfloat16, device="cuda")
    for t in range(Ttot):
        dynconv_decode_step(x[:, t].cuda(), w[:, t].cuda(), cache, t, 1, out=yb[:, D : 2 * D])
        assert_close(f"y[{t}]", yb[:, D : 2 * D], ref[:, t], torch.bfloat16)
    assert torch.count_nonzero(big[:, 0]) == 0 and torch.count_nonzero(big[:, W:]) == 0
    assert torch.count_nonzero(big[:, :, :D]) == 0
    assert torch.count_nonzero(yb[:, :D]) == 0 and torch.count_nonzero(yb[:, 2 * D :]) == 0
