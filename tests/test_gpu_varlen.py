"""GPU parity of packed sequences (several documents per row, per-token segment ids)
against the float64 oracle, through the C ABI.

Rows hold documents of random lengths (synth.segments) led by documents of 1, 2 and 3
tokens, shorter than the filter, so that taps are cut at every distance; the kernels'
time chunks and token tiles fall at arbitrary offsets to the document starts. The oracle
(oracle.conv_fwd / conv_bwd / lowrank_* with seq_idx) is pinned by packed == separate
documents in tests/test_oracle_pins.py. Tolerances as in the other parity tests.
"""
import numpy as np
import pytest
import torch

import synth
from dynamic_short_convolution_amd import (dynconv_bwd, dynconv_cache_fill, dynconv_decode_step, dynconv_fwd,
                                           dynconv_lowrank_bwd, dynconv_lowrank_fwd)
from oracle import conv_bwd, conv_fwd, lowrank_bwd, lowrank_fwd
from tests.parity import assert_close, to64

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    yield
    torch.cuda.synchronize()


def _stream_case(B, T, D, W, H, dtype, static, seed, mean_len=20.0, seq=None):
    x = synth.draw((B, T, D), 1.0, seed, "x", dtype)
    dy = synth.draw((B, T, D), 1.0, seed, "dy", dtype)
    w = synth.draw((D // H, W) if static else (B, T, D // H, W), (1.0 / W) ** 0.5, seed, "w", dtype)
    if seq is None:
        seq = synth.segments(B, T, mean_len, seed, first=(1, 2, 3))
    xg, wg, dyg = x.cuda(), w.cuda(), dy.cuda()
    sg = seq.cuda()
    y = dynconv_fwd(xg, wg, H, seq_idx=sg)
    dx, dw = dynconv_bwd(xg, wg, dyg, H, seq_idx=sg)
    s64 = seq.cpu().numpy()
    x64, w64, dy64 = to64(x), to64(w), to64(dy)
    td = DT[dtype]
    assert_close("y", y, conv_fwd(x64, w64, H, s64), td)
    rdx, rdw = conv_bwd(x64, w64, dy64, H, s64)
    assert_close("dx", dx, rdx, td)
    if static:
        assert_close("dw_static", dw, rdw, torch.float32, rtol=1e-5, atol=1e-5)
    else:
        assert_close("dw", dw, rdw, td)
    return y, dx, dw


STREAM = []
for dtype in ("f32", "bf16", "f16"):
    for W in (1, 2, 3, 4, 5, 6, 8):
        for H, static in ((1, False), (4, False), (16, False), (1, True), (4, True)):
            STREAM.append((dtype, W, H, static))
    for W in (3, 4):
        for H, static in ((6, False), (3, True), (12, False)):
            STREAM.append((dtype, W, H, static))


@pytest.mark.parametrize("dtype,W,H,static", STREAM)
def test_packed_stream_parity(dtype, W, H, static):
    D = 136 if H == 1 else (264 if H % 3 == 0 else 256)
    _stream_case(2, 300, D, W, H, dtype, static, seed=300 + 10 * W + H + int(static))


@pytest.mark.parametrize("mean_len", [1.0, 4.0, 500.0])
def test_packed_stream_document_lengths(mean_len):
    """Every token its own document (no tap survives but k = 0), short documents, and
    documents longer than a time chunk."""
    _stream_case(3, 257, 200, 4, 1, "bf16", False, seed=7, mean_len=mean_len)
    _stream_case(2, 257, 256, 3, 8, "bf16", True, seed=8, mean_len=mean_len)


def test_packed_single_segment_equals_unpacked():
    """One segment per row: bit for bit the call without segment ids."""
    for H, static in ((1, False), (4, False), (1, True)):
        B, T, D, W = 2, 190, 256, 4
        x = synth.draw((B, T, D), 1.0, 5, "x", "bf16").cuda()
        dy = synth.draw((B, T, D), 1.0, 5, "dy", "bf16").cuda()
        w = synth.draw((D // H, W) if static else (B, T, D // H, W), 0.5, 5, "w", "bf16").cuda()
        seq = torch.full((B, T), 7, dtype=torch.int32, device="cuda")
        assert torch.equal(dynconv_fwd(x, w, H, seq_idx=seq), dynconv_fwd(x, w, H))
        a, b = dynconv_bwd(x, w, dy, H, seq_idx=seq), dynconv_bwd(x, w, dy, H)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_packed_strided_segment_ids():
    """Segment ids as a transposed [T, B] tensor and as every other column of a wider one."""
    B, T = 2, 150
    seq = synth.segments(B, T, 9.0, 11, first=(1, 2))
    tr = seq.t().contiguous().cuda().t()          # strides (1, B)
    wide = torch.zeros((B, 2 * T), dtype=torch.int32)
    wide[:, ::2] = seq
    wd = wide.cuda()[:, ::2]                      # strides (2T, 2)
    assert tr.stride() == (1, B) and wd.stride() == (2 * T, 2)
    for sg in (tr, wd):
        x = synth.draw((B, T, 64), 1.0, 12, "x", "bf16")
        w = synth.draw((B, T, 64, 4), 0.5, 12, "w", "bf16")
        dy = synth.draw((B, T, 64), 1.0, 12, "dy", "bf16")
        y = dynconv_fwd(x.cuda(), w.cuda(), 1, seq_idx=sg)
        dx, dw = dynconv_bwd(x.cuda(), w.cuda(), dy.cuda(), 1, seq_idx=sg)
        s64 = seq.numpy()
        assert_close("y", y, conv_fwd(to64(x), to64(w), 1, s64), torch.bfloat16)
        rdx, rdw = conv_bwd(to64(x), to64(w), to64(dy), 1, s64)
        assert_close("dx", dx, rdx, torch.bfloat16)
        assert_close("dw", dw, rdw, torch.bfloat16)


LOWRANK = [("bf16", 4, 64, 128, 1), ("bf16", 2, 32, 128, 1), ("bf16", 3, 64, 192, 1), ("bf16", 5, 40, 72, 1),
           ("f32", 1, 16, 64, 1), ("f32", 3, 64, 136, 1), ("f32", 4, 128, 64, 1), ("bf16", 4, 64, 128, 4),
           ("f32", 3, 32, 64, 8), ("f16", 4, 64, 128, 1), ("f16", 3, 40, 96, 2), ("bf16", 4, 64, 512, 4),
           ("bf16", 3, 32, 320, 2), ("bf16", 5, 64, 192, 2),
           ("bf16", 4, 64, 1024, 8), ("bf16", 4, 64, 1024, 16), ("bf16", 2, 32, 512, 8),
           ("bf16", 4, 64, 192, 6), ("f32", 3, 20, 96, 3), ("f16", 5, 40, 240, 12),
           ("bf16", 6, 64, 128, 1), ("f32", 8, 32, 96, 2), ("f16", 7, 100, 72, 1)]


@pytest.mark.parametrize("dtype,W,R,D,H", LOWRANK)
def test_packed_lowrank_parity(dtype, W, R, D, H):
    """Includes bf16 shapes that would take the fast kernels without segment ids, and
    head-wise generation."""
    B, T, seed = 2, 300, 700 + W + R + H
    td = DT[dtype]
    G = D // H
    x = synth.draw((B, T, D), 1.0, seed, "x", dtype)
    dy = synth.draw((B, T, D), 1.0, seed, "dy", dtype)
    z = synth.draw((B, T, R), 1.0, seed, "z", dtype)
    U = synth.draw((R, G * W), 0.3 / R**0.5, seed, "U", dtype)
    b = synth.draw((G * W,), 0.3, seed, "b", dtype)
    seq = synth.segments(B, T, 24.0, seed, first=(1, 2, 3))
    xg, zg, Ug, bg, dyg, sg = x.cuda(), z.cuda(), U.cuda(), b.cuda(), dy.cuda(), seq.cuda()
    x64, z64, U64, b64, dy64, s64 = to64(x), to64(z), to64(U), to64(b), to64(dy), seq.numpy()
    y = dynconv_lowrank_fwd(xg, zg, Ug, bg, W, H, seq_idx=sg)
    assert_close("y", y, lowrank_fwd(x64, z64, U64, b64, W, H, s64), td)
    dx, dz, dU, db = dynconv_lowrank_bwd(xg, zg, Ug, bg, dyg, W, H, seq_idx=sg)
    rdx, rdz, rdU, rdb = lowrank_bwd(x64, z64, U64, b64, dy64, W, H, s64)
    assert_close("dx", dx, rdx, td)
    _, gabs = conv_bwd(np.abs(x64), np.zeros((B, T, G, W)), np.abs(dy64), H)
    gabs = gabs.reshape(B * T, G * W)
    u = {torch.bfloat16: 2.0**-8, torch.float16: 2.0**-11}.get(td, 2.0**-22)
    assert_close("dz", dz, rdz, td, extra=(u * (gabs @ np.abs(U64).T)).reshape(B, T, R))
    rt = torch.float32 if td == torch.float32 else td
    assert_close("dU", dU, rdU, rt, rtol=1e-5, atol=1e-5, extra=u * (np.abs(z64).reshape(B * T, R).T @ gabs))
    assert_close("db", db, rdb, rt, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("W", [2, 4, 5, 8])
def test_packed_prompt_cache_fill_and_decode(W):
    """The cache after a packed prompt holds only the last document's tokens; decoding
    then continues that document (row t of the oracle over the packed row, with the new
    tokens in the last segment)."""
    B, T0, Ttot, D = 3, 11, 16, 72
    seq = synth.segments(B, Ttot, 4.0, 40 + W, first=(1, 2))
    # the decoded tokens continue the prompt's last document
    seq[:, T0:] = seq[:, T0 - 1 : T0]
    x = synth.draw((B, Ttot, D), 1.0, 41 + W, "x", "bf16")
    w = synth.draw((B, Ttot, D, W), 0.5, 41 + W, "w", "bf16")
    ref = conv_fwd(to64(x), to64(w), 1, seq.numpy())
    xg, wg = x.cuda(), w.cuda()
    cache = dynconv_cache_fill(xg[:, :T0], W, seq_idx=seq[:, :T0].contiguous().cuda())
    want = torch.zeros((B, W - 1, D), dtype=torch.bfloat16)
    for b in range(B):
        for s in range(T0 - W + 1, T0):
            if s >= 0 and seq[b, s] == seq[b, T0 - 1]:
                want[b, s % (W - 1)] = x[b, s]
    assert torch.equal(cache.cpu(), want)
    for t in range(T0, Ttot):
        yt = dynconv_decode_step(xg[:, t], wg[:, t], cache, t, 1)
        assert_close(f"y[{t}]", yt, ref[:, t], torch.bfloat16)


def test_full_packed_perchannel():
    """B8 T4096 D2048 W4 with documents of mean length 512, every element (one sequence at a
    time), in the launch configuration of the benchmark's packed rows."""
    wl = synth.workloads()["perchannel_h1"]
    x, w, dy = wl.x(), wl.w(), wl.dy()
    seq = synth.segments(wl.B, wl.T, 512.0, wl.seed, first=(1, 2, 3))
    xg, wg, dyg, sg = x.cuda(), w.cuda(), dy.cuda(), seq.cuda()
    y = dynconv_fwd(xg, wg, 1, seq_idx=sg).cpu()
    dx, dw = dynconv_bwd(xg, wg, dyg, 1, seq_idx=sg)
    dx, dw = dx.cpu(), dw.cpu()
    del xg, wg, dyg
    torch.cuda.empty_cache()
    s64 = seq.numpy()
    for b in range(wl.B):
        x64, w64, sq = to64(x[b : b + 1]), to64(w[b : b + 1]), s64[b : b + 1]
        assert_close(f"y[{b}]", y[b : b + 1], conv_fwd(x64, w64, 1, sq), torch.bfloat16)
        rdx, rdw = conv_bwd(x64, w64, to64(dy[b : b + 1]), 1, sq)
        assert_close(f"dx[{b}]", dx[b : b + 1], rdx, torch.bfloat16)
        assert_close(f"dw[{b}]", dw[b : b + 1], rdw, torch.bfloat16)


def test_full_packed_lowrank():
    """B8 T4096 D2048 W4 R64 with documents of mean length 512 (the fast kernels with
    segment ids), every element of y, dx, dz, dU and db."""
    from tests.test_gpu_lowrank import check_lowrank_full_bwd

    wl = synth.workloads()["lowrank_r64"]
    x, z, U, b, dy = wl.x(), wl.z(), wl.U(), wl.b(), wl.dy()
    W = wl.W
    seq = synth.segments(wl.B, wl.T, 512.0, wl.seed, first=(1, 2, 3))
    xg, zg, Ug, bg, sg = x.cuda(), z.cuda(), U.cuda(), b.cuda(), seq.cuda()
    y = dynconv_lowrank_fwd(xg, zg, Ug, bg, W, seq_idx=sg).cpu()
    got = dynconv_lowrank_bwd(xg, zg, Ug, bg, dy.cuda(), W, seq_idx=sg)
    s64 = seq.numpy()
    U64, b64 = to64(U), to64(b)
    for bb in range(wl.B):
        ref = lowrank_fwd(to64(x[bb : bb + 1]), to64(z[bb : bb + 1]), U64, b64, W, 1, s64[bb : bb + 1])
        assert_close(f"y[{bb}]", y[bb : bb + 1], ref, torch.bfloat16)
    check_lowrank_full_bwd(x, z, U, b, dy, W, torch.bfloat16, got, seq_idx=s64)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("W", [4, 5])
@pytest.mark.parametrize("R", [20, 64])
def test_packed_lowrank_fast_padded_rank(R, W):
    """Packed sequences on the fast low-rank kernels with a rank that is zero-padded (20:
    4-byte z pieces) and one that is not, at W = 4 and W = 5 (a fifth tap reaching the
    previous lane's first token)."""
    B, T, D = 2, 640, 256
    seed = 400 + R + 13 * W
    x = synth.draw((B, T, D), 1.0, seed, "x", "bf16")
    dy = synth.draw((B, T, D), 1.0, seed, "dy", "bf16")
    z = synth.draw((B, T, R), 1.0, seed, "z", "bf16")
    U = synth.draw((R, D * W), 0.3 / R**0.5, seed, "U", "bf16")
    b = synth.draw((D * W,), 0.3, seed, "b", "bf16")
    seq = synth.segments(B, T, 40.0, seed, first=(1, 2, 3))
    sg = seq.cuda()
    y = dynconv_lowrank_fwd(x.cuda(), z.cuda(), U.cuda(), b.cuda(), W, seq_idx=sg)
    x64, z64, U64, b64, dy64, s64 = to64(x), to64(z), to64(U), to64(b), to64(dy), seq.numpy()
    assert_close("y", y, lowrank_fwd(x64, z64, U64, b64, W, 1, s64), torch.bfloat16)
    dx, dz, dU, db = dynconv_lowrank_bwd(x.cuda(), z.cuda(), U.cuda(), b.cuda(), dy.cuda(), W, seq_idx=sg)
    rdx, rdz, rdU, rdb = lowrank_bwd(x64, z64, U64, b64, dy64, W, 1, s64)
    _, gabs = conv_bwd(np.abs(x64), np.zeros((B, T, D, W)), np.abs(dy64), 1, s64)
    gabs = gabs.reshape(B * T, D * W)
    u = 2.0**-8
    assert_close("dx", dx, rdx, torch.bfloat16)
    assert_close("dz", dz, rdz, torch.bfloat16, extra=(u * (gabs @ np.abs(U64).T)).reshape(B, T, R))
    assert_close("dU", dU, rdU, torch.bfloat16, rtol=1e-5, atol=1e-5,
                 extra=u * (np.abs(z64).reshape(B * T, R).T @ gabs))
    assert_close("db", db, rdb, torch.bfloat16, rtol=1e-5, atol=1e-5)
