"""Every global load and store of the DMA-staged and chunk-loop kernels stays inside its
tensor, over sweeps of dtype, W, R, H, D, T and strided layouts (host emulation of the
kernels' index arithmetic, tests/kernel_bounds.py). Each case also checks that the
emulated stores cover the whole output, so that an emulation which drops work cannot pass.
"""
import itertools

import numpy as np
import pytest

import kernel_bounds as kb


def _full(acc, name, B, T, C):
    cov = acc.cover(name, B, T, C)
    assert cov.all(), f"{name}: {int((~cov).sum())} of {cov.size} elements never touched"


# ---------------------------------------------------------------------------------------
# projection + convolution
# ---------------------------------------------------------------------------------------
GEMM = [
    # B, T, K, N, W, H
    (1, 1, 64, 128, 4, 1),
    (2, 300, 128, 256, 3, 2),
    (1, 481, 64, 384, 5, 16),
    (3, 100, 192, 128, 1, 4),
    (1, 2000, 64, 256, 4, 8),
]


@pytest.mark.parametrize("B,T,K,N,W,H", GEMM)
def test_gemm_conv_bounds(B, T, K, N, W, H):
    acc = kb.gemm_conv(B, T, K, N, W, H)
    G = N // H
    acc.check({"A": (B, T, K), "Wp": (1, N, K), "w": (B, T, G * W), "y": (B, T, N)})
    _full(acc, "y", B, T, N)
    _full(acc, "A", B, T, K)


@pytest.mark.parametrize("B,T,K,N,W,H", GEMM)
@pytest.mark.parametrize("R", [8, 20, 64, 100, 128])
@pytest.mark.parametrize("vec", [True, False])
def test_gemm_lowrank_bounds(B, T, K, N, W, H, R, vec):
    zvec = vec and R % 8 == 0
    acc = kb.gemm_conv(B, T, K, N, W, H, R=R, lowrank=True, zvec=zvec, uvec=vec, has_bias=R % 2 == 0)
    J = (N // H) * W
    acc.check({"A": (B, T, K), "Wp": (1, N, K), "z": (B, T, R), "U": (1, R, J), "bias": (1, 1, J),
               "y": (B, T, N)})
    _full(acc, "y", B, T, N)
    _full(acc, "U", 1, R, J)


# ---------------------------------------------------------------------------------------
# fast low-rank forward and fused backward
# ---------------------------------------------------------------------------------------
FAST_SHAPES = [
    # B, T, D
    (1, 1, 64),
    (2, 4, 64),
    (1, 63, 128),
    (2, 64, 64),
    (1, 65, 192),
    (2, 200, 128),
    (1, 1000, 64),
]
FAST_RANKS = [2, 20, 26, 64, 100, 128]


def _fast_cases(widths=(1, 2, 3, 4, 5), ok=kb.fast_width_ok):
    for (B, T, D), W, H, R in itertools.product(FAST_SHAPES, widths, [1, 4, 16], FAST_RANKS):
        if D % H or not ok(W, (R + 31) // 32):
            continue
        for ZB in ([16, 4] if R % 8 == 0 else [4]):
            yield B, T, D, W, H, R, ZB


FAST_CASES = list(_fast_cases())
# a deterministic subset keeps the CPU suite short; every shape, W, H, R and ZB appears
FAST_PICK = FAST_CASES[::7]
# the forward alone also takes six to eight taps (up to 64 ranks)
FAST_FWD_WIDE = list(_fast_cases((6, 7, 8), kb.fwd_fast_width_ok))[::5]


def _layout(D, R, ZB, strided):
    """Row strides: dense, or views into wider rows (16-byte multiples for the activations,
    ZB-byte multiples for z)."""
    if not strided:
        return D, R, D, D
    zpad = 8 if ZB == 16 else 2
    return D + 64, (R + zpad + (zpad - 1)) // zpad * zpad, D + 8, D + 128


@pytest.mark.parametrize("B,T,D,W,H,R,ZB", FAST_PICK + FAST_FWD_WIDE)
@pytest.mark.parametrize("strided", [False, True])
def test_lowrank_fwd_fast_bounds(B, T, D, W, H, R, ZB, strided):
    xs1, zs1, dys1, os1 = _layout(D, R, ZB, strided)
    seg = T % 4 == 0 and T >= 4
    acc = kb.lowrank_fwd_fast(B, T, D, W, H, R, ZB, xs1, zs1, os1, seg=seg, has_bias=(T % 2 == 0))
    J = (D // H) * W
    acc.check({"x": (B, T, D), "z": (B, T, R), "U": (1, R, J), "bias": (1, 1, J), "y": (B, T, D),
               "seg": (B, T, 1)})
    _full(acc, "y", B, T, D)
    _full(acc, "x", B, T, D)
    _full(acc, "z", B, T, R)


@pytest.mark.parametrize("B,T,D,W,H,R,ZB", FAST_PICK)
@pytest.mark.parametrize("strided", [False, True])
def test_lowrank_bwd_fused_bounds(B, T, D, W, H, R, ZB, strided):
    xs1, zs1, dys1, os1 = _layout(D, R, ZB, strided)
    seg = T % 4 == 0 and T >= 4
    acc, nTr = kb.lowrank_bwd_fused(B, T, D, W, H, R, ZB, xs1, zs1, dys1, os1, seg=seg, has_bias=(T % 2 == 1))
    J = (D // H) * W
    nR = B * nTr
    acc.check({"x": (B, T, D), "dy": (B, T, D), "z": (B, T, R), "U": (1, R, J), "bias": (1, 1, J),
               "dx": (B, T, D), "seg": (B, T, 1), "part_dU": (1, nR * R, J), "part_db": (1, nR, J)})
    _full(acc, "dx", B, T, D)
    _full(acc, "part_dU", 1, nR * R, J)
    _full(acc, "part_db", 1, nR, J)
    _full(acc, "dy", B, T, D)


def test_fast_case_list_is_wide():
    ws = {c[3] for c in FAST_PICK}
    hs = {c[4] for c in FAST_PICK}
    rs = {c[5] for c in FAST_PICK}
    zbs = {c[6] for c in FAST_PICK}
    shapes = {c[:3] for c in FAST_PICK}
    assert ws == {1, 2, 3, 4, 5} and hs == {1, 4, 16} and rs == set(FAST_RANKS) and zbs == {4, 16}
    assert shapes == set(FAST_SHAPES)


# ---------------------------------------------------------------------------------------
# DMA dz
# ---------------------------------------------------------------------------------------

def _dz_cases():
    for W, H, R, T in itertools.product(range(1, 9), [1, 2, 4, 8, 16], [2, 20, 64, 100, 128], [64, 130]):
        KS = (R + 31) // 32
        s = kb.dz_dma_shape(W, KS, H)
        if not s["ok"]:
            continue
        D = s["CHC"] * (2 if H <= 4 else 1)
        yield 1, T, D, W, H, R


DZ_CASES = list(_dz_cases())


@pytest.mark.parametrize("B,T,D,W,H,R", DZ_CASES[::3])
@pytest.mark.parametrize("strided", [False, True])
def test_dz_dma_bounds(B, T, D, W, H, R, strided):
    J = (D // H) * W
    xs1, dys1, ldu = (D + 64, D + 8, J + 8) if strided else (D, D, J)
    acc = kb.dz_dma(B, T, D, W, H, R, xs1, dys1, ldu)
    acc.check({"x": (B, T, D), "dy": (B, T, D), "U": (1, R, J), "dz": (B, T, R)})
    T64 = T // 64 * 64
    _full(acc, "dz", B, T64, R)
    _full(acc, "U", 1, R, J)


def test_dz_cases_cover_every_group_size_and_width():
    assert {c[4] for c in DZ_CASES[::3]} == {1, 2, 4, 8, 16}
    assert {c[3] for c in DZ_CASES[::3]} == set(range(1, 9))


# ---------------------------------------------------------------------------------------
# fixed-order reduce
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("nchunk", [1, 7, 8, 63, 64, 200])
@pytest.mark.parametrize("n", [1, 3, 4, 31, 33, 600, 2052])
def test_reduce_partials_bounds(nchunk, n):
    for vec4 in ([False, True] if n % 4 == 0 else [False]):
        acc = kb.reduce_partials(nchunk, n, vec4)
        acc.check({"part": (1, nchunk, n), "out": (1, 1, n)})
        _full(acc, "part", 1, nchunk, n)  # every partial summed ...
        assert sum(int(w.sum()) for *_, w in acc.spans["part"]) == nchunk * n  # ... once
        _full(acc, "out", 1, 1, n)


# ---------------------------------------------------------------------------------------
# decoding
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("B,D,H", [(1, 8, 1), (3, 72, 4), (5, 130, 5), (17, 96, 6)])
@pytest.mark.parametrize("W", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("t", [0, 1, 2, 7, 20])
def test_decode_bounds(B, D, H, W, t):
    S = max(W - 1, 1)
    fill = kb.cache_fill(B, t, D, W, seg=t > 0)
    fill.check({"x": (B, max(t, 1), D), "cache": (B, S, D), "seg": (B, max(t, 1), 1)})
    if W > 1:
        _full(fill, "cache", B, S, D)
    for static in (False, True):
        acc = kb.decode_step(B, D, W, H, t, static=static, cbias=True)
        acc.check({"w": (1 if static else B, 1, (D // H) * W), "x": (B, 1, D), "cbias": (1, 1, D),
                   "cache": (B, S, D), "y": (B, 1, D)})
        _full(acc, "y", B, 1, D)


@pytest.mark.parametrize("B,D,H", [(1, 8, 1), (19, 136, 1), (16, 64, 4), (33, 72, 3)])
@pytest.mark.parametrize("W", [1, 2, 4, 5, 8])
@pytest.mark.parametrize("R", [1, 8, 20, 64, 96, 128])
@pytest.mark.parametrize("t", [0, 3])
def test_lowrank_decode_bounds(B, D, H, W, R, t):
    vec = R % 8 == 0
    S = max(W - 1, 1)
    J = (D // H) * W
    acc, voffs = kb.lowrank_decode_step(B, D, W, H, R, t, vec, has_bias=R % 3 != 0, cbias=True)
    acc.check({"x": (B, 1, D), "cache": (B, S, D), "z": (B, 1, R), "U": (1, R, J), "bias": (1, 1, J),
               "cbias": (1, 1, D), "y": (B, 1, D)})
    _full(acc, "y", B, 1, D)
    # vector loads: z pieces of 8 ranks at multiples of 8 (16-byte aligned rows), U taps at
    # multiples of W (rows ldu = J, a multiple of W)
    for name, row, col in voffs:
        assert col % (8 if name == "z" else W) == 0, (name, row, col)


# ---------------------------------------------------------------------------------------
# register-path dz (every dtype, ragged T and D, any H; the blocks the DMA path leaves)
# ---------------------------------------------------------------------------------------
DZ_REG = [
    # B, T, D, H
    (1, 1, 8, 1),
    (2, 65, 40, 2),
    (1, 130, 96, 3),
    (1, 200, 72, 12),
    (2, 64, 256, 16),
]


@pytest.mark.parametrize("B,T,D,H", DZ_REG)
@pytest.mark.parametrize("W", [1, 3, 4, 5, 7, 8])
@pytest.mark.parametrize("R", [1, 20, 64, 100, 128])
@pytest.mark.parametrize("eb", [2, 4])
def test_lowrank_dz_register_bounds(B, T, D, H, W, R, eb):
    J = (D // H) * W
    strided = (T + W + R) % 2 == 1
    xs1, dys1, ldu = (D + 24, D + 8, J + 5) if strided else (D, D, J)
    acc = kb.lowrank_dz_register(B, T, D, W, H, R, eb, xs1, dys1, ldu, seg=T % 2 == 1)
    acc.check({"x": (B, T, D), "dy": (B, T, D), "U": (1, R, J), "dz": (B, T, R), "seg": (B, T, 1)})
    _full(acc, "dz", B, T, R)
    _full(acc, "x", B, T, D)
    _full(acc, "dy", B, T, D)


def test_lowrank_dz_register_tail_blocks():
    """The blocks after the DMA path's whole ones (tbb0 > 0): only the tail's tokens of dz."""
    B, T, D, W, H, R = 2, 200, 64, 4, 1, 64
    acc = kb.lowrank_dz_register(B, T, D, W, H, R, 2, D, D, D * W, tbb0=3, nTbL=1)
    acc.check({"x": (B, T, D), "dy": (B, T, D), "U": (1, R, D * W), "dz": (B, T, R)})
    cov = acc.cover("dz", B, T, R)
    assert cov[:, 192:].all() and not cov[:, :192].any()


# ---------------------------------------------------------------------------------------
# general kernels
# ---------------------------------------------------------------------------------------
GEN = [
    # B, T, D, H
    (1, 1, 8, 1),
    (2, 17, 40, 2),
    (1, 100, 130, 1),
    (1, 300, 96, 4),
    (2, 45, 36, 3),
    (1, 70, 120, 12),
]


@pytest.mark.parametrize("B,T,D,H", GEN)
@pytest.mark.parametrize("W", [1, 3, 4, 5, 7, 8])
@pytest.mark.parametrize("R", [1, 3, 20, 64, 100])
@pytest.mark.parametrize("eb", [2, 4])
def test_lowrank_fwd_general_bounds(B, T, D, H, W, R, eb):
    vec = (T + W + R) % 2 == 0
    acc = kb.lowrank_fwd_general(B, T, D, W, H, R, eb, act16=vec, z16=not vec, seg=T % 3 == 1,
                                 has_bias=R % 2 == 0)
    J = (D // H) * W
    acc.check({"x": (B, T, D), "z": (B, T, R), "U": (1, R, J), "bias": (1, 1, J), "y": (B, T, D), "seg": (B, T, 1)})
    _full(acc, "y", B, T, D)
    _full(acc, "x", B, T, D)


GEN_BWD = [
    # B, T, D, H
    (1, 1, 16, 1),
    (2, 5, 40, 2),
    (1, 64, 32, 1),
    (1, 65, 48, 4),
    (1, 150, 96, 1),
    (2, 300, 64, 2),
    (1, 70, 96, 6),
    (2, 33, 60, 5),
]


@pytest.mark.parametrize("B,T,D,H", GEN_BWD)
@pytest.mark.parametrize("W", [1, 2, 4, 5, 6, 8])
@pytest.mark.parametrize("R", [3, 32, 64, 100, 128])
@pytest.mark.parametrize("eb", [2, 4])
def test_lowrank_bwd_general_bounds(B, T, D, H, W, R, eb):
    fast = R % 32 == 0
    acc, nTr = kb.lowrank_bwd_general(B, T, D, W, H, R, eb, fast, seg=T % 2 == 1, has_bias=W % 2 == 0,
                                      want_db=R != 64,
                                      lean=(eb == 2 and W <= 4 and D % 64 == 0 and H in (1, 2, 4, 8, 16)))
    J = (D // H) * W
    nR = B * nTr
    acc.check({"x": (B, T, D), "dy": (B, T, D), "z": (B, T, R), "U": (1, R, J), "bias": (1, 1, J),
               "dx": (B, T, D), "seg": (B, T, 1), "part_dU": (1, nR * H * R, J), "part_db": (1, nR * H, J)})
    _full(acc, "dx", B, T, D)
    _full(acc, "part_dU", 1, nR * H * R, J)


# ---------------------------------------------------------------------------------------
# streaming kernels (materialised and static filters), every group size the ABI admits
# ---------------------------------------------------------------------------------------
STREAM = [
    # B, T, D, H
    (1, 1, 2, 1),
    (2, 37, 200, 1),
    (1, 300, 768, 1),
    (2, 50, 96, 2),
    (1, 129, 1024, 16),
    (3, 40, 198, 3),
    (1, 70, 390, 5),
    (2, 33, 1152, 6),
    (1, 90, 1536, 12),
    (1, 20, 2304, 96),
    (1, 17, 1536, 384),
    (2, 25, 126, 63),
    (1, 40, 1280, 10),
    (2, 30, 2560, 80),
    (1, 20, 2560, 640),
]


def _stream_cases():
    for (B, T, D, H), eb, align in itertools.product(STREAM, (2, 4), (4, 8, 16)):
        if (D * eb) % align == 0 and kb.stream_layout_ok(D, H, eb, align):
            yield B, T, D, H, eb, align


STREAM_CASES = list(_stream_cases())


@pytest.mark.parametrize("B,T,D,H,eb,align", STREAM_CASES)
@pytest.mark.parametrize("W", [1, 3, 4, 8])
@pytest.mark.parametrize("static", [False, True])
def test_stream_fwd_bounds(B, T, D, H, eb, align, W, static):
    acc, _ = kb.stream_fwd(B, T, D, W, H, eb, align, static=static, seg=T % 2 == 1, cbias=W % 2 == 0)
    G = D // H
    wext = (1, 1, G * W) if static else (B, T, G * W)
    acc.check({"x": (B, T, D), "y": (B, T, D), "w": wext, "seg": (B, T, 1), "cbias": (1, 1, D)})
    _full(acc, "y", B, T, D)


@pytest.mark.parametrize("B,T,D,H,eb,align", STREAM_CASES)
@pytest.mark.parametrize("W", [1, 3, 4, 8])
@pytest.mark.parametrize("static", [False, True])
@pytest.mark.parametrize("want", ["dx", "dw", "both"])
def test_stream_bwd_bounds(B, T, D, H, eb, align, W, static, want):
    want_dx, want_dw = want in ("dx", "both"), want in ("dw", "both")
    cb = T % 2 == 0
    acc, pl = kb.stream_bwd(B, T, D, W, H, eb, align, static=static, want_dx=want_dx, want_dw=want_dw,
                            seg=W % 2 == 1, cb=cb)
    G = D // H
    nch = B * pl["nTw"]
    wext = (1, 1, G * W) if static else (B, T, G * W)
    acc.check({"x": (B, T, D), "dy": (B, T, D), "dx": (B, T, D), "w": wext, "dw": (B, T, G * W),
               "seg": (B, T, 1), "cb_partial": (1, nch, D), "partial": (1, nch, G * W)})
    if want_dx:
        _full(acc, "dx", B, T, D)
    if want_dw:
        _full(acc, "partial" if static else "dw", *((1, nch, G * W) if static else (B, T, G * W)))
    if cb:
        _full(acc, "cb_partial", 1, nch, D)


def test_stream_cases_cover_odd_and_mixed_groups():
    """The sweep reaches groups of 3, 5 and 63 lanes (suffix scan, idle lanes past
    lanes_in_use), one 16-bit channel per lane, and 6 or 10 channels per lane for 16-bit
    groups of 3 * 2^k and 5 * 2^k channels (power-of-two lanes per group)."""
    plans = [kb.plan_stream(B, T, D, 4, H, eb, al, True, False) for B, T, D, H, eb, al in STREAM_CASES]
    assert {3, 5, 63} <= {p["lpg"] for p in plans}
    assert {1, 6, 10} <= {p["vec"] for p in plans}
    assert any(p["vec"] == 6 and p["lpg"] > 1 for p in plans) and any(p["vec"] == 10 and p["lpg"] > 1 for p in plans)


def test_stream_group_check_catches_a_straddling_group():
    """A wave slice of all 64 lanes with groups of 7 lanes would split a group between two
    waves: the group check must see it."""
    B, T, D, H, eb, align = 1, 8, 196, 7, 2, 4
    pl = kb.plan_stream(B, T, D, 4, H, eb, align, True, False)
    assert pl["lpg"] == 7 and pl["lpw"] == 63
    bad = dict(pl, lpw=64, nDw=(D + 63) // 64)
    lane = np.arange(64)
    c0 = lane * bad["vec"] + 64 * bad["vec"]  # the second slice
    valid = c0 < D
    with pytest.raises(AssertionError):
        kb._check_groups(c0, valid, bad, H)


# ---------------------------------------------------------------------------------------
# column sums of dy (the low-rank form's convolution-bias gradient)
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("B,T,D", [(1, 1, 2), (2, 5, 200), (1, 300, 1024), (8, 4096, 2048), (3, 3000, 192),
                                   (1000, 37, 64)])
@pytest.mark.parametrize("eb", [2, 4])
def test_column_partials_bounds(B, T, D, eb):
    acc, nchunk = kb.column_partials(B, T, D, eb)
    acc.check({"dy": (B, T, D), "part": (1, B * nchunk, D)})
    _full(acc, "dy", B, T, D)
    _full(acc, "part", 1, B * nchunk, D)


# ---------------------------------------------------------------------------------------
# 32-bit offsets at the largest row strides the ABI admits
# ---------------------------------------------------------------------------------------
BIG = kb.MAX_ROW_STRIDE - 64  # a multiple of 16 bytes for every dtype


def test_largest_admitted_strides_keep_32bit_offsets():
    kb.dz_dma(1, 64, 64, 4, 1, 128, BIG, BIG, BIG).check({"x": (1, 64, 64), "dy": (1, 64, 64),
                                                          "U": (1, 128, 256), "dz": (1, 64, 128)})
    acc, nTr = kb.lowrank_bwd_general(1, 70, 32, 4, 1, 128, 2, True, xs1=BIG, zs1=BIG, dys1=BIG, os1=BIG)
    acc.check({"x": (1, 70, 32), "dy": (1, 70, 32), "z": (1, 70, 128), "U": (1, 128, 128), "bias": (1, 1, 128),
               "dx": (1, 70, 32), "part_dU": (1, nTr * 128, 128), "part_db": (1, nTr, 128)})


def test_strides_past_the_bound_would_overflow():
    """The reason for the ABI's bound: a few times past it the kernels' 32-bit offsets wrap
    (U's 128 rank rows at twice the bound, a 64-token step's rows at four times)."""
    over = 4 * kb.MAX_ROW_STRIDE
    with pytest.raises(AssertionError, match="32-bit offset"):
        kb.dz_dma(1, 64, 64, 4, 1, 128, 64, 64, over).check({})
    with pytest.raises(AssertionError, match="32-bit offset"):
        kb.lowrank_bwd_general(1, 70, 32, 4, 1, 128, 2, True, xs1=over)[0].check({})


def test_emulation_detects_a_misplaced_row():
    """A planted off-by-one (the fast forward's last partial step reading row T instead of
    T - 1) is reported."""
    orig = kb.step_rows
    try:
        kb.step_rows = lambda t0, rl, T: t0 + rl
        acc = kb.lowrank_fwd_fast(1, 65, 64, 4, 1, 64, 16, 64, 64, 64)
        with pytest.raises(AssertionError, match="x: access"):
            acc.check({"x": (1, 65, 64), "z": (1, 65, 64), "U": (1, 64, 256), "bias": (1, 1, 256),
                       "y": (1, 65, 64)})
    finally:
        kb.step_rows = orig
