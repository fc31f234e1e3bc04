"""Host emulation of the global-memory accesses of the DMA-staged and chunk-loop kernels.

Each emulator restates, for every workgroup, wave, lane and pipeline step of one launch,
the index arithmetic of one kernel's loads and stores (the expressions of the kernel
source, with its variable names) and records every access as
(tensor, sequence b, row t, first element of the row, width in elements). `Accesses.check`
then asserts that each access lies inside its tensor's logical extent [B, T, C], so that a
strided view's gaps and the rows of other sequences count as outside too. Pieces that a
kernel reads from a static zero word, and stores that the hardware drops (buffer stores
past the resource's extent, whose own bound is checked), are counted, not recorded.
Offsets that a kernel forms in 32-bit arithmetic are recorded with `int32` and checked to
stay in range (below 2^31, or 2^32 where the kernel takes them as unsigned).

Kernels (dynamic_short_convolution_amd/csrc):
  k_gemm_conv            projection + convolution (per-token or low-rank filters)
  k_lowrank_fwd_fast     low-rank forward, LDS DMA ring
  k_lowrank_bwd_fast     fused low-rank backward: dx role and filter-gradient role
  k_lowrank_dz_dma       dz over whole 64-token blocks, LDS DMA stages
  k_lowrank_fwd          general low-rank forward (16-token tiles, register staging)
  k_lowrank_bwd          general low-rank backward (64-token steps; FAST and masked
                         loads, including the surplus threads' "safe" chunk)
  k_stream_fwd/_bwd      materialised and static filters: a wave sweeps a run of tokens
                         over lpw lanes of VEC channels (head-wise groups of H / VEC lanes)
  k_column_partials      column sums of dy (the low-rank form's convolution-bias gradient)
"""
from __future__ import annotations

import math
from collections import defaultdict

import numpy as np

STEP = 64  # tokens per pipeline step (fast kernels, general backward, dz blocks)
TT = 16  # tokens per tile of the general forward


def lr_halo(W):
    """Rows before a range that the general low-rank kernels stage (lr_halo)."""
    return 4 if W <= 5 else W - 1


I32 = 1 << 31
U32 = 1 << 32
MAX_ROW_STRIDE = 1 << 24  # the ABI's bound on the low-rank form's row strides


def xcd_logical_block(bid, n):
    """The kernels' XCD-grouping map of workgroup ids (a bijection of 0 .. n-1)."""
    bid = np.asarray(bid)
    q, r = n // 8, n % 8
    x = bid % 8
    return x * q + np.minimum(x, r) + bid // 8


class Accesses:
    def __init__(self):
        self.spans = defaultdict(list)
        self.zero = 0  # pieces read from a static zero word
        self.dropped = 0  # 16-byte stores past a buffer resource's extent
        self.i32 = []  # (what, max, min, limit)

    def add(self, name, b, t, c0, width):
        b, t, c0, width = np.broadcast_arrays(np.asarray(b), np.asarray(t), np.asarray(c0), np.asarray(width))
        if b.size:
            self.spans[name].append((b.ravel().astype(np.int64), t.ravel().astype(np.int64),
                                     c0.ravel().astype(np.int64), width.ravel().astype(np.int64)))

    def int32(self, what, values, limit=I32):
        v = np.asarray(values, dtype=np.int64)
        if v.size:
            self.i32.append((what, int(v.max()), int(v.min()), limit))

    def check(self, extents):
        """extents: tensor name -> (B, T, C). Raises AssertionError naming the first bad access."""
        for what, hi, lo, limit in self.i32:
            assert lo >= 0 and hi < limit, f"32-bit offset {what} reaches {lo} .. {hi} (limit {limit})"
        for name, lst in self.spans.items():
            B, T, C = extents[name]
            for b, t, c0, w in lst:
                bad = (b < 0) | (b >= B) | (t < 0) | (t >= T) | (c0 < 0) | (w < 1) | (c0 + w > C)
                if np.any(bad):
                    i = int(np.argmax(bad))
                    raise AssertionError(f"{name}: access b={b[i]} t={t[i]} elements {c0[i]}..{c0[i] + w[i] - 1}"
                                         f" outside [B={B}, T={T}, C={C}]")
        return True

    def cover(self, name, B, T, C):
        """Boolean [B, T, C] map of the elements a tensor's accesses touch."""
        m = np.zeros((B, T, C), dtype=bool)
        for b, t, c0, w in self.spans.get(name, []):
            for wv in np.unique(w):
                sel = w == wv
                for k in range(int(wv)):
                    m[b[sel], t[sel], c0[sel] + k] = True
        return m


def _log2(h):
    assert h >= 1 and h & (h - 1) == 0
    return h.bit_length() - 1


# ---------------------------------------------------------------------------------------
# k_gemm_conv: 256 computed rows (16 of them the halo of the next 240) x 128 columns per
# workgroup, K in steps of 64, 8 waves (4 along the rows, 2 along the columns)
# ---------------------------------------------------------------------------------------

def gemm_conv(B, T, K, N, W, H, R=0, lowrank=False, zvec=True, uvec=True, has_bias=True):
    GBM, GHALO, GBN, GKT, GNT = 256, 16, 128, 64, 512
    GBMO = GBM - GHALO
    M = B * T
    nTm, nTn = (M + GBMO - 1) // GBMO, N // GBN
    nk = K // GKT
    CPR = GKT // 8
    AI, BI = GBM * GKT * 2 // 16 // GNT, GBN * GKT * 2 // 16 // GNT
    hsh = _log2(H)
    acc = Accesses()
    nblk = nTm * nTn
    lb = xcd_logical_block(np.arange(nblk), nblk)
    per_group = 8 * nTn
    grp, rem = lb // per_group, lb % per_group
    rows_in_grp = np.minimum(8, nTm - 8 * grp)
    tm = 8 * grp + rem % rows_in_grp
    tn = rem // rows_in_grp
    assert len(set(zip(tm.tolist(), tn.tolist()))) == nblk, "tile map is not a bijection"
    assert tm.max() < nTm and tn.max() < nTn
    m0 = tm * GBMO - GHALO
    n0 = tn * GBN
    swz = (lambda r: r & 7) if GKT == 64 else (lambda r: (r >> 2) & 3)
    for wv in range(8):
        for i in range(AI):
            pidx = (wv + 8 * i) * 64 + np.arange(64)
            row, c = pidx // CPR, (pidx % CPR) ^ swz(pidx // CPR)
            m = np.clip(m0[:, None] + row[None, :], 0, M - 1)
            for s in range(nk):
                acc.add("A", m // T, m % T, 8 * c[None, :] + s * GKT, 8)
        for i in range(BI):
            pidx = (wv + 8 * i) * 64 + np.arange(64)
            row, c = pidx // CPR, (pidx % CPR) ^ swz(pidx // CPR)
            for s in range(nk):
                acc.add("Wp", 0, n0[:, None] + row[None, :], 8 * c[None, :] + s * GKT, 8)
    # epilogue: tile row r is token m0 + r (clamped into 0 .. M-1 for loads)
    r = np.arange(GBM)
    m = m0[:, None] + r[None, :]
    mc = np.clip(m, 0, M - 1)
    out = (r[None, :] >= GHALO) & (m < M)
    acc.add("y", (mc // T)[out], (mc % T)[out], np.broadcast_to(n0[:, None], m.shape)[out], GBN)
    bb, tt = (mc // T)[:, :, None], (mc % T)[:, :, None]
    col = n0[:, None, None] + np.arange(GBN)[None, None, :]
    if not lowrank:
        acc.add("w", bb, tt, (col >> hsh) * W, W)
        return acc
    KS = (R + 31) // 32
    # z fragments of every tile row: ranks 32 ks + 8 q (+ e) below R
    ranks = np.arange(32 * KS)
    if zvec:
        acc.add("z", bb, tt, ranks[(ranks % 8 == 0) & (ranks < R)][None, None, :], 8)
    else:
        acc.add("z", bb, tt, ranks[ranks < R][None, None, :], 1)
    # U: the tile's columns (groups G0 .. G0 + 128/H - 1, all taps), rank rows below R
    G0 = n0 // H
    ucols = (GBN >> hsh) * W
    assert ucols % 8 == 0
    rr = np.arange(R)
    if uvec:
        ch = np.arange(ucols // 8)
        acc.add("U", 0, rr[None, :, None], (G0 * W)[:, None, None] + 8 * ch[None, None, :], 8)
    else:
        acc.add("U", 0, rr[None, :, None], (G0 * W)[:, None, None] + np.arange(ucols)[None, None, :], 1)
    if has_bias:
        acc.add("bias", 0, 0, (col[:, 0, :] >> hsh) * W, W)
    return acc


# ---------------------------------------------------------------------------------------
# fast low-rank kernels (64 channels per workgroup, 64-token steps staged by LDS DMA)
# ---------------------------------------------------------------------------------------

def rot_quarter(r):
    return r >> 2


def rot_double(r):
    return 2 * r


def rot_fused(r):
    return 2 * r + (r >> 2)


def z_pieces(ZB, KS, R, rot):
    """(row, first element, valid) of every z piece of a stage (piece idx = (wv + 4 i) 64 + lane)."""
    ZROW = 16 * 4 * KS
    ZCPR = ZROW // 16
    idx = np.arange(STEP * ZROW // ZB)
    o = idx * ZB
    row, ob = o // ZROW, o % ZROW
    c = ((ob // 16 - rot(row)) % ZCPR + ZCPR) % ZCPR
    gb = 16 * c + (ob & 15)
    return row, gb // 2, gb // 2 < R


def step_rows(t0, rl, T):
    """Row that staged row rl of the step at t0 reads: rows past T - 1 read row T - 1."""
    if t0 + STEP <= T:
        return t0 + rl
    return np.minimum(t0 + rl, T - 1)


def _x_chunks(rot):
    """(row, logical chunk) of the 512 x (or dy) pieces of a step: 8 chunks of a 64-channel row."""
    idx = np.arange(STEP * 8)
    rl, pc = idx // 8, idx % 8
    return rl, (pc - rot(rl)) & 7


def _seg_loads(acc, b, t0, T, ih=4):
    sc = np.arange((STEP + ih) // 4)  # id chunk sc: tokens t0 - ih + 4 sc .. + 3, clamped into 0 .. T - 4
    tk = np.minimum(np.maximum(t0 - ih + 4 * sc, 0), T - 4)
    acc.add("seg", b, tk, 0, 1)
    acc.add("seg", b, tk + 3, 0, 1)


def _fast_generation_operands(acc, c_base, H, W, R, KS, has_bias):
    """U^T rows and bias of the 64 channels: rank rows clamped to R - 1, taps (0..3, and
    4..7 when W > 4) clamped to W - 1; U stands in for a missing bias (element 0 .. W - 1)."""
    hsh = _log2(H)
    ch = c_base + np.arange(64)
    r = np.minimum(np.arange(32 * KS), R - 1)
    acc.add("U", 0, r[:, None], ((ch >> hsh) * W)[None, :], W)
    if has_bias:
        acc.add("bias", 0, 0, (ch >> hsh) * W, W)
    else:
        acc.add("U", 0, 0, 0, W)


def _fast_offsets(acc, what, stride):
    # (rl * int(stride) + 8 c) as int, then times 2 as unsigned; rl < 64
    acc.int32(what + " (elements, int)", 63 * stride + 56)
    acc.int32(what + " (bytes, unsigned)", (63 * stride + 56) * 2 + 16, U32)


def plan_fwd_fast(B, T, D, KS):
    lds = 3 * 8192 + 2 * STEP * 64 * KS + 2 * 8192 + 3 * 320  # with the id stages
    resident = min(160 * 1024 // lds, 2)
    nCs = D // 64
    per_seq = (256 * resident + B * nCs - 1) // (B * nCs)
    per_seq = max(1, min(per_seq, (T + STEP - 1) // STEP))
    L = (T + per_seq - 1) // per_seq
    L = (L + STEP - 1) // STEP * STEP
    return nCs, L, (T + L - 1) // L


def fast_width_ok(W, KS):
    return 1 <= W <= 4 or (W == 5 and KS <= 2)


def fwd_fast_width_ok(W, KS):
    """The forward reaches two row groups back: up to eight taps."""
    return 1 <= W <= 4 or (W <= 8 and KS <= 2)


def fast_fwd_ok(T, D, W, H, R, xs1, zs1, os1):
    KS = (R + 31) // 32
    return (KS in (1, 2, 4) and R % 2 == 0 and fwd_fast_width_ok(W, KS) and H in (1, 2, 4, 8, 16) and D % 64 == 0
            and (T + STEP) * os1 * 2 < I32 and STEP * xs1 < (1 << 30) and STEP * zs1 < (1 << 30))


def lowrank_fwd_fast(B, T, D, W, H, R, ZB, xs1, zs1, os1, seg=False, has_bias=True):
    assert fast_fwd_ok(T, D, W, H, R, xs1, zs1, os1) and (ZB == 4 or R % 8 == 0)
    KS = (R + 31) // 32
    nCs, L, nTr = plan_fwd_fast(B, T, D, KS)
    acc = Accesses()
    HR = W - 1
    XD = 1  # x and z are fetched one step ahead
    zrow, zel, zval = z_pieces(ZB, KS, R, rot_quarter)
    rl, c = _x_chunks(rot_quarter)
    _fast_offsets(acc, "x piece", xs1)
    _fast_offsets(acc, "z piece", zs1)
    nblk = B * nTr * nCs
    assert sorted(xcd_logical_block(np.arange(nblk), nblk).tolist()) == list(range(nblk))
    for lb in range(nblk):
        cs, tr, b = lb % nCs, (lb // nCs) % nTr, lb // (nCs * nTr)
        c_base, t_first = cs * 64, tr * L
        t_end = min(T, t_first + L)
        nsteps = (t_end - t_first + STEP - 1) // STEP
        for s in range(nsteps + XD):  # the prologue's step 0 and, at step s, step s + 1
            t0 = t_first + s * STEP
            acc.add("x", b, step_rows(t0, rl, T), c_base + 8 * c, 8)
            acc.add("z", b, step_rows(t0, zrow[zval], T), zel[zval], ZB // 2)
            acc.zero += int((~zval).sum())
            if seg:
                _seg_loads(acc, b, t0, T, ih=8 if W > 5 else 4)
        if HR > 0 and t_first > 0:
            acc.add("x", b, t_first - HR + np.arange(HR)[:, None], c_base + 8 * np.arange(8)[None, :], 8)
        _fast_generation_operands(acc, c_base, H, W, R, KS, has_bias)
        # y: 16-byte pieces of rows t0 .. t0 + 63 through a buffer resource whose extent ends
        # with row T - 1 (32-bit byte offsets ygo + t0 * ystep)
        for s in range(nsteps):
            t = t_first + s * STEP + np.arange(STEP)
            keep = t < T
            acc.add("y", b, t[keep][:, None], c_base + 8 * np.arange(8)[None, :], 8)
            acc.dropped += int((~keep).sum()) * 8
            acc.int32("y store offset", (t * os1 + c_base + 56) * 2)
    acc.int32("y buffer extent", ((T - 1) * os1 + D) * 2)
    return acc


def plan_lowrank_bwd(B, T, D, W, H, R, lean):
    """Token ranges of the backward (the lean plan where the fast kernels can serve it)."""
    KS = (R + 31) // 32
    WP = 8 if W > 4 else 4
    DC = 4 * 2 * 16 // WP
    nCs = (D + DC - 1) // DC
    target = 512 if lean else 2048
    slices = D // 64 if lean else nCs
    per_seq = (target + B * slices - 1) // (B * slices)
    per_seq = max(1, min(per_seq, (T + TT - 1) // TT))
    L = (T + per_seq - 1) // per_seq
    L = (L + STEP - 1) // STEP * STEP
    return nCs, L, (T + L - 1) // L, DC, KS


def fast_bwd_ok(T, D, W, H, R, xs1, zs1, dys1, os1):
    KS = (R + 31) // 32
    return (KS in (1, 2, 4) and R % 2 == 0 and fast_width_ok(W, KS) and H in (1, 2, 4, 8, 16) and D % 64 == 0
            and (T + STEP) * os1 * 2 < I32 and STEP * dys1 < (1 << 30) and STEP * zs1 < (1 << 30)
            and STEP * xs1 < (1 << 30))


def lowrank_bwd_fused(B, T, D, W, H, R, ZB, xs1, zs1, dys1, os1, seg=False, has_bias=True, want_db=True):
    """The fast backward: up to 64 ranks k_lowrank_bwd_fast (both roles, the gradient role
    staging steps 0 .. nsteps for both); at 128 ranks k_lowrank_bwd_dx_fast over its own
    token ranges (about 512 workgroups; it stages dy and z itself, steps 0 .. nsteps) and
    k_lowrank_bwd_gdu_fast over the planned ranges (steps 0 .. nsteps - 1)."""
    assert fast_bwd_ok(T, D, W, H, R, xs1, zs1, dys1, os1) and (ZB == 4 or R % 8 == 0)
    _, L, nTr, _, KS = plan_lowrank_bwd(B, T, D, W, H, R, lean=True)
    split = KS == 4
    slices = D // 64
    acc = Accesses()
    HR = W - 1
    hsh = _log2(H)
    zrow, zel, zval = z_pieces(ZB, KS, R, rot_fused)
    rl, c = _x_chunks(rot_fused)
    for what, st in (("x piece", xs1), ("dy piece", dys1), ("z piece", zs1)):
        _fast_offsets(acc, what, st)
    for lb in range(B * nTr * slices):
        cs, tr, b = lb % slices, (lb // slices) % nTr, lb // (slices * nTr)
        c_base, t_first = cs * 64, tr * L
        t_end = min(T, t_first + L)
        nsteps = (t_end - t_first + STEP - 1) // STEP
        # filter-gradient role (waves 4..7): stages of steps 0 .. nsteps (dx's tail step too);
        # the standalone gradient kernel stops before the tail step
        for s in range(nsteps + (0 if split else 1)):
            t0 = t_first + s * STEP
            rows = step_rows(t0, rl, T)
            acc.add("x", b, rows, c_base + 8 * c, 8)
            acc.add("dy", b, rows, c_base + 8 * c, 8)
            acc.add("z", b, step_rows(t0, zrow[zval], T), zel[zval], ZB // 2)
            acc.zero += int((~zval).sum())
            if seg:
                _seg_loads(acc, b, t0, T)
        if HR > 0 and t_first > 0:
            acc.add("x", b, t_first - HR + np.arange(HR)[:, None], c_base + 8 * np.arange(8)[None, :], 8)
        rng = b * nTr + tr
        cols = (64 >> hsh) * W
        acc.add("part_dU", 0, rng * R + np.arange(R)[:, None], (c_base >> hsh) * W + np.arange(0, cols, 4)[None, :], 4)
        if want_db:
            acc.add("part_db", 0, rng, (((c_base + np.arange(64)) >> hsh) * W)[:, None] + np.arange(W)[None, :], 1)
        if not split:
            _dx_role(acc, b, c_base, t_first, t_end, T, D, W, H, R, KS, os1, has_bias)
    if split:
        # the standalone dx kernel: its own ranges, dy and z staged for steps 0 .. nsteps
        nCs = D // 64
        per_seq = max(1, min((512 + B * nCs - 1) // (B * nCs), (T + STEP - 1) // STEP))
        Ld = (T + per_seq - 1) // per_seq
        Ld = (Ld + STEP - 1) // STEP * STEP
        nTd = (T + Ld - 1) // Ld
        zrow_q, zel_q, zval_q = z_pieces(ZB, KS, R, rot_quarter)
        rlq, cq = _x_chunks(rot_quarter)
        for lb in range(B * nTd * nCs):
            cs, tr, b = lb % nCs, (lb // nCs) % nTd, lb // (nCs * nTd)
            c_base, t_first = cs * 64, tr * Ld
            t_end = min(T, t_first + Ld)
            nsteps = (t_end - t_first + STEP - 1) // STEP
            for s in range(nsteps + 1):
                t0 = t_first + s * STEP
                acc.add("dy", b, step_rows(t0, rlq, T), c_base + 8 * cq, 8)
                acc.add("z", b, step_rows(t0, zrow_q[zval_q], T), zel_q[zval_q], ZB // 2)
                acc.zero += int((~zval_q).sum())
                if seg:
                    _seg_loads(acc, b, t0, T)
            _dx_role(acc, b, c_base, t_first, t_end, T, D, W, H, R, KS, os1, has_bias)
    acc.int32("dx buffer extent", ((T - 1) * os1 + D) * 2)
    return acc, nTr


def _dx_role(acc, b, c_base, t_first, t_end, T, D, W, H, R, KS, os1, has_bias):
    """dx stores of one (sequence, token range, 64-channel slice): tile rows r of steps
    0 .. nsteps are tokens t0 - DXH + r (DXH = 3 rows of delay, 4 at W = 5); the first step
    keeps rows >= DXH, the tail rows < DXH, the rest are pushed out (offset 0x80000000,
    past every extent)."""
    nsteps = (t_end - t_first + STEP - 1) // STEP
    _fast_generation_operands(acc, c_base, H, W, R, KS, has_bias)
    DXH = 4 if W > 4 else 3
    for s in range(nsteps + 1):
        t0 = t_first + s * STEP
        r = np.arange(STEP)
        keep = ((s > 0) | (r >= DXH)) & ((s < nsteps) | (r < DXH))
        t = t0 - DXH + r[keep]
        inb = t < T
        acc.add("dx", b, t[inb][:, None], c_base + 8 * np.arange(8)[None, :], 8)
        acc.dropped += int((~inb).sum()) * 8
        acc.int32("dx store offset", (t * os1 + c_base + 56) * 2)


# ---------------------------------------------------------------------------------------
# k_lowrank_dz_dma: one workgroup per 64-token block inside T, chunks of CH filter groups
# ---------------------------------------------------------------------------------------

DZ_STAGES = 2  # the DMA dz kernel's ring (LRDZ_NST)


def dz_dma_shape(W, KS, HG, stages=DZ_STAGES):
    GL = 8 if HG <= 4 else 32 // HG
    CH = 4 * GL
    CHC, UC = CH * HG, CH * W
    RP = 32 * KS
    UCPR, XCPR = UC // 8, CHC // 8
    XR = STEP + lr_halo(W)
    UCH, XCH, DCH = RP * UCPR, XR * XCPR, STEP * XCPR
    ni = lambda n: (n + 63) // 64  # noqa: E731
    stage = (ni(UCH) + ni(XCH) + ni(DCH)) * 64 * 16
    place_ok = lambda cpr: cpr % 8 == 4 or cpr in (8, 16, 24, 32)  # noqa: E731 (lds_place_ok)
    ok = (GL * W) % 8 == 0 and place_ok(UCPR) and place_ok(XCPR) and stages * stage <= 150 * 1024
    return dict(GL=GL, CH=CH, CHC=CHC, UC=UC, UCPR=UCPR, XCPR=XCPR, XR=XR, UCH=UCH, XCH=XCH, DCH=DCH, ok=ok)


def dz_dma(B, T, D, W, H, R, xs1, dys1, ldu):
    KS = (R + 31) // 32
    S = dz_dma_shape(W, KS, H)
    assert S["ok"] and D % S["CHC"] == 0
    HALO = lr_halo(W)
    nchunk = D // S["CHC"]
    acc = Accesses()
    pidx = np.arange(S["UCH"])
    r, pc = pidx // S["UCPR"], pidx % S["UCPR"]
    uz = r >= R  # a padding rank: the zero word, never a row past U
    acc.int32("U offset r*int(ldu) + 8c", r[~uz] * ldu + 8 * (S["UCPR"] - 1))
    acc.int32("x offset row*int(xs1) + 8c", (S["XR"] - 1) * xs1 + 8 * (S["XCPR"] - 1))
    acc.int32("dy offset row*int(dys1) + 8c", (STEP - 1) * dys1 + 8 * (S["XCPR"] - 1))
    xp = np.arange(S["XCH"])
    xrow, xc = xp // S["XCPR"], xp % S["XCPR"]
    dp = np.arange(S["DCH"])
    drow, dc = dp // S["XCPR"], dp % S["XCPR"]
    for b in range(B):
        for tb in range(T // STEP):
            tb0 = tb * STEP
            # issue(ci) for ci = 0 .. nchunk - 1 + (stages - 1), clamped to the last chunk;
            # the chunk positions within a row are a permutation of 0 .. CPR - 1
            for ci in sorted({min(i, nchunk - 1) for i in range(nchunk + DZ_STAGES - 1)}):
                acc.add("U", 0, r[~uz], ci * S["UC"] + 8 * pc[~uz], 8)
                acc.zero += int(uz.sum())
                xr = np.maximum(xrow, HALO - tb0)  # rows before token 0 read token 0
                acc.add("x", b, tb0 - HALO + xr, ci * S["CHC"] + 8 * xc, 8)
                acc.add("dy", b, tb0 + drow, ci * S["CHC"] + 8 * dc, 8)
            acc.add("dz", b, tb0 + np.arange(STEP)[:, None], np.arange(R)[None, :], 1)
    return acc


# ---------------------------------------------------------------------------------------
# fixed-order reduce of float32 partials: k_reduce_partials (one column per thread, 8
# groups of chunks) and k_reduce_partials4 / 4x2 (4 columns per thread, 16-byte loads,
# G = 8 groups, or 32 from 64 chunks on)
# ---------------------------------------------------------------------------------------

def reduce_partials(nchunk, n, vec4):
    acc = Accesses()
    tid = np.arange(256)
    if vec4:
        assert n % 4 == 0
        G = 32 if nchunk >= 64 else 8
        C = 256 // G
        col, grp = tid % C, tid // C
        for blk in range((n + 4 * C - 1) // (4 * C)):
            i = blk * 4 * C + 4 * col
            for g, ii in zip(grp[i < n], i[i < n]):
                acc.add("part", 0, np.arange(g, nchunk, G), ii, 4)
            st = (grp == 0) & (i < n)
            acc.add("out", 0, 0, i[st], 4)
    else:
        col, grp = tid % 32, tid // 32
        for blk in range((n + 31) // 32):
            i = blk * 32 + col
            for g, ii in zip(grp[i < n], i[i < n]):
                acc.add("part", 0, np.arange(g, nchunk, 8), ii, 1)
            st = (grp == 0) & (i < n)
            acc.add("out", 0, 0, i[st], 1)
    return acc


# ---------------------------------------------------------------------------------------
# decoding: k_cache_fill, k_decode_step, k_lowrank_decode_step
# ---------------------------------------------------------------------------------------

def cache_fill(B, t, D, W, seg=False):
    """One thread per (sequence, cache slot, channel): slot m holds token s, the one of
    t - (W-1) .. t-1 with s = m (mod W-1); tokens before 0 (and, packed, of another
    document than token t-1) store zero without a load."""
    S = W - 1
    acc = Accesses()
    if S == 0:
        return acc
    idx = np.arange(B * S * D)
    d, m, b = idx % D, (idx // D) % S, idx // (D * S)
    s0 = t - S
    s_ = s0 + ((m - s0) % S + S) % S
    keep = s_ >= 0
    if seg:
        acc.add("seg", b[keep], s_[keep], 0, 1)
        acc.add("seg", b[keep], t - 1, 0, 1)
    acc.add("x", b[keep], s_[keep], d[keep], 1)
    acc.add("cache", b, m, d, 1)
    return acc


def decode_step(B, D, W, H, t, static=False, cbias=False):
    """One thread per (sequence, channel): the W taps of its group, x_t, the W-1 cached
    inputs and the optional bias; stores y and the cache slot of token t."""
    S = W - 1
    acc = Accesses()
    idx = np.arange(B * D)
    d, b = idx % D, idx // D
    wb = 0 if static else b
    acc.add("w", np.broadcast_to(np.asarray(wb), d.shape), 0, (d // H) * W, W)
    acc.add("x", b, 0, d, 1)
    if cbias:
        acc.add("cbias", 0, 0, d, 1)
    for kk in range(1, W):
        acc.add("cache", b, ((t - kk) % S + S) % S, d, 1)
    if S > 0:
        acc.add("cache", b, t % S, d, 1)
    acc.add("y", b, 0, d, 1)
    return acc


def lowrank_decode_step(B, D, W, H, R, t, vec, has_bias=True, cbias=False):
    """Workgroups of 64 lanes over (16 channels, 16 sequences): lane (l, q) generates the
    filters of channel c0 + l (clamped to D-1) for sequences b0 + 4q + i (clamped to B-1),
    from z rows b0 + l (clamped) and U rows r < 32 NK (clamped to R-1); VEC: 16-byte z
    pieces at rank min(32 s + 8 q, R - 8) (R % 8 == 0). Stores only for c0 + l < D and
    sequences below B. Returns the accesses and the element offsets of the vector loads."""
    S = W - 1
    NK = (R + 31) // 32
    acc = Accesses()
    vec_offsets = []
    for by in range((B + 15) // 16):
        for bx in range((D + 15) // 16):
            b0, c0 = by * 16, bx * 16
            for lane in range(64):
                l, q = lane & 15, lane >> 4
                ca = min(c0 + l, D - 1)
                bs = [min(b0 + 4 * q + i, B - 1) for i in range(4)]
                acc.add("x", bs, 0, ca, 1)
                for kk in range(1, W):
                    acc.add("cache", bs, ((t - kk) % S + S) % S, ca, 1)
                zb = min(b0 + l, B - 1)
                for s_ in range(NK):
                    k0 = 32 * s_ + 8 * q
                    if vec:
                        acc.add("z", zb, 0, min(k0, R - 8), 8)
                        vec_offsets.append(("z", zb, min(k0, R - 8)))
                    else:
                        acc.add("z", zb, 0, [min(k0 + e, R - 1) for e in range(8)], 1)
                    for e in range(8):
                        r = min(32 * s_ + 8 * q + e, R - 1)
                        acc.add("U", 0, r, (ca // H) * W, W)
                        if vec and W in (2, 4):
                            vec_offsets.append(("U", r, (ca // H) * W))
                if has_bias:
                    acc.add("bias", 0, 0, (ca // H) * W, W)
                if cbias:
                    acc.add("cbias", 0, 0, ca, 1)
                if c0 + l < D:
                    for i in range(4):
                        b = b0 + 4 * q + i
                        if b >= B:
                            break
                        acc.add("y", b, 0, ca, 1)
                        if S > 0:
                            acc.add("cache", b, t % S, ca, 1)
    return acc, vec_offsets


# ---------------------------------------------------------------------------------------
# k_lowrank_dz: register-staged dz (any storage type, ragged token blocks and D, any H)
# ---------------------------------------------------------------------------------------
DZ_CHUNK = 32  # channels per chunk (kLowrankDzChunk)


def lowrank_dz_register(B, T, D, W, H, R, eb, xs1, dys1, ldu, tbb0=0, nTbL=None, seg=False):
    """One workgroup per (sequence, 64-token block tbb0 ..): every chunk of CH channels stages
    the chunk's U columns (all ranks; head-wise: each channel's group columns, element by
    element), the x rows from HALO tokens before the block and the dy rows, each 16-byte
    piece clipped to the chunk's end in D and to rows 0 .. T-1; prefetches run two chunks
    past the last one and load nothing there."""
    KS = (R + 31) // 32
    CE = 16 // eb
    CH, TB, HALO, RP = DZ_CHUNK, STEP, lr_halo(W), 32 * KS
    UC = CH * W
    XR = TB + HALO
    UCH, XCH, DCH = RP * UC // CE, XR * CH // CE, TB * CH // CE
    US, AS = (UCH + 255) // 256, (XCH + DCH + 255) // 256
    nblk = (T + TB - 1) // TB
    nTbL = nblk - tbb0 if nTbL is None else nTbL
    nchunk = (D + CH - 1) // CH
    acc = Accesses()
    ck = np.arange(US * 256)
    ur, uc = ck // (UC // CE), (ck % (UC // CE)) * CE
    ak = np.arange(AS * 256)
    isx = ak < XCH
    k2 = np.where(isx, ak, ak - XCH)
    arow, ac = k2 // (CH // CE), (k2 % (CH // CE)) * CE
    acc.int32("U offset r*int(ldu) + c", ur[(ck < UCH) & (ur < R)] * ldu + UC)
    acc.int32("x offset row*int(xs1) + c", arow[isx] * xs1 + CH)
    acc.int32("dy offset row*int(dys1) + c", arow[~isx & (k2 < DCH)] * dys1 + CH)
    e = np.arange(CE)
    for b in range(B):
        for tb in range(tbb0, tbb0 + nTbL):
            tb0 = tb * TB
            for c0 in range(0, (nchunk + 2) * CH, CH):
                climit, jlimit = D - c0, (D - c0) * W
                ok = (ck < UCH) & (ur < R) & (uc < jlimit)
                if H == 1:
                    acc.add("U", 0, ur[ok], c0 * W + uc[ok], np.minimum(CE, jlimit - uc[ok]))
                else:
                    # element e reads column c + min(e, limit - 1) of the chunk
                    lim = jlimit - uc[ok]
                    jj = uc[ok][:, None] + np.minimum(e[None, :], lim[:, None] - 1)
                    col = ((c0 + jj // W) // H) * W + jj % W
                    acc.add("U", 0, np.broadcast_to(ur[ok][:, None], col.shape), col, 1)
                t = np.where(isx, tb0 - HALO + arow, tb0 + arow)
                okx = (isx | (k2 < DCH)) & (t >= 0) & (t < T) & (ac < climit)
                w = np.minimum(CE, climit - ac)
                acc.add("x", b, t[okx & isx], c0 + ac[okx & isx], w[okx & isx])
                acc.add("dy", b, t[okx & ~isx], c0 + ac[okx & ~isx], w[okx & ~isx])
            nt = np.arange(TB)
            if seg:
                tt = np.minimum(tb0 + nt, T - 1)
                acc.add("seg", b, tt, 0, 1)
                for k in range(1, W):
                    acc.add("seg", b, (tt - k)[tt - k >= 0], 0, 1)
            t = tb0 + nt
            t = t[t < T]
            acc.add("dz", b, t[:, None], np.arange(R)[None, :], 1)
    return acc


# ---------------------------------------------------------------------------------------
# general low-rank kernels (register-staged 16-byte chunks; any dtype, ragged D)
# ---------------------------------------------------------------------------------------

def _chunk_span(c, limit, CE, vec):
    """Elements that load_chunk reads: the whole chunk when vec and c + CE <= limit, else
    elements c .. min(c + CE, limit) - 1 one by one."""
    c = np.asarray(c)
    return np.where(vec & (c + CE <= limit), CE, np.minimum(CE, limit - c))


def plan_fwd_general(B, T, D, W, R):
    KS = (R + 31) // 32
    MT = 8 if KS <= 2 else 4
    WP = 8 if W > 4 else 4
    DC = 4 * MT * 16 // WP
    nCs = (D + DC - 1) // DC
    per_seq = (1024 + B * nCs - 1) // (B * nCs)
    per_seq = max(1, min(per_seq, (T + TT - 1) // TT))
    L = (T + per_seq - 1) // per_seq
    L = (L + TT - 1) // TT * TT
    return nCs, L, (T + L - 1) // L, DC, KS, MT


def lowrank_fwd_general(B, T, D, W, H, R, eb, act16, z16, seg=False, has_bias=True):
    nCs, L, nTr, DC, KS, MT = plan_fwd_general(B, T, D, W, R)
    CE = 16 // eb
    RP = 32 * KS
    WP = 8 if W > 4 else 4
    CPW = MT * 4 // (WP // 4)
    HALO = lr_halo(W)
    acc = Accesses()
    zck = np.arange(TT * RP // CE)
    zrow, zc = zck // (RP // CE), (zck % (RP // CE)) * CE
    xck = np.arange(TT * DC // CE)
    xrow, xc = xck // (DC // CE), (xck % (DC // CE)) * CE
    hck = np.arange(HALO * DC // CE)
    hrow, hc = hck // (DC // CE), (hck % (DC // CE)) * CE
    for b in range(B):
        for tr in range(nTr):
            t_first = tr * L
            t_end = min(T, t_first + L)
            if t_first >= T:
                continue
            for cs in range(nCs):
                c_base = cs * DC
                lim = D - c_base
                t = t_first - HALO + hrow
                ok = (t >= 0) & (hc < lim)
                acc.add("x", b, t[ok], c_base + hc[ok], _chunk_span(hc[ok], lim, CE, act16))
                for t0 in range(t_first, t_end, TT):
                    tz = t0 + zrow
                    okz = (tz < t_end) & (zc < R)
                    acc.add("z", b, tz[okz], zc[okz], _chunk_span(zc[okz], R, CE, z16))
                    tx = t0 + xrow
                    okx = (tx < t_end) & (xc < lim)
                    acc.add("x", b, tx[okx], c_base + xc[okx], _chunk_span(xc[okx], lim, CE, act16))
                    if seg:
                        ts = t0 + np.arange(TT)
                        acc.add("seg", b, ts[ts < t_end], 0, 1)
                if seg:
                    ts = t_first - HALO + np.arange(HALO)
                    acc.add("seg", b, ts[ts >= 0], 0, 1)
                # y: each lane's run of MT channels, clipped at D
                for wv in range(4):
                    for q in range(4):
                        cg = c_base + wv * CPW + (q // (WP // 4)) * MT
                        if cg < D:
                            acc.add("y", b, np.arange(t_first, t_end), cg, min(MT, D - cg))
                ch = c_base + np.arange(DC)
                ch = ch[ch < D]
                acc.add("U", 0, np.arange(R)[:, None], ((ch // H) * W)[None, :], W)
                if has_bias:
                    acc.add("bias", 0, 0, (ch // H) * W, W)
    return acc


def lowrank_bwd_general(B, T, D, W, H, R, eb, fast, seg=False, has_bias=True, want_db=True, xs1=None, zs1=None,
                        dys1=None, os1=None, lean=False):
    """k_lowrank_bwd over every channel slice it is launched on: with `fast`, the FAST
    instantiation covers the slices inside D (16-byte loads; R % 32 == 0) and the other
    one the rest (masked element loads)."""
    nCs, L, nTr, DC, KS = plan_lowrank_bwd(B, T, D, W, H, R, lean)
    xs1 = D if xs1 is None else xs1
    zs1 = R if zs1 is None else zs1
    dys1 = D if dys1 is None else dys1
    os1 = D if os1 is None else os1
    CE = 16 // eb
    RP = 32 * KS
    S = STEP
    MT = 2
    WP = 8 if W > 4 else 4
    LPC = WP // 4
    CPW = MT * 4 // LPC
    ZCH, XCH = S * RP // CE, S * DC // CE
    NT = 256
    ZS, XS = (ZCH + NT - 1) // NT, (XCH + NT - 1) // NT
    HALO = lr_halo(W)
    HCH = HALO * DC // CE
    assert not fast or R % 32 == 0
    acc = Accesses()
    acc.int32("z row offset row*int(zs1) + c", (S - 1) * zs1 + RP)
    acc.int32("x row offset row*int(xs1) + c", (S - 1) * xs1 + DC)
    acc.int32("dy row offset row*int(dys1) + c", (S - 1) * dys1 + DC)
    acc.int32("dx row offset (sub TT + n - (W-1))*int(os1) + cl", (S - 1) * os1 + D)
    nfull = D // DC if fast else 0
    tid = np.arange(NT)
    safe = lambda name, n: acc.add(name, 0, 0, 0, np.full(int(n), CE))  # noqa: E731
    for b in range(B):
        for tr in range(nTr):
            t_first = tr * L
            t_end = min(T, t_first + L)
            t_need = min(T, t_end + HALO)
            rng = b * nTr + tr
            for cs in range(nCs):
                FAST = cs < nfull
                c_base = cs * DC
                xlimit = D - c_base
                # the HALO rows of x and dy before the range (zeros before t = 0)
                th = tid[tid < 2 * HCH]
                k2 = th % HCH
                isx = th < HCH
                row, c = k2 // (DC // CE), (k2 % (DC // CE)) * CE
                t = t_first - HALO + row
                ok = (t >= 0) & (c < xlimit)
                w = np.full(c.shape, CE) if FAST else np.minimum(CE, xlimit - c)
                acc.add("x", b, t[ok & isx], c_base + c[ok & isx], w[ok & isx])
                acc.add("dy", b, t[ok & ~isx], c_base + c[ok & ~isx], w[ok & ~isx])
                if FAST:
                    safe("x", (~ok & isx).sum())
                    safe("dy", (~ok & ~isx).sum())
                # steps t0 = t_first, t_first + S, ... while t0 - (W - 1) < t_end, two per
                # pass; prefetched: t_first, t_first + S and t0 + 2 S at each step
                steps = []
                t0 = t_first
                while t0 - (W - 1) < t_end:
                    steps.append(t0)
                    if not (t0 + S - (W - 1) < t_end):
                        break
                    steps.append(t0 + S)
                    t0 += 2 * S
                for t0 in sorted({t_first, t_first + S} | {s + 2 * S for s in steps}):
                    if seg:
                        tt = t0 + tid[tid < S]
                        acc.add("seg", b, tt[tt < t_need], 0, 1)
                    if FAST and t0 + S <= t_end:
                        for i in range(ZS):
                            ck = tid + i * NT
                            acc.add("z", b, t0 + ck // (RP // CE), (ck % (RP // CE)) * CE, CE)
                        for i in range(XS):
                            ck = tid + i * NT
                            inn = ck < XCH
                            row, c = ck // (DC // CE), (ck % (DC // CE)) * CE
                            acc.add("x", b, t0 + row[inn], c_base + c[inn], CE)
                            acc.add("dy", b, t0 + row[inn], c_base + c[inn], CE)
                            safe("x", (~inn).sum())
                            safe("dy", (~inn).sum())
                        continue
                    for i in range(ZS):
                        ck = tid + i * NT
                        row, c = ck // (RP // CE), (ck % (RP // CE)) * CE
                        ok = (ck < ZCH) & (t0 + row < t_need) & (c < R)
                        w = np.full(c.shape, CE) if FAST else np.minimum(CE, R - c)
                        acc.add("z", b, t0 + row[ok], c[ok], w[ok])
                        if FAST:
                            safe("z", (~ok).sum())
                    for i in range(XS):
                        ck = tid + i * NT
                        row, c = ck // (DC // CE), (ck % (DC // CE)) * CE
                        ok = (ck < XCH) & (c < xlimit)
                        okx, okd = ok & (t0 + row < t_end), ok & (t0 + row < t_need)
                        w = np.full(c.shape, CE) if FAST else np.minimum(CE, xlimit - c)
                        acc.add("x", b, t0 + row[okx], c_base + c[okx], w[okx])
                        acc.add("dy", b, t0 + row[okd], c_base + c[okd], w[okd])
                        if FAST:
                            safe("x", (~okx).sum())
                            safe("dy", (~okd).sum())
                # dx: token s of the range from the lanes whose run of MT channels starts
                # inside D (clipped at D)
                for wv in range(4):
                    for q in range(0, 4, LPC):
                        cl = c_base + wv * CPW + (q // LPC) * MT
                        if cl < D:
                            acc.add("dx", b, np.arange(t_first, t_end), cl, min(MT, D - cl))
                # partial sums, one per (range, channel of the group), and the generation
                # operands of the wave's channels
                for wv in range(4):
                    ch = c_base + wv * CPW + np.arange(CPW)
                    ch = ch[ch < D]
                    cols = (ch // H) * W
                    prow = rng * H + ch % H
                    acc.add("part_dU", 0, prow[None, :] * R + np.arange(R)[:, None], cols[None, :], W)
                    if want_db:
                        acc.add("part_db", 0, prow, cols, W)
                    acc.add("U", 0, np.arange(R)[:, None], cols[None, :], W)
                    if has_bias:
                        acc.add("bias", 0, 0, cols, W)
    return acc, nTr


# ---------------------------------------------------------------------------------------
# k_stream_fwd / k_stream_bwd (plan_stream, wave_tile and the per-lane loads and stores)
# ---------------------------------------------------------------------------------------
STREAM_WAVES = dict(fwd=8, fwd_group=12, fwd_wide=4, bwd=16, bwd_group=12, bwd_static=8, bwd_wide=8)


def group_vec(H, eb, align, bwd):
    """Channels per lane of a head-wise group: the largest power of two dividing H that fits
    the lane vector (align bytes), or 2m for 16-bit groups of m * 2^k channels (m = 3 or 5,
    k >= 1) in the backward, and 6 in the forward for m = 3 when the power of two is below 6."""
    v = align // eb
    while v > 1 and H % v:
        v //= 2
    m = H
    while m % 2 == 0:
        m //= 2
    if eb == 2 and m in (3, 5) and H % (2 * m) == 0:
        if bwd:
            return 2 * m
        if m == 3 and v < 6:
            return 6
    if eb == 2 and m in (3, 5) and H == m:
        return m
    return v


def stream_layout_ok(D, H, eb, align):
    """The ABI's check of the lane layout (check_stream_layout)."""
    if D % (4 // eb):
        return False
    return H == 1 or H // group_vec(H, eb, align, True) <= 64


def plan_stream(B, T, D, W, H, eb, align, bwd, static):
    if H == 1:
        vec, lpg = 4 // eb, 1
    else:
        vec = group_vec(H, eb, align, bwd)
        lpg = H // vec
    lpw = (64 // lpg) * lpg if bwd else 64
    span = lpw * vec
    nDw = (D + span - 1) // span
    WD = 4 if nDw >= 4 else (2 if nDw >= 2 else 1)
    WT = 4 // WD
    nDb = (nDw + WD - 1) // WD
    wide = H == 1 and not static and W >= 7
    if not bwd:
        waves = STREAM_WAVES["fwd_wide"] if wide else (
            STREAM_WAVES["fwd_group"] if H > 1 and not static else STREAM_WAVES["fwd"])
    else:
        waves = STREAM_WAVES["bwd_static"] if static else (
            STREAM_WAVES["bwd_group"] if H > 1 else (STREAM_WAVES["bwd_wide"] if wide else STREAM_WAVES["bwd"]))
    target = 256.0 * waves / 4
    min_len = 64 if (bwd and static) else 16
    max_chunks = 1 if T <= min_len else (T + min_len - 1) // min_len
    per_seq = target * WT / (B * nDb)
    lo, hi = int(per_seq / 4), int(per_seq * 4) + 1
    lo = max(lo, 1)
    hi = min(hi, max_chunks)
    lo = min(lo, hi)
    best, bestL = -1e30, T
    for c in range(lo, hi + 1):
        L = (T + c - 1) // c
        L = (L + 3) // 4 * 4
        nTw = (T + L - 1) // L
        blocks = B * nDb * ((nTw + WT - 1) // WT)
        per_cu = (blocks + 255) // 256
        score = blocks / (256 * per_cu) - 0.25 * abs(math.log(blocks / target))
        if score > best + 1e-12:
            best, bestL = score, L
    nTw = (T + bestL - 1) // bestL
    nTb = (nTw + WT - 1) // WT
    return dict(vec=vec, lpg=lpg, lpw=lpw, nDw=nDw, WD=WD, WT=WT, nDb=nDb, L=bestL, nTw=nTw, nTb=nTb,
                blocks=B * nDb * nTb)


def _stream_waves(pl, B, T, D, channel_fastest, xcd):
    """(b, c0 per lane, valid per lane, t0, t1, chunk) of every wave of the launch."""
    lane = np.arange(64)
    n = pl["blocks"]
    for bid in range(n):
        lb = int(xcd_logical_block(bid, n)) if xcd else bid
        if channel_fastest:
            db = lb % pl["nDb"]
            lb //= pl["nDb"]
            tb = lb % pl["nTb"]
            b = lb // pl["nTb"]
        else:
            tb = lb % pl["nTb"]
            lb //= pl["nTb"]
            db = lb % pl["nDb"]
            b = lb // pl["nDb"]
        for wv in range(4):
            dsl = db * pl["WD"] + wv % pl["WD"]
            tch = tb * pl["WT"] + wv // pl["WD"]
            c0 = (dsl * pl["lpw"] + lane) * pl["vec"]
            valid = (dsl < pl["nDw"]) & (tch < pl["nTw"]) & (lane < pl["lpw"]) & (c0 < D)
            t0 = tch * pl["L"]
            yield b, c0, valid, t0, min(T, t0 + pl["L"]), b * pl["nTw"] + tch


def _check_groups(c0, valid, pl, H):
    """The group reductions read the H / VEC consecutive lanes from each group's first one
    (pos = lane % lpg): all of them valid and of that group."""
    lpg = pl["lpg"]
    g = c0 // H
    for lane in np.nonzero(valid)[0]:
        lead = lane - lane % lpg
        assert lead + lpg <= pl["lpw"], f"group at lane {lead} straddles the lanes in use"
        assert valid[lead:lead + lpg].all(), f"group at lane {lead} partly invalid"
        assert (g[lead:lead + lpg] == g[lane]).all(), f"lane {lane} is not in the group of lane {lead}"
        assert c0[lead] % H == 0, f"group at lane {lead} does not start a filter group"


def stream_fwd(B, T, D, W, H, eb, align, static=False, seg=False, cbias=False):
    pl = plan_stream(B, T, D, W, H, eb, align, False, static)
    vec = pl["vec"]
    perch = H == 1
    nw = vec * W if perch else W
    acc = Accesses()
    for b, c0, valid, t0, t1, _ in _stream_waves(pl, B, T, D, static, False):
        c0 = c0[valid]
        if c0.size == 0:
            continue
        gcol = (c0 if perch else c0 // H) * W
        for k in range(1, W):
            if t0 - k >= 0:
                acc.add("x", b, t0 - k, c0, vec)
                if seg:
                    acc.add("seg", b, t0 - k, 0, 1)
        if static:
            acc.add("w", 0, 0, gcol, nw)
        if cbias:
            acc.add("cbias", 0, 0, c0, vec)
        t = np.arange(t0, t1)[:, None]
        acc.add("x", b, t, c0[None, :], vec)
        acc.add("y", b, t, c0[None, :], vec)
        if not static:
            acc.add("w", b, t, gcol[None, :], nw)
        if seg:
            acc.add("seg", b, t, 0, 1)
    return acc, pl


def stream_bwd(B, T, D, W, H, eb, align, static=False, want_dx=True, want_dw=True, seg=False, cb=False):
    pl = plan_stream(B, T, D, W, H, eb, align, True, static)
    vec = pl["vec"]
    perch = H == 1
    nw = vec * W if perch else W
    acc = Accesses()
    for b, c0_all, valid, t0, t1, chunk in _stream_waves(pl, B, T, D, static, True):
        if not perch:
            _check_groups(c0_all, valid, pl, H)
        lane = np.arange(64)[valid]
        c0 = c0_all[valid]
        if c0.size == 0:
            continue
        lead = lane % pl["lpg"] == 0
        gcol = (c0 if perch else c0 // H) * W
        if want_dw:
            for k in range(1, W):
                if t0 - k >= 0:
                    acc.add("x", b, t0 - k, c0, vec)
        if seg:
            for k in range(1, W):
                if t0 - k >= 0:
                    acc.add("seg", b, t0 - k, 0, 1)
        if static:
            acc.add("w", 0, 0, gcol, nw)
        if want_dx:
            for e in range(W - 1):
                tt = t1 + e
                if tt < T:
                    acc.add("dy", b, tt, c0, vec)
                    if seg:
                        acc.add("seg", b, tt, 0, 1)
                    if not static:
                        acc.add("w", b, tt, gcol, nw)
        t = np.arange(t0, t1)[:, None]
        acc.add("dy", b, t, c0[None, :], vec)
        if seg:
            acc.add("seg", b, t, 0, 1)
        if want_dw:
            acc.add("x", b, t, c0[None, :], vec)
        if not static and want_dx:
            acc.add("w", b, t, gcol[None, :], nw)
        if want_dx:
            # steps t0 .. t1 + W - 2 (the last W - 1 on the future halo) store row s = t - (W - 1)
            s_ = np.arange(t0, t1 + W - 1) - (W - 1)
            s_ = s_[(s_ >= t0) & (s_ < t1)][:, None]
            acc.add("dx", b, s_, c0[None, :], vec)
        if want_dw and not static:
            if perch:
                acc.add("dw", b, t, gcol[None, :], nw)
            else:
                acc.add("dw", b, t, gcol[lead][None, :], W)
        if cb:
            acc.add("cb_partial", 0, chunk, c0, vec)
        if static and want_dw:
            if perch:
                acc.add("partial", 0, chunk, gcol, nw)
            else:
                acc.add("partial", 0, chunk, gcol[lead], W)
    return acc, pl


# ---------------------------------------------------------------------------------------
# k_column_partials (launch_column_sums): 256 lanes of one 32-bit word of channels per
# workgroup, a chunk of tokens each, partial sums per (sequence, chunk)
# ---------------------------------------------------------------------------------------

def colsum_chunks(B, T, D):
    per_seq = (2048 + B * ((D + 255) // 256) - 1) // (B * ((D + 255) // 256))
    most = (T + 63) // 64
    return 1 if per_seq < 1 else (max(most, 1) if per_seq > most else per_seq)


def column_partials(B, T, D, eb):
    nchunk = colsum_chunks(B, T, D)
    L = (T + nchunk - 1) // nchunk
    V = 4 // eb
    nDb = (D + 256 * V - 1) // (256 * V)
    acc = Accesses()
    lane = np.arange(256)
    for bid in range(B * nchunk * nDb):
        db, chunk = bid % nDb, bid // nDb
        b, tc = chunk // nchunk, chunk % nchunk
        c = (db * 256 + lane) * V
        c = c[c < D]
        t0, t1 = tc * L, min(T, tc * L + L)
        if t1 > t0:
            acc.add("dy", b, np.arange(t0, t1)[:, None], c[None, :], V)
        acc.add("part", 0, chunk, c, V)
    return acc, nchunk
