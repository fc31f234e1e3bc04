"""Pins of the float64 oracle against facts that do not come from the oracle itself.

Sources of truth used here (all from "Dynamic Short Convolutions Improve Transformers",
reading note, section "Parameterization", and plain mathematics):

* hand-worked examples of eq. 1-3, the head-wise and the low-rank parameterisation
  (tests/golden/handworked.json, every value derived by hand with its arithmetic);
* eq. 1 is an ordinary causal FIR filter, so the static form must agree with
  numpy.convolve, scipy.signal.lfilter and torch's grouped conv1d (cross-correlation,
  hence a flipped kernel);
* the banded-matrix form of eq. 2 + 3, built entry by entry from index arithmetic:
  y = M x and, since the loss <dy, y> is linear, dx = M^T dy;
* <dy, y> is affine in every single scalar input (y is linear in x for fixed filters
  and linear in the filters for fixed x; the low-rank filters are affine in z, U, b),
  so central differences give every gradient exactly up to rounding;
* closed forms (zero filters, one-hot taps, constant input), causality, batch
  independence and the adjoint identities.

The mutation tests at the end plant typical mistakes in copies of the oracle and
check that these pins reject every one of them.
"""
import json
import os

import numpy as np
import pytest
import scipy.signal
import torch

from oracle import conv_bwd, conv_fwd, lowrank_bwd, lowrank_filters, lowrank_fwd

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "handworked.json")


def _rng(*seed):
    return np.random.default_rng(list(seed))


def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


# ----------------------------------------------------------------------------------
# pin helpers, parametrised over the implementation so that mutants can be checked
# ----------------------------------------------------------------------------------


def pin_golden_fwd(fwd) -> bool:
    ok = True
    for c in _golden_cases():
        x = np.array(c["x"], float)[None]
        H = c["H"]
        if "w" in c:
            y = fwd(x, np.array(c["w"], float)[None], H)
        elif "w_static" in c:
            y = fwd(x, np.array(c["w_static"], float), H)
        else:
            continue
        ok &= np.array_equal(y[0], np.array(c["y"], float))
    return bool(ok)


def pin_golden_bwd(bwd) -> bool:
    ok = True
    for c in _golden_cases():
        x = np.array(c["x"], float)[None]
        dy = np.array(c["dy"], float)[None]
        H = c["H"]
        if "w" in c:
            dx, dw = bwd(x, np.array(c["w"], float)[None], dy, H)
            ok &= np.array_equal(dx[0], c["dx"]) and np.array_equal(dw[0], c["dw"])
        elif "w_static" in c:
            dx, dw = bwd(x, np.array(c["w_static"], float), dy, H)
            ok &= np.array_equal(dx[0], c["dx"]) and np.array_equal(dw, c["dw_static"])
    return bool(ok)


def _banded_matrix(wfull_bd, T, W):
    """M[t, s] = [t == s] + w^{(t)}_{t-s} for 0 <= t - s < W (eq. 2 + 3 for one channel)."""
    M = np.zeros((T, T))
    for t in range(T):
        M[t, t] += 1.0
        for s in range(T):
            k = t - s
            if 0 <= k < W:
                M[t, s] += wfull_bd[t][k]
    return M


def _channel_filters(w, b, d, H, T):
    """Filter taps of channel d of sequence b at every t, by explicit index arithmetic."""
    g = d // H
    if w.ndim == 2:
        return [w[g] for _ in range(T)]
    return [w[b, t, g] for t in range(T)]


def pin_matrix_form(fwd, bwd, B, T, D, W, H, static, seed) -> bool:
    r = _rng(11, seed)
    x = r.standard_normal((B, T, D))
    dy = r.standard_normal((B, T, D))
    w = r.standard_normal((D // H, W)) if static else r.standard_normal((B, T, D // H, W))
    y = fwd(x, w, H)
    dx, _ = bwd(x, w, dy, H)
    ok = True
    for b in range(B):
        for d in range(D):
            M = _banded_matrix(_channel_filters(w, b, d, H, T), T, W)
            ok &= np.allclose(y[b, :, d], M @ x[b, :, d], rtol=0, atol=1e-13)
            ok &= np.allclose(dx[b, :, d], M.T @ dy[b, :, d], rtol=0, atol=1e-13)
    return bool(ok)


def pin_static_library(fwd, B, T, D, W, H, seed) -> bool:
    r = _rng(12, seed)
    x = r.standard_normal((B, T, D))
    w = r.standard_normal((D // H, W))
    y = fwd(x, w, H)
    ok = True
    for b in range(B):
        for d in range(D):
            taps = w[d // H]
            ref = np.convolve(x[b, :, d], taps)[:T]  # true convolution, no flip
            ok &= np.allclose(y[b, :, d] - x[b, :, d], ref, rtol=0, atol=1e-13)
            ref2 = scipy.signal.lfilter(taps, [1.0], x[b, :, d])  # causal FIR
            ok &= np.allclose(y[b, :, d] - x[b, :, d], ref2, rtol=0, atol=1e-12)
    # torch conv1d is cross-correlation: flip the taps and pad W-1 zeros on the left
    xt = torch.from_numpy(x).permute(0, 2, 1)  # (B, D, T)
    wt = torch.from_numpy(np.repeat(w, H, axis=0)[:, ::-1].copy()).unsqueeze(1)  # (D, 1, W)
    ref3 = torch.nn.functional.conv1d(torch.nn.functional.pad(xt, (W - 1, 0)), wt, groups=D)
    ok &= np.allclose(y - x, ref3.permute(0, 2, 1).numpy(), rtol=0, atol=1e-12)
    return bool(ok)


def _fd_check(loss, arrays, grads, tol=1e-10) -> bool:
    """Central differences of an affine-per-coordinate loss, every coordinate."""
    ok = True
    for a, g in zip(arrays, grads):
        flat = a.reshape(-1)
        gf = np.asarray(g).reshape(-1)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + 1.0
            lp = loss()
            flat[i] = old - 1.0
            lm = loss()
            flat[i] = old
            fd = (lp - lm) / 2.0
            ok &= abs(fd - gf[i]) <= tol * max(1.0, abs(fd))
    return bool(ok)


def pin_fd_conv(fwd, bwd, B, T, D, W, H, static, seed) -> bool:
    r = _rng(13, seed)
    x = r.standard_normal((B, T, D))
    dy = r.standard_normal((B, T, D))
    w = r.standard_normal((D // H, W)) if static else r.standard_normal((B, T, D // H, W))
    dx, dw = bwd(x, w, dy, H)
    return _fd_check(lambda: float(np.sum(dy * fwd(x, w, H))), [x, w], [dx, dw])


def pin_fd_lowrank(fwd, bwd, B, T, D, W, H, R, seed) -> bool:
    r = _rng(14, seed)
    G = D // H
    x = r.standard_normal((B, T, D))
    dy = r.standard_normal((B, T, D))
    z = r.standard_normal((B, T, R))
    U = r.standard_normal((R, G * W))
    bias = r.standard_normal(G * W)
    dx, dz, dU, db = bwd(x, z, U, bias, dy, W, H)
    loss = lambda: float(np.sum(dy * fwd(x, z, U, bias, W, H)))  # noqa: E731
    return _fd_check(loss, [x, z, U, bias], [dx, dz, dU, db])


# ----------------------------------------------------------------------------------
# the pins applied to the oracle
# ----------------------------------------------------------------------------------


def test_golden_handworked_fwd_bwd():
    assert pin_golden_fwd(conv_fwd)
    assert pin_golden_bwd(conv_bwd)


def test_golden_handworked_lowrank():
    for c in _golden_cases():
        if "z" not in c:
            continue
        x = np.array(c["x"], float)[None]
        z = np.array(c["z"], float)[None]
        U = np.array(c["U"], float)
        bias = np.array(c["b"], float)
        dy = np.array(c["dy"], float)[None]
        W = U.shape[1] // x.shape[2] * c["H"]
        y = lowrank_fwd(x, z, U, bias, W, c["H"])
        dx, dz, dU, db = lowrank_bwd(x, z, U, bias, dy, W, c["H"])
        assert np.array_equal(y[0], c["y"])
        assert np.array_equal(dx[0], c["dx"])
        assert np.array_equal(dz[0], c["dz"])
        assert np.array_equal(dU, c["dU"])
        assert np.array_equal(db, c["db"])


@pytest.mark.parametrize("W", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("H", [1, 2, 4])
@pytest.mark.parametrize("T", [1, 3, 9])
@pytest.mark.parametrize("static", [False, True])
def test_matrix_form(W, H, T, static):
    assert pin_matrix_form(conv_fwd, conv_bwd, 2, T, 8, W, H, static, seed=W * 100 + H * 10 + T)


@pytest.mark.parametrize("W", [1, 3, 4, 5, 8])
@pytest.mark.parametrize("H", [1, 4])
def test_static_matches_library_fir(W, H):
    assert pin_static_library(conv_fwd, 2, 17, 8, W, H, seed=W + 7 * H)


def test_constant_in_t_dynamic_equals_static():
    r = _rng(15)
    B, T, D, W, H = 2, 13, 8, 4, 2
    x = r.standard_normal((B, T, D))
    ws = r.standard_normal((D // H, W))
    wd = np.broadcast_to(ws, (B, T, D // H, W)).copy()
    dy = r.standard_normal((B, T, D))
    assert np.allclose(conv_fwd(x, wd, H), conv_fwd(x, ws, H), rtol=0, atol=1e-14)
    dxd, dwd = conv_bwd(x, wd, dy, H)
    dxs, dws = conv_bwd(x, ws, dy, H)
    assert np.allclose(dxd, dxs, rtol=0, atol=1e-13)
    assert np.allclose(dwd.sum(axis=(0, 1)), dws, rtol=0, atol=1e-12)


@pytest.mark.parametrize("static", [False, True])
@pytest.mark.parametrize("W,H,T", [(1, 1, 4), (3, 2, 5), (4, 1, 6), (5, 4, 3), (4, 2, 7), (8, 1, 10), (7, 2, 5)])
def test_finite_differences_conv(W, H, T, static):
    assert pin_fd_conv(conv_fwd, conv_bwd, 2, T, 4 * H if H > 1 else 4, W, H, static, seed=W * 31 + T)


@pytest.mark.parametrize("W,H,R,T", [(4, 1, 3, 6), (2, 2, 2, 5), (5, 1, 1, 4), (3, 4, 5, 7), (6, 2, 3, 7), (8, 1, 2, 10)])
def test_finite_differences_lowrank(W, H, R, T):
    assert pin_fd_lowrank(lowrank_fwd, lowrank_bwd, 2, T, 8, W, H, R, seed=W * 17 + R)


def test_closed_form_zero_filter():
    r = _rng(16)
    x = r.standard_normal((2, 11, 8))
    dy = r.standard_normal((2, 11, 8))
    w = np.zeros((2, 11, 8, 4))
    assert np.array_equal(conv_fwd(x, w), x)
    dx, _ = conv_bwd(x, w, dy)
    assert np.array_equal(dx, dy)


@pytest.mark.parametrize("j", [0, 1, 2, 3, 4])
def test_closed_form_one_hot_tap(j):
    r = _rng(17, j)
    B, T, D, W = 2, 9, 6, 5
    x = r.standard_normal((B, T, D))
    w = np.zeros((B, T, D, W))
    w[..., j] = 1.0
    expect = x.copy()
    expect[:, j:, :] += x[:, : T - j, :]  # y_t = x_t + x_{t-j} for t >= j
    assert np.array_equal(conv_fwd(x, w), expect)


def test_closed_form_constant_input():
    r = _rng(18)
    B, T, D, W, H = 2, 7, 4, 4, 2
    c = 1.75
    x = np.full((B, T, D), c)
    w = r.standard_normal((B, T, D // H, W))
    y = conv_fwd(x, w, H)
    for b in range(B):
        for t in range(T):
            for d in range(D):
                taps = sum(w[b, t, d // H, k] for k in range(min(W - 1, t) + 1))
                assert abs(y[b, t, d] - c * (1.0 + taps)) < 1e-13


def test_causality_band():
    r = _rng(19)
    B, T, D, W, H = 2, 12, 4, 4, 2
    x = r.standard_normal((B, T, D))
    w = r.standard_normal((B, T, D // H, W))
    y0 = conv_fwd(x, w, H)
    for (b, s, d) in [(0, 0, 0), (1, 5, 3), (0, 11, 2), (1, 9, 1)]:
        xp = x.copy()
        xp[b, s, d] += 1.0
        dif = conv_fwd(xp, w, H) - y0
        expect = np.zeros_like(dif)
        for t in range(s, min(T, s + W)):
            expect[b, t, d] = (1.0 if t == s else 0.0) + w[b, t, d // H, t - s]
        assert np.allclose(dif, expect, rtol=0, atol=1e-13)


def test_headwise_equals_broadcast_perchannel():
    r = _rng(20)
    B, T, D, W, H = 2, 10, 16, 3, 4
    x = r.standard_normal((B, T, D))
    dy = r.standard_normal((B, T, D))
    w = r.standard_normal((B, T, D // H, W))
    wb = np.zeros((B, T, D, W))
    for d in range(D):  # explicit: channel d takes the filter of group d // H
        wb[:, :, d, :] = w[:, :, d // H, :]
    assert np.allclose(conv_fwd(x, w, H), conv_fwd(x, wb, 1), rtol=0, atol=1e-14)
    dxh, dwh = conv_bwd(x, w, dy, H)
    dxp, dwp = conv_bwd(x, wb, dy, 1)
    assert np.allclose(dxh, dxp, rtol=0, atol=1e-13)
    grouped = np.zeros_like(dwh)
    for d in range(D):
        grouped[:, :, d // H, :] += dwp[:, :, d, :]
    assert np.allclose(dwh, grouped, rtol=0, atol=1e-13)


@pytest.mark.parametrize("zero", ["U", "z"])
def test_lowrank_reduces_to_static_bias_filter(zero):
    r = _rng(21)
    B, T, D, W, H, R = 2, 9, 8, 4, 2, 3
    x = r.standard_normal((B, T, D))
    z = r.standard_normal((B, T, R))
    U = r.standard_normal((R, D // H * W))
    bias = r.standard_normal(D // H * W)
    if zero == "U":
        U[:] = 0
    else:
        z[:] = 0
    y = lowrank_fwd(x, z, U, bias, W, H)
    taps = bias.reshape(D // H, W)  # column j = g * W + k
    for b in range(B):
        for d in range(D):
            ref = np.convolve(x[b, :, d], taps[d // H])[:T]
            assert np.allclose(y[b, :, d] - x[b, :, d], ref, rtol=0, atol=1e-13)


def test_lowrank_rank_one_closed_form():
    """R = 1, U = u (one row): w^{(t)} = z_t u + b, so y - x is linear in z_t per tap."""
    r = _rng(22)
    B, T, D, W = 1, 8, 4, 3
    x = r.standard_normal((B, T, D))
    z = r.standard_normal((B, T, 1))
    U = r.standard_normal((1, D * W))
    bias = r.standard_normal(D * W)
    y = lowrank_fwd(x, z, U, bias, W, 1)
    for t in range(T):
        for d in range(D):
            acc = x[0, t, d]
            for k in range(W):
                if t - k >= 0:
                    acc += (z[0, t, 0] * U[0, d * W + k] + bias[d * W + k]) * x[0, t - k, d]
            assert abs(acc - y[0, t, d]) < 1e-12


@pytest.mark.parametrize("H,static", [(1, False), (4, False), (1, True), (4, True)])
def test_adjoint_identities(H, static):
    r = _rng(23, H, int(static))
    B, T, D, W = 2, 96, 32, 4
    x = r.standard_normal((B, T, D))
    dy = r.standard_normal((B, T, D))
    w = r.standard_normal((D // H, W)) if static else r.standard_normal((B, T, D // H, W))
    dx, dw = conv_bwd(x, w, dy, H)
    dlx = r.standard_normal(x.shape)
    dlw = r.standard_normal(w.shape)
    lhs = np.sum((dx - dy) * dlx)
    rhs = np.sum(dy * (conv_fwd(dlx, w, H) - dlx))
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(rhs))
    lhs = np.sum(dw * dlw)
    rhs = np.sum(dy * (conv_fwd(x, dlw, H) - x))
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(rhs))


def test_adjoint_identities_lowrank():
    r = _rng(24)
    B, T, D, W, H, R = 2, 64, 16, 4, 1, 6
    G = D // H
    x = r.standard_normal((B, T, D))
    dy = r.standard_normal((B, T, D))
    z = r.standard_normal((B, T, R))
    U = r.standard_normal((R, G * W))
    bias = r.standard_normal(G * W)
    dx, dz, dU, db = lowrank_bwd(x, z, U, bias, dy, W, H)

    def cx(filters):  # the conv part as a linear map of the filters, x fixed
        return conv_fwd(x, filters, H) - x

    dz_dir = r.standard_normal(z.shape)
    dU_dir = r.standard_normal(U.shape)
    db_dir = r.standard_normal(bias.shape)
    checks = [
        (np.sum(dz * dz_dir), np.sum(dy * cx(lowrank_filters(dz_dir, U, None, W)))),
        (np.sum(dU * dU_dir), np.sum(dy * cx(lowrank_filters(z, dU_dir, None, W)))),
        (np.sum(db * db_dir), np.sum(dy * cx(np.broadcast_to(db_dir.reshape(G, W), (B, T, G, W))))),
    ]
    for lhs, rhs in checks:
        assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(rhs))


def test_batch_independence():
    r = _rng(25)
    B, T, D, W, H = 3, 10, 8, 4, 2
    x = r.standard_normal((B, T, D))
    dy = r.standard_normal((B, T, D))
    w = r.standard_normal((B, T, D // H, W))
    perm = [2, 0, 1]
    y = conv_fwd(x, w, H)
    assert np.array_equal(conv_fwd(x[perm], w[perm], H), y[perm])
    dx, dw = conv_bwd(x, w, dy, H)
    dxp, dwp = conv_bwd(x[perm], w[perm], dy[perm], H)
    assert np.array_equal(dxp, dx[perm]) and np.array_equal(dwp, dw[perm])


# ----------------------------------------------------------------------------------
# planted mistakes: each mutant of the oracle must be rejected by at least one pin
# ----------------------------------------------------------------------------------


def _mut_fwd_flipped(x, w, H=1):
    return conv_fwd(x, w[..., ::-1], H)


def _mut_fwd_no_residual(x, w, H=1):
    return conv_fwd(x, w, H) - np.asarray(x, float)


def _mut_fwd_off_by_one(x, w, H=1):
    x = np.asarray(x, float)
    w = np.asarray(w, float)
    B, T, D = x.shape
    W = w.shape[-1]
    y = x.copy()
    for b in range(B):
        wf = np.repeat(w, H, axis=0) if w.ndim == 2 else np.repeat(w[b], H, axis=1)
        for k in range(W):
            s = k + 1  # wrong: reads x_{t-k-1}
            if s >= T:
                break
            y[b, s:, :] += (wf[None, :, k] if wf.ndim == 2 else wf[s:, :, k]) * x[b, : T - s, :]
    return y


def _mut_fwd_wraparound(x, w, H=1):
    x = np.asarray(x, float)
    w = np.asarray(w, float)
    B, T, D = x.shape
    y = x.copy()
    for b in range(B):
        wf = np.repeat(w, H, axis=0)[None] if w.ndim == 2 else np.repeat(w[b], H, axis=1)
        for k in range(w.shape[-1]):
            y[b] += wf[..., k] * np.roll(x[b], k, axis=0)  # wrong: circular instead of zeros
    return y


def _mut_fwd_group_modulo(x, w, H=1):
    w = np.asarray(w, float)
    D = np.asarray(x).shape[2]
    G = D // H
    idx = np.arange(D) % G  # wrong: tiles the filters instead of repeating them
    if w.ndim == 2:
        return conv_fwd(x, w[idx], 1)
    return conv_fwd(x, w[:, :, idx, :], 1)


def _mut_fwd_filter_of_source(x, w, H=1):
    """Wrong token index: uses w^{(t-k)} instead of w^{(t)} for the tap reading x_{t-k}."""
    x = np.asarray(x, float)
    w = np.asarray(w, float)
    if w.ndim == 2:
        return conv_fwd(x, w, H)
    B, T, D = x.shape
    y = x.copy()
    for b in range(B):
        wf = np.repeat(w[b], H, axis=1)
        for k in range(w.shape[-1]):
            if k >= T:
                break
            y[b, k:, :] += wf[: T - k, :, k] * x[b, : T - k, :]
    return y


def _mut_bwd_dx_same_token(x, w, dy, H=1):
    """Wrong: dx uses w^{(s)} instead of w^{(s+k)}."""
    x = np.asarray(x, float)
    w = np.asarray(w, float)
    dy = np.asarray(dy, float)
    _, dw = conv_bwd(x, w, dy, H)
    if w.ndim == 2:
        return conv_bwd(x, w, dy, H)
    B, T, D = x.shape
    dx = dy.copy()
    for b in range(B):
        wf = np.repeat(w[b], H, axis=1)
        for k in range(w.shape[-1]):
            if k >= T:
                break
            dx[b, : T - k, :] += wf[: T - k, :, k] * dy[b, k:, :]
    return dx, dw


def _mut_bwd_dw_flipped(x, w, dy, H=1):
    dx, dw = conv_bwd(x, w, dy, H)
    return dx, dw[..., ::-1]


def _mut_bwd_dw_no_group_sum(x, w, dy, H=1):
    dx, dw = conv_bwd(x, w, dy, H)
    return dx, dw / H  # wrong: averages instead of summing the H channels


FWD_MUTANTS = [
    _mut_fwd_flipped,
    _mut_fwd_no_residual,
    _mut_fwd_off_by_one,
    _mut_fwd_wraparound,
    _mut_fwd_group_modulo,
    _mut_fwd_filter_of_source,
]
BWD_MUTANTS = [_mut_bwd_dx_same_token, _mut_bwd_dw_flipped, _mut_bwd_dw_no_group_sum]


@pytest.mark.parametrize("mutant", FWD_MUTANTS, ids=lambda f: f.__name__)
def test_pins_reject_forward_mutant(mutant):
    verdicts = [
        pin_golden_fwd(mutant),
        pin_matrix_form(mutant, conv_bwd, 1, 7, 8, 3, 2, False, seed=1),
        pin_static_library(mutant, 1, 9, 8, 3, 2, seed=2),
    ]
    assert not all(verdicts)


@pytest.mark.parametrize("mutant", BWD_MUTANTS, ids=lambda f: f.__name__)
def test_pins_reject_backward_mutant(mutant):
    verdicts = [
        pin_golden_bwd(mutant),
        pin_fd_conv(conv_fwd, mutant, 1, 5, 4, 3, 2, False, seed=3),
    ]
    assert not all(verdicts)


def _mut_lr_dU_transposed_z(x, z, U, bias, dy, W, H=1):
    dx, dz, dU, db = lowrank_bwd(x, z, U, bias, dy, W, H)
    return dx, dz, dU[::-1], db  # wrong row order of dU


def _mut_lr_dz_no_taps(x, z, U, bias, dy, W, H=1):
    dx, dz, dU, db = lowrank_bwd(x, z, U, bias, dy, W, H)
    return dx, dz * 0.5, dU, db


def _mut_lr_column_order(x, z, U, bias, W, H=1):
    """Wrong column order: j = k * G + g instead of g * W + k."""
    wf = lowrank_filters(z, U, bias, W)
    B, T, G, _ = wf.shape
    flat = wf.reshape(B, T, G * W)
    return conv_fwd(x, flat.reshape(B, T, W, G).transpose(0, 1, 3, 2), H)


def test_pins_reject_lowrank_mutants():
    for mut in (_mut_lr_dU_transposed_z, _mut_lr_dz_no_taps):
        assert not pin_fd_lowrank(lowrank_fwd, mut, 1, 5, 4, 3, 1, 2, seed=5)
    # the column-order mutant: the hand-worked case has D/H = 1 so it cannot tell; the
    # U = 0 reduction to a static filter b reshaped (D/H, W) does
    r = _rng(26)
    B, T, D, W, R = 1, 9, 4, 3, 2
    x = r.standard_normal((B, T, D))
    z = r.standard_normal((B, T, R))
    U = np.zeros((R, D * W))
    bias = r.standard_normal(D * W)
    y = _mut_lr_column_order(x, z, U, bias, W)
    taps = bias.reshape(D, W)
    ref = np.stack([np.convolve(x[0, :, d], taps[d])[:T] for d in range(D)], axis=1)
    assert not np.allclose(y[0] - x[0], ref, atol=1e-12)


# ----------------------------------------------------------------------------------
# packed sequences (segment ids): a row holding several documents must give, on each
# document, exactly what that document gives alone as its own zero-padded sequence
# ----------------------------------------------------------------------------------

PACKED_DOCS = ([1, 4, 2, 6], [7, 1, 1, 4])  # per row; lengths 1 and 2 are shorter than W - 1


def _packed_inputs(W, H, static, seed, D=8):
    r = _rng(seed)
    T = sum(PACKED_DOCS[0])
    assert all(sum(d) == T for d in PACKED_DOCS)
    B = len(PACKED_DOCS)
    seq = np.zeros((B, T), dtype=np.int32)
    for b, docs in enumerate(PACKED_DOCS):
        seq[b] = np.repeat(np.arange(len(docs)) + 10 * b, docs)
    x = r.standard_normal((B, T, D))
    dy = r.standard_normal((B, T, D))
    w = r.standard_normal((D // H, W) if static else (B, T, D // H, W))
    return x, w, dy, seq


def _doc_ranges(b):
    s = 0
    for n in PACKED_DOCS[b]:
        yield s, s + n
        s += n


def pin_packed_fwd(fwd, W, H, static, seed):
    x, w, _, seq = _packed_inputs(W, H, static, seed)
    y = fwd(x, w, H, seq)
    for b in range(x.shape[0]):
        for s, e in _doc_ranges(b):
            wd = w if static else w[b : b + 1, s:e]
            if not np.array_equal(y[b, s:e], conv_fwd(x[b : b + 1, s:e], wd, H)[0]):
                return False
    return True


def pin_packed_bwd(bwd, W, H, static, seed):
    x, w, dy, seq = _packed_inputs(W, H, static, seed)
    dx, dw = bwd(x, w, dy, H, seq)
    dw_sum = np.zeros_like(w) if static else None
    for b in range(x.shape[0]):
        for s, e in _doc_ranges(b):
            wd = w if static else w[b : b + 1, s:e]
            rdx, rdw = conv_bwd(x[b : b + 1, s:e], wd, dy[b : b + 1, s:e], H)
            if not np.array_equal(dx[b, s:e], rdx[0]):
                return False
            if static:
                dw_sum += rdw
            elif not np.array_equal(dw[b, s:e], rdw[0]):
                return False
    return (not static) or np.allclose(dw, dw_sum, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("W", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("H,static", [(1, False), (2, False), (1, True), (4, True)])
def test_packed_equals_separate_documents(W, H, static):
    assert pin_packed_fwd(conv_fwd, W, H, static, seed=40 + W)
    assert pin_packed_bwd(conv_bwd, W, H, static, seed=50 + W)


@pytest.mark.parametrize("W", [2, 4, 5, 7])
def test_packed_equals_separate_documents_lowrank(W):
    r = _rng(60 + W)
    B, T, D, R = 2, sum(PACKED_DOCS[0]), 6, 3
    _, _, _, seq = _packed_inputs(W, 1, False, 61)
    x, dy = r.standard_normal((B, T, D)), r.standard_normal((B, T, D))
    z, U, bias = r.standard_normal((B, T, R)), r.standard_normal((R, D * W)), r.standard_normal(D * W)
    y = lowrank_fwd(x, z, U, bias, W, 1, seq)
    dx, dz, dU, db = lowrank_bwd(x, z, U, bias, dy, W, 1, seq)
    sU, sb = np.zeros_like(dU), np.zeros_like(db)
    for b in range(B):
        for s, e in _doc_ranges(b):
            args = (x[b : b + 1, s:e], z[b : b + 1, s:e], U, bias)
            np.testing.assert_allclose(y[b, s:e], lowrank_fwd(*args, W)[0], rtol=1e-13, atol=1e-13)
            rdx, rdz, rdU, rdb = lowrank_bwd(*args, dy[b : b + 1, s:e], W)
            np.testing.assert_allclose(dx[b, s:e], rdx[0], rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(dz[b, s:e], rdz[0], rtol=1e-12, atol=1e-12)
            sU += rdU
            sb += rdb
    np.testing.assert_allclose(dU, sU, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(db, sb, rtol=1e-12, atol=1e-12)


def test_single_segment_equals_unpacked():
    x, w, dy, _ = _packed_inputs(4, 2, False, 70)
    seq = np.full(x.shape[:2], 3, dtype=np.int32)
    assert np.array_equal(conv_fwd(x, w, 2, seq), conv_fwd(x, w, 2))
    for a, b in zip(conv_bwd(x, w, dy, 2, seq), conv_bwd(x, w, dy, 2)):
        assert np.array_equal(a, b)


def _mut_packed_adjacent_only(x, w, H=1, seq_idx=None):
    """Wrong: a tap is cut only when token t-1 (not t-k) is in another segment."""
    x = np.asarray(x, float)
    seq = np.asarray(seq_idx)
    y = conv_fwd(x, w, H)
    B, T, _ = x.shape
    for b in range(B):
        for t in range(1, T):
            if seq[b, t] != seq[b, t - 1]:
                # start of a segment: drop every tap of this token only
                y[b, t] = conv_fwd(x[b : b + 1, t : t + 1], w if np.ndim(w) == 2 else w[b : b + 1, t : t + 1], H)[0, 0]
    return y


def _mut_packed_bwd_unmasked_dx(x, w, dy, H=1, seq_idx=None):
    """Wrong: dw is masked but dx still collects the next segment's terms."""
    _, dw = conv_bwd(x, w, dy, H, seq_idx)
    dx, _ = conv_bwd(x, w, dy, H)
    return dx, dw


def test_pins_reject_packed_mutants():
    assert not all(pin_packed_fwd(_mut_packed_adjacent_only, W, 1, False, 80 + W) for W in (3, 4))
    assert not pin_packed_bwd(_mut_packed_bwd_unmasked_dx, 4, 1, False, 81)


# ----------------------------------------------------------------------------------
# optional convolution bias (a per-channel vector added to every output token)
# ----------------------------------------------------------------------------------
from oracle import conv_bias_grad  # noqa: E402


def pin_conv_bias(fwd, bgrad, seed):
    """Zero filters: y = x + c exactly at every token, including t < W - 1; dc from central
    differences of <dy, y> (affine in c) and equal to the plain sum of dy."""
    r = _rng(seed)
    B, T, D, W = 2, 7, 6, 4
    x, dy, c = r.standard_normal((B, T, D)), r.standard_normal((B, T, D)), r.standard_normal(D)
    if not np.array_equal(fwd(x, np.zeros((B, T, D, W)), 1, None, c), x + c[None, None, :]):
        return False
    w = r.standard_normal((B, T, D, W))
    dc = bgrad(dy)
    h = 0.5
    for d in range(D):
        e = np.zeros(D)
        e[d] = h
        num = (np.sum(dy * fwd(x, w, 1, None, c + e)) - np.sum(dy * fwd(x, w, 1, None, c - e))) / (2 * h)
        if abs(num - dc[d]) > 1e-9 * (1 + abs(dc[d])):
            return False
    return True


def test_conv_bias():
    assert pin_conv_bias(conv_fwd, conv_bias_grad, 90)
    # the bias does not change the other gradients: y is c plus terms free of c
    r = _rng(91)
    x, w, dy = r.standard_normal((2, 9, 8)), r.standard_normal((2, 9, 4, 3)), r.standard_normal((2, 9, 8))
    assert np.array_equal(conv_fwd(x, w, 2, None, np.zeros(8)), conv_fwd(x, w, 2))


def _mut_bias_full_window_only(x, w, H=1, seq_idx=None, conv_bias=None):
    """Wrong: the bias is added only once the filter window is full (t >= W - 1)."""
    y = conv_fwd(x, w, H, seq_idx)
    if conv_bias is not None:
        y[:, np.shape(w)[-1] - 1 :, :] += np.asarray(conv_bias, float)[None, None, :]
    return y


def _mut_bias_grad_mean(dy):
    return np.asarray(dy, float).mean(axis=(0, 1))  # wrong: averages instead of summing


def test_pins_reject_conv_bias_mutants():
    assert not pin_conv_bias(_mut_bias_full_window_only, conv_bias_grad, 92)
    assert not pin_conv_bias(conv_fwd, _mut_bias_grad_mean, 93)


def _lowrank_as_conv(x, w, H=1, seq_idx=None, conv_bias=None):
    """The low-rank form with U = I (R = (D/H) W, no generator bias): z U reproduces any
    filter tensor, so the convolution-bias pin applies to the low-rank forward as is."""
    B, T, G, W = np.shape(w)
    return lowrank_fwd(x, np.reshape(w, (B, T, G * W)), np.eye(G * W), None, W, H, seq_idx, conv_bias)


def test_lowrank_conv_bias():
    assert pin_conv_bias(_lowrank_as_conv, conv_bias_grad, 94)
    assert not pin_conv_bias(
        lambda x, w, H=1, s=None, c=None: _lowrank_as_conv(x, w, H, s, None if c is None else 2 * c),
        conv_bias_grad, 95)  # a bias counted twice


# ----------------------------------------------------------------------------------
# The convolution on a projection's output (the epilogue fusion of the end-to-end
# throughput section): X = A W_p^T, then eq. 2 + eq. 3 on X.
# ----------------------------------------------------------------------------------
from oracle import gemm_conv_fwd, gemm_lowrank_fwd, projection  # noqa: E402


def _brute_gemm_conv(A, Wp, w, H):
    """Pure-Python loops: X[b,t,n] = sum_k A[b,t,k] Wp[n,k]; y = X + sum_j w[b,t,n//H,j] X[b,t-j,n]."""
    B, T, K = A.shape
    N = Wp.shape[0]
    W = w.shape[-1]
    X = [[[sum(float(A[b, t, k]) * float(Wp[n, k]) for k in range(K)) for n in range(N)] for t in range(T)]
         for b in range(B)]
    y = np.zeros((B, T, N))
    for b in range(B):
        for t in range(T):
            for n in range(N):
                acc = X[b][t][n]
                for j in range(W):
                    if t - j >= 0:
                        f = w[n // H, j] if w.ndim == 2 else w[b, t, n // H, j]
                        acc += float(f) * X[b][t - j][n]
                y[b, t, n] = acc
    return y


def pin_gemm_conv(fn, seed) -> bool:
    """Brute force on tiny shapes, identity and permutation projections, linearity in A."""
    rng = _rng(seed, 90)
    ok = True
    for (B, T, K, N, W, H) in ((1, 6, 3, 4, 4, 1), (2, 5, 5, 4, 3, 2), (1, 3, 2, 2, 5, 1)):
        A = rng.standard_normal((B, T, K))
        Wp = rng.standard_normal((N, K))
        w = rng.standard_normal((B, T, N // H, W))
        ok &= np.allclose(fn(A, Wp, w, H), _brute_gemm_conv(A, Wp, w, H), rtol=1e-13, atol=1e-13)
    B, T, N, W = 2, 9, 6, 4
    A = rng.standard_normal((B, T, N))
    w = rng.standard_normal((B, T, N, W))
    ok &= np.array_equal(fn(A, np.eye(N), w, 1), conv_fwd(A, w, 1))  # identity projection
    perm = np.array([2, 0, 5, 1, 3, 4])  # not an involution: a transposed W_p picks other columns
    P = np.zeros((N, N))
    P[np.arange(N), perm] = 1.0  # output column n reads input column perm[n]
    ok &= np.array_equal(fn(A, P, w, 1), conv_fwd(A[..., perm], w, 1))
    K = 7
    A1, A2 = rng.standard_normal((B, T, K)), rng.standard_normal((B, T, K))
    Wp = rng.standard_normal((N, K))
    ok &= np.allclose(fn(A1 + A2, Wp, w, 1), fn(A1, Wp, w, 1) + fn(A2, Wp, w, 1), rtol=1e-12, atol=1e-12)
    return bool(ok)


def test_gemm_conv_pins():
    assert pin_gemm_conv(gemm_conv_fwd, 1)


def test_gemm_conv_static_filter_and_projection_shape():
    rng = _rng(3, 91)
    A = rng.standard_normal((2, 7, 5))
    Wp = rng.standard_normal((8, 5))
    w = rng.standard_normal((4, 3))
    assert projection(A, Wp).shape == (2, 7, 8)
    assert np.allclose(gemm_conv_fwd(A, Wp, w, 2), _brute_gemm_conv(A, Wp, w, 2), rtol=1e-13, atol=1e-13)


def test_gemm_lowrank_equals_materialised_filters():
    """Low-rank filters in the epilogue == the materialised z U + b on the same projection;
    with the identity projection == the low-rank convolution of A itself."""
    rng = _rng(4, 92)
    B, T, K, N, W, R, H = 2, 11, 6, 8, 4, 3, 2
    A = rng.standard_normal((B, T, K))
    Wp = rng.standard_normal((N, K))
    z = rng.standard_normal((B, T, R))
    U = rng.standard_normal((R, (N // H) * W))
    bias = rng.standard_normal(((N // H) * W,))
    wf = np.einsum("btr,rj->btj", z, U) + bias
    ref = _brute_gemm_conv(A, Wp, wf.reshape(B, T, N // H, W), H)
    assert np.allclose(gemm_lowrank_fwd(A, Wp, z, U, bias, W, H), ref, rtol=1e-12, atol=1e-12)
    A2 = rng.standard_normal((B, T, N))
    assert np.array_equal(gemm_lowrank_fwd(A2, np.eye(N), z, U, bias, W, H), lowrank_fwd(A2, z, U, bias, W, H))


def _mut_gemm_transposed(A, Wp, w, H=1):
    return conv_fwd(np.matmul(A, Wp) if Wp.shape[0] == Wp.shape[1] else projection(A, Wp), w, H)


def _mut_gemm_conv_first(A, Wp, w, H=1):
    # the convolution on A, then the projection: only equal when W_p commutes with it
    if A.shape[-1] != Wp.shape[0]:
        return gemm_conv_fwd(A, Wp, w, H) + 1.0
    return projection(conv_fwd(A, w, H), Wp)


def test_pins_reject_gemm_mutants():
    assert not pin_gemm_conv(_mut_gemm_transposed, 1)
    assert not pin_gemm_conv(_mut_gemm_conv_first, 1)
