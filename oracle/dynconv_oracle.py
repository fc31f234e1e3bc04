"""Plain float64 CPU oracle for the dynamic short convolution.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute
this module; only the tests, the package smoke check and the benchmark's CPU-baseline
leg use it. It shares no code with the HIP library and imports nothing from it.

What it computes, from "Dynamic Short Convolutions Improve Transformers" (reading
note, section "Parameterization"):

* eq. 1 (static): y_t = sum_{k=0}^{W-1} w_k * x_{t-k}, one filter w in R^{W x D}
  for every t;
* eq. 2 (dynamic): the same sum with a per-token filter w^{(t)};
* eq. 3 (residual placement on Q, K, V): X <- X + dynamicShortConv(X);
* head-wise parameterisation: one filter of W taps is shared by H consecutive
  channels, so the per-token filter tensor is B x T x (D/H) x W (section
  "Efficient training (Triton kernels)");
* low-rank parameterisation: the generator D -> R -> W*D is affine ("all transforms
  have a bias"); the fused kernel takes the rank-R activations z (B x T x R) and the
  second projection U (R x (D*W)) and forms z U + b.

Readings where the page leaves a step open (each also listed in the design notes):

* positions before t = 0 of every sequence hold zeros (the sum simply has no term
  for t - k < 0);
* the filter tensor keeps the W taps of one group contiguous: w[b, t, g, k], with
  channel d using group g = d // H;
* the low-rank column index of U and b is j = g * W + k, so z U + b reshapes directly
  to (D/H, W);
* the filters carry no nonlinearity (affine generator), and the convolution itself
  has no bias;
* the generator's input is the normalised block input, not X itself, so x and w are
  independent inputs and dx has no path through w;
* optional convolution bias (the Conv1D module of the convolution technical report, whose
  initialisation study randomises both its weights and its bias; the dynamic-convolution
  page itself has no bias in the convolution): a per-channel vector c added to every output token,
  y_t = x_t + sum_k w_k x_{t-k} + c, with gradient dc = sum over (b, t) of dy;
* packed sequences (several documents in one row; the RubiConv page's point that a
  convolution must not read across a document start): an optional segment id per token,
  seq_idx (B, T) of integers, and tap k of token t is present only when token t - k
  carries the same id as token t. Without seq_idx every row is one document.

* the convolution in the epilogue of the producing projection (the closing analysis of
  the end-to-end throughput section: fusing the dynamic convolution into the matmul
  epilogue cuts memory traffic; the "Parameterization" section places the convolution
  on the outputs of the QKV projection): the projection output X = A W_p^T, with A the
  (B, T, K) activations and W_p the (N, K) weight of a linear layer, followed by eq. 2 +
  eq. 3 on X. The fused kernel never stores X; the oracle forms it with a plain matmul
  and calls the convolution above.

Everything is float64; bfloat16 and float32 inputs are exact in float64. Arrays are
processed one sequence (one b) at a time; no blocking, fusion or reordering beyond
the sums written out below.
"""
from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _filters_for_sequence(w: np.ndarray, b: int, D: int, H: int) -> np.ndarray:
    """Per-channel filters of sequence b as a (T, D, W) or (D, W) array.

    Head-wise sharing: channel d reads group d // H, i.e. each filter is repeated over H
    consecutive channels ("Parameterization", head-wise parameterisation).
    Static filters (eq. 1) have shape (D/H, W) and are the same for every (b, t).
    """
    if w.ndim == 2:  # static (D/H, W)
        return np.repeat(w, H, axis=0)
    return np.repeat(w[b], H, axis=1)  # (T, D/H, W) -> (T, D, W)


def _same_segment(seq_idx, b: int, k: int, T: int):
    """(T - k, 1) array: 1.0 where token t - k has the segment id of token t (t = k .. T-1),
    else 0.0; all ones without seq_idx."""
    if seq_idx is None:
        return np.ones((T - k, 1))
    s = np.asarray(seq_idx)[b]
    return (s[k:] == s[: T - k]).astype(np.float64)[:, None]


def conv_fwd(x, w, H: int = 1, seq_idx=None, conv_bias=None) -> np.ndarray:
    """Forward of eq. 2 + eq. 3: y_t = x_t + sum_{k<W} w_k^{(t)} * x_{t-k}, zero for t-k < 0
    (and, with seq_idx, for t-k in another segment than t), plus conv_bias (D,) if given.

    x: (B, T, D). w: (B, T, D/H, W) per-token filters, or (D/H, W) for a static filter
    (eq. 1). Returns y: (B, T, D) in float64.
    """
    x = _f64(x)
    w = _f64(w)
    B, T, D = x.shape
    W = w.shape[-1]
    y = x.copy()  # residual, eq. 3
    for b in range(B):
        wf = _filters_for_sequence(w, b, D, H)
        for k in range(W):
            if k >= T:
                break
            # term k reads x_{t-k}; rows t < k have no term (zeros before t = 0)
            m = _same_segment(seq_idx, b, k, T)
            if wf.ndim == 2:
                y[b, k:, :] += m * wf[None, :, k] * x[b, : T - k, :]
            else:
                y[b, k:, :] += m * wf[k:, :, k] * x[b, : T - k, :]
    if conv_bias is not None:
        y += _f64(conv_bias)[None, None, :]  # every token, every sequence
    return y


def conv_bias_grad(dy) -> np.ndarray:
    """Gradient of <dy, y> with respect to the convolution bias: y is c plus terms free of
    c, so dc[d] = sum over every (b, t) of dy[b, t, d]. Returns (D,) float64."""
    return _f64(dy).sum(axis=(0, 1))


def conv_bwd(x, w, dy, H: int = 1, seq_idx=None):
    """Gradients of <dy, y> for y = conv_fwd(x, w, H, seq_idx).

    Since y is bilinear in (x, w):
      dx_s = dy_s + sum_k w_k^{(s+k)} * dy_{s+k}            (terms with s + k < T and,
                                                            with seq_idx, s in the segment of s + k),
      dwfull[t, d, k] = dy_t[d] * x_{t-k}[d]               (zero for t - k < 0 or across segments),
      dw[t, g, k] = sum over the H channels d of group g of dwfull[t, d, k];
    for a static filter, dw[g, k] is additionally summed over every (b, t).
    Returns (dx, dw) in float64, dw in the layout of w.
    """
    x = _f64(x)
    w = _f64(w)
    dy = _f64(dy)
    B, T, D = x.shape
    W = w.shape[-1]
    G = D // H
    dx = dy.copy()  # residual path
    if w.ndim == 2:
        dw = np.zeros((G, W))
    else:
        dw = np.zeros((B, T, G, W))
    for b in range(B):
        wf = _filters_for_sequence(w, b, D, H)
        dwf = np.zeros((T, D, W))
        for k in range(W):
            if k >= T:
                break
            m = _same_segment(seq_idx, b, k, T)  # m[t - k]: tap k of token t present
            if wf.ndim == 2:
                dx[b, : T - k, :] += m * wf[None, :, k] * dy[b, k:, :]
            else:
                dx[b, : T - k, :] += m * wf[k:, :, k] * dy[b, k:, :]
            dwf[k:, :, k] = m * dy[b, k:, :] * x[b, : T - k, :]
        dwg = dwf.reshape(T, G, H, W).sum(axis=2)  # sum over the H channels of a group
        if w.ndim == 2:
            dw += dwg.sum(axis=0)
        else:
            dw[b] = dwg
    return dx, dw


def lowrank_filters(z, U, bias, W: int) -> np.ndarray:
    """Per-token filters of the low-rank generator's second projection: w = z U + b.

    z: (B, T, R); U: (R, (D/H)*W); bias: ((D/H)*W,) or None. Column j = g*W + k.
    Returns (B, T, D/H, W) float64.
    """
    z = _f64(z)
    U = _f64(U)
    B, T, R = z.shape
    J = U.shape[1]
    wf = np.matmul(z.reshape(B * T, R), U).reshape(B, T, J)
    if bias is not None:
        wf = wf + _f64(bias)[None, None, :]
    return wf.reshape(B, T, J // W, W)


def lowrank_fwd(x, z, U, bias, W: int, H: int = 1, seq_idx=None, conv_bias=None) -> np.ndarray:
    """Low-rank form: filters z U + b (never stored by the kernel), then eq. 2 + eq. 3, plus
    the optional convolution bias c (its gradient is conv_bias_grad(dy), whatever the
    filters)."""
    return conv_fwd(x, lowrank_filters(z, U, bias, W), H, seq_idx, conv_bias)


def lowrank_bwd(x, z, U, bias, dy, W: int, H: int = 1, seq_idx=None):
    """Gradients of <dy, y> for y = lowrank_fwd(x, z, U, bias, W, H, seq_idx).

    With g_t = dw_t flattened to (D/H)*W columns (from conv_bwd):
      dz_t = g_t U^T,   dU = sum_t z_t^T g_t,   db = sum_t g_t.
    Returns (dx, dz, dU, db) in float64.
    """
    z = _f64(z)
    U = _f64(U)
    wf = lowrank_filters(z, U, bias, W)
    dx, dw = conv_bwd(x, wf, dy, H, seq_idx)
    B, T, R = z.shape
    J = U.shape[1]
    g = dw.reshape(B * T, J)
    zf = z.reshape(B * T, R)
    dz = np.matmul(g, U.T).reshape(B, T, R)
    dU = np.matmul(zf.T, g)
    db = g.sum(axis=0)
    return dx, dz, dU, db


def projection(A, Wp) -> np.ndarray:
    """X = A W_p^T: A (B, T, K) activations, W_p (N, K) a linear layer's weight (out x in).
    Returns (B, T, N) float64."""
    A = _f64(A)
    Wp = _f64(Wp)
    B, T, K = A.shape
    return np.matmul(A.reshape(B * T, K), Wp.T).reshape(B, T, Wp.shape[0])


def gemm_conv_fwd(A, Wp, w, H: int = 1) -> np.ndarray:
    """The convolution applied to the projection's output: y = X + conv(X) with
    X = A W_p^T and per-token (B, T, N/H, W) or static (N/H, W) filters w."""
    return conv_fwd(projection(A, Wp), w, H)


def gemm_lowrank_fwd(A, Wp, z, U, bias, W: int, H: int = 1) -> np.ndarray:
    """The same with low-rank filters z U + bias (U: (R, (N/H)*W), column j = g*W + k)."""
    return lowrank_fwd(projection(A, Wp), z, U, bias, W, H)
