"""Comparison helpers for GPU-vs-oracle parity tests.

Gate (per output tensor): normwise relative max error
    max|gpu - ref| / max|ref|  <=  1e-5 (float32 path)  or  2e-2 (bf16 path, fp32 accumulate).
The pages state no float16 gate; the one here is derived the same way: the bf16 gate is
about 5 unit roundoffs of bf16 (2e-2 ~ 5 * 2^-8), so float16 gets 5 * 2^-11 ~ 2.5e-3.
Diagnostic bound (also asserted): elementwise
    |gpu - ref| <= rtol * |ref| + atol * max|ref|
with rtol = the unit roundoff of the stored 16-bit result (2^-8 bf16, 2^-11 float16) and
1e-6 for float32, plus atol for accumulation error.
"""
from __future__ import annotations

import numpy as np
import torch

GATE = {torch.float32: 1e-5, torch.bfloat16: 2e-2, torch.float16: 2.5e-3}
UNIT_ROUNDOFF = {torch.bfloat16: 2.0**-8, torch.float16: 2.0**-11}


def to64(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu").to(torch.float64).numpy()


def rel_max_err(got, ref) -> float:
    got = to64(got)
    ref = np.asarray(ref, dtype=np.float64)
    denom = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if denom == 0.0:
        return num
    return num / denom


def assert_close(name, got, ref, dtype, rtol=None, atol=None, extra=None):
    """Asserts the normwise gate and the elementwise bound; returns the normwise error.

    `extra` is an optional per-element allowance added to the bound (used where an
    operand is rounded to bf16 before a matrix-core product: 2^-8 * sum |terms|).
    """
    got64 = to64(got)
    ref = np.asarray(ref, dtype=np.float64)
    assert got64.shape == ref.shape, f"{name}: shape {got64.shape} != {ref.shape}"
    assert np.all(np.isfinite(got64)), f"{name}: non-finite values in the GPU output"
    err = rel_max_err(got64, ref)
    gate = GATE[dtype]
    assert err <= gate, f"{name}: normwise rel max err {err:.3e} > {gate:.0e}"
    if rtol is None:
        rtol = UNIT_ROUNDOFF.get(dtype, 1e-6)
    if atol is None:
        atol = 1e-5 if dtype in UNIT_ROUNDOFF else 2e-6
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    bound = rtol * np.abs(ref) + atol * scale
    if extra is not None:
        bound = bound + np.asarray(extra, dtype=np.float64)
    bad = np.abs(got64 - ref) > bound
    if np.any(bad):
        idx = np.argwhere(bad)[0]
        raise AssertionError(
            f"{name}: elementwise bound broken at {tuple(idx)}: got {got64[tuple(idx)]!r} ref {ref[tuple(idx)]!r} "
            f"({int(bad.sum())} of {bad.size} elements)"
        )
    return err
