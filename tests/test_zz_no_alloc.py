"""GPU test of the allocation-free backward, dynconv_bwd_ex_noalloc, through the C ABI.

It must give what dynconv_bwd_ex gives with a caller's workspace (same kernels, same plan,
same fixed-order reduce, so the results are bit-identical), on two calls in a row where the
second is smaller: the scratch array keeps the first call's partial sums, and every one the
second call reads must be its own. A static filter with a convolution bias uses both
partial-sum regions; a per-token filter with a bias uses only the bias partials.
"""
import pytest
import torch

import synth
from dynamic_short_convolution_amd.ops import dynconv_bwd, dynconv_bwd_ex_noalloc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    yield
    torch.cuda.synchronize()


def _inputs(B, T, D, W, H, static, seed, dtype="bf16", packed=False):
    x = synth.draw((B, T, D), 1.0, seed, "x", dtype).cuda()
    dy = synth.draw((B, T, D), 1.0, seed, "dy", dtype).cuda()
    w = synth.draw((D // H, W) if static else (B, T, D // H, W), (1.0 / W) ** 0.5, seed, "w", dtype).cuda()
    seq = synth.segments(B, T, 15.0, seed, first=(1, 2)).cuda() if packed else None
    return x, w, dy, seq


def _outputs(x, w, H):
    B, T, D = x.shape
    W = w.shape[-1]
    dx = torch.full_like(x, float("nan"))
    dw = torch.full((D // H, W) if w.dim() == 2 else (B, T, D // H, W), float("nan"),
                    dtype=torch.float32 if w.dim() == 2 else x.dtype, device=x.device)
    dcb = torch.full((D,), float("nan"), dtype=torch.float32, device=x.device)
    return dx, dw, dcb


def _same(name, got, ref):
    assert got.shape == ref.shape, name
    assert torch.equal(got.view(torch.int16) if got.element_size() == 2 else got.view(torch.int32),
                       ref.view(torch.int16) if ref.element_size() == 2 else ref.view(torch.int32)), \
        f"{name}: the allocation-free call differs from the call with a workspace"


@pytest.mark.parametrize("static,H,W,dtype,packed", [
    (True, 1, 3, "bf16", False),
    (True, 4, 4, "f32", False),
    (False, 1, 4, "bf16", False),
    (False, 16, 4, "f16", True),
])
def test_noalloc_equals_workspace_call_twice(static, H, W, dtype, packed):
    # first call: many time chunks and channels; second: a smaller one on the same scratch
    for i, (B, T, D) in enumerate(((4, 3000, 1024), (2, 333, 256))):
        x, w, dy, seq = _inputs(B, T, D, W, H, static, 40 + i, dtype, packed)
        rdx, rdw, rdcb = dynconv_bwd(x, w, dy, H, seq_idx=seq, want_dconv_bias=True)
        dx, dw, dcb = _outputs(x, w, H)
        dynconv_bwd_ex_noalloc(x, w, dy, H, dx=dx, dw=dw, dconv_bias=dcb, seq_idx=seq)
        torch.cuda.synchronize()
        print(f"noalloc call {i}: B={B} T={T} D={D} W={W} H={H} static={static} {dtype}", flush=True)
        _same("dx", dx, rdx)
        _same("dw", dw, rdw)
        _same("dconv_bias", dcb, rdcb)


def test_noalloc_static_dw_without_bias_and_dx_only():
    """dw of a static filter alone (no bias), then dx alone (no scratch use at all)."""
    B, T, D, W, H = 3, 700, 512, 4, 1
    x, w, dy, _ = _inputs(B, T, D, W, H, True, 51)
    _, rdw = dynconv_bwd(x, w, dy, H, need_dx=False)
    dw = torch.full((D, W), float("nan"), dtype=torch.float32, device=x.device)
    dynconv_bwd_ex_noalloc(x, w, dy, H, dw=dw)
    _same("dw", dw, rdw)
    rdx, _ = dynconv_bwd(x, w, dy, H, need_dw=False)
    dx = torch.full_like(x, float("nan"))
    dynconv_bwd_ex_noalloc(x, w, dy, H, dx=dx)
    torch.cuda.synchronize()
    _same("dx", dx, rdx)

