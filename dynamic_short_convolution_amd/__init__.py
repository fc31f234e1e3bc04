"""MI355X-native dynamic short convolution: HIP kernels for gfx950 behind a C ABI.

The Python surface mirrors the C entry points of include/dynconv.h:
dynconv_fwd, dynconv_bwd, dynconv_lowrank_fwd, dynconv_lowrank_bwd (and the workspace
queries), and for inference dynconv_cache_fill, dynconv_decode_step and
dynconv_lowrank_decode_step (with new_cache for a zeroed rolling cache), and the
convolution fused into its producing projection, dynconv_gemm_fwd and
dynconv_gemm_lowrank_fwd. Importing this package does not load the library; the first call does, and
fails loudly if it has not been built.
"""
from .ops import (  # noqa: F401
    dynconv_bwd,
    dynconv_bwd_workspace_size,
    dynconv_cache_fill,
    dynconv_decode_step,
    dynconv_fwd,
    dynconv_gemm_fwd,
    dynconv_gemm_lowrank_fwd,
    dynconv_lowrank_bwd,
    dynconv_lowrank_bwd_workspace_size,
    dynconv_lowrank_decode_step,
    dynconv_lowrank_fwd,
    new_cache,
)
from ._lib import DynconvError, load  # noqa: F401
