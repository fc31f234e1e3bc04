"""MI355X-native dynamic short convolution: HIP kernels for gfx950 behind a C ABI.

The Python surface mirrors the C entry points of include/dynconv.h:
dynconv_fwd, dynconv_bwd, dynconv_lowrank_fwd, dynconv_lowrank_bwd (and the workspace
queries). Importing this package does not load the library; the first call does, and
fails loudly if it has not been built.
"""
from .ops import (  # noqa: F401
    dynconv_bwd,
    dynconv_bwd_workspace_size,
    dynconv_fwd,
    dynconv_lowrank_bwd,
    dynconv_lowrank_bwd_workspace_size,
    dynconv_lowrank_fwd,
)
from ._lib import DynconvError, load  # noqa: F401
