"""float64 CPU oracle of the dynamic short convolution (test infrastructure only).

Used by the tests, the package smoke check and the benchmark's CPU-baseline leg; never
by the product path. See ``dynconv_oracle`` for what it computes and where it comes from.
"""
from .dynconv_oracle import (  # noqa: F401
    conv_bias_grad,
    conv_bwd,
    conv_fwd,
    gemm_conv_fwd,
    gemm_lowrank_fwd,
    lowrank_bwd,
    lowrank_filters,
    lowrank_fwd,
    projection,
)
