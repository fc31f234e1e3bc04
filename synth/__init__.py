"""Seeded synthetic inputs for the dynamic short convolution.

This module is shared by the tests, the benchmark and the oracle checks. It holds
none of the convolution's arithmetic: it only draws i.i.d. Gaussian values with a
counter-seeded NumPy generator, scales them to a stated standard deviation and
rounds them to the storage dtype (round-to-nearest-even for bfloat16, via torch's
own cast). The same bits are handed to the HIP path and, upcast to float64, to the
oracle.

Distribution notation: ``N(0, v)`` in the workload descriptions means variance
``v`` (plain N(mu, sigma^2) notation), so ``std = sqrt(v)``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

# Fixed stream index per named tensor, so every tensor of a workload has its own stream.
TENSOR_STREAM = {
    "x": 0,
    "w": 1,
    "dy": 2,
    "z": 3,
    "U": 4,
    "b": 5,
    "w_static": 6,
    "probe": 7,
    "seg": 8,
    "c": 9,  # convolution bias (the low-rank tests, whose "b" is the generator bias)
}

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def draw(shape, std: float, seed: int, name: str, dtype: str) -> torch.Tensor:
    """Return a CPU tensor of ``shape`` with i.i.d. N(0, std**2) values in ``dtype``.

    The generator is ``numpy.random.default_rng([seed, TENSOR_STREAM[name]])``; values
    are drawn in float32, multiplied by ``std`` in float32 and cast to the storage dtype.
    """
    rng = np.random.default_rng([int(seed), TENSOR_STREAM[name]])
    n = int(np.prod(shape)) if len(shape) else 1
    out = torch.empty(n, dtype=DTYPES[dtype])
    # Chunked so that very large tensors do not need a second full-size float32 copy.
    chunk = 1 << 24
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        a = rng.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            a *= np.float32(std)
        out[s:e] = torch.from_numpy(a).to(DTYPES[dtype])
    return out.reshape(shape)


def segments(B: int, T: int, mean_len: float, seed: int, first=()) -> torch.Tensor:
    """Segment ids int32 [B, T] of packed sequences: each row is a run of documents whose
    lengths are 1 + round(Exponential(mean_len - 1)) (the last one cut at T), with ids
    0, 1, 2, ... along the row. ``first`` lists the lengths of row 0's leading documents
    (e.g. 1 and 2 to put documents shorter than the filter at the start).
    Generator: ``numpy.random.default_rng([seed, TENSOR_STREAM["seg"]])``."""
    rng = np.random.default_rng([int(seed), TENSOR_STREAM["seg"]])
    out = np.zeros((B, T), dtype=np.int32)
    for b in range(B):
        lens = list(first) if b == 0 else []
        while sum(lens) < T:
            lens.append(1 + int(round(rng.exponential(max(mean_len - 1.0, 1e-9)))))
        pos = 0
        for i, n in enumerate(lens):
            out[b, pos : min(T, pos + n)] = i
            pos += n
            if pos >= T:
                break
    return torch.from_numpy(out)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a CPU tensor (bf16 and f32 values are exact in f64)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


@dataclass
class Workload:
    """One synthetic workload: shapes, dtype, form and the distributions of its tensors."""

    name: str
    B: int
    T: int
    D: int
    W: int
    H: int = 1
    R: int = 0  # 0: materialised filters; >0: low-rank generator of rank R
    dtype: str = "bf16"
    static: bool = False
    seed: int = 0
    w_var: float | None = None  # variance of materialised / static filters
    u_scale: float = 0.1  # U = u_scale * N(0, 1/R)
    b_var: float = 0.1  # bias ~ N(0, b_var)
    split: tuple = field(default_factory=tuple)  # channel split of a fused launch (Q|K|V)

    @property
    def G(self) -> int:
        return self.D // self.H

    @property
    def J(self) -> int:
        return self.G * self.W

    def x(self) -> torch.Tensor:
        return draw((self.B, self.T, self.D), 1.0, self.seed, "x", self.dtype)

    def dy(self) -> torch.Tensor:
        return draw((self.B, self.T, self.D), 1.0, self.seed, "dy", self.dtype)

    def w(self) -> torch.Tensor:
        var = self.w_var if self.w_var is not None else 1.0 / self.W
        if self.static:
            return draw((self.G, self.W), math.sqrt(var), self.seed, "w_static", self.dtype)
        return draw((self.B, self.T, self.G, self.W), math.sqrt(var), self.seed, "w", self.dtype)

    def z(self) -> torch.Tensor:
        return draw((self.B, self.T, self.R), 1.0, self.seed, "z", self.dtype)

    def U(self) -> torch.Tensor:
        return draw((self.R, self.J), self.u_scale / math.sqrt(self.R), self.seed, "U", self.dtype)

    def b(self) -> torch.Tensor:
        return draw((self.J,), math.sqrt(self.b_var), self.seed, "b", self.dtype)


def workloads() -> dict:
    """The named workloads, with the shapes of the pages' 150M-2B models (D=2048, T=4096)."""
    return {
        # Tiny per-channel case the oracle finishes instantly.
        "tiny_perchannel_f32": Workload("tiny_perchannel_f32", 1, 64, 32, 4, 1, dtype="f32", seed=1),
        # Head-wise (16 channels per filter), bf16.
        "headwise_h16": Workload("headwise_h16", 8, 4096, 2048, 4, 16, seed=2),
        # Static W=3 filter, same activations as the head-wise case.
        "static_w3": Workload("static_w3", 8, 4096, 2048, 3, 1, static=True, seed=2, w_var=1.0 / 3.0),
        # Post-QKV GQA shape: Q 2048 | K 512 | V 512 channels in one launch.
        "qkv_gqa_fused": Workload("qkv_gqa_fused", 4, 8192, 3072, 4, 1, seed=3, split=(2048, 512, 512)),
        # Low-rank generator, rank 64.
        "lowrank_r64": Workload("lowrank_r64", 8, 4096, 2048, 4, 1, R=64, seed=4),
        # Per-channel / head-wise backward sweep shapes.
        "perchannel_h1": Workload("perchannel_h1", 8, 4096, 2048, 4, 1, seed=5),
        "headwise_h4": Workload("headwise_h4", 8, 4096, 2048, 4, 4, seed=5),
        "headwise_h16_bwd": Workload("headwise_h16_bwd", 8, 4096, 2048, 4, 16, seed=5),
        "lowrank_r64_bwd": Workload("lowrank_r64_bwd", 8, 4096, 2048, 4, 1, R=64, seed=5),
        # Head-wise groups whose size is not a power of two: 12 channels per filter, D = 3072.
        "headwise_h12": Workload("headwise_h12", 8, 4096, 3072, 4, 12, seed=6),
    }
