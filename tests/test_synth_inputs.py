"""The seeded input generator: determinism, distributions and bf16 round-to-nearest-even."""
import numpy as np
import torch

import synth


def _rne_bf16_bits(a32: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even of finite float32 values to bfloat16, on the bit pattern."""
    u = a32.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def test_bf16_rounding_is_rne():
    rng = np.random.default_rng([3, synth.TENSOR_STREAM["x"]])
    a = rng.standard_normal(1 << 16, dtype=np.float32) * np.float32(0.5)
    t = synth.draw((1 << 16,), 0.5, 3, "x", "bf16")
    got = t.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, _rne_bf16_bits(a))


def test_ties_round_to_even():
    # 1 + 2^-8 lies exactly between two bf16 values (1 and 1 + 2^-7): ties go to the even one (1)
    a = np.array([1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8], dtype=np.float32)
    got = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, _rne_bf16_bits(a))
    assert got[0] == 0x3F80 and got[1] == 0x3F82


def test_deterministic_and_distinct_streams():
    a = synth.draw((4, 8), 1.0, 7, "x", "f32")
    b = synth.draw((4, 8), 1.0, 7, "x", "f32")
    c = synth.draw((4, 8), 1.0, 7, "dy", "f32")
    assert torch.equal(a, b) and not torch.equal(a, c)


def test_std_follows_variance_notation():
    wl = synth.Workload("t", 2, 512, 64, 4, 1, dtype="f32", seed=9)
    w = wl.w().numpy()
    assert abs(w.std() - 0.5) < 0.01  # N(0, 1/W) with W = 4 has std 1/2
    wl = synth.Workload("t", 2, 512, 64, 4, 1, R=64, dtype="f32", seed=9)
    assert abs(wl.U().numpy().std() - 0.1 / 8) < 0.001
    assert abs(wl.b().numpy().std() - np.sqrt(0.1)) < 0.02
