"""The BF16 half-ulp term of the output bound matches torch's BF16 rounding (CPU)."""
import numpy as np
import torch

from gpu_util import bf16_half_ulp


def test_half_ulp_bounds_round_to_nearest():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 0.1, 1.0, 3.0, 100.0)])
    r = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    err = np.abs(r - x)
    hu = bf16_half_ulp(x)
    # correct rounding never exceeds half an ulp (plus the float32 step of the input)
    assert np.all(err <= hu * (1 + 1e-6) + np.abs(x) * 2.0 ** -24)
    # and the bound is tight: some values get close to it
    assert (err / hu).max() > 0.99


def test_half_ulp_values():
    assert bf16_half_ulp(1.0) == 2.0 ** -8
    assert bf16_half_ulp(1.99) == 2.0 ** -8
    assert bf16_half_ulp(2.0) == 2.0 ** -7
    assert bf16_half_ulp(-3.5) == 2.0 ** -7
    assert bf16_half_ulp(0.5) == 2.0 ** -9
