"""The bf16 output allowance used by the parity checks is exactly the format's
rounding bound: half an ulp at the tensor's largest magnitude."""
import numpy as np

from tests.parity import bf16_half_ulp


def test_half_ulp_values():
    assert bf16_half_ulp(np.array([0.0])) == 0.0
    assert bf16_half_ulp(np.array([1.0])) == 2.0 ** -8
    assert bf16_half_ulp(np.array([-9.3, 0.5])) == 2.0 ** -5
    assert bf16_half_ulp(np.array([0.3])) == 2.0 ** -10


def test_half_ulp_bounds_round_to_nearest():
    import torch
    r = np.random.default_rng(0)
    for lo in (0.01, 0.9, 8.0, 100.0):
        x = r.uniform(lo, 2 * lo, size=20000).astype(np.float32)
        xb = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
        err = np.abs(xb - x.astype(np.float64))
        assert err.max() <= bf16_half_ulp(x)
        # and it is nearly attained: the bound is not loose
        assert err.max() >= 0.9 * bf16_half_ulp(x)
