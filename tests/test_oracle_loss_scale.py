"""Pins of the loss-scaling oracle: special values, exactness of power-of-two
scaling, and agreement with torch's own fused check-and-unscale routine."""
import numpy as np
import torch

import oracle


def test_special_values():
    for bad in (np.inf, -np.inf, np.nan):
        g, found = oracle.unscale_check_finite([1.0, bad, 3.0], 0.5)
        assert found
    g, found = oracle.unscale_check_finite([1.0, -2.0, 3.5e38], 1.0)
    assert not found


def test_power_of_two_scaling_is_exact():
    x = np.random.default_rng(1).standard_normal(1000).astype(np.float32)
    g, found = oracle.unscale_check_finite(x, 2.0 ** -12)
    assert not found
    np.testing.assert_array_equal(g, x.astype(np.float64) * 2.0 ** -12)
    np.testing.assert_array_equal((g * 2.0 ** 12).astype(np.float32), x)


def test_matches_torch_fused_routine():
    rng = np.random.default_rng(2)
    for planted in (False, True):
        x = rng.standard_normal(257).astype(np.float32) * 1000
        if planted:
            x[100] = np.nan
        t = [torch.from_numpy(x.copy())]
        flag = torch.zeros(1)
        torch._amp_foreach_non_finite_check_and_unscale_(t, flag, torch.tensor(1.0 / 1024))
        g, found = oracle.unscale_check_finite(x, 1.0 / 1024)
        assert found == bool(flag.item())
        np.testing.assert_allclose(t[0].numpy(), g, rtol=1e-7, equal_nan=True)
