"""The GPU tests' own acceptance checks, on the CPU: each fails on a planted
error of the kind it is meant to catch and passes the noise it allows."""
import numpy as np
import pytest


def _fp8_case(seed=0, rows=256, d=128):
    g = np.random.default_rng(seed)
    o_ref = g.standard_normal((rows, d)) * 0.05
    lse = g.standard_normal(rows)
    return o_ref, lse


def test_check_fp8_unbiased_noise_passes():
    from test_attn_fp8_gpu import check_fp8
    o_ref, lse = _fp8_case()
    noise = np.random.default_rng(1).standard_normal(o_ref.shape) * 0.02 * np.abs(o_ref).mean()
    check_fp8(o_ref + noise, lse, o_ref, lse)


@pytest.mark.parametrize("factor", [0.99, 1.01])
def test_check_fp8_systematic_scale_fails(factor):
    """A 1% shrink or growth of every output passes the normwise and max
    gates (5e-2) but not the unbiasedness gate (5e-3)."""
    from test_attn_fp8_gpu import check_fp8
    o_ref, lse = _fp8_case()
    with pytest.raises(AssertionError, match="along o_ref"):
        check_fp8(o_ref * factor, lse, o_ref, lse)
