"""The output bar of the parity tests (tests/_ref.py), checked on the CPU:
its exact rounding agrees with torch's casts, and the bar accepts exactly
the roundings of values within 2e-3 (1e-5 for fp32) of the oracle."""

import numpy as np
import pytest
import torch

from _ref import assert_close, round_to

TD = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
def test_round_to_matches_torch_casts(dt):
    r = np.random.default_rng(3)
    x = np.concatenate([r.standard_normal(20000) * s for s in (1e-6, 1e-3, 1.0, 100.0)])
    if dt != "f32":  # float32 inputs: torch rounds them once, as round_to does
        x = x.astype(np.float32).astype(np.float64)
    want = torch.from_numpy(x).to(TD[dt]).to(torch.float64).numpy()
    assert np.array_equal(round_to(x, dt), want)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_bar_accepts_roundings_within_it_and_nothing_else(dt):
    r = np.random.default_rng(4)
    ref = r.standard_normal(5000) * 2.0
    ok = round_to(ref + r.uniform(-2e-3, 2e-3, ref.size), dt)     # kernel results within the bar
    assert_close(ok, ref, dt)
    far = round_to(ref + 2.6e-3 * np.sign(r.standard_normal(ref.size)), dt)
    # only the values whose rounding step is coarse enough to land back in
    # [rn(ref - 2e-3), rn(ref + 2e-3)] may pass; the small ones must fail
    small = np.abs(ref) < 0.25
    with pytest.raises(AssertionError):
        assert_close(far[small], ref[small], dt)


def test_fp32_bar():
    ref = np.linspace(-3, 3, 101)
    assert_close(ref + 0.9e-5, ref, "f32")
    with pytest.raises(AssertionError):
        assert_close(ref + 1.2e-5, ref, "f32")
