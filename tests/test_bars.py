"""CPU pins of the parity bar used by the GPU tests (tests/_bars.py)."""
import numpy as np
import pytest
import torch

import _bars as bars


def test_bf16_ulp_is_the_spacing_of_bf16_numbers():
    # bf16 keeps 8 significant bits: spacing 2^-7 on [1, 2), 2^-4 on [8, 16)
    for v, ulp in [(1.0, 2.0 ** -7), (1.99, 2.0 ** -7), (2.0, 2.0 ** -6), (7.99, 2.0 ** -5),
                   (8.0, 2.0 ** -4), (-9.5, 2.0 ** -4), (16.0, 2.0 ** -3), (0.3, 2.0 ** -9)]:
        assert bars.bf16_ulp(v) == ulp, v
    # against the bf16 format itself: the gap from a positive bf16 number to the next one up
    b = torch.from_numpy(np.random.default_rng(1).uniform(1e-3, 100.0, 4096)).to(torch.bfloat16)
    nxt = (b.view(torch.int16) + 1).view(torch.bfloat16)
    gap = (nxt.double() - b.double()).numpy()
    np.testing.assert_array_equal(bars.bf16_ulp(b.double().numpy()), gap)


def test_bound_is_2e2_below_4_and_one_ulp_from_4():
    ref = np.array([0.0, 3.9, -4.0, 7.99, 8.0, -12.0, 20.0])
    np.testing.assert_array_equal(
        bars.abs_bound(ref), [2e-2, 2e-2, 2.0 ** -5, 2.0 ** -5, 2.0 ** -4, 2.0 ** -4, 2.0 ** -3])


def test_exact_results_rounded_to_bf16_pass_and_offsets_fail():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((64, 256)) * 6.0          # values up to about 25 in magnitude
    got = torch.from_numpy(ref).float().to(torch.bfloat16)
    bars.check_close(got, ref, "rounded exact")         # the output's own rounding passes
    small = np.full((4, 4), 3.0)
    with pytest.raises(AssertionError):
        bars.check_close(torch.from_numpy(small + 0.021).float(), small, "offset below 4")
    big = np.full((4, 4), 10.0)
    bars.check_close(torch.from_numpy(big + 0.06).float(), big, "within an ulp above 8")
    with pytest.raises(AssertionError):
        bars.check_close(torch.from_numpy(big + 0.07).float(), big, "offset above 8")


def test_act_rounding_matches_bf16_conversion():
    import _fullsize as fs
    a = np.random.default_rng(2).standard_normal(100_000) * np.exp(
        np.random.default_rng(3).uniform(-8, 8, 100_000))
    want = torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(fs.round_act_bf16(a), want)
