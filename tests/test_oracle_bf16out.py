"""Pins for the oracle's bfloat16 output rounding (CPU only): round to
nearest, ties to even, in one step from the exact value.  Checked against
torch's float32 -> bfloat16 conversion (round to nearest even) on float32
inputs, hand-made ties and near-ties (including one that rounding through
float32 first would get wrong), exact bfloat16 values (unchanged), signs and
powers of two."""
import numpy as np
import torch

import oracle


def test_matches_torch_on_float32_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(0, 1, 20000), rng.normal(0, 1e3, 5000),
                        rng.normal(0, 1e-3, 5000)]).astype(np.float32)
    ref = torch.from_numpy(x).bfloat16().float().double().numpy()
    assert np.array_equal(oracle.round_to_bf16(x.astype(np.float64)), ref)


def test_ties_go_to_even():
    u = 2.0 ** -7  # spacing of bfloat16 values in [1, 2)
    x = np.array([1 + u / 2, 1 + 3 * u / 2, -(1 + u / 2), 2 + u, 0.5 + u / 4])
    want = np.array([1.0, 1 + 2 * u, -1.0, 2.0, 0.5])
    assert np.array_equal(oracle.round_to_bf16(x), want)


def test_one_step_rounding():
    """1 + 2^-8 + 2^-40 lies above the midpoint between 1 and 1 + 2^-7: it
    rounds up.  Rounding to float32 first gives the tie 1 + 2^-8, which
    would then go to the even neighbour 1."""
    x = np.array([1 + 2.0 ** -8 + 2.0 ** -40, 1 + 2.0 ** -8 - 2.0 ** -40])
    assert np.array_equal(oracle.round_to_bf16(x), [1 + 2.0 ** -7, 1.0])


def test_exact_values_and_powers_of_two_unchanged():
    vals = torch.randn(5000, dtype=torch.float32).bfloat16().double().numpy()
    assert np.array_equal(oracle.round_to_bf16(vals), vals)
    p = np.ldexp(1.0, np.arange(-120, 120))
    assert np.array_equal(oracle.round_to_bf16(p), p)
    assert np.array_equal(oracle.round_to_bf16(-p), -p)
    # just below a power of two rounds up to it
    assert np.array_equal(oracle.round_to_bf16(np.nextafter(p, 0)), p)
    assert oracle.round_to_bf16(np.array([0.0]))[0] == 0.0


def test_values_next_to_powers_of_two_use_the_right_spacing():
    """Brute force: every value on a fine grid just below and above 2^k
    rounds to the nearest of the bfloat16 values around it."""
    for k in (-3, 0, 5, 17):
        p = 2.0 ** k
        grid = np.concatenate([p * (1 - np.arange(1, 400) * 2.0 ** -12),
                               p * (1 + np.arange(0, 400) * 2.0 ** -12)])
        cand = np.concatenate([p * (1 - np.arange(0, 40) * 2.0 ** -8),
                               p * (1 + np.arange(0, 40) * 2.0 ** -7)])
        got = oracle.round_to_bf16(grid)
        for x, g in zip(grid, got):
            d = np.abs(cand - x)
            best = cand[d == d.min()]
            assert g in best, (k, x, g, best)
