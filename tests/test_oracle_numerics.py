"""Pins for the oracle's storage roundings and the input generator's bf16 encoding.

bf16 rounding is pinned against PyTorch's own fp32 -> bfloat16 conversion (an
independent library routine) and against hand-worked ties.
"""

import numpy as np
import pytest
import torch

from mdm_inputs import bf16_bits_from_f32, bf16_bits_to_f32
from oracle.numerics import round_bf16, round_f32, table_values


def _torch_bf16(x32):
    return torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()


def test_round_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000), rng.standard_normal(20000) * 1e-20,
                        rng.standard_normal(20000) * 1e20]).astype(np.float32)
    assert np.array_equal(round_bf16(x.astype(np.float64)), _torch_bf16(x))


def test_round_bf16_ties_go_to_even():
    # spacing of bf16 just above 1 is 2**-7
    assert round_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0                    # tie -> even (1.0)
    assert round_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6      # tie -> even (..10)
    assert round_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -30]))[0] == 1 + 2.0 ** -7   # above tie
    assert round_bf16(np.array([-(1 + 3 * 2.0 ** -8)]))[0] == -(1 + 2.0 ** -6)


def test_round_bf16_float64_inputs_round_once():
    # a float64 just above a bf16 tie must round up; rounding through fp32 first
    # would land exactly on the tie and go to even (down)
    x = np.array([1 + 2.0 ** -8 + 2.0 ** -40])
    assert round_bf16(x)[0] == 1 + 2.0 ** -7
    assert _torch_bf16(x.astype(np.float32))[0] == 1.0


def test_round_bf16_rejects_out_of_range():
    with pytest.raises(ValueError):
        round_bf16(np.array([1e39]))
    with pytest.raises(ValueError):
        round_bf16(np.array([1e-39]))


def test_round_f32():
    x = np.array([1 + 2.0 ** -24, 1 + 3 * 2.0 ** -24, 0.1])
    assert round_f32(x)[0] == 1.0
    assert round_f32(x)[1] == 1 + 2.0 ** -22
    assert round_f32(x)[2] == float(np.float32(0.1))


def test_generator_bf16_encoding_matches_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(100000).astype(np.float32)
    bits = bf16_bits_from_f32(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, want)
    assert np.array_equal(bf16_bits_to_f32(bits).astype(np.float64), table_values(bits))


def test_top_two_matches_a_scan_with_ties():
    """The two best (index, value) pairs per row, pinned by a plain scan that
    keeps the first index of equal values; rows with ties included."""
    from oracle.logits import top_two
    rng = np.random.default_rng(5)
    z = rng.integers(-4, 5, size=(300, 17)).astype(np.float64)      # many equal values
    z[:5] = 2.0                                                     # all equal
    idx, val = top_two(z)
    for r in range(z.shape[0]):
        row = list(z[r])
        b1 = 0
        for j in range(len(row)):
            if row[j] > row[b1]:
                b1 = j
        b2 = 1 if b1 == 0 else 0
        for j in range(len(row)):
            if j != b1 and row[j] > row[b2]:
                b2 = j
        assert (idx[r, 0], idx[r, 1]) == (b1, b2)
        assert (val[r, 0], val[r, 1]) == (row[b1], row[b2])
