"""The ulp helpers every parity comparison goes through (tests/ulp.py), against an independent
definition: the distance between two finite bf16 values is how many representable values apart
they are, counted in the sorted list of all finite bf16 values with +0 and -0 as one value."""
import numpy as np
import torch

from ulp import is_nan, ulp_diff


def _finite_values_sorted():
    """Positions of every finite bf16 pattern in the sorted list of distinct finite values."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    finite = np.isfinite(vals)
    distinct = np.unique(vals[finite])  # -0.0 == +0.0, so the two zeros are one value
    pos = np.full(1 << 16, -1, dtype=np.int64)
    pos[finite] = np.searchsorted(distinct, vals[finite])
    return bits, vals, finite, pos


def test_ulp_diff_counts_representable_values_between():
    bits, vals, finite, pos = _finite_values_sorted()
    fin = bits[finite]
    rng = np.random.default_rng(3)
    a = rng.choice(fin, 200_000)
    b = rng.choice(fin, 200_000)
    # pairs a few values apart, where the 1-ulp decisions are taken
    near = rng.choice(fin, 50_000)
    step = rng.integers(-3, 4, near.size)
    idx = np.clip(pos[near] + step, 0, pos[finite].max())
    inv = np.full(pos.max() + 1, 0, dtype=np.uint16)
    inv[pos[finite]] = bits[finite]
    a = np.concatenate([a, near])
    b = np.concatenate([b, inv[idx]])
    assert np.array_equal(ulp_diff(a, b), np.abs(pos[a] - pos[b]))


def test_ulp_diff_edge_cases():
    z, nz = np.uint16(0x0000), np.uint16(0x8000)
    assert ulp_diff(z, nz) == 0                              # +0 and -0 are the same value
    assert ulp_diff(np.uint16(0x0001), np.uint16(0x8001)) == 2  # across zero
    assert ulp_diff(np.uint16(0x3F80), np.uint16(0x3F81)) == 1  # 1.0 and its successor
    assert ulp_diff(np.uint16(0x3F80), np.uint16(0xBF80)) == 2 * 0x3F80
    assert ulp_diff(np.uint16(0x7F7F), np.uint16(0x7F80)) == 1  # largest finite to +inf


def test_is_nan_matches_the_float_view():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(is_nan(bits), np.isnan(vals))
