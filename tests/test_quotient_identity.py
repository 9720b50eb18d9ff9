"""The bulk E4M3 quantiser forms x / scale as fp32((double)x * (1 / (double)scale))
instead of an fp32 division.  These host tests check, with numpy's correctly
rounded float32 division as the reference, that the two agree wherever the
quotient is a normal fp32 number, and that below that range they encode to
the same E4M3 code (the oracle's encoder decides)."""
from __future__ import annotations

import numpy as np

from oracle import e4m3


def _via_double(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    inv = 1.0 / s.astype(np.float64)
    return (x.astype(np.float64) * inv).astype(np.float32)


def _check(x: np.ndarray, s: np.ndarray) -> int:
    with np.errstate(all="ignore"):
        want = (x / s).astype(np.float32)
        got = _via_double(x, s)
    normal = np.abs(want) >= np.float32(2.0 ** -126)
    assert np.array_equal(want[normal].view(np.uint32), got[normal].view(np.uint32))
    tiny = ~normal
    if tiny.any():
        clip = lambda v: np.clip(v.astype(np.float64), -448.0, 448.0)
        assert np.array_equal(e4m3.encode(clip(want[tiny])), e4m3.encode(clip(got[tiny])))
    return int(normal.sum())


def test_random_pairs_over_the_quantisers_range():
    rng = np.random.default_rng(20)
    n = 2_000_000
    amax = np.exp2(rng.uniform(-20, 20, n)).astype(np.float32)
    s = (amax / np.float32(448.0)).astype(np.float32)
    x = (amax * rng.uniform(-1, 1, n)).astype(np.float32)
    assert _check(x, s) > 0.99 * n


def test_quotients_next_to_fp32_rounding_midpoints():
    """x = fp32(m * s) for m an fp32 rounding midpoint (a 25-bit odd
    significand): the quotient x / s then lies as close to a midpoint as
    fp32 operands allow."""
    rng = np.random.default_rng(21)
    n = 2_000_000
    sig = (rng.integers(1 << 24, 1 << 25, n) | 1).astype(np.float64)   # 25-bit odd
    m = sig * np.exp2(rng.integers(-30, 8, n) - 24.0)
    s = np.exp2(rng.uniform(-10, 10, n)).astype(np.float32)
    x = (m * s.astype(np.float64)).astype(np.float32)
    assert _check(x, s) > 0.99 * n


def test_power_of_two_scales_and_signed_zeros():
    x = np.array([0.0, -0.0, 1e-45, -1e-45, 3e-45, 448.0, -448.0, 1.0, -1.5], dtype=np.float32)
    for s in (np.float32(1.0), np.float32(0.5), np.float32(2.0 ** -20), np.float32(3.0)):
        _check(x, np.full_like(x, s))
    got = _via_double(np.array([-0.0], np.float32), np.array([2.0], np.float32))
    assert got.view(np.uint32)[0] == 0x80000000
