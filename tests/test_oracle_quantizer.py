"""Pins of the oracle's quantiser against what the pages and arithmetic fix.

The quantiser is the asymmetric min-max group quantiser of the KIVI paper card
(method paragraph) and news article (asymmetry paragraph); scale = range / L,
zero = min, round half to even.  These tests do not re-type that formula: they
check invariants any correct implementation must satisfy (constant groups
reproduced exactly, error within half a step, extremes hit 0 and L, nearest
level, hand-worked ties) and the pages' qualitative claim that per-channel key
groups beat per-token key groups on outlier-channel keys.
"""
import numpy as np
import pytest

import oracle

FLT_MIN = np.float32(np.finfo(np.float32).tiny)


def _bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 value (as fp32), ties to even."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32)


def _groups(rng, n, bits_scale=1.0):
    for _ in range(n):
        kind = rng.integers(4)
        if kind == 0:
            x = rng.standard_normal(32) * bits_scale
        elif kind == 1:
            x = rng.uniform(-1e-3, 1e-3, 32)
        elif kind == 2:
            x = rng.standard_normal(32) * 40.0 + 100.0
        else:
            x = rng.standard_normal(32) * 1e-20
        yield _bf16_round(x.astype(np.float32))


@pytest.mark.parametrize("bits", [2, 4])
def test_constant_group_is_exact(bits):
    for val in [0.0, -3.25, 1e-30, 7.0e4, -2.0 ** -130]:
        x = _bf16_round(np.full(32, val, np.float32))
        codes, s, z = oracle.quantize_values(x, bits)
        assert s == 0.0 and np.all(codes == 0)
        deq = codes.astype(np.float64) * np.float64(s) + np.float64(z)
        assert np.array_equal(deq, x.astype(np.float64))


@pytest.mark.parametrize("bits", [2, 4])
def test_error_within_half_step(bits):
    L = (1 << bits) - 1
    rng = np.random.default_rng(bits)
    checked = 0
    for x in _groups(rng, 2000):
        codes, s, z = oracle.quantize_values(x, bits)
        assert codes.max() <= L
        assert z == x.min()
        if s < FLT_MIN:
            assert np.all(codes == 0)
            continue
        deq = codes.astype(np.float64) * np.float64(s) + np.float64(z)
        err = np.abs(x.astype(np.float64) - deq)
        bound = np.float64(s) * (0.5 + 3 * L * 2.0 ** -24)
        assert np.all(err <= bound), (x, codes, s, z)
        checked += 1
    assert checked > 1000


@pytest.mark.parametrize("bits", [2, 4])
def test_extremes_map_to_zero_and_top(bits):
    L = (1 << bits) - 1
    rng = np.random.default_rng(10 + bits)
    for x in _groups(rng, 500):
        codes, s, z = oracle.quantize_values(x, bits)
        if s < FLT_MIN:
            continue
        assert codes[np.argmin(x)] == 0
        assert codes[np.argmax(x)] == L


@pytest.mark.parametrize("bits", [2, 4])
def test_code_is_nearest_level(bits):
    L = (1 << bits) - 1
    rng = np.random.default_rng(20 + bits)
    for x in _groups(rng, 500):
        codes, s, z = oracle.quantize_values(x, bits)
        if s < FLT_MIN:
            continue
        levels = np.arange(L + 1, dtype=np.float64) * np.float64(s) + np.float64(z)
        dist = np.abs(x.astype(np.float64)[:, None] - levels[None, :])
        best = np.argmin(dist, axis=1)
        # near a midpoint two levels are equally good up to fp32 rounding
        t = (x.astype(np.float64) - np.float64(z)) / np.float64(s)
        near_mid = np.abs(t - np.floor(t) - 0.5) <= 3 * L * 2.0 ** -24 * 4
        assert np.all((codes == best) | near_mid)


def test_worked_ties_two_bit():
    # group {0, 0.5, 1.5, 2.5, 3, 3, ...}: min 0, max 3, scale 1, 1/scale 1
    # 0.5 -> rint 0 (half to even), 1.5 -> 2, 2.5 -> 2, 3 -> 3
    x = np.array([0.0, 0.5, 1.5, 2.5, 3.0] + [3.0] * 27, np.float32)
    codes, s, z = oracle.quantize_values(x, 2)
    assert (s, z) == (1.0, 0.0)
    assert list(codes[:5]) == [0, 0, 2, 2, 3]


def test_worked_ties_four_bit():
    # min 0, max 15 -> scale 1: 7.5 -> 8, 8.5 -> 8, 0.5 -> 0, 14.5 -> 14
    x = np.array([0.0, 15.0, 7.5, 8.5, 0.5, 14.5] + [1.0] * 26, np.float32)
    codes, s, z = oracle.quantize_values(x, 4)
    assert (s, z) == (1.0, 0.0)
    assert list(codes[:6]) == [0, 15, 8, 8, 0, 14]


def test_scaled_grid_is_reproduced():
    # values on an exact grid k*s + z are quantised to k and dequantise exactly
    for bits in (2, 4):
        L = (1 << bits) - 1
        k = np.array(list(range(L + 1)) * 32, np.int64)[:32]
        k[0], k[1] = 0, L
        x = (k * 0.25 - 1.5).astype(np.float32)
        codes, s, z = oracle.quantize_values(x, bits)
        assert s == 0.25 and z == -1.5
        assert np.array_equal(codes, k.astype(np.uint8))


def test_subnormal_range_gives_zero_codes():
    x = np.zeros(32, np.float32)
    x[5] = np.float32(2.0 ** -130)  # bf16-representable subnormal
    codes, s, z = oracle.quantize_values(x, 2)
    assert 0 < s < FLT_MIN and np.all(codes == 0) and z == 0.0


def test_per_channel_keys_beat_per_token_keys():
    """News article, asymmetry paragraph: keys carry outlier channels, so
    grouping them per token gives noticeably larger error than per channel."""
    rng = np.random.default_rng(7)
    k = rng.standard_normal((32, 128)).astype(np.float32)
    k[:, [5, 60, 99]] *= 10.0
    k = _bf16_round(k)

    def mse(groups):
        tot = 0.0
        for x in groups:
            c, s, z = oracle.quantize_values(x, 2)
            tot += float(np.sum((c * np.float64(s) + np.float64(z) - x) ** 2))
        return tot / k.size

    per_channel = mse(k[:, c].copy() for c in range(128))
    per_token = mse(k[t, j * 32:(j + 1) * 32].copy() for t in range(32) for j in range(4))
    assert per_channel < 0.5 * per_token
