"""Pins of the oracle's 16-bit scale/zero format (fp16 scale, bf16 zero).

No page fixes a metadata format (the catalog record's byte basis counts none),
so the reading is: the zero is the group minimum, a bf16 input, kept exactly
in bf16; the scale range / L is rounded to fp16 (nearest, ties to even,
saturating at 65504) and the codes are computed from the rounded scale.  The
tests do not re-type the formula.  They pin the fp16 rounding to numpy's
float16 conversion (a library routine), the zero to the exact minimum, the
codes through invariants (constant groups exact, error within half a step
of the rounded scale, nearest level, the same codes as the fp32 format
whenever the scale is exactly an fp16 number), and the cache layout and
streaming behaviour of the format (stored bytes equal the per-group
results; appending with flushes equals prefilling the longer sequence;
attention equals library SDPA over the dequantised cache).
"""
import math

import numpy as np
import pytest
import torch

import oracle

FLT_MIN = np.float32(np.finfo(np.float32).tiny)


def _bf16_round(x):
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32)


def _groups(rng, n):
    for _ in range(n):
        kind = rng.integers(5)
        if kind == 0:
            x = rng.standard_normal(32)
        elif kind == 1:
            x = rng.uniform(-1e-3, 1e-3, 32)
        elif kind == 2:
            x = rng.standard_normal(32) * 40.0 + 100.0
        elif kind == 3:
            x = rng.standard_normal(32) * 1e-6   # fp16-subnormal scales
        else:
            x = rng.standard_normal(32) * 3e3
        yield _bf16_round(x.astype(np.float32))


def _f16(bits):
    return np.uint16(bits).view(np.float16).astype(np.float64)


def _bf(bits):
    return float((np.uint32(bits) << np.uint32(16)).view(np.float32))


@pytest.mark.parametrize("bits", [2, 4])
def test_scale_is_fp16_rounding_and_zero_is_exact_min(bits):
    L = (1 << bits) - 1
    rng = np.random.default_rng(40 + bits)
    for x in _groups(rng, 3000):
        _, sh, zh = oracle.quantize_values(x, bits, meta=1)
        s32 = np.float32(np.float32(x.max()) - np.float32(x.min())) / np.float32(L)
        assert sh == np.float16(s32).view(np.uint16), (s32, sh)
        assert _bf(zh) == float(x.min())


@pytest.mark.parametrize("bits", [2, 4])
def test_constant_group_is_exact(bits):
    for val in [0.0, -3.25, 1e-30, 7.0e4, -2.0 ** -130]:
        x = _bf16_round(np.full(32, val, np.float32))
        codes, sh, zh = oracle.quantize_values(x, bits, meta=1)
        assert sh == 0 and np.all(codes == 0)
        assert np.all(_bf(zh) == x)


@pytest.mark.parametrize("bits", [2, 4])
def test_error_within_half_step_of_rounded_scale(bits):
    """|x - dequant| <= s16/2 (plus fp32 slack) where fp16 holds the scale to
    11 bits (normal range: L * |s32 - s16| < s16 / 2, so no code clamps);
    in the fp16 subnormal range the top codes may clamp, and the bound gains
    the L * |s32 - s16| the rounding of the scale moved the top level by."""
    L = (1 << bits) - 1
    rng = np.random.default_rng(50 + bits)
    n_sub = 0
    for x in _groups(rng, 3000):
        codes, sh, zh = oracle.quantize_values(x, bits, meta=1)
        s, z = _f16(sh), _bf(zh)
        assert codes.max() <= L
        if s == 0:
            assert np.all(codes == 0)
            continue
        s32 = float(np.float32(np.float32(x.max()) - np.float32(x.min())) / np.float32(L))
        deq = codes.astype(np.float64) * s + z
        err = np.abs(deq - x.astype(np.float64)).max()
        half = s * (0.5 + 3 * L * 2.0 ** -24)
        if s >= 2.0 ** -14:
            assert err <= half
        else:
            n_sub += 1
            assert err <= half + L * abs(s32 - s)
    assert n_sub > 100


@pytest.mark.parametrize("bits", [2, 4])
def test_code_is_nearest_level_of_rounded_grid(bits):
    L = (1 << bits) - 1
    rng = np.random.default_rng(60 + bits)
    for x in _groups(rng, 1000):
        codes, sh, zh = oracle.quantize_values(x, bits, meta=1)
        s, z = _f16(sh), _bf(zh)
        if s == 0:
            continue
        levels = np.arange(L + 1) * s + z
        d = np.abs(x.astype(np.float64)[:, None] - levels[None, :])
        best = d.argmin(axis=1)
        # away from a midpoint the nearest level is unique
        gap = np.sort(d, axis=1)[:, 1] - np.sort(d, axis=1)[:, 0]
        sure = gap > 6 * L * 2.0 ** -24 * s
        assert np.array_equal(codes[sure], best[sure])


@pytest.mark.parametrize("bits", [2, 4])
def test_same_codes_as_fp32_format_when_scale_is_an_fp16_number(bits):
    L = (1 << bits) - 1
    rng = np.random.default_rng(70 + bits)
    for e in range(-12, 12):
        s = 2.0 ** e * 1.25
        k = rng.integers(0, L + 1, 32)
        k[0], k[1] = 0, L
        x = (k * s - 3.0).astype(np.float32)
        x = _bf16_round(x)
        c32, s32, z32 = oracle.quantize_values(x, bits)
        c16, sh, zh = oracle.quantize_values(x, bits, meta=1)
        if np.float16(s32) == s32:
            assert np.array_equal(c16, c32) and _f16(sh) == s32 and _bf(zh) == z32


def test_saturated_scale():
    x = _bf16_round(np.array([-2.0e5] + [0.0] * 30 + [2.0e5], np.float32))
    codes, sh, zh = oracle.quantize_values(x, 2, meta=1)
    assert sh == 0x7BFF                        # 65504, the largest finite fp16
    assert codes[0] == 0 and codes[-1] == 3    # clamped at the top level


def _cache(rng, B, H, S, bits, meta):
    x = rng.standard_normal((2, B, H, S, 128)).astype(np.float32)
    x[0, :, :, :, [3, 42, 85]] *= 10
    kb = (_bf16_round(x[0]).view(np.uint32) >> 16).astype(np.uint16)
    vb = (_bf16_round(x[1]).view(np.uint32) >> 16).astype(np.uint16)
    g = oracle.Geom(B, H, 2, bits=bits, max_tokens=32 * (S // 32 + 2), meta=meta)
    return g, kb, vb


@pytest.mark.parametrize("bits", [2, 4])
def test_stored_bytes_equal_per_group_results(bits):
    rng = np.random.default_rng(80 + bits)
    g, kb, vb = _cache(rng, 1, 2, 300, bits, 1)
    c = oracle.prefill(g, kb, vb)
    assert c.k_scale.dtype == np.uint16 and c.n_q == 160
    f = lambda a: (a.astype(np.uint32) << 16).view(np.float32)
    for h in range(2):
        for gi in range(c.n_q // 32):
            for ch in (0, 3, 77, 127):
                x = f(kb[0, h, 32 * gi:32 * gi + 32, ch])
                _, sh, zh = oracle.quantize_values(x, bits, meta=1)
                assert c.k_scale[0, h, gi, ch] == sh and c.k_zero[0, h, gi, ch] == zh
            for t in (0, 13, 31):
                for j in range(4):
                    x = f(vb[0, h, 32 * gi + t, 32 * j:32 * j + 32])
                    _, sh, zh = oracle.quantize_values(x, bits, meta=1)
                    assert c.v_scale[0, h, gi, j, t] == sh and c.v_zero[0, h, gi, j, t] == zh
    # dequantised keys of one group: codes times fp16 scale plus bf16 zero
    k, _ = oracle.dequant_unit(c, 1)
    x = f(kb[0, 1, 32:64, 5])
    codes, sh, zh = oracle.quantize_values(x, bits, meta=1)
    np.testing.assert_array_equal(k[32:64, 5], codes * _f16(sh) + _bf(zh))


@pytest.mark.parametrize("bits", [2, 4])
def test_streaming_equals_prefill_16bit(bits):
    rng = np.random.default_rng(90 + bits)
    g, kb, vb = _cache(rng, 2, 1, 260, bits, 1)
    c = oracle.prefill(g, kb[:, :, :150].copy(), vb[:, :, :150].copy())
    for t in range(150, 260):
        oracle.append(c, kb[:, :, t].copy(), vb[:, :, t].copy())
        oracle.flush(c)
    ref = oracle.prefill(g, kb, vb)
    assert (c.n_q, c.n_res) == (ref.n_q, ref.n_res)
    ng = ref.n_q // 32
    for name in ("k_scale", "k_zero", "v_scale", "v_zero"):
        np.testing.assert_array_equal(getattr(c, name)[:, :, :ng], getattr(ref, name)[:, :, :ng])
    np.testing.assert_array_equal(c.k_codes[:, :, :ref.n_q], ref.k_codes[:, :, :ref.n_q])
    np.testing.assert_array_equal(c.v_codes[:, :, :ng], ref.v_codes[:, :, :ng])


def test_attention_equals_sdpa_on_dequantised_16bit():
    rng = np.random.default_rng(99)
    g, kb, vb = _cache(rng, 1, 2, 230, 2, 1)
    c = oracle.prefill(g, kb, vb)
    q = (_bf16_round(rng.standard_normal((1, 4, 128)).astype(np.float32)).view(np.uint32)
         >> 16).astype(np.uint16)
    scale = 1 / math.sqrt(128)
    out = oracle.attention(c, q, scale)
    qf = (q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for h in range(2):
        k, v = oracle.dequant_unit(c, h)
        t = [torch.from_numpy(a)[None] for a in (qf[0, 2 * h:2 * h + 2], k, v)]
        ref = torch.nn.functional.scaled_dot_product_attention(*t, scale=scale)[0].numpy()
        np.testing.assert_allclose(out[0, 2 * h:2 * h + 2], ref, rtol=0, atol=1e-6)
