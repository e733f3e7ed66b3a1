"""Pins of the oracle's decode attention.

Attention over the mixed cache is exact softmax attention over the
dequantised history plus the bf16 residual (paper card, method paragraph:
the attention kernel reads the per-channel K / per-token V cache; catalog
record, KV bytes basis: grouped history plus bf16 residual).  Pins:
library SDPA in float64 (on raw bf16 K/V when nothing is quantised, on the
oracle's dequantised K/V otherwise), closed forms (equal keys or q = 0 give
the mean of V; one token gives that token's V), order independence of the
ring, and a brute-force triple loop on tiny inputs.
"""
import numpy as np
import pytest
import torch

import oracle


def _bits(x):
    return (np.ascontiguousarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _f(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _sdpa(q, k, v, scale):
    """Library scaled-dot-product attention in float64: q [m][D], k, v [n][D]."""
    t = [torch.from_numpy(np.ascontiguousarray(a, np.float64))[None] for a in (q, k, v)]
    return torch.nn.functional.scaled_dot_product_attention(*t, scale=scale)[0].numpy()


def _cache(rng, B, H, QPK, S, bits=2, D=128, residual=128, outlier=True):
    x = rng.standard_normal((2, B, H, S, D)).astype(np.float32)
    if outlier:
        x[0, :, :, :, [3, 42, 85]] *= 10
    k, v = _bits(x[0]), _bits(x[1])
    T = 32 * (S // 32 + 2)
    g = oracle.Geom(B, H, QPK, head_dim=D, bits=bits, group=32, residual=residual,
                    max_tokens=T)
    q = _bits(rng.standard_normal((B, H * QPK, D)).astype(np.float32))
    return g, oracle.prefill(g, k, v), k, v, q


def test_no_quantised_part_equals_sdpa_on_raw():
    rng = np.random.default_rng(1)
    g, c, k, v, q = _cache(rng, 2, 2, 2, 150)
    assert c.n_q == 0
    scale = 128 ** -0.5
    out = oracle.attention(c, q, scale)
    for b in range(2):
        for hq in range(4):
            h = hq // 2
            ref = _sdpa(_f(q[b, hq])[None], _f(k[b, h]), _f(v[b, h]), scale)[0]
            np.testing.assert_allclose(out[b, hq], ref, rtol=0, atol=1e-6)


@pytest.mark.parametrize("bits", [2, 4])
def test_mixed_cache_equals_sdpa_on_dequantised(bits):
    rng = np.random.default_rng(2 + bits)
    B, H, QPK, S = 1, 2, 4, 600
    g, c, k, v, q = _cache(rng, B, H, QPK, S, bits=bits)
    assert c.n_q == 448 and c.n_res == 152
    scale = 0.07
    out = oracle.attention(c, q, scale)
    for u in range(B * H):
        kd, vd = oracle.dequant_unit(c, u)
        for j in range(QPK):
            hq = (u % H) * QPK + j
            qd = _f(q[u // H, hq])
            ref = _sdpa(qd[None], kd, vd, scale)[0]
            np.testing.assert_allclose(out[u // H, hq], ref.astype(np.float32),
                                       rtol=1e-6, atol=1e-7)


def test_dequantised_cache_is_close_to_raw():
    # the history dequantises to within half a step of the raw keys/values
    rng = np.random.default_rng(5)
    g, c, k, v, q = _cache(rng, 1, 1, 1, 512)
    kd, vd = oracle.dequant_unit(c, 0)
    ks = np.repeat(c.k_scale[0, 0, :c.n_q // 32], 32, axis=0)
    assert np.all(np.abs(kd[:c.n_q] - _f(k[0, 0, :c.n_q])) <= ks * 0.5 + 1e-6)
    assert np.array_equal(kd[c.n_q:], _f(k[0, 0, c.n_q:]))
    # values: per token and block of 32 channels
    vs = np.repeat(c.v_scale[0, 0, :c.n_q // 32].transpose(0, 2, 1).reshape(c.n_q, 4), 32,
                   axis=1)
    assert np.all(np.abs(vd[:c.n_q] - _f(v[0, 0, :c.n_q])) <= vs * 0.5 + 1e-6)
    assert np.array_equal(vd[c.n_q:], _f(v[0, 0, c.n_q:]))


def test_equal_keys_or_zero_query_give_mean_of_values():
    rng = np.random.default_rng(6)
    g, c, k, v, q = _cache(rng, 1, 1, 2, 400)
    _, vd = oracle.dequant_unit(c, 0)
    q0 = np.zeros_like(q)
    out = oracle.attention(c, q0, 0.1)
    np.testing.assert_allclose(out[0, 0], vd.mean(axis=0), rtol=1e-6, atol=1e-7)
    # identical keys: every score equal
    kk = np.tile(k[:, :, :1], (1, 1, 400, 1))
    g2 = oracle.Geom(1, 1, 2, bits=2, max_tokens=448)
    c2 = oracle.prefill(g2, kk, v)
    _, vd2 = oracle.dequant_unit(c2, 0)
    out2 = oracle.attention(c2, q, 0.1)
    np.testing.assert_allclose(out2[0, 1], vd2.mean(axis=0), rtol=1e-6, atol=1e-7)


def test_single_token_returns_its_value():
    rng = np.random.default_rng(7)
    g, c, k, v, q = _cache(rng, 1, 1, 3, 1)
    out = oracle.attention(c, q, 0.3)
    for j in range(3):
        assert np.array_equal(out[0, j], _f(v[0, 0, 0]).astype(np.float32))


def test_ring_order_does_not_change_attention():
    rng = np.random.default_rng(8)
    B, H, D = 1, 1, 128
    x = rng.standard_normal((2, 1, 1, 500, D)).astype(np.float32)
    k, v = _bits(x[0]), _bits(x[1])
    q = _bits(rng.standard_normal((1, 1, D)).astype(np.float32))
    g = oracle.Geom(B, H, 1, max_tokens=512)
    c = oracle.prefill(g, k[:, :, :300], v[:, :, :300])
    for t in range(300, 500):
        oracle.append(c, k[:, :, t], v[:, :, t])
        oracle.flush(c)
    assert c.res_start != 0
    out = oracle.attention(c, q, 0.09)
    # same logical cache with the residual rotated back to slot 0
    c2 = c.copy()
    slots = g.slots
    order = [(c.res_start + i) % slots for i in range(slots)]
    c2.k_res[0, 0] = c.k_res[0, 0, order]
    c2.v_res[0, 0] = c.v_res[0, 0, order]
    c2.res_start = 0
    out2 = oracle.attention(c2, q, 0.09)
    np.testing.assert_allclose(out, out2, rtol=1e-6, atol=1e-7)


def test_brute_force_tiny():
    rng = np.random.default_rng(9)
    for n in [1, 2, 7, 33, 64]:
        q = rng.standard_normal(16)
        k = rng.standard_normal((n, 16))
        v = rng.standard_normal((n, 16))
        s = 0.25
        o = oracle.attend_row(q, k, v, s)
        w = [np.exp(s * sum(q[c] * k[t, c] for c in range(16))) for t in range(n)]
        ref = [sum(w[t] * v[t, c] for t in range(n)) / sum(w) for c in range(16)]
        np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_large_scores_do_not_overflow():
    q = np.full(8, 50.0)
    k = np.stack([np.full(8, 10.0), np.full(8, 9.0)])
    v = np.array([[1.0] * 8, [3.0] * 8])
    o = oracle.attend_row(q, k, v, 1.0)   # scores 4000 and 3600
    np.testing.assert_allclose(o, np.ones(8), rtol=0, atol=1e-12)
