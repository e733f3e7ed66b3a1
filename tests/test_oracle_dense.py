"""Pins of the oracle's attention over an uncompressed bf16 cache, the
baseline the pages measure KIVI against (paper card: the comparison with the
FP16 cache; catalog record, Methodology: throughput over the FP16 baseline).

It is plain softmax attention, so it is pinned to library SDPA in float64
(with the grouped-query head mapping written out), to a brute-force loop on a
tiny case, to the fact that tokens past seq_len are never read, and to the
mixed-cache oracle on a cache whose tokens all sit in the bf16 residual.
"""
import math

import numpy as np
import torch

import oracle


def _bits(x):
    return (np.ascontiguousarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _f(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _inputs(rng, B, H, QPK, T, D=128):
    k = _bits(rng.standard_normal((B, H, T, D)).astype(np.float32) * 2)
    v = _bits(rng.standard_normal((B, H, T, D)).astype(np.float32))
    q = _bits(rng.standard_normal((B, H * QPK, D)).astype(np.float32))
    return oracle.Geom(B, H, QPK, head_dim=D), k, v, q


def test_dense_equals_library_sdpa_with_head_groups():
    rng = np.random.default_rng(31)
    B, H, QPK, T, S = 2, 3, 4, 96, 77
    g, k, v, q = _inputs(rng, B, H, QPK, T)
    scale = 1 / math.sqrt(128)
    out = oracle.attention_dense(g, k, v, S, q, scale)
    # library routine: queries [B][Hq][1][D], keys repeated per query head
    qt = torch.from_numpy(_f(q))[:, :, None, :]
    kt = torch.from_numpy(_f(k[:, :, :S])).repeat_interleave(QPK, dim=1)
    vt = torch.from_numpy(_f(v[:, :, :S])).repeat_interleave(QPK, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[:, :, 0].numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-6)


def test_dense_brute_force_tiny():
    rng = np.random.default_rng(32)
    g, k, v, q = _inputs(rng, 1, 2, 2, 8, D=16)
    s = 0.3
    out = oracle.attention_dense(g, k, v, 5, q, s)
    for hq in range(4):
        h = hq // 2
        w = [math.exp(s * sum(_f(q)[0, hq, c] * _f(k)[0, h, t, c] for c in range(16)))
             for t in range(5)]
        ref = [sum(w[t] * _f(v)[0, h, t, c] for t in range(5)) / sum(w) for c in range(16)]
        np.testing.assert_allclose(out[0, hq], ref, rtol=1e-6, atol=1e-7)


def test_tokens_past_seq_len_are_not_read():
    rng = np.random.default_rng(33)
    g, k, v, q = _inputs(rng, 1, 2, 1, 64)
    a = oracle.attention_dense(g, k, v, 40, q, 0.1)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 40:] = 0x7F80   # +inf
    v2[:, :, 40:] = 0x7FC0   # NaN
    b = oracle.attention_dense(g, k2, v2, 40, q, 0.1)
    np.testing.assert_array_equal(a, b)


def test_dense_equals_mixed_cache_without_quantised_part():
    """A cache of S <= R tokens holds everything in the bf16 residual, so the
    mixed-cache attention and the dense attention see the same tokens."""
    rng = np.random.default_rng(34)
    B, H, QPK, S = 2, 2, 3, 130
    g, k, v, q = _inputs(rng, B, H, QPK, S)
    gm = oracle.Geom(B, H, QPK, max_tokens=64)
    c = oracle.prefill(gm, k, v)
    assert c.n_q == 0 and c.n_res == S
    np.testing.assert_array_equal(oracle.attention(c, q, 0.09),
                                  oracle.attention_dense(g, k, v, S, q, 0.09))
