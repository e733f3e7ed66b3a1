"""Pins of the oracle's cache layout, prefill split and streaming behaviour.

* Packed bytes of constructed groups against hand-derived bytes
  (tests/golden/packed_bytes.txt).
* The prefill split leaves whole groups of 32 and a residual of at least 128
  tokens (catalog record kivi-2bit-llama3-8b-gqa-8k, KV bytes basis: the
  grouped term covers S-R tokens, 8064 = 252 groups of 32 at S = 8192).
* Appending tokens one at a time with flushes yields, byte for byte, the cache
  that a prefill of the longer sequence yields (the grouped history is a pure
  function of the token index; the residual keeps the most recent tokens).
"""
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "packed_bytes.txt")


def _golden():
    rows = {}
    for line in open(GOLD):
        line = line.split("#")[0].strip()
        if not line:
            continue
        parts = line.split()
        key = tuple(parts[:3]) if parts[0].startswith("v") else tuple(parts[:2])
        rows[key] = [int(b, 16) for b in parts[len(key):]]
    return rows


def _bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, np.float32).view(np.uint32).__rshift__(16).astype(np.uint16)


def _pattern_cache(bits):
    L = (1 << bits) - 1
    t = np.arange(32)[:, None]
    c = np.arange(32)[None, :]
    if bits == 2:
        xk = (t + c) % 4
        xv = (t // 2 + 3 * c) % 4
    else:
        xk = (t + c) % 16
        xv = (t + c) % 16
    assert xk.max() == L
    k = _bits(xk.astype(np.float32))[None, None]
    v = _bits(xv.astype(np.float32))[None, None]
    g = oracle.Geom(1, 1, 1, head_dim=32, bits=bits, group=32, residual=0, max_tokens=32)
    return oracle.prefill(g, k, v), xk, xv


@pytest.mark.parametrize("bits", [2, 4])
def test_packed_bytes_match_hand_derivation(bits):
    gold = _golden()
    cache, xk, xv = _pattern_cache(bits)
    assert cache.n_q == 32 and cache.n_res == 0
    assert np.all(cache.k_scale == 1.0) and np.all(cache.k_zero == 0.0)
    assert np.all(cache.v_scale == 1.0) and np.all(cache.v_zero == 0.0)
    n = 0
    for key, want in gold.items():
        if key[0] == f"k{bits}":
            t = int(key[1].split("=")[1])
            assert list(cache.k_codes[0, 0, t]) == want, key
            n += 1
        if key[0] == f"v{bits}":
            o = int(key[1].split("=")[1])
            c = int(key[2].split("=")[1])
            assert list(cache.v_codes[0, 0, 0, o, c]) == want, key
            n += 1
    assert n >= 2
    # dequantising the pattern cache gives the pattern back exactly
    kd, vd = oracle.dequant_unit(cache, 0)
    assert np.array_equal(kd, xk.astype(np.float64))
    assert np.array_equal(vd, xv.astype(np.float64))


@pytest.mark.parametrize("S,n_q", [(1, 0), (127, 0), (128, 0), (159, 0), (160, 32),
                                   (256, 128), (4096, 3968), (8192, 8064), (32768, 32640)])
def test_prefill_split(S, n_q):
    assert oracle.prefill_split(S, 32, 128) == n_q
    r = S - n_q
    assert r == S if S < 128 else 128 <= r < 160


def _random_kv(rng, B, H, S, D):
    x = rng.standard_normal((2, B, H, S, D)).astype(np.float32)
    x[0, :, :, :, 3] *= 10
    return _bits(x[0]), _bits(x[1])


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("residual", [0, 32, 128])
def test_streaming_equals_prefill(bits, residual):
    rng = np.random.default_rng(bits * 100 + residual)
    B, H, D, G = 2, 2, 64, 32
    S0, N = residual + 5, 3 * G + 7
    total = S0 + N
    k, v = _random_kv(rng, B, H, total, D)
    g = oracle.Geom(B, H, 1, head_dim=D, bits=bits, group=G, residual=residual,
                    max_tokens=G * (total // G + 1))
    c = oracle.prefill(g, k[:, :, :S0], v[:, :, :S0])
    flushes = 0
    for t in range(S0, total):
        oracle.append(c, k[:, :, t], v[:, :, t])
        flushes += oracle.flush(c)
        assert residual <= c.n_res < residual + G or c.n_q == 0
    ref = oracle.prefill(g, k, v)
    assert flushes > 0
    assert (c.n_q, c.n_res) == (ref.n_q, ref.n_res)
    nq, NG = ref.n_q, ref.n_q // G
    assert np.array_equal(c.k_codes[:, :, :nq], ref.k_codes[:, :, :nq])
    assert np.array_equal(c.v_codes[:, :, :NG], ref.v_codes[:, :, :NG])
    for a, b_ in [(c.k_scale, ref.k_scale), (c.k_zero, ref.k_zero),
                  (c.v_scale, ref.v_scale), (c.v_zero, ref.v_zero)]:
        assert np.array_equal(a[:, :, :NG].view(np.uint32), b_[:, :, :NG].view(np.uint32))
    for u in range(B * H):
        k1, v1 = oracle.dequant_unit(c, u)
        k2, v2 = oracle.dequant_unit(ref, u)
        assert np.array_equal(k1, k2) and np.array_equal(v1, v2)


def test_residual_holds_most_recent_tokens_in_order():
    rng = np.random.default_rng(3)
    B, H, D = 1, 1, 32
    k, v = _random_kv(rng, B, H, 300, D)
    g = oracle.Geom(B, H, 1, head_dim=D, bits=2, group=32, residual=64, max_tokens=320)
    c = oracle.prefill(g, k[:, :, :100], v[:, :, :100])
    for t in range(100, 300):
        oracle.append(c, k[:, :, t], v[:, :, t])
        oracle.flush(c)
    kd, vd = oracle.dequant_unit(c, 0)
    r = c.n_res
    raw_k = (k[0, 0, 300 - r:].astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(kd[c.n_q:], raw_k.astype(np.float64))
    assert c.n_q + r == 300


def test_append_refuses_full_ring_and_flush_refuses_full_history():
    rng = np.random.default_rng(4)
    k, v = _random_kv(rng, 1, 1, 200, 32)
    g = oracle.Geom(1, 1, 1, head_dim=32, bits=2, group=32, residual=32, max_tokens=64)
    c = oracle.prefill(g, k[:, :, :63], v[:, :, :63])   # n_q 0? -> 63-32=31 -> 0, r 63
    assert (c.n_q, c.n_res) == (0, 63)
    oracle.append(c, k[:, :, 63], v[:, :, 63])
    with pytest.raises(ValueError):
        oracle.append(c, k[:, :, 64], v[:, :, 64])
    assert oracle.flush(c) == 1 and (c.n_q, c.n_res) == (32, 32)
    for t in range(64, 96):
        oracle.append(c, k[:, :, t], v[:, :, t])
    assert oracle.flush(c) == 1 and c.n_q == 64
    for t in range(96, 128):
        oracle.append(c, k[:, :, t], v[:, :, t])
    with pytest.raises(ValueError):
        oracle.flush(c)
