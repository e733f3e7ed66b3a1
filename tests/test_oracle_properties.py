"""Property tests of the oracle over random small geometries (hypothesis).

The fixed-case pins elsewhere check these invariants on chosen shapes; here
hypothesis draws the geometry (batch, kv heads, query heads per kv head,
head_dim, group size, residual length, bit width, scale/zero format), the
prefill length, the number of streamed tokens and the value magnitudes:

* streaming equals prefill: appending tokens one at a time and flushing a
  group whenever the ring holds R + G tokens leaves the same bytes as one
  prefill of all tokens (catalog record kivi-2bit-llama3-8b-gqa-8k, KV bytes
  basis: the most recent R tokens stay in bf16, older ones are flushed into
  groups of G);
* every group's dequantised values lie within half a quantisation step of
  its inputs (paper card, method paragraph: asymmetric min-max groups;
  fp32 scale/zero format);
* decode attention equals library scaled-dot-product attention in float64
  over the oracle's dequantised cache (exact softmax attention over the
  mixed cache).

Examples are derandomised, so the suite is reproducible.
"""
import numpy as np
import torch
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle

FLT_MIN = np.float32(np.finfo(np.float32).tiny)


def _bits(x):
    """float32 -> bf16 bit patterns (truncation: any bf16 input will do)."""
    return (np.ascontiguousarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _f(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@st.composite
def geometries(draw):
    G = draw(st.sampled_from([16, 32, 64]))
    D = G * draw(st.integers(1, 128 // G if G <= 64 else 1))
    residual = G * draw(st.integers(0, 4))
    return dict(B=draw(st.integers(1, 2)), H=draw(st.integers(1, 3)),
                QPK=draw(st.integers(1, 4)), D=D, G=G, residual=residual,
                bits=draw(st.sampled_from([2, 4])), meta=draw(st.sampled_from([0, 1])))


def _values(seed, shape, log2_mag):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32) * np.float32(2.0 ** log2_mag)
    if shape[-1] > 3:
        x[..., 3] *= 10   # an outlier channel
    return x


def _geom(p, total):
    return oracle.Geom(p["B"], p["H"], p["QPK"], head_dim=p["D"], bits=p["bits"],
                       group=p["G"], residual=p["residual"],
                       max_tokens=p["G"] * (total // p["G"] + 2), meta=p["meta"])


def _same_bytes(a, b):
    return np.array_equal(np.ascontiguousarray(a).view(np.uint8),
                          np.ascontiguousarray(b).view(np.uint8))


@settings(max_examples=40, deadline=None, derandomize=True)
@given(p=geometries(), s0=st.integers(0, 200), n=st.integers(1, 140),
       seed=st.integers(0, 2 ** 31), mag=st.integers(-12, 12))
def test_streaming_equals_prefill(p, s0, n, seed, mag):
    total = s0 + n
    x = _values(seed, (2, p["B"], p["H"], total, p["D"]), mag)
    k, v = _bits(x[0]), _bits(x[1])
    g = _geom(p, total)
    c = oracle.prefill(g, k[:, :, :s0].copy(), v[:, :, :s0].copy())
    G, R = p["G"], p["residual"]
    for t in range(s0, total):
        oracle.append(c, k[:, :, t].copy(), v[:, :, t].copy())
        oracle.flush(c)
        assert c.n_res < R + G
    ref = oracle.prefill(g, k, v)
    assert (c.n_q, c.n_res) == (ref.n_q, ref.n_res)
    NG = ref.n_q // G
    assert _same_bytes(c.k_codes[:, :, :ref.n_q], ref.k_codes[:, :, :ref.n_q])
    assert _same_bytes(c.v_codes[:, :, :NG], ref.v_codes[:, :, :NG])
    for a, b in [(c.k_scale, ref.k_scale), (c.k_zero, ref.k_zero),
                 (c.v_scale, ref.v_scale), (c.v_zero, ref.v_zero)]:
        assert _same_bytes(a[:, :, :NG], b[:, :, :NG])
    for u in range(p["B"] * p["H"]):
        k1, v1 = oracle.dequant_unit(c, u)
        k2, v2 = oracle.dequant_unit(ref, u)
        assert np.array_equal(k1, k2) and np.array_equal(v1, v2)


@settings(max_examples=200, deadline=None, derandomize=True)
@given(bits=st.sampled_from([2, 4]), size=st.sampled_from([8, 16, 32, 64]),
       seed=st.integers(0, 2 ** 31), mag=st.integers(-120, 120),
       offset=st.floats(-4.0, 4.0))
def test_group_error_within_half_step(bits, size, seed, mag, offset):
    L = (1 << bits) - 1
    rng = np.random.default_rng(seed)
    x = ((rng.standard_normal(size) + offset) * 2.0 ** mag).astype(np.float32)
    x = _f(_bits(x)).astype(np.float32)
    codes, s, z = oracle.quantize_values(x, bits)
    assert codes.max() <= L and z == x.min()
    if s < FLT_MIN:
        assert np.all(codes == 0)
        return
    deq = codes.astype(np.float64) * np.float64(s) + np.float64(z)
    err = np.abs(x.astype(np.float64) - deq)
    assert np.all(err <= np.float64(s) * (0.5 + 3 * L * 2.0 ** -24))


@settings(max_examples=30, deadline=None, derandomize=True)
@given(p=geometries(), S=st.integers(1, 300), seed=st.integers(0, 2 ** 31),
       mag=st.integers(-6, 6), scale=st.sampled_from([0.01, 0.09, 0.5, 2.0]))
def test_attention_equals_sdpa_on_dequantised(p, S, seed, mag, scale):
    x = _values(seed, (2, p["B"], p["H"], S, p["D"]), mag)
    k, v = _bits(x[0]), _bits(x[1])
    g = _geom(p, S)
    c = oracle.prefill(g, k, v)
    rng = np.random.default_rng(seed + 1)
    q = _bits(rng.standard_normal((p["B"], p["H"] * p["QPK"], p["D"])).astype(np.float32))
    out = oracle.attention(c, q, scale)
    for u in range(p["B"] * p["H"]):
        b, h = divmod(u, p["H"])
        kd, vd = oracle.dequant_unit(c, u)
        qd = _f(q[b, h * p["QPK"]:(h + 1) * p["QPK"]])
        t = [torch.from_numpy(np.ascontiguousarray(a))[None] for a in (qd, kd, vd)]
        ref = torch.nn.functional.scaled_dot_product_attention(*t, scale=scale)[0].numpy()
        got = out[b, h * p["QPK"]:(h + 1) * p["QPK"]].astype(np.float64)
        tol = 1e-6 * np.abs(ref).max(axis=1, keepdims=True) + 1e-30
        assert np.all(np.abs(got - ref) <= tol)
