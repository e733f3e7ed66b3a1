"""Pins of the oracle quantiser's exact floating-point sequence.

The reading of the asymmetric min-max quantiser ("KIVI: A Tuning-Free
Asymmetric 2bit Quantization for KV Cache", method paragraph; the pages give
no formula) takes every step as one IEEE binary32 operation rounded to
nearest even: s = (mx - mn) / L, one reciprocal inv = 1 / s per group, codes
rint((x - mn) * inv); the 16-bit format rounds s to binary16 first.

The invariant pins elsewhere (half-step error, nearest level) cannot see the
last bit of the scale or a code next to a rounding midpoint, where the
plausible variants of that sequence differ.  Here the expected bits come
from exact rational arithmetic with IEEE rounding written from its
definition (tests/golden/make_quantizer_sequence.py, which uses no float
arithmetic and no oracle code), on constructed groups that separate the
variants, plus random groups.  Each variant, run here in numpy float32, must
fail at least one constructed case.
"""
import importlib.util
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "quantizer_fp32_sequence.txt")


def _deriv():
    spec = importlib.util.spec_from_file_location(
        "make_quantizer_sequence", os.path.join(HERE, "golden", "make_quantizer_sequence.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _cases():
    out, cur = [], None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, rest = line.split(" ", 1)
        if key == "case":
            f = rest.split()
            cur = {"name": f[0], "bits": int(f[1].split("=")[1]), "meta": int(f[2].split("=")[1])}
            out.append(cur)
        elif key == "x":
            bits = np.array([int(t, 16) for t in rest.split()], np.uint32)
            cur["x"] = (bits << 16).view(np.float32)
        elif key == "scale":
            f = rest.split()
            cur["scale"], cur["zero"] = int(f[0], 16), int(f[2], 16)
        elif key == "codes":
            cur["codes"] = np.array([int(t) for t in rest.split()], np.uint8)
    return out


CASES = _cases()


def _stored_bits(v, meta):
    return int(v) if meta == 1 else int(np.float32(v).view(np.uint32))


def test_golden_file_is_the_exact_derivation():
    """The stored file is what the exact-arithmetic script writes."""
    assert open(GOLDEN).read() == _deriv().render()
    assert [c["name"] for c in CASES] == [c[0] for c in _deriv().CASES]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_oracle_reproduces_the_derived_bits(case):
    codes, s, z = oracle.quantize_values(case["x"], case["bits"], meta=case["meta"])
    assert _stored_bits(s, case["meta"]) == case["scale"]
    assert _stored_bits(z, case["meta"]) == case["zero"]
    np.testing.assert_array_equal(codes, case["codes"])


# ---- plausible variants of the sequence, in numpy float32 (each op is one
# correctly rounded binary32 operation)

def _variant(x, bits, meta, kind):
    f32 = np.float32
    L = f32((1 << bits) - 1)
    mn, mx = f32(x.min()), f32(x.max())
    d = f32(mx - mn)
    s = f32(d * f32(f32(1) / L)) if kind == "scale_times_recip" else f32(d / L)
    if meta == 1:
        s = f32(np.float16(min(s, f32(65504.0))))
    tiny = s < np.finfo(np.float32).tiny
    y = (x - mn).astype(np.float32)
    if kind == "per_element_divide":
        t = (y / s).astype(np.float32) if not tiny else np.zeros_like(y)
    else:
        if tiny:
            inv = f32(0)
        elif kind == "direct_recip":
            inv = f32(L / d)
        else:
            inv = f32(f32(1) / s)
        t = (y * inv).astype(np.float32)
    codes = np.clip(np.rint(t), 0, L).astype(np.uint8)
    return codes, s


@pytest.mark.parametrize("kind,meta", [("scale_times_recip", 0), ("per_element_divide", 0),
                                       ("direct_recip", 0), ("per_element_divide", 1)])
def test_each_plausible_variant_fails_a_case(kind, meta):
    fails = []
    for c in CASES:
        if c["meta"] != meta:
            continue
        codes, s = _variant(c["x"], c["bits"], meta, kind)
        sb = int(s.astype(np.float16).view(np.uint16)) if meta == 1 else int(s.view(np.uint32))
        if sb != c["scale"] or not np.array_equal(codes, c["codes"]):
            fails.append(c["name"])
    assert fails, f"{kind} (meta {meta}) is not told apart from the derived sequence"


def test_the_sequence_itself_passes_every_case():
    """The variant-free numpy float32 sequence agrees with the exact
    derivation (so the cases separate variants, not rounding artefacts)."""
    for c in CASES:
        codes, s = _variant(c["x"], c["bits"], c["meta"], "reference")
        sb = (int(s.astype(np.float16).view(np.uint16)) if c["meta"] == 1
              else int(s.view(np.uint32)))
        assert sb == c["scale"], c["name"]
        np.testing.assert_array_equal(codes, c["codes"], c["name"])


def _bf16(x):
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32)


@pytest.mark.parametrize("bits,meta", [(2, 0), (4, 0), (2, 1), (4, 1)])
def test_random_groups_match_the_exact_derivation(bits, meta):
    from fractions import Fraction
    dv = _deriv()
    rng = np.random.default_rng(900 + 2 * bits + meta)
    for i in range(120):
        scale = [1.0, 1e-3, 40.0, 1e-6, 3e3][i % 5]
        x = _bf16((rng.standard_normal(32) * scale + (100.0 if i % 7 == 3 else 0.0))
                  .astype(np.float32))
        r = dv.derive([Fraction(float(v)) for v in x], bits, meta)
        codes, s, z = oracle.quantize_values(x, bits, meta=meta)
        assert _stored_bits(s, meta) == r["s_bits"], (i, x)
        assert _stored_bits(z, meta) == r["z_bits"], (i, x)
        np.testing.assert_array_equal(codes, np.array(r["codes"], np.uint8), str(i))
