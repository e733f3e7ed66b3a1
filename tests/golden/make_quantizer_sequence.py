"""Writes quantizer_fp32_sequence.txt: constructed quantiser groups whose
scale bits and codes follow from exact rational arithmetic.

The quantiser reading (the pages fix "asymmetric", min-max, per-channel K and
per-token V groups, but no formula; "KIVI: A Tuning-Free Asymmetric 2bit
Quantization for KV Cache", method paragraph): with every step one IEEE
binary32 operation rounded to nearest, ties to even,
    d = mx - mn,  s = d / L,  inv = 1 / s (0 when s < 2^-126),
    code = clamp(rint((x - mn) * inv), 0, L),
and, in the 16-bit scale/zero format, s rounded on to binary16 (ties to
even, saturating at 65504) before inv is taken from it.

Every rounding below is written from the definition of IEEE rounding to
nearest even on exact rationals (fractions.Fraction); no float arithmetic and
no oracle code is used.  The groups were chosen so that plausible variants of
that sequence give different bits:
  - a scale taken as d * (1/L) instead of the divide d / L;
  - codes from a per-element divide (x - mn) / s instead of the per-group
    reciprocal;
  - a reciprocal taken directly as L / d instead of 1 / s;
  - the same per-element divide with the 16-bit scale.
Run from the repository root:  python tests/golden/make_quantizer_sequence.py
"""
from __future__ import annotations

import os
import struct
from fractions import Fraction

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "quantizer_fp32_sequence.txt")

# binary32: 24 significant bits, smallest normal exponent -126;
# binary16: 11 bits, -14
F32 = (24, -126)
F16 = (11, -14)


def ilog2(a: Fraction) -> int:
    """floor(log2 a) for a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def rne(q: Fraction, fmt=F32) -> Fraction:
    """The value of the format nearest to q, ties to the even significand
    (subnormals below the smallest normal exponent; no overflow here)."""
    if q == 0:
        return Fraction(0)
    p, emin = fmt
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = max(ilog2(a), emin)
    ulp = Fraction(2) ** (e - p + 1)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def rint_even(t: Fraction) -> int:
    """Nearest integer, ties to even."""
    fl = t.numerator // t.denominator
    rem = t - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def f32_bits(v: Fraction) -> int:
    return struct.unpack("<I", struct.pack("<f", float(v)))[0]


def f16_bits(v: Fraction) -> int:
    return struct.unpack("<H", struct.pack("<e", float(v)))[0]


def bf16_value(bits: int) -> Fraction:
    return Fraction(struct.unpack("<f", struct.pack("<I", bits << 16))[0])


def bf16_bits(v: Fraction) -> int:
    b = f32_bits(v)
    assert b & 0xFFFF == 0, "not a bf16 value"
    return b >> 16


FLT_MIN = Fraction(2) ** -126
F16_MAX = Fraction(65504)


def derive(xs: list[Fraction], bits: int, meta: int):
    """Scale (fp32 value), its stored bits, zero bits, codes, and the
    intermediate values of the derivation."""
    L = (1 << bits) - 1
    mn, mx = min(xs), max(xs)
    d = rne(mx - mn)
    s32 = rne(d / L)
    if meta == 1:
        s = rne(min(s32, F16_MAX), F16)
        s_bits = f16_bits(s)
        z_bits = bf16_bits(mn)
    else:
        s = s32
        s_bits = f32_bits(s)
        z_bits = f32_bits(mn)
    inv = rne(1 / s) if s >= FLT_MIN else Fraction(0)
    codes, steps = [], []
    for x in xs:
        y = rne(x - mn)
        t = rne(y * inv)
        c = min(max(rint_even(t), 0), L)
        codes.append(c)
        steps.append((y, t))
    return dict(L=L, mn=mn, mx=mx, d=d, s32=s32, s=s, s_bits=s_bits, z_bits=z_bits, inv=inv,
                codes=codes, steps=steps)


def _fill(mn: Fraction, mx: Fraction, n: int) -> list[Fraction]:
    """n bf16 values spread over [mn, mx] (each the bf16 value just below
    mn + (mx - mn) * i / (n + 1), bit patterns chosen without rounding)."""
    out = []
    for i in range(1, n + 1):
        target = mn + (mx - mn) * Fraction(i, n + 1)
        # bf16 has 8 significant bits: truncate the target to them
        if target == 0:
            out.append(Fraction(0))
            continue
        e = ilog2(abs(target))
        ulp = Fraction(2) ** (e - 7)
        v = (abs(target) / ulp).numerator // (abs(target) / ulp).denominator * ulp
        out.append(v if target > 0 else -v)
    return out


# (name, bits, meta, mn, mx, the separating element x or None, what it pins)
CASES = [
    ("scale_L3", 2, 0, Fraction(-1, 2), Fraction(33, 64), None,
     "d = 1.015625: d/3 rounds to 0x3EAD5555, d*(1/3) to 0x3EAD5556"),
    ("scale_L15", 4, 0, Fraction(-1, 2), Fraction(9, 16), None,
     "d = 1.0625: d/15 rounds to 0x3D911111, d*(1/15) to 0x3D911112"),
    ("code_L3", 2, 0, Fraction(-1), Fraction(13, 32), Fraction(11, 64),
     "y = 1.171875 = 2.5 s exactly: y*inv rounds above 2.5 (code 3), y/s is the tie 2.5 (code 2)"),
    ("code_L3_inv", 2, 0, Fraction(-1), Fraction(67, 64), Fraction(3, 128),
     "y = 1.0234375: y*inv gives code 1; y/s and y*(3/d) give code 2"),
    ("code_L15", 4, 0, Fraction(-1), Fraction(29, 64), Fraction(27, 128),
     "y = 1.2109375: y*inv gives code 13; y/s and y*(15/d) give code 12"),
    ("code16_L3", 2, 1, Fraction(-2), Fraction(55, 64), Fraction(-73, 128),
     "16-bit scale: y = 1.4296875, y*inv gives code 1, y/s gives code 2"),
    ("code16_L15", 4, 1, Fraction(-1), Fraction(131, 64), Fraction(41, 128),
     "16-bit scale: y = 1.3203125, y*inv gives code 7, y/s gives code 6"),
]


def case_inputs(mn, mx, x):
    xs = [mn, mx] + ([x] if x is not None else [])
    xs += _fill(mn, mx, 32 - len(xs))
    for v in xs:
        bf16_bits(v)   # every input is a bf16 value
    return xs


def render() -> str:
    lines = [
        "# Constructed quantiser groups; scale bits and codes derived by exact",
        "# rational arithmetic with IEEE round-to-nearest-even written from its",
        "# definition (tests/golden/make_quantizer_sequence.py; no float",
        "# arithmetic, no oracle).  Format per case:",
        "#   case <name> bits=<b> meta=<0 fp32 | 1 fp16 scale + bf16 zero>",
        "#   x <32 bf16 bit patterns, hex>",
        "#   scale <stored scale bits, hex> zero <stored zero bits, hex>",
        "#   codes <32 codes>",
        "# preceded by comment lines with the derivation of the scale and of",
        "# the separating element.",
        "",
    ]
    for name, bits, meta, mn, mx, x, what in CASES:
        xs = case_inputs(mn, mx, x)
        r = derive(xs, bits, meta)
        L = r["L"]
        q = r["d"] / L
        lo, hi = rne(q), None
        lines.append(f"# {name}: {what}")
        lines.append(f"#   mn = {float(mn)!r}, mx = {float(mx)!r}, d = mx - mn = {r['d']} (exact)")
        lines.append(f"#   d / L = {q} = {float(q)!r}; nearest binary32 {float(lo)!r} "
                     f"(0x{f32_bits(lo):08X}), |error| = {float(abs(lo - q)):.3e}, "
                     f"half ulp = {float(Fraction(2) ** (ilog2(abs(lo)) - 24)):.3e}")
        if meta == 1:
            lines.append(f"#   rounded to binary16: {float(r['s'])!r} (0x{r['s_bits']:04X})")
        lines.append(f"#   inv = rne(1 / s) = {float(r['inv'])!r} (0x{f32_bits(r['inv']):08X})")
        if x is not None:
            i = xs.index(x)
            y, t = r["steps"][i]
            lines.append(f"#   element {i}: x = {float(x)!r}, y = x - mn = {float(y)!r}, "
                         f"y * inv = {y * r['inv']} exactly, rounded {float(t)!r}, "
                         f"code {r['codes'][i]}; y / s = {float(y / r['s'])!r} exactly")
        lines.append(f"case {name} bits={bits} meta={meta}")
        lines.append("x " + " ".join(f"{bf16_bits(v):04X}" for v in xs))
        w = 4 if meta == 1 else 8
        lines.append(f"scale {r['s_bits']:0{w}X} zero {r['z_bits']:0{w}X}")
        lines.append("codes " + " ".join(str(c) for c in r["codes"]))
        lines.append("")
    return "\n".join(lines)


if __name__ == "__main__":
    with open(OUT, "w") as f:
        f.write(render())
    print(OUT)
