"""CPU oracle of the KIVI hot path (ctypes wrapper around kivi_oracle.c).

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the product path never does.
It shares no code with the HIP library (``decode_attention_channel_amd``)
and does not import it.

The C source states what each function computes and which page passage it
follows.  Arrays are numpy; bf16 tensors travel as uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kivi_oracle.c")
_LIB = os.path.join(_HERE, "libkivi_oracle.so")
_CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile kivi_oracle.c with gcc (no FMA contraction, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


class _Geom(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "batch", "kv_heads", "q_per_kv", "head_dim", "bits", "group", "residual",
        "max_tokens", "meta")]


class _Cache(ctypes.Structure):
    _fields_ = [
        ("k_codes", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
        ("k_zero", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p), ("v_zero", ctypes.c_void_p),
        ("k_res", ctypes.c_void_p), ("v_res", ctypes.c_void_p),
        ("n_q", ctypes.c_int), ("n_res", ctypes.c_int), ("res_start", ctypes.c_int),
    ]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        G = ctypes.POINTER(_Geom)
        C = ctypes.POINTER(_Cache)
        L.kivio_quantize_values.argtypes = [P, ctypes.c_int, ctypes.c_int, P, P, P]
        L.kivio_quantize_values.restype = None
        L.kivio_quantize_values_h.argtypes = [P, ctypes.c_int, ctypes.c_int, P, P, P]
        L.kivio_quantize_values_h.restype = None
        L.kivio_prefill_split.argtypes = [ctypes.c_int] * 3
        L.kivio_prefill_split.restype = ctypes.c_int
        L.kivio_prefill.argtypes = [G, C, P, P, ctypes.c_int]
        L.kivio_prefill.restype = ctypes.c_int
        L.kivio_append.argtypes = [G, C, P, P]
        L.kivio_append.restype = ctypes.c_int
        L.kivio_flush.argtypes = [G, C]
        L.kivio_flush.restype = ctypes.c_int
        L.kivio_dequant_unit.argtypes = [G, C, ctypes.c_long, P, P]
        L.kivio_dequant_unit.restype = None
        L.kivio_attend_row.argtypes = [P, P, P, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_double, P]
        L.kivio_attend_row.restype = None
        L.kivio_attention_unit.argtypes = [G, C, ctypes.c_long, P, ctypes.c_float, P]
        L.kivio_attention_unit.restype = ctypes.c_int
        L.kivio_attention_dense_unit.argtypes = [G, P, P, ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_long, P, ctypes.c_float, P]
        L.kivio_attention_dense_unit.restype = ctypes.c_int
        L.kivio_bytes_per_token.argtypes = [ctypes.c_int] * 7 + [P]
        L.kivio_bytes_per_token.restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


@dataclasses.dataclass(frozen=True)
class Geom:
    batch: int
    kv_heads: int
    q_per_kv: int
    head_dim: int = 128
    bits: int = 2
    group: int = 32
    residual: int = 128
    max_tokens: int = 0
    meta: int = 0   # scale/zero format: 0 = fp32/fp32, 1 = fp16 scale, bf16 zero

    @property
    def units(self) -> int:
        return self.batch * self.kv_heads

    @property
    def n_groups(self) -> int:
        return self.max_tokens // self.group

    @property
    def slots(self) -> int:
        return self.residual + self.group

    def _c(self) -> _Geom:
        if self.head_dim > 256 or self.group > 64 or self.group % 8:
            raise ValueError("oracle supports head_dim <= 256 and group <= 64, group % 8 == 0")
        if self.max_tokens % self.group:
            raise ValueError("max_tokens must be a multiple of group")
        if self.meta not in (0, 1):
            raise ValueError("meta must be 0 (fp32 scale/zero) or 1 (fp16 scale, bf16 zero)")
        return _Geom(*dataclasses.astuple(self))


class Cache:
    """Host copy of every cache buffer, shaped by the documented layout."""

    def __init__(self, g: Geom):
        U, T, D, b, G = g.units, g.max_tokens, g.head_dim, g.bits, g.group
        NG = g.n_groups
        self.geom = g
        self.k_codes = np.zeros((g.batch, g.kv_heads, T, D * b // 8), np.uint8)
        mt = np.uint16 if g.meta == 1 else np.float32   # fp16 / bf16 bits, or fp32
        self.k_scale = np.zeros((g.batch, g.kv_heads, NG, D), mt)
        self.k_zero = np.zeros_like(self.k_scale)
        self.v_codes = np.zeros((g.batch, g.kv_heads, NG, G // 8, D, b), np.uint8)
        self.v_scale = np.zeros((g.batch, g.kv_heads, NG, D // G, G), mt)
        self.v_zero = np.zeros_like(self.v_scale)
        self.k_res = np.zeros((g.batch, g.kv_heads, g.slots, D), np.uint16)
        self.v_res = np.zeros_like(self.k_res)
        self.n_q = 0
        self.n_res = 0
        self.res_start = 0
        del U

    def buffers(self):
        return (self.k_codes, self.k_scale, self.k_zero, self.v_codes, self.v_scale,
                self.v_zero, self.k_res, self.v_res)

    def _c(self) -> _Cache:
        return _Cache(*[_p(a).value for a in self.buffers()], self.n_q, self.n_res,
                      self.res_start)

    def _take(self, c: _Cache):
        self.n_q, self.n_res, self.res_start = c.n_q, c.n_res, c.res_start

    def copy(self) -> "Cache":
        out = Cache(self.geom)
        for dst, src in zip(out.buffers(), self.buffers()):
            dst[...] = src
        out.n_q, out.n_res, out.res_start = self.n_q, self.n_res, self.res_start
        return out


def quantize_values(x: np.ndarray, bits: int, meta: int = 0):
    """Asymmetric min-max quantisation of one group: (codes, scale, zero);
    with meta=1, scale and zero are the fp16 / bf16 bit patterns (uint16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.zeros(x.size, np.uint8)
    mt = np.uint16 if meta == 1 else np.float32
    s = np.zeros(1, mt)
    z = np.zeros(1, mt)
    fn = lib().kivio_quantize_values_h if meta == 1 else lib().kivio_quantize_values
    fn(_p(x), x.size, bits, _p(codes), _p(s), _p(z))
    return codes, s[0], z[0]


def prefill_split(seq_len: int, group: int = 32, residual: int = 128) -> int:
    return lib().kivio_prefill_split(seq_len, group, residual)


def prefill(g: Geom, k: np.ndarray, v: np.ndarray) -> Cache:
    """k, v: uint16 (bf16 bits) [B][H][S][D]."""
    k = np.ascontiguousarray(k, np.uint16)
    v = np.ascontiguousarray(v, np.uint16)
    assert k.shape == v.shape and k.shape[:2] == (g.batch, g.kv_heads)
    assert k.shape[3] == g.head_dim
    c = Cache(g)
    cc = c._c()
    if lib().kivio_prefill(ctypes.byref(g._c()), ctypes.byref(cc), _p(k), _p(v),
                           k.shape[2]) != 0:
        raise ValueError("prefill does not fit the cache capacity")
    c._take(cc)
    return c


def append(c: Cache, k_new: np.ndarray, v_new: np.ndarray) -> None:
    """k_new, v_new: uint16 [B][H][D]; raises when the ring is full."""
    k_new = np.ascontiguousarray(k_new, np.uint16)
    v_new = np.ascontiguousarray(v_new, np.uint16)
    cc = c._c()
    if lib().kivio_append(ctypes.byref(c.geom._c()), ctypes.byref(cc), _p(k_new),
                          _p(v_new)) != 0:
        raise ValueError("residual ring full")
    c._take(cc)


def flush(c: Cache) -> int:
    cc = c._c()
    r = lib().kivio_flush(ctypes.byref(c.geom._c()), ctypes.byref(cc))
    if r < 0:
        raise ValueError("quantised history full")
    c._take(cc)
    return r


def dequant_unit(c: Cache, unit: int):
    """(k, v) float64 [n_q + n_res][D] of unit b*H + h (history then residual)."""
    n = c.n_q + c.n_res
    D = c.geom.head_dim
    k = np.zeros((n, D), np.float64)
    v = np.zeros((n, D), np.float64)
    lib().kivio_dequant_unit(ctypes.byref(c.geom._c()), ctypes.byref(c._c()), unit,
                             _p(k), _p(v))
    return k, v


def attend_row(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    q = np.ascontiguousarray(q, np.float64)
    k = np.ascontiguousarray(k, np.float64)
    v = np.ascontiguousarray(v, np.float64)
    o = np.zeros(q.shape[0], np.float64)
    lib().kivio_attend_row(_p(q), _p(k), _p(v), k.shape[0], k.shape[1], scale, _p(o))
    return o


def attention(c: Cache, q: np.ndarray, scale: float, units=None,
              out: np.ndarray | None = None) -> np.ndarray:
    """Decode attention.  q: uint16 [B][H*QPK][D]; returns float32 of the same
    shape.  With `units`, only the rows of those units are computed (the other
    rows of `out` are left as they are, zero by default)."""
    g = c.geom
    q = np.ascontiguousarray(q, np.uint16)
    assert q.shape == (g.batch, g.kv_heads * g.q_per_kv, g.head_dim)
    if out is None:
        out = np.zeros(q.shape, np.float32)
    gc, cc = g._c(), c._c()
    for u in (range(g.units) if units is None else units):
        if lib().kivio_attention_unit(ctypes.byref(gc), ctypes.byref(cc), int(u), _p(q),
                                      scale, _p(out)) != 0:
            raise ValueError("empty cache")
    return out


def attention_dense(g: Geom, k: np.ndarray, v: np.ndarray, seq_len: int, q: np.ndarray,
                    scale: float, units=None, out: np.ndarray | None = None) -> np.ndarray:
    """Decode attention over an uncompressed bf16 cache (the baseline).
    k, v: uint16 [B][H][T][D] (the first seq_len tokens are attended);
    q: uint16 [B][H*QPK][D]; returns float32 [B][H*QPK][D]."""
    k = np.ascontiguousarray(k, np.uint16)
    v = np.ascontiguousarray(v, np.uint16)
    q = np.ascontiguousarray(q, np.uint16)
    assert k.shape == v.shape and k.shape[:2] == (g.batch, g.kv_heads) and k.shape[3] == g.head_dim
    assert q.shape == (g.batch, g.kv_heads * g.q_per_kv, g.head_dim)
    if out is None:
        out = np.zeros(q.shape, np.float32)
    gc = g._c()
    for u in (range(g.units) if units is None else units):
        if lib().kivio_attention_dense_unit(ctypes.byref(gc), _p(k), _p(v), int(seq_len),
                                            k.shape[2], int(u), _p(q), scale, _p(out)) != 0:
            raise ValueError("seq_len out of range")
    return out


def bytes_per_token(layers, kv_heads, head_dim, bits, group, residual, ctx):
    """(bf16, catalog convention, exact codes, stored incl. fp32 scale/zero,
    stored with fp16 scale + bf16 zero) B/token."""
    out = np.zeros(5, np.float64)
    lib().kivio_bytes_per_token(layers, kv_heads, head_dim, bits, group, residual, ctx,
                                _p(out))
    return tuple(float(x) for x in out)
