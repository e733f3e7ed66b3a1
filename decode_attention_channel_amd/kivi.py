"""ctypes binding of libkivi.so (include/kivi.h): argument marshalling only.

Buffers are torch tensors on the current HIP device; the calls enqueue work
on torch's current stream.  Every step of the method runs in the HIP kernels
of libkivi.so.  There is no fallback: if the library is missing or fails to
load, importing this module raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os

import numpy as np
import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkivi.so")

STATUS = {
    0: "KIVI_OK", 1: "KIVI_E_NULL", 2: "KIVI_E_GEOMETRY", 3: "KIVI_E_UNSUPPORTED",
    4: "KIVI_E_SEQLEN", 5: "KIVI_E_CAPACITY", 6: "KIVI_E_RESIDUAL_FULL",
    7: "KIVI_E_WORKSPACE", 8: "KIVI_E_HIP", 9: "KIVI_E_STATE",
}
EXPORTS = (
    "kivi_cache_layout", "kivi_decode_workspace_bytes", "kivi_quantize_prefill",
    "kivi_append_token", "kivi_flush_residual", "kivi_decode_attention",
    "kivi_decode_step", "kivi_dense_decode_attention", "kivi_ragged_prefill",
    "kivi_ragged_decode_step", "kivi_paged_layout", "kivi_paged_prefill",
    "kivi_paged_decode_step", "kivi_decode_step_noalloc", "kivi_status_string",
    "kivi_last_hip_error",
)
BUFFERS = ("records", "k_res", "v_res")   # order of the KIVI_BUF_* sizes
META_FP32, META_FP16_BF16 = 0, 1   # scale/zero formats (kivi_geom.meta_format)
FLAG_DETERMINISTIC = 1              # kivi_geom.flags: bitwise-repeatable decode launches
SEQ_BAD_LENGTH, SEQ_FULL = 1, 2     # per-sequence state flags (mixed-length batches)


class KiviError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        name = STATUS.get(status, str(status))
        msg = f"{where}: {name} ({_lib.kivi_status_string(status).decode()})"
        if status == 8:
            msg += f", hipError {_lib.kivi_last_hip_error()}"
        super().__init__(msg)


class _Geom(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "kv_heads", "q_per_kv", "head_dim", "bits", "group", "residual",
        "max_tokens", "meta_format", "flags")]


class _Cache(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in BUFFERS] + [
        ("n_q", ctypes.c_int32), ("n_res", ctypes.c_int32), ("res_start", ctypes.c_int32)]


class _PagedCache(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in BUFFERS] + [
        ("block_table", ctypes.c_void_p), ("page_groups", ctypes.c_int32),
        ("num_pages", ctypes.c_int32)]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built: run `python "
                          "decode_attention_channel_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(_LIB_PATH)
    G, C, P = ctypes.POINTER(_Geom), ctypes.POINTER(_Cache), ctypes.c_void_p
    sz = ctypes.POINTER(ctypes.c_size_t)
    lib.kivi_cache_layout.argtypes = [G, sz]
    lib.kivi_decode_workspace_bytes.argtypes = [G, ctypes.c_int32, ctypes.c_int32]
    lib.kivi_quantize_prefill.argtypes = [G, C, P, P, ctypes.c_int32, P]
    lib.kivi_append_token.argtypes = [G, C, P, P, P]
    lib.kivi_flush_residual.argtypes = [G, C, ctypes.POINTER(ctypes.c_int32), P]
    lib.kivi_decode_attention.argtypes = [G, C, P, P, ctypes.c_float, P, ctypes.c_size_t, P]
    lib.kivi_decode_step.argtypes = [G, C, P, P, P, P, ctypes.c_float, P, ctypes.c_size_t,
                                     ctypes.POINTER(ctypes.c_int32), P]
    lib.kivi_decode_step_noalloc.argtypes = [G, C, P, P, P, P, ctypes.c_float,
                                             ctypes.POINTER(ctypes.c_int32), P]
    lib.kivi_dense_decode_attention.argtypes = [G, P, P, ctypes.c_int32, P, P, ctypes.c_float, P,
                                                ctypes.c_size_t, P]
    lib.kivi_ragged_prefill.argtypes = [G, C, P, P, ctypes.c_int32, P, P, P]
    lib.kivi_ragged_decode_step.argtypes = [G, C, P, P, P, P, P, P, ctypes.c_float, P,
                                            ctypes.c_size_t, P]
    PC = ctypes.POINTER(_PagedCache)
    lib.kivi_paged_layout.argtypes = [G, ctypes.c_int32, ctypes.c_int32, sz,
                                      ctypes.POINTER(ctypes.c_int32)]
    lib.kivi_paged_prefill.argtypes = [G, PC, P, P, ctypes.c_int32, P, P, P]
    lib.kivi_paged_decode_step.argtypes = [G, PC, P, P, P, P, P, P, ctypes.c_float, P,
                                           ctypes.c_size_t, P]
    for f in EXPORTS[:-2]:
        getattr(lib, f).restype = ctypes.c_int
    lib.kivi_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.kivi_status_string.argtypes = [ctypes.c_int]
    lib.kivi_status_string.restype = ctypes.c_char_p
    lib.kivi_last_hip_error.restype = ctypes.c_int32
    return lib


_lib = _load()


def library_path() -> str:
    return _LIB_PATH


def raw_library():
    return _lib


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
    meta_format: int = META_FP32
    flags: int = 0

    def c(self) -> _Geom:
        return _Geom(*dataclasses.astuple(self))

    @property
    def q_heads(self) -> int:
        return self.kv_heads * self.q_per_kv

    @property
    def slots(self) -> int:
        return self.residual + self.group


def _check(status: int, where: str):
    if status != 0:
        raise KiviError(status, where)


def cache_layout(g: Geom) -> list[int]:
    """Byte sizes of the cache buffers, in the order of BUFFERS."""
    out = (ctypes.c_size_t * len(BUFFERS))()
    _check(_lib.kivi_cache_layout(ctypes.byref(g.c()), out), "kivi_cache_layout")
    return list(out)


def workspace_bytes(g: Geom, n_q: int | None = None, n_res: int | None = None) -> int:
    """kivi_decode_workspace_bytes; by default for the fullest cache state
    (n_q = max_tokens, n_res = R+G), which serves every state."""
    n_q = g.max_tokens if n_q is None else n_q
    n_res = g.slots if n_res is None else n_res
    n = _lib.kivi_decode_workspace_bytes(ctypes.byref(g.c()), n_q, n_res)
    if n == 0:
        raise ValueError(f"kivi_decode_workspace_bytes: invalid geometry or counts "
                         f"({g}, n_q={n_q}, n_res={n_res})")
    return n


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: torch.Tensor, dtype, shape=None, name="tensor") -> ctypes.c_void_p:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def record_bytes(g: Geom) -> int:
    return 1024 * (g.bits + (1 if g.meta_format == META_FP16_BF16 else 2))


def records_to_arrays(rec: np.ndarray, bits: int, meta: int) -> dict:
    """Group records [N][bytes] -> per-array layout of N groups (kivi.h):
    k_codes [N][G][D*b/8], k_scale/k_zero [N][D], v_codes [N][G/8][D][b],
    v_scale/v_zero [N][D/G][G]; scale/zero as fp32 or as 16-bit patterns."""
    N = rec.shape[0]
    r = rec.reshape(N, -1, 64, 16)
    t = np.arange(32)[:, None]
    j = np.arange(4)[None, :]
    lane = 16 * j + 4 * (t >> 3) + (t & 3)              # [32][4]: 32-channel block j of row t
    tile = np.broadcast_to((t >> 2) & 1, lane.shape)
    if bits == 2:
        kc = r[:, 0][:, lane[..., None], 8 * tile[..., None] + np.arange(8)]   # [N][32][4][8]
    else:
        kc = r[:, tile, lane, :]                                                # [N][32][4][16]
    kc = kc.reshape(N, 32, 16 * bits)
    o = np.arange(4)[:, None]
    c4 = np.arange(32)[None, :]
    vl = 16 * o + (c4 >> 1)                                                     # [4][32]
    if bits == 2:
        vc = r[:, 1][:, vl[..., None], 8 * np.broadcast_to(c4 & 1, vl.shape)[..., None] + np.arange(8)]
    else:
        vc = r[:, 2 + np.broadcast_to(c4 & 1, vl.shape), vl, :]
    vc = vc.reshape(N, 4, 128, bits)
    if meta == 1:
        m = np.ascontiguousarray(r[:, bits]).view(np.uint16).reshape(N, 64, 8)
        ks, kz, vs, vz = (m[:, :, 2 * i:2 * i + 2].reshape(N, 128) for i in range(4))
    else:
        m0 = np.ascontiguousarray(r[:, bits]).view(np.float32).reshape(N, 64, 4)
        m1 = np.ascontiguousarray(r[:, bits + 1]).view(np.float32).reshape(N, 64, 4)
        ks, kz = m0[:, :, 0:2].reshape(N, 128), m0[:, :, 2:4].reshape(N, 128)
        vs, vz = m1[:, :, 0:2].reshape(N, 128), m1[:, :, 2:4].reshape(N, 128)
    return {"k_codes": kc, "k_scale": ks, "k_zero": kz, "v_codes": vc,
            "v_scale": vs.reshape(N, 4, 32), "v_zero": vz.reshape(N, 4, 32)}


class Cache:
    """The cache buffers (torch tensors, shaped by the documented layout:
    records uint8 [B][H][NG][record bytes], k_res / v_res bf16 [B][H][R+G][D])
    and the host-side counters."""

    def __init__(self, g: Geom, device=None):
        device = torch.device("cuda", torch.cuda.current_device()) if device is None else device
        sizes = cache_layout(g)
        B, H, D = g.batch, g.kv_heads, g.head_dim
        NG, S = g.max_tokens // g.group, g.residual + g.group
        shapes = {"records": ((B, H, NG, record_bytes(g)), torch.uint8),
                  "k_res": ((B, H, S, D), torch.bfloat16),
                  "v_res": ((B, H, S, D), torch.bfloat16)}
        self.geom = g
        for (name, (shape, dt)), nbytes in zip(shapes.items(), sizes):
            t = torch.empty(shape, dtype=dt, device=device)
            assert t.numel() * t.element_size() == nbytes, name
            setattr(self, name, t)
        self._c = _Cache(*[ctypes.c_void_p(getattr(self, n).data_ptr()) for n in BUFFERS],
                         0, 0, 0)

    @property
    def n_q(self) -> int:
        return self._c.n_q

    @property
    def n_res(self) -> int:
        return self._c.n_res

    @property
    def res_start(self) -> int:
        return self._c.res_start

    def set_counters(self, n_q: int, n_res: int, res_start: int):
        self._c.n_q, self._c.n_res, self._c.res_start = n_q, n_res, res_start

    def nbytes(self) -> int:
        return sum(getattr(self, n).numel() * getattr(self, n).element_size() for n in BUFFERS)

    # geometry fields that fix the buffers' meaning (flags only pick a launch)
    _STATE_GEOM = ("batch", "kv_heads", "q_per_kv", "head_dim", "bits", "group", "residual",
                   "meta_format")

    def state_dict(self) -> dict:
        """Snapshot for checkpointing: host copies of the live group records
        (the first n_q / G of every unit), the whole residual ring, and the
        counters, as tensors and ints (loadable with torch.load(...,
        weights_only=True)).  Enqueued work on the cache must have finished:
        the copies synchronise with the current stream."""
        g = self.geom
        ng = self.n_q // g.group
        return {"geom": {k: getattr(g, k) for k in self._STATE_GEOM},
                "n_q": self.n_q, "n_res": self.n_res, "res_start": self.res_start,
                "records": self.records[:, :, :ng].cpu().contiguous(),
                "k_res": self.k_res.cpu(), "v_res": self.v_res.cpu()}

    def load_state_dict(self, sd: dict) -> None:
        """Restore a state_dict() snapshot into this cache (same geometry; its
        max_tokens may be larger): the stream continues exactly as it would
        have from the snapshot."""
        g = self.geom
        want = {k: getattr(g, k) for k in self._STATE_GEOM}
        if sd["geom"] != want:
            raise ValueError(f"snapshot geometry {sd['geom']} does not match {want}")
        n_q, n_res, res_start = int(sd["n_q"]), int(sd["n_res"]), int(sd["res_start"])
        ng = n_q // g.group
        if (n_q % g.group or not 0 <= n_q <= g.max_tokens or not 0 <= n_res <= g.slots or
                not 0 <= res_start < g.slots or res_start % g.group or
                tuple(sd["records"].shape) != tuple(self.records.shape[:2]) + (ng, self.records.shape[3]) or
                sd["k_res"].shape != self.k_res.shape or sd["v_res"].shape != self.v_res.shape):
            raise ValueError("snapshot counters or buffer shapes do not fit this cache")
        self.records[:, :, :ng].copy_(sd["records"])
        self.k_res.copy_(sd["k_res"])
        self.v_res.copy_(sd["v_res"])
        self.set_counters(n_q, n_res, res_start)

    def history(self) -> dict:
        """Host copy of the quantised history in the per-array layout
        (k_codes [B][H][T][D*b/8], k_scale ..., as numpy arrays) from the
        group records the cache keeps."""
        g = self.geom
        B, H, NG = g.batch, g.kv_heads, g.max_tokens // g.group
        arr = records_to_arrays(self.records.cpu().numpy().reshape(B * H * NG, -1), g.bits,
                                g.meta_format)
        out = {n: a.reshape((B, H, NG) + a.shape[1:]) for n, a in arr.items()}
        out["k_codes"] = out["k_codes"].reshape(B, H, NG * g.group, -1)
        return out


def paged_layout(g: Geom, page_groups: int, num_pages: int) -> tuple[list[int], int]:
    out = (ctypes.c_size_t * len(BUFFERS))()
    mp = ctypes.c_int32(0)
    _check(_lib.kivi_paged_layout(ctypes.byref(g.c()), page_groups, num_pages, out,
                                  ctypes.byref(mp)), "kivi_paged_layout")
    return list(out), mp.value


class PagedCache:
    """Pools of a paged history (shaped [slots][...] by the documented
    layout), the residual rings and the block table (int32 [B][max_pages],
    all entries -1 = unassigned until the caller assigns pages)."""

    def __init__(self, g: Geom, page_groups: int, num_pages: int, device=None):
        device = torch.device("cuda", torch.cuda.current_device()) if device is None else device
        sizes, self.max_pages = paged_layout(g, page_groups, num_pages)
        B, H, D = g.batch, g.kv_heads, g.head_dim
        n, S = num_pages * H * page_groups, g.residual + g.group
        shapes = {"records": ((n, record_bytes(g)), torch.uint8),
                  "k_res": ((B, H, S, D), torch.bfloat16),
                  "v_res": ((B, H, S, D), torch.bfloat16)}
        self.geom, self.page_groups, self.num_pages = g, page_groups, num_pages
        for (name, (shape, dt)), nbytes in zip(shapes.items(), sizes):
            t = torch.empty(shape, dtype=dt, device=device)
            assert t.numel() * t.element_size() == nbytes, name
            setattr(self, name, t)
        self.block_table = torch.full((B, self.max_pages), -1, dtype=torch.int32, device=device)
        self._c = _PagedCache(*[ctypes.c_void_p(getattr(self, n).data_ptr()) for n in BUFFERS],
                              ctypes.c_void_p(self.block_table.data_ptr()), page_groups,
                              num_pages)

    def pool_history(self) -> dict:
        """Host copy of the pool in the per-array per-slot layout (k_codes
        [slots][G][D*b/8], k_scale [slots][D], ...) from its group records."""
        g = self.geom
        return records_to_arrays(self.records.cpu().numpy(), g.bits, g.meta_format)

    def slot(self, b: int, h: int, g: int, table=None) -> int:
        """Pool slot of group g of (sequence b, kv head h); -1 without a page."""
        table = self.block_table.cpu() if table is None else table
        e = int(table[b, g // self.page_groups])
        if e < 0 or e >= self.num_pages:
            return -1
        return (e * self.geom.kv_heads + h) * self.page_groups + g % self.page_groups


def paged_prefill(g: Geom, c: PagedCache, k: torch.Tensor, v: torch.Tensor,
                  seq_lens: torch.Tensor, state: torch.Tensor | None = None) -> torch.Tensor:
    """Mixed-length prefill into a paged cache (see ragged_prefill)."""
    stride = k.shape[2] if k.dim() == 4 else -1
    shape = (g.batch, g.kv_heads, stride, g.head_dim)
    if state is None:
        state = torch.empty(g.batch, 4, dtype=torch.int32, device=k.device)
    _check(_lib.kivi_paged_prefill(ctypes.byref(g.c()), ctypes.byref(c._c),
                                   _ptr(k, torch.bfloat16, shape, "k"),
                                   _ptr(v, torch.bfloat16, shape, "v"), stride,
                                   _ptr(seq_lens, torch.int32, (g.batch,), "seq_lens"),
                                   _ptr(state, torch.int32, (g.batch, 4), "state"), _stream()),
           "kivi_paged_prefill")
    return state


def paged_decode_step(g: Geom, c: PagedCache, state_in: torch.Tensor, state_out: torch.Tensor,
                      k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                      out: torch.Tensor | None = None, softmax_scale: float | None = None,
                      ws: Workspace | None = None) -> torch.Tensor:
    """One mixed-length step over a paged cache (see ragged_decode_step)."""
    shape = (g.batch, g.q_heads, g.head_dim)
    tok = (g.batch, g.kv_heads, g.head_dim)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=q.device)
    if ws is None:
        ws = Workspace(g, q.device)
    scale = 1.0 / math.sqrt(g.head_dim) if softmax_scale is None else float(softmax_scale)
    _check(_lib.kivi_paged_decode_step(
        ctypes.byref(g.c()), ctypes.byref(c._c),
        _ptr(state_in, torch.int32, (g.batch, 4), "state_in"),
        _ptr(state_out, torch.int32, (g.batch, 4), "state_out"),
        _ptr(k_new, torch.bfloat16, tok, "k_new"), _ptr(v_new, torch.bfloat16, tok, "v_new"),
        _ptr(q, torch.bfloat16, shape, "q"), _ptr(out, torch.float32, shape, "out"), scale,
        ctypes.c_void_p(ws.buf.data_ptr()), ws.nbytes, _stream()), "kivi_paged_decode_step")
    return out


def quantize_prefill(g: Geom, c: Cache, k: torch.Tensor, v: torch.Tensor) -> None:
    """k, v: bf16 [B][H][S][D] on the device."""
    S = k.shape[2] if k.dim() == 4 else -1
    shape = (g.batch, g.kv_heads, S, g.head_dim)
    _check(_lib.kivi_quantize_prefill(ctypes.byref(g.c()), ctypes.byref(c._c),
                                      _ptr(k, torch.bfloat16, shape, "k"),
                                      _ptr(v, torch.bfloat16, shape, "v"), S, _stream()),
           "kivi_quantize_prefill")


def append_token(g: Geom, c: Cache, k_new: torch.Tensor, v_new: torch.Tensor) -> None:
    shape = (g.batch, g.kv_heads, g.head_dim)
    _check(_lib.kivi_append_token(ctypes.byref(g.c()), ctypes.byref(c._c),
                                  _ptr(k_new, torch.bfloat16, shape, "k_new"),
                                  _ptr(v_new, torch.bfloat16, shape, "v_new"), _stream()),
           "kivi_append_token")


def flush_residual(g: Geom, c: Cache) -> int:
    flushed = ctypes.c_int32(0)
    _check(_lib.kivi_flush_residual(ctypes.byref(g.c()), ctypes.byref(c._c),
                                    ctypes.byref(flushed), _stream()), "kivi_flush_residual")
    return flushed.value


class Workspace:
    """Device workspace for decode attention, zero-filled once (the calls
    leave its arrival counters at zero).  Sized by kivi_decode_workspace_bytes
    for a cache of n_q quantised and n_res residual tokens; by default for the
    fullest state of the geometry, which serves every call on it."""

    def __init__(self, g: Geom, device=None, n_q: int | None = None, n_res: int | None = None):
        device = torch.device("cuda", torch.cuda.current_device()) if device is None else device
        self.nbytes = workspace_bytes(g, n_q, n_res)
        self.buf = torch.zeros(max(self.nbytes, 16), dtype=torch.uint8, device=device)


def decode_attention(g: Geom, c: Cache, q: torch.Tensor, out: torch.Tensor | None = None,
                     softmax_scale: float | None = None, ws: Workspace | None = None
                     ) -> torch.Tensor:
    """q: bf16 [B][H*QPK][D] -> fp32 [B][H*QPK][D]."""
    shape = (g.batch, g.q_heads, g.head_dim)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=q.device)
    if ws is None:
        ws = Workspace(g, q.device)
    scale = 1.0 / math.sqrt(g.head_dim) if softmax_scale is None else float(softmax_scale)
    _check(_lib.kivi_decode_attention(ctypes.byref(g.c()), ctypes.byref(c._c),
                                      _ptr(q, torch.bfloat16, shape, "q"),
                                      _ptr(out, torch.float32, shape, "out"), scale,
                                      ctypes.c_void_p(ws.buf.data_ptr()), ws.nbytes, _stream()),
           "kivi_decode_attention")
    return out


def decode_step(g: Geom, c: Cache, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                out: torch.Tensor | None = None, softmax_scale: float | None = None,
                ws: Workspace | None = None) -> tuple[torch.Tensor, int]:
    """Append k_new/v_new (bf16 [B][H][D]), flush if the ring is full, attend
    with q (bf16 [B][H*QPK][D]); returns (out fp32 [B][H*QPK][D], flushed)."""
    shape = (g.batch, g.q_heads, g.head_dim)
    tok = (g.batch, g.kv_heads, g.head_dim)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=q.device)
    if ws is None:
        ws = Workspace(g, q.device)
    scale = 1.0 / math.sqrt(g.head_dim) if softmax_scale is None else float(softmax_scale)
    flushed = ctypes.c_int32(0)
    _check(_lib.kivi_decode_step(ctypes.byref(g.c()), ctypes.byref(c._c),
                                 _ptr(k_new, torch.bfloat16, tok, "k_new"),
                                 _ptr(v_new, torch.bfloat16, tok, "v_new"),
                                 _ptr(q, torch.bfloat16, shape, "q"),
                                 _ptr(out, torch.float32, shape, "out"), scale,
                                 ctypes.c_void_p(ws.buf.data_ptr()), ws.nbytes,
                                 ctypes.byref(flushed), _stream()),
           "kivi_decode_step")
    return out, flushed.value


def decode_step_noalloc(g: Geom, c: Cache, k_new: torch.Tensor, v_new: torch.Tensor,
                        q: torch.Tensor, out: torch.Tensor, softmax_scale: float | None = None
                        ) -> int:
    """kivi_decode_step_noalloc: decode_step with the library's static device
    workspace (no workspace argument; `out` must be given, so that nothing is
    allocated).  Returns 1 if a group was flushed, else 0."""
    shape = (g.batch, g.q_heads, g.head_dim)
    tok = (g.batch, g.kv_heads, g.head_dim)
    scale = 1.0 / math.sqrt(g.head_dim) if softmax_scale is None else float(softmax_scale)
    flushed = ctypes.c_int32(0)
    _check(_lib.kivi_decode_step_noalloc(ctypes.byref(g.c()), ctypes.byref(c._c),
                                         _ptr(k_new, torch.bfloat16, tok, "k_new"),
                                         _ptr(v_new, torch.bfloat16, tok, "v_new"),
                                         _ptr(q, torch.bfloat16, shape, "q"),
                                         _ptr(out, torch.float32, shape, "out"), scale,
                                         ctypes.byref(flushed), _stream()),
           "kivi_decode_step_noalloc")
    return flushed.value


def dense_decode_attention(g: Geom, k: torch.Tensor, v: torch.Tensor, seq_len: int,
                           q: torch.Tensor, out: torch.Tensor | None = None,
                           softmax_scale: float | None = None, ws: Workspace | None = None
                           ) -> torch.Tensor:
    """Baseline attention over an uncompressed cache: k, v bf16
    [B][H][g.max_tokens][D], first seq_len tokens; q bf16 [B][H*QPK][D] ->
    fp32 [B][H*QPK][D].  A workspace passed in must hold
    workspace_bytes(g, 0, seq_len)."""
    shape = (g.batch, g.q_heads, g.head_dim)
    kv_shape = (g.batch, g.kv_heads, g.max_tokens, g.head_dim)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=q.device)
    if ws is None:
        ws = Workspace(g, q.device, n_q=0, n_res=int(seq_len))
    scale = 1.0 / math.sqrt(g.head_dim) if softmax_scale is None else float(softmax_scale)
    _check(_lib.kivi_dense_decode_attention(ctypes.byref(g.c()),
                                            _ptr(k, torch.bfloat16, kv_shape, "k"),
                                            _ptr(v, torch.bfloat16, kv_shape, "v"), int(seq_len),
                                            _ptr(q, torch.bfloat16, shape, "q"),
                                            _ptr(out, torch.float32, shape, "out"), scale,
                                            ctypes.c_void_p(ws.buf.data_ptr()), ws.nbytes,
                                            _stream()),
           "kivi_dense_decode_attention")
    return out


def ragged_prefill(g: Geom, c: Cache, k: torch.Tensor, v: torch.Tensor,
                   seq_lens: torch.Tensor, state: torch.Tensor | None = None) -> torch.Tensor:
    """Mixed-length prefill.  k, v: bf16 [B][H][stride][D]; seq_lens: int32
    [B] on the device.  Returns the per-sequence state, int32 [B][4]
    {n_q, n_res, res_start, flags} (written into `state` if given)."""
    stride = k.shape[2] if k.dim() == 4 else -1
    shape = (g.batch, g.kv_heads, stride, g.head_dim)
    if state is None:
        state = torch.empty(g.batch, 4, dtype=torch.int32, device=k.device)
    _check(_lib.kivi_ragged_prefill(ctypes.byref(g.c()), ctypes.byref(c._c),
                                    _ptr(k, torch.bfloat16, shape, "k"),
                                    _ptr(v, torch.bfloat16, shape, "v"), stride,
                                    _ptr(seq_lens, torch.int32, (g.batch,), "seq_lens"),
                                    _ptr(state, torch.int32, (g.batch, 4), "state"), _stream()),
           "kivi_ragged_prefill")
    return state


def ragged_decode_step(g: Geom, c: Cache, state_in: torch.Tensor, state_out: torch.Tensor,
                       k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                       out: torch.Tensor | None = None, softmax_scale: float | None = None,
                       ws: Workspace | None = None) -> torch.Tensor:
    """One step of a mixed-length batch: reads state_in, writes state_out
    (int32 [B][4] each), returns out fp32 [B][H*QPK][D]."""
    shape = (g.batch, g.q_heads, g.head_dim)
    tok = (g.batch, g.kv_heads, g.head_dim)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=q.device)
    if ws is None:
        ws = Workspace(g, q.device)
    scale = 1.0 / math.sqrt(g.head_dim) if softmax_scale is None else float(softmax_scale)
    _check(_lib.kivi_ragged_decode_step(
        ctypes.byref(g.c()), ctypes.byref(c._c),
        _ptr(state_in, torch.int32, (g.batch, 4), "state_in"),
        _ptr(state_out, torch.int32, (g.batch, 4), "state_out"),
        _ptr(k_new, torch.bfloat16, tok, "k_new"), _ptr(v_new, torch.bfloat16, tok, "v_new"),
        _ptr(q, torch.bfloat16, shape, "q"), _ptr(out, torch.float32, shape, "out"), scale,
        ctypes.c_void_p(ws.buf.data_ptr()), ws.nbytes, _stream()), "kivi_ragged_decode_step")
    return out


class LayerStepper:
    """Pre-marshalled arguments of one layer's decode step (append, flush,
    attend as separate calls, or step() for the fused kivi_decode_step) for
    tight loops: the geometry, cache, workspace, q/out buffers,
    softmax scale and stream (torch's current stream at construction) are
    converted once; append() checks only the new token's tensors."""

    def __init__(self, g: Geom, c: Cache, ws: Workspace, q: torch.Tensor, out: torch.Tensor,
                 softmax_scale: float | None = None):
        shape_q = (g.batch, g.q_heads, g.head_dim)
        self.geom, self.cache = g, c
        self._g = g.c()
        self._gp, self._cp = ctypes.byref(self._g), ctypes.byref(c._c)
        self._q = _ptr(q, torch.bfloat16, shape_q, "q")
        self._out = _ptr(out, torch.float32, shape_q, "out")
        self._keep = (q, out, ws)
        self._ws, self._wsn = ctypes.c_void_p(ws.buf.data_ptr()), ws.nbytes
        scale = 1.0 / math.sqrt(g.head_dim) if softmax_scale is None else float(softmax_scale)
        self._scale = ctypes.c_float(scale)
        self._stream = _stream()
        self._flushed = ctypes.c_int32(0)
        self._tok_shape = (g.batch, g.kv_heads, g.head_dim)

    def _check_token(self, k_new: torch.Tensor, v_new: torch.Tensor) -> None:
        if (k_new.shape != self._tok_shape or v_new.shape != self._tok_shape or
                k_new.dtype != torch.bfloat16 or v_new.dtype != torch.bfloat16 or
                not k_new.is_contiguous() or not v_new.is_contiguous()):
            raise ValueError("k_new / v_new must be contiguous bf16 [B][H][D]")

    def append(self, k_new: torch.Tensor, v_new: torch.Tensor) -> None:
        self._check_token(k_new, v_new)
        _check(_lib.kivi_append_token(self._gp, self._cp, ctypes.c_void_p(k_new.data_ptr()),
                                      ctypes.c_void_p(v_new.data_ptr()), self._stream),
               "kivi_append_token")

    def flush(self) -> int:
        _check(_lib.kivi_flush_residual(self._gp, self._cp, ctypes.byref(self._flushed),
                                        self._stream), "kivi_flush_residual")
        return self._flushed.value

    def attend(self) -> None:
        _check(_lib.kivi_decode_attention(self._gp, self._cp, self._q, self._out, self._scale,
                                          self._ws, self._wsn, self._stream),
               "kivi_decode_attention")

    def step(self, k_new: torch.Tensor, v_new: torch.Tensor) -> int:
        self._check_token(k_new, v_new)
        _check(_lib.kivi_decode_step(self._gp, self._cp, ctypes.c_void_p(k_new.data_ptr()),
                                     ctypes.c_void_p(v_new.data_ptr()), self._q, self._out,
                                     self._scale, self._ws, self._wsn,
                                     ctypes.byref(self._flushed), self._stream),
               "kivi_decode_step")
        return self._flushed.value


class RaggedStepper:
    """Pre-marshalled kivi_ragged_decode_step (kivi_paged_decode_step for a
    PagedCache) of one layer for tight loops
    and graph capture: the new token, q and out buffers are fixed (the
    caller refills them), and the two state buffers alternate, step(0)
    reading state_a and writing state_b, step(1) the other way round.  The
    stream is torch's current stream at each call, so that a capture sees
    its capture stream."""

    def __init__(self, g: Geom, c: Cache, ws: Workspace, state_a: torch.Tensor,
                 state_b: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                 q: torch.Tensor, out: torch.Tensor, softmax_scale: float | None = None):
        shape_q = (g.batch, g.q_heads, g.head_dim)
        tok = (g.batch, g.kv_heads, g.head_dim)
        self.geom, self.cache = g, c
        self._g = g.c()
        self._gp, self._cp = ctypes.byref(self._g), ctypes.byref(c._c)
        self._fn = (_lib.kivi_paged_decode_step if isinstance(c, PagedCache)
                    else _lib.kivi_ragged_decode_step)
        st = [_ptr(x, torch.int32, (g.batch, 4), "state") for x in (state_a, state_b)]
        if st[0].value == st[1].value:
            raise ValueError("state_a and state_b must be distinct buffers")
        self._st = st
        self._k = _ptr(k_new, torch.bfloat16, tok, "k_new")
        self._v = _ptr(v_new, torch.bfloat16, tok, "v_new")
        self._q = _ptr(q, torch.bfloat16, shape_q, "q")
        self._out = _ptr(out, torch.float32, shape_q, "out")
        self._keep = (ws, state_a, state_b, k_new, v_new, q, out)
        self._ws, self._wsn = ctypes.c_void_p(ws.buf.data_ptr()), ws.nbytes
        scale = 1.0 / math.sqrt(g.head_dim) if softmax_scale is None else float(softmax_scale)
        self._scale = ctypes.c_float(scale)

    def step(self, parity: int) -> None:
        a, b = self._st[parity & 1], self._st[(parity & 1) ^ 1]
        _check(self._fn(self._gp, self._cp, a, b, self._k, self._v, self._q, self._out,
                        self._scale, self._ws, self._wsn, _stream()), self._fn.__name__)
