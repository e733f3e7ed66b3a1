"""CPU checks of the C ABI: the library loads, exports every function that
include/kivi.h declares, sizes its buffers as the header documents, and
rejects invalid arguments on the host before touching any device (so these
calls are safe without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
kivi = pytest.importorskip("decode_attention_channel_amd.kivi")


def _declared():
    src = open(os.path.join(ROOT, "include", "kivi.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kivi_[a-z_]+)\s*\(", src)))


# the boundary planned before any kernel was written: buffer sizes, workspace
# bytes for a cache state, prefill, append, flush, decode attention, and the
# two error helpers
PLANNED = ("kivi_cache_layout", "kivi_decode_workspace_bytes", "kivi_quantize_prefill",
           "kivi_append_token", "kivi_flush_residual", "kivi_decode_attention",
           "kivi_status_string", "kivi_last_hip_error")


def test_exports_every_declared_function():
    names = _declared()
    assert len(names) == 16
    lib = ctypes.CDLL(kivi.library_path())
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(kivi.EXPORTS)
    assert set(PLANNED) <= set(names)


def _g(**kw):
    base = dict(batch=2, kv_heads=3, q_per_kv=4, head_dim=128, bits=2, group=32, residual=128,
                max_tokens=1024)
    base.update(kw)
    return kivi.Geom(**base)


def _ws(U, qpk, n_q, n_res, c):
    """The workspace size kivi.h documents: counters, then split partials."""
    s = min(max((n_q // 32 * c + -(-n_res // 32) * 16) // (8 * c), 1), 256)
    return 256 * -(-4 * U // 256) + U * qpk * 528 * s


@pytest.mark.parametrize("bits", [2, 4])
def test_layout_sizes(bits):
    U, T, D, NG, S = 6, 1024, 128, 32, 160
    # one record per group in the records buffer, of the bytes of the
    # per-array layout (codes, fp32 scale/zero) in 1 KiB planes, for every
    # number of query heads per kv head
    rec = 1024 * (bits + 2)
    assert rec == 32 * D * bits // 8 * 2 + 4 * D * 4
    for qpk in (1, 4):
        g = _g(bits=bits, q_per_kv=qpk)
        assert kivi.cache_layout(g) == [U * NG * rec, U * S * D * 2, U * S * D * 2]
        assert kivi.workspace_bytes(g) == _ws(U, qpk, T, S, bits + 2)
        assert kivi.workspace_bytes(g, 0, 1) == _ws(U, qpk, 0, 1, bits + 2)
        assert kivi.workspace_bytes(g, 512, 140) == _ws(U, qpk, 512, 140, bits + 2)


def test_workspace_bytes_grows_with_the_state():
    lib = kivi.raw_library()
    g = _g(max_tokens=1 << 20)
    P = ctypes.byref
    prev = 0
    for n_q in range(0, 1 << 20, 4096):
        n = lib.kivi_decode_workspace_bytes(P(g.c()), n_q, 150)
        assert n >= prev and n >= lib.kivi_decode_workspace_bytes(P(g.c()), n_q, 100)
        prev = n
    # capped at 256 partials per (sequence, kv head)
    assert prev == _ws(6, 4, 1 << 20, 150, 4) == 256 + 6 * 4 * 528 * 256
    # invalid counts or geometry: 0
    for n_q, n_res in [(-32, 0), (33, 0), ((1 << 20) + 32, 0), (0, -1)]:
        assert lib.kivi_decode_workspace_bytes(P(g.c()), n_q, n_res) == 0
    assert lib.kivi_decode_workspace_bytes(None, 0, 0) == 0
    assert lib.kivi_decode_workspace_bytes(P(_g(bits=3).c()), 0, 0) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), 2), (dict(kv_heads=-1), 2), (dict(bits=3), 3), (dict(bits=8), 3),
    (dict(head_dim=64), 3), (dict(group=64), 3), (dict(residual=100), 3),
    (dict(q_per_kv=17), 3), (dict(max_tokens=1000), 3), (dict(residual=-32), 2),
    (dict(flags=2), 3), (dict(flags=-1), 3),
    # a (sequence, kv head) may hold at most 2^30 bytes of group records
    (dict(max_tokens=((1 << 18) + 1) * 32), 3),                    # 2-bit, 4 KiB records
    (dict(bits=4, max_tokens=((1 << 30) // 6144 + 1) * 32), 3),   # 4-bit, 6 KiB records
    (dict(bits=2, meta_format=1, max_tokens=((1 << 30) // 3072 + 1) * 32), 3),
])
def test_geometry_rejected(kw, status):
    with pytest.raises(kivi.KiviError) as e:
        kivi.cache_layout(_g(**kw))
    assert e.value.status == status


def test_largest_record_range_accepted():
    for bits, meta, rec in [(2, 0, 4096), (4, 0, 6144), (2, 1, 3072), (4, 1, 5120)]:
        ng = (1 << 30) // rec
        g = _g(bits=bits, meta_format=meta, max_tokens=ng * 32, batch=1, kv_heads=1)
        assert kivi.cache_layout(g)[0] == ng * rec <= 1 << 30
    assert kivi.cache_layout(_g(flags=kivi.FLAG_DETERMINISTIC))[0] > 0


def _cache_struct(n_q=0, n_res=0, res_start=0, null=None):
    ptrs = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(3)]
    if null is not None:
        ptrs[null] = ctypes.c_void_p(0)
    return kivi._Cache(*ptrs, n_q, n_res, res_start)


def _call(fn, *args):
    return getattr(kivi.raw_library(), fn)(*args)


def test_host_validation_before_any_device_work():
    g = _g().c()
    fake = ctypes.c_void_p(0x2000)
    P = ctypes.byref
    # NULL geometry / cache / buffers / inputs
    assert _call("kivi_quantize_prefill", None, P(_cache_struct()), fake, fake, 10, None) == 1
    assert _call("kivi_quantize_prefill", P(g), None, fake, fake, 10, None) == 1
    # a cache needs the records and the rings
    for geom in (g, _g(q_per_kv=1).c()):
        for i in (0, 1, 2):
            assert _call("kivi_quantize_prefill", P(geom), P(_cache_struct(null=i)), fake, fake,
                         10, None) == 1
    assert _call("kivi_quantize_prefill", P(g), P(_cache_struct()), None, fake, 10, None) == 1
    # sequence length and capacity
    assert _call("kivi_quantize_prefill", P(g), P(_cache_struct()), fake, fake, 0, None) == 4
    c = _cache_struct()
    assert _call("kivi_quantize_prefill", P(g), P(c), fake, fake, 1024 + 160, None) == 5
    assert (c.n_q, c.n_res, c.res_start) == (0, 0, 0)
    # append on a full ring, with counters left unchanged
    c = _cache_struct(n_q=64, n_res=160, res_start=32)
    assert _call("kivi_append_token", P(g), P(c), fake, fake, None) == 6
    assert (c.n_q, c.n_res, c.res_start) == (64, 160, 32)
    # flush: nothing to do (no device work) and history full
    flushed = ctypes.c_int32(7)
    c = _cache_struct(n_q=64, n_res=150)
    assert _call("kivi_flush_residual", P(g), P(c), P(flushed), None) == 0
    assert flushed.value == 0 and (c.n_q, c.n_res) == (64, 150)
    c = _cache_struct(n_q=1024, n_res=160)
    assert _call("kivi_flush_residual", P(g), P(c), P(flushed), None) == 5
    # inconsistent counters
    for bad in [dict(n_q=33), dict(n_q=-32), dict(n_res=161), dict(res_start=16),
                dict(res_start=160), dict(n_q=1056)]:
        c = _cache_struct(**bad)
        assert _call("kivi_append_token", P(g), P(c), fake, fake, None) == 9, bad
    # decode: empty cache, workspace (sized for the cache's counters), scale
    ws_need = kivi.workspace_bytes(_g(), 64, 130)
    assert ws_need < kivi.workspace_bytes(_g())
    args = (fake, fake, ctypes.c_float(0.1))
    assert _call("kivi_decode_attention", P(g), P(_cache_struct()), *args, fake, ws_need,
                 None) == 9
    c = _cache_struct(n_q=64, n_res=130)
    assert _call("kivi_decode_attention", P(g), P(c), *args, fake, ws_need - 1, None) == 7
    assert _call("kivi_decode_attention", P(g), P(c), *args, None, ws_need, None) == 7
    assert _call("kivi_decode_attention", P(g), P(c), fake, fake, ctypes.c_float(float("nan")),
                 fake, ws_need, None) == 2
    assert _call("kivi_decode_attention", P(g), P(c), None, fake, ctypes.c_float(0.1), fake,
                 ws_need, None) == 1


def test_decode_step_validation_before_any_device_work():
    g = _g().c()
    fake = ctypes.c_void_p(0x2000)
    P = ctypes.byref
    # the attention of a step runs over the counters after it: 64 + 141
    ws_need = kivi.workspace_bytes(_g(), 64, 141)
    flushed = ctypes.c_int32(7)

    def step(c, k=fake, v=fake, q=fake, out=fake, scale=0.1, ws=fake, nbytes=ws_need, geom=g):
        return _call("kivi_decode_step", P(geom), P(c), k, v, q, out, ctypes.c_float(scale), ws,
                     nbytes, P(flushed), None)

    c = _cache_struct(n_q=64, n_res=140)
    assert step(c, k=None) == 1 and step(c, v=None) == 1
    assert step(c, q=None) == 1 and step(c, out=None) == 1
    assert step(c, ws=None) == 7 and step(c, nbytes=ws_need - 1) == 7
    assert step(c, scale=float("inf")) == 2
    g1 = _g(q_per_kv=1)
    for i in (0, 1, 2):   # records and rings
        assert step(_cache_struct(n_q=64, n_res=140, null=i)) == 1
        assert step(_cache_struct(n_q=64, n_res=140, null=i), geom=g1.c(),
                    nbytes=kivi.workspace_bytes(g1)) == 1
    # a full ring on entry, as for kivi_append_token
    c = _cache_struct(n_q=64, n_res=160, res_start=32)
    assert step(c) == 6
    # a flush is due (n_res == R+G-1) but the history is at capacity
    c = _cache_struct(n_q=1024, n_res=159)
    assert step(c) == 5
    # inconsistent counters
    assert step(_cache_struct(n_q=33, n_res=140)) == 9
    assert step(_cache_struct(n_q=64, n_res=140, res_start=8)) == 9
    # nothing was enqueued and no counter moved on any error
    assert (c.n_q, c.n_res, c.res_start) == (1024, 159, 0)
    assert flushed.value == 7


def test_noalloc_step_validation_before_any_device_work():
    """kivi_decode_step_noalloc checks everything, including that the step's
    workspace fits the library's 16 MiB array, before it touches a device."""
    g = _g().c()
    fake = ctypes.c_void_p(0x2000)
    P = ctypes.byref
    flushed = ctypes.c_int32(7)

    def step(c, k=fake, v=fake, q=fake, out=fake, scale=0.1, geom=g):
        return _call("kivi_decode_step_noalloc", P(geom), P(c), k, v, q, out,
                     ctypes.c_float(scale), P(flushed), None)

    c = _cache_struct(n_q=64, n_res=140)
    assert step(c, k=None) == 1 and step(c, v=None) == 1
    assert step(c, q=None) == 1 and step(c, out=None) == 1
    assert step(c, scale=float("nan")) == 2
    assert step(_cache_struct(n_q=64, n_res=140, null=0)) == 1
    assert step(_cache_struct(n_q=64, n_res=160)) == 6
    assert step(_cache_struct(n_q=33, n_res=140)) == 9
    # 512 (sequence, kv head) pairs x 4 query heads at 24K tokens: ~106 MB of
    # partials, beyond the array
    big = _g(batch=64, kv_heads=8, max_tokens=32768)
    assert kivi.workspace_bytes(big, 24576, 141) > 16 << 20
    c = _cache_struct(n_q=24576, n_res=140)
    assert step(c, geom=big.c()) == 7
    assert (c.n_q, c.n_res, c.res_start) == (24576, 140, 0) and flushed.value == 7


def test_dense_attention_validation_before_any_device_work():
    g = _g().c()
    fake = ctypes.c_void_p(0x2000)
    ws_need = kivi.workspace_bytes(_g(), 0, 100)

    def dense(k=fake, v=fake, n=100, q=fake, out=fake, scale=0.1, ws=fake, nbytes=ws_need):
        return _call("kivi_dense_decode_attention", ctypes.byref(g), k, v, n, q, out,
                     ctypes.c_float(scale), ws, nbytes, None)

    assert dense(k=None) == 1 and dense(v=None) == 1 and dense(q=None) == 1
    assert dense(out=None) == 1
    assert dense(n=0) == 4 and dense(n=1025) == 4
    assert dense(ws=None) == 7 and dense(nbytes=ws_need - 1) == 7
    assert dense(scale=float("nan")) == 2
    assert _call("kivi_dense_decode_attention", None, fake, fake, 10, fake, fake,
                 ctypes.c_float(0.1), fake, ws_need, None) == 1
    big = _g(max_tokens=(1 << 24) + 32).c()
    assert _call("kivi_dense_decode_attention", ctypes.byref(big), fake, fake, 10, fake, fake,
                 ctypes.c_float(0.1), fake, ws_need, None) == 3


def test_16bit_meta_layout_and_rejected_formats():
    U, T, D, NG, S = 6, 1024, 128, 32, 160
    # 2-bit records with 16-bit scale/zero: two code planes, one meta plane
    assert 3072 == 32 * D * 2 // 8 * 2 + 4 * D * 2
    for qpk in (1, 4):
        g = _g(meta_format=kivi.META_FP16_BF16, q_per_kv=qpk)
        assert kivi.cache_layout(g) == [U * NG * 3072, U * S * D * 2, U * S * D * 2]
        assert kivi.workspace_bytes(g) == _ws(U, qpk, T, S, 3)
    for bad in (2, -1):
        with pytest.raises(kivi.KiviError) as e:
            kivi.cache_layout(_g(meta_format=bad))
        assert e.value.status == 3


def test_ragged_calls_validation_before_any_device_work():
    g = _g().c()
    fake = ctypes.c_void_p(0x2000)
    fake2 = ctypes.c_void_p(0x3000)
    P = ctypes.byref
    ws_need = kivi.workspace_bytes(_g())   # the fullest state: lengths live on the device
    c = _cache_struct()
    assert _call("kivi_ragged_prefill", P(g), P(c), None, fake, 100, fake, fake, None) == 1
    assert _call("kivi_ragged_prefill", P(g), P(c), fake, fake, 100, None, fake, None) == 1
    assert _call("kivi_ragged_prefill", P(g), P(c), fake, fake, 100, fake, None, None) == 1
    assert _call("kivi_ragged_prefill", P(g), P(c), fake, fake, 0, fake, fake, None) == 4
    assert _call("kivi_ragged_prefill", P(g), P(_cache_struct(null=0)), fake, fake, 100, fake,
                 fake, None) == 1
    assert _call("kivi_ragged_prefill", P(_g(q_per_kv=1).c()), P(_cache_struct(null=2)), fake,
                 fake, 100, fake, fake, None) == 1

    def step(geom=g, si=fake, so=fake2, nbytes=ws_need):
        return _call("kivi_ragged_decode_step", P(geom), P(c), si, so, fake, fake, fake, fake,
                     ctypes.c_float(0.1), fake, nbytes, None)

    assert step(si=None) == 1 and step(so=None) == 1
    assert step(so=fake) == 9           # state_in and state_out must differ
    assert step(nbytes=ws_need - 1) == 7
    assert step(geom=_g(residual=0).c()) == 3   # the fused append needs R >= G


def _paged_struct(P=4, pages=20, null=None):
    ptrs = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(4)]
    if null is not None:
        ptrs[null] = ctypes.c_void_p(0)
    return kivi._PagedCache(*ptrs, P, pages)


@pytest.mark.parametrize("bits,meta", [(2, 0), (4, 1)])
def test_paged_layout_sizes(bits, meta):
    n = 10 * 3 * 4                         # pages * kv heads * groups per page
    for qpk in (1, 4):                     # a pool of group records
        g = _g(bits=bits, meta_format=meta, q_per_kv=qpk)
        sizes, max_pages = kivi.paged_layout(g, 4, 10)
        assert max_pages == 8              # 32 groups of capacity / 4
        assert sizes == [n * 1024 * (bits + (1 if meta else 2)), 6 * 160 * 128 * 2,
                         6 * 160 * 128 * 2]
    assert kivi.paged_layout(g, 16, 1)[1] == 2
    assert kivi.paged_layout(g, 64, 1)[1] == 1


def test_paged_calls_validation_before_any_device_work():
    g = _g().c()
    fake = ctypes.c_void_p(0x2000)
    fake2 = ctypes.c_void_p(0x3000)
    P = ctypes.byref
    out = (ctypes.c_size_t * 3)()
    mp = ctypes.c_int32(0)
    for pg, pages, status in [(3, 10, 3), (0, 10, 3), (1 << 21, 1, 3), (4, 0, 3), (4, 1, 0),
                              (1 << 20, 1, 3)]:   # the last: pools of 2 GiB and more
        assert _call("kivi_paged_layout", P(g), pg, pages, out, P(mp)) == status, (pg, pages)
    assert _call("kivi_paged_layout", P(g), 4, 10, None, P(mp)) == 1
    assert _call("kivi_paged_layout", P(g), 4, 10, out, None) == 0
    ws_need = kivi.workspace_bytes(_g())
    for geom in (g, _g(q_per_kv=1).c()):
        for null in (0, 1, 2, 3):   # record pool, rings, block table
            assert _call("kivi_paged_prefill", P(geom), P(_paged_struct(null=null)), fake, fake,
                         100, fake, fake, None) == 1, null
    assert _call("kivi_paged_prefill", P(g), P(_paged_struct(P=6)), fake, fake, 100, fake, fake,
                 None) == 3
    assert _call("kivi_paged_prefill", P(g), P(_paged_struct()), fake, fake, 0, fake, fake,
                 None) == 4
    assert _call("kivi_paged_prefill", P(g), None, fake, fake, 100, fake, fake, None) == 1

    def step(geom=g, pc=_paged_struct(), si=fake, so=fake2, nbytes=ws_need):
        return _call("kivi_paged_decode_step", P(geom), P(pc), si, so, fake, fake, fake, fake,
                     ctypes.c_float(0.1), fake, nbytes, None)

    assert step(si=None) == 1 and step(so=None) == 1
    assert step(so=fake) == 9
    assert step(nbytes=ws_need - 1) == 7
    assert step(pc=_paged_struct(pages=0)) == 3
    assert step(pc=_paged_struct(null=3)) == 1   # block table
    assert step(geom=_g(residual=0).c()) == 3


def test_status_strings():
    lib = kivi.raw_library()
    for s in range(10):
        assert lib.kivi_status_string(s)
    assert lib.kivi_status_string(99) == b"unknown status"
    assert lib.kivi_last_hip_error() == 0
