"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

* quantised history (packed codes, scale, zero) and residual: byte-exact;
* decode attention: max over rows of ||o - o_ref||_inf / ||o_ref||_inf <= 1e-3;
* outputs are poisoned (NaN) before each launch; every case runs twice in the
  default launch (whose waves may merge in the order they finish, so repeats
  agree to within REPEAT_TOL (2e-4) row-relative) and twice with the deterministic flag
  (repeats bitwise equal), and each result is checked against the oracle.

Inputs are seeded synthetic K/V/q with outlier key channels (synth.py).
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from kivi_testutil import ATTN_TOL, REPEAT_TOL, assert_same_cache, bits_to_dev, host_cache, row_rel_err, to_np

kivi = pytest.importorskip("decode_attention_channel_amd.kivi")

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _wl(B, H, QPK, S, bits, outliers=3, factor=8.0):
    return synth.Workload("case", B, H, QPK, S, bits, 1, outliers, factor)


def _geoms(w: synth.Workload, extra_tokens=0):
    T = 32 * ((max(w.seq_len + extra_tokens - 128, 0)) // 32 + 1)
    kg = kivi.Geom(w.batch, w.kv_heads, w.q_per_kv, bits=w.bits, max_tokens=T)
    og = oracle.Geom(w.batch, w.kv_heads, w.q_per_kv, bits=w.bits, max_tokens=T)
    return kg, og


def _attend_and_check(kg, gc, oc, q_bits, scale=None, rows_units=None):
    scale = 1.0 / math.sqrt(128) if scale is None else scale
    q = bits_to_dev(q_bits)
    ws = kivi.Workspace(kg)
    kd = dataclasses.replace(kg, flags=kg.flags | kivi.FLAG_DETERMINISTIC)
    outs = []
    for g in (kg, kg, kd, kd):
        out = torch.full((kg.batch, kg.q_heads, 128), float("nan"), device=DEV)
        kivi.decode_attention(g, gc, q, out=out, softmax_scale=scale, ws=ws)
        outs.append(out)
    torch.cuda.synchronize()
    o = [to_np(x) for x in outs]
    for x in o:
        assert np.isfinite(x).all(), "unwritten or non-finite output"
    assert row_rel_err(o[0], o[1]) <= REPEAT_TOL, "default launches disagree"
    assert np.array_equal(o[2].view(np.uint32), o[3].view(np.uint32)), "not deterministic"
    ref = oracle.attention(oc, q_bits, scale, units=rows_units)
    if rows_units is not None:
        H, QPK = kg.kv_heads, kg.q_per_kv
        rows = [(u // H, (u % H) * QPK + j) for u in rows_units for j in range(QPK)]
        o = [np.stack([x[b, hq] for b, hq in rows]) for x in o]
        ref = np.stack([ref[b, hq] for b, hq in rows])
    err = max(row_rel_err(o[0], ref), row_rel_err(o[2], ref))
    assert err <= ATTN_TOL, f"attention row-relative error {err:.3e}"
    return err


CASES = [
    # B, H, QPK, S, bits
    (1, 1, 1, 256, 2),
    (2, 2, 1, 1, 2),
    (2, 2, 1, 127, 2),
    (1, 2, 1, 128, 2),
    (1, 1, 1, 129, 2),
    (1, 3, 1, 159, 2),
    (1, 1, 1, 160, 2),
    (2, 1, 1, 293, 2),
    (2, 2, 1, 1509, 2),
    (2, 2, 1, 1509, 4),
    (2, 2, 4, 293, 2),
    (1, 2, 4, 1000, 2),
    (1, 2, 4, 1509, 2),
    (2, 1, 4, 1509, 4),
    (2, 1, 2, 700, 4),
    (1, 2, 3, 500, 2),
    (1, 1, 5, 300, 2),
    (1, 1, 8, 600, 2),
    (1, 2, 16, 400, 4),
    (3, 1, 4, 161, 4),
]


@pytest.mark.parametrize("B,H,QPK,S,bits", CASES)
def test_prefill_and_attention(B, H, QPK, S, bits):
    print(f"case B={B} H={H} QPK={QPK} S={S} bits={bits}", flush=True)
    w = _wl(B, H, QPK, S, bits)
    seed = 1000 + B * 100 + H * 10 + QPK + S + bits
    k, v = synth.prefill_kv(w, seed)
    kb, vb = synth.bits_u16(k), synth.bits_u16(v)
    kg, og = _geoms(w)
    gc = kivi.Cache(kg)
    kivi.quantize_prefill(kg, gc, bits_to_dev(kb), bits_to_dev(vb))
    oc = oracle.prefill(og, kb, vb)
    torch.cuda.synchronize()
    assert_same_cache(host_cache(gc, og), oc)
    q = synth.bits_u16(synth.query(w, seed))
    _attend_and_check(kg, gc, oc, q)


@pytest.mark.parametrize("B,H,QPK", [(32, 32, 1), (16, 64, 4)])
def test_one_workgroup_per_unit(B, H, QPK):
    """1024 (sequence, kv head) units at 300 tokens: more units than the
    chip holds at once, so the launch is the static variant with one
    workgroup per unit, which writes its output directly from its merge (no
    partial, no combine).  Checked against the oracle in the default launch
    and with the deterministic flag."""
    S, bits = 300, 2
    print(f"one workgroup per unit: B={B} H={H} QPK={QPK} S={S}", flush=True)
    w = _wl(B, H, QPK, S, bits)
    seed = 7100 + B + H + QPK
    k, v = synth.prefill_kv(w, seed)
    kb, vb = synth.bits_u16(k), synth.bits_u16(v)
    kg, og = _geoms(w)
    gc = kivi.Cache(kg)
    kivi.quantize_prefill(kg, gc, bits_to_dev(kb), bits_to_dev(vb))
    oc = oracle.prefill(og, kb, vb)
    torch.cuda.synchronize()
    q = synth.bits_u16(synth.query(w, seed))
    _attend_and_check(kg, gc, oc, q)


def test_tiny_workload_exact():
    """Tiny single head, S = 256: 4 key groups + 128 residual, 4 fixed outlier
    channels x10, one prefill and one decode step."""
    w = synth.WORKLOADS["tiny"]
    k, v = synth.prefill_kv(w, 1)
    kb, vb = synth.bits_u16(k), synth.bits_u16(v)
    kg, og = _geoms(w)
    gc = kivi.Cache(kg)
    kivi.quantize_prefill(kg, gc, bits_to_dev(kb), bits_to_dev(vb))
    oc = oracle.prefill(og, kb, vb)
    torch.cuda.synchronize()
    assert (gc.n_q, gc.n_res) == (128, 128)
    assert_same_cache(host_cache(gc, og), oc)
    _attend_and_check(kg, gc, oc, synth.bits_u16(synth.query(w, 1)))


@pytest.mark.parametrize("bits,QPK", [(2, 1), (2, 4), (4, 4), (4, 1)])
def test_streaming_append_flush_attend(bits, QPK):
    B, H, S0, N = 2, 2, 150, 100
    w = _wl(B, H, QPK, S0 + N, bits)
    seed = 77 + bits + QPK
    k, v = synth.prefill_kv(w, seed)
    kb, vb = synth.bits_u16(k), synth.bits_u16(v)
    kg, og = _geoms(w)
    gc = kivi.Cache(kg)
    kivi.quantize_prefill(kg, gc, bits_to_dev(kb[:, :, :S0].copy()), bits_to_dev(vb[:, :, :S0].copy()))
    oc = oracle.prefill(og, kb[:, :, :S0].copy(), vb[:, :, :S0].copy())
    flushes = 0
    for t in range(S0, S0 + N):
        kn, vn = kb[:, :, t].copy(), vb[:, :, t].copy()
        kivi.append_token(kg, gc, bits_to_dev(kn), bits_to_dev(vn))
        f = kivi.flush_residual(kg, gc)
        oracle.append(oc, kn, vn)
        assert oracle.flush(oc) == f
        flushes += f
        assert (gc.n_q, gc.n_res, gc.res_start) == (oc.n_q, oc.n_res, oc.res_start)
        if t % 23 == 0 or f:
            q = synth.bits_u16(synth.query(w, seed, step=t))
            _attend_and_check(kg, gc, oc, q)
    assert flushes == 3
    torch.cuda.synchronize()
    assert_same_cache(host_cache(gc, og), oc)
    # streaming == prefill of the whole sequence, on the GPU side as well
    gp = kivi.Cache(kg)
    kivi.quantize_prefill(kg, gp, bits_to_dev(kb), bits_to_dev(vb))
    torch.cuda.synchronize()
    assert_same_cache(host_cache(gc, og), host_cache(gp, og))


def test_subnormal_and_constant_groups():
    """Groups whose range is zero, subnormal, or spans subnormals: the GPU must
    keep IEEE denormals exactly like the oracle."""
    B, H, S = 1, 2, 128 + 64
    rng = np.random.default_rng(5)
    x = np.zeros((2, B, H, S, 128), np.float32)
    x[:, :, 0, :32] = 3.5                                # constant groups
    x[:, :, 0, 32:64] = rng.standard_normal((2, B, 32, 128)) * 2.0 ** -128   # subnormal range
    x[:, :, 1] = rng.standard_normal((2, B, S, 128)) * 2.0 ** -120
    bits16 = (x.view(np.uint32) >> 16).astype(np.uint16)
    kb, vb = bits16[0].copy(), bits16[1].copy()
    for bits in (2, 4):
        kg = kivi.Geom(B, H, 2, bits=bits, max_tokens=64)
        og = oracle.Geom(B, H, 2, bits=bits, max_tokens=64)
        gc = kivi.Cache(kg)
        kivi.quantize_prefill(kg, gc, bits_to_dev(kb), bits_to_dev(vb))
        oc = oracle.prefill(og, kb, vb)
        torch.cuda.synchronize()
        assert_same_cache(host_cache(gc, og), oc)


def test_softmax_scale_and_large_scores():
    """A large softmax scale makes the scores span hundreds (log2 units),
    exercising the running-max rescale across groups and splits."""
    w = _wl(1, 2, 4, 1509, 2, outliers=6, factor=30.0)
    k, v = synth.prefill_kv(w, 9)
    kb, vb = synth.bits_u16(k), synth.bits_u16(v)
    kg, og = _geoms(w)
    gc = kivi.Cache(kg)
    kivi.quantize_prefill(kg, gc, bits_to_dev(kb), bits_to_dev(vb))
    oc = oracle.prefill(og, kb, vb)
    q = synth.bits_u16(synth.query(w, 9))
    for scale in (0.01, 0.3, 2.0):
        _attend_and_check(kg, gc, oc, q, scale=scale)


def test_query_head_mapping():
    """Query head hq reads kv head hq // q_per_kv: a query that is zero except
    in one head must reproduce that head's own attention only."""
    w = _wl(1, 3, 4, 700, 2)
    k, v = synth.prefill_kv(w, 3)
    kb, vb = synth.bits_u16(k), synth.bits_u16(v)
    kg, og = _geoms(w)
    gc = kivi.Cache(kg)
    kivi.quantize_prefill(kg, gc, bits_to_dev(kb), bits_to_dev(vb))
    oc = oracle.prefill(og, kb, vb)
    q = np.zeros((1, 12, 128), np.uint16)
    q[0, 7] = synth.bits_u16(synth.query(w, 3))[0, 7]
    _attend_and_check(kg, gc, oc, q)
