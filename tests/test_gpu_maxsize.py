"""GPU parity at the largest accepted geometry: one (sequence, kv head) whose
quantised history fills the 2^30-byte record limit of a unit (8,388,608
tokens at 2-bit and 5,592,384 at 4-bit with fp32 scale/zero; 11,184,800 and
6,710,880 with 16-bit scale/zero; kivi.h, geometry limits), plus a full
residual of R = 128 bf16 tokens.

Every history group but the last holds the same 32 tokens A; the last group
B (at the largest record offset) and the residual have their keys shifted
along the sum of the query heads, so that their scores are about 15 and 12
higher and both carry a large share of the softmax weight.  The expected
values follow from the oracle on a 192-token cache A, B, residual (catalog
record kivi-2bit-llama3-8b-gqa-8k, KV bytes basis: grouped history plus bf16
residual; paper card, method paragraph: per-channel K / per-token V groups):
* every A record of the large cache equals the A record of the small one,
  the last record equals its B record, and the live ring slots equal its
  ring; the small cache is checked byte for byte against the oracle;
* attention is softmax attention in which each A token carries weight
  n_groups - 1: out = ((n-1) sum_A e^s v + sum_B e^s v + sum_res e^s v) /
  ((n-1) sum_A e^s + sum_B e^s + sum_res e^s), in float64 over the oracle's
  dequantised A, B and residual.
Both the default and the bitwise-repeatable launch are checked.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from kivi_testutil import ATTN_TOL, assert_same_cache, bits_to_dev, host_cache, row_rel_err, to_np

kivi = pytest.importorskip("decode_attention_channel_amd.kivi")

pytestmark = pytest.mark.gpu

G, R, D, QPK = 32, 128, 128, 4
# (bits, scale/zero format) -> the most tokens whose records fit 2^30 bytes
MAX_TOKENS = {(2, 0): 8_388_608, (4, 0): 5_592_384, (2, 1): 11_184_800, (4, 1): 6_710_880}


def _f(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("bits,meta", sorted(MAX_TOKENS))
def test_largest_geometry(bits, meta):
    T = MAX_TOKENS[(bits, meta)]
    n = T // G
    print(f"max size: bits={bits} meta={meta} max_tokens={T} groups={n}", flush=True)
    rng = np.random.default_rng(40 + bits)
    qf = rng.standard_normal((QPK, D)).astype(np.float32)
    qb = (qf.view(np.uint32) >> 16).astype(np.uint16)[None]
    x = rng.standard_normal((2, 1, 1, 2 * G + R, D)).astype(np.float32)
    x[0, :, :, :, [5, 77]] *= 8.0   # outlier key channels
    x[0, :, :, G:2 * G] = x[0, :, :, :G]   # B: the A tokens ...
    u = _f((qf.view(np.uint32) >> 16).astype(np.uint16)).sum(axis=0)
    unit = (u / (u @ u)).astype(np.float32)
    # ... shifted so that scores rise by ~15 (B) and ~12 (residual), per head
    # about (q_h . u) / (u . u) of that
    x[0, :, :, G:2 * G] += (15 * QPK * math.sqrt(D)) * unit
    x[0, :, :, 2 * G:] += (12 * QPK * math.sqrt(D)) * unit
    small = (x.view(np.uint32) >> 16).astype(np.uint16)
    kb, vb = small[0].copy(), small[1].copy()

    # the 192-token cache: GPU against the oracle, byte for byte
    og = oracle.Geom(1, 1, QPK, bits=bits, max_tokens=2 * G, meta=meta)
    oc = oracle.prefill(og, kb, vb)
    assert (oc.n_q, oc.n_res) == (2 * G, R)
    gs_geom = kivi.Geom(1, 1, QPK, bits=bits, max_tokens=2 * G, meta_format=meta)
    gs = kivi.Cache(gs_geom)
    kivi.quantize_prefill(gs_geom, gs, bits_to_dev(kb), bits_to_dev(vb))
    torch.cuda.synchronize()
    assert_same_cache(host_cache(gs, og), oc)

    # the largest cache: A repeated n - 1 times, B, then the residual
    k_small, v_small = bits_to_dev(kb), bits_to_dev(vb)
    k = torch.cat([k_small[:, :, :G].repeat(1, 1, n - 1, 1), k_small[:, :, G:]], dim=2)
    v = torch.cat([v_small[:, :, :G].repeat(1, 1, n - 1, 1), v_small[:, :, G:]], dim=2)
    del k_small, v_small
    outs = {}
    for flags in (0, kivi.FLAG_DETERMINISTIC):
        g = kivi.Geom(1, 1, QPK, bits=bits, max_tokens=T, meta_format=meta, flags=flags)
        gc = kivi.Cache(g)
        kivi.quantize_prefill(g, gc, k, v)
        torch.cuda.synchronize()
        assert (gc.n_q, gc.n_res) == (T, R)
        rec = gc.records.view(n, -1)
        ref_a, ref_b = gs.records.view(2, -1)
        for i in sorted({0, 1, n // 3, n // 2, n - 2}):
            assert torch.equal(rec[i], ref_a), f"group {i} differs from group A"
        assert torch.equal(rec[n - 1], ref_b), "the last group differs from group B"
        # the live ring slots (both caches start the ring at slot 0)
        assert gc.res_start == 0 and gs.res_start == 0
        assert torch.equal(gc.k_res[:, :, :R], gs.k_res[:, :, :R])
        assert torch.equal(gc.v_res[:, :, :R], gs.v_res[:, :, :R])
        out = torch.full((1, QPK, D), float("nan"), device="cuda")
        scale = 1.0 / math.sqrt(D)
        kivi.decode_attention(g, gc, bits_to_dev(qb), out=out, softmax_scale=scale,
                              ws=kivi.Workspace(g))
        torch.cuda.synchronize()
        outs[flags] = to_np(out)
        del gc
        torch.cuda.empty_cache()

    kd, vd = oracle.dequant_unit(oc, 0)          # rows: A, B, then the residual
    s = scale * (_f(qb[0]) @ kd.T)                # [QPK][2G + R]
    m = s.max(axis=1, keepdims=True)
    wts = np.exp(s - m)
    wts[:, :G] *= n - 1
    share = wts.sum(axis=1)
    # B and the residual each hold a real share of every head's weight
    assert (wts[:, G:2 * G].sum(axis=1) > 0.02 * share).all()
    assert (wts[:, 2 * G:].sum(axis=1) > 0.01 * share).all()
    ref = (wts @ vd) / share[:, None]
    for flags, o in outs.items():
        assert np.isfinite(o).all()
        err = row_rel_err(o, ref)
        assert err <= ATTN_TOL, f"flags={flags}: row-relative error {err:.3e}"
