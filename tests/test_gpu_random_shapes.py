"""GPU parity over seeded random geometries inside the supported set.

Each case draws batch, kv heads, query heads per kv head (1-16), bit width,
scale/zero format, residual length R (0-128), prefill length (1-2500, so
empty, group-aligned and ragged histories all occur; every eighth case has
192-512 (sequence, kv head) units, mostly more than the chip holds at
once), a number of fused decode steps (crossing flushes), the softmax scale and the launch flag from
numpy's default_rng(2024).  The launcher then picks its variant and split
count from the shape, so the sweep reaches launches the fixed cases do not
name.  Checks: the cache after prefill and after the steps byte-exact
against the oracle, the last step's output and a final decode_attention
within the attention tolerance of the oracle, and outputs poisoned with NaN
before every launch."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from kivi_testutil import ATTN_TOL, assert_same_cache, bits_to_dev, host_cache, row_rel_err, to_np

kivi = pytest.importorskip("decode_attention_channel_amd.kivi")

pytestmark = pytest.mark.gpu


def _cases(n=64, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        wide = i % 8 == 7   # more units than the chip holds at once: many-round launches
        B = int(rng.integers(16, 33)) if wide else int(rng.integers(1, 7))
        H = int(rng.integers(12, 17)) if wide else int(rng.integers(1, 7))
        QPK = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 12, 16]))
        bits = int(rng.choice([2, 4]))
        meta = int(rng.integers(0, 2))
        R = int(rng.choice([0, 32, 64, 128]))
        if wide:
            S0 = int(rng.integers(1, 601))
        elif i % 2:
            S0 = int(np.exp(rng.uniform(0, math.log(2500))))   # short histories often
        else:
            S0 = int(rng.integers(1, 2501))
        N = int(rng.integers(0, 9)) if wide else int(rng.integers(0, 41))
        flags = int(rng.integers(0, 2))
        scale = float(rng.choice([0.25, 0.5, 1.0, 2.0, 4.0])) / math.sqrt(128)
        out.append((i, B, H, QPK, bits, meta, R, S0, N, flags, scale))
    return out


@pytest.mark.parametrize("i,B,H,QPK,bits,meta,R,S0,N,flags,scale", _cases())
def test_random_geometry(i, B, H, QPK, bits, meta, R, S0, N, flags, scale):
    print(f"random case {i}: B={B} H={H} QPK={QPK} bits={bits} meta={meta} R={R} S0={S0} "
          f"N={N} flags={flags} scale={scale:.4f}", flush=True)
    w = synth.Workload("case", B, H, QPK, S0 + N, bits, 1, 3, 8.0)
    seed = 5000 + i
    k, v = synth.prefill_kv(w, seed)
    kb, vb = synth.bits_u16(k), synth.bits_u16(v)
    T = 32 * ((S0 + N) // 32 + 2)
    kg = kivi.Geom(B, H, QPK, bits=bits, residual=R, max_tokens=T, meta_format=meta, flags=flags)
    og = oracle.Geom(B, H, QPK, bits=bits, residual=R, max_tokens=T, meta=meta)
    gc = kivi.Cache(kg)
    kivi.quantize_prefill(kg, gc, bits_to_dev(kb[:, :, :S0].copy()), bits_to_dev(vb[:, :, :S0].copy()))
    oc = oracle.prefill(og, kb[:, :, :S0].copy(), vb[:, :, :S0].copy())
    torch.cuda.synchronize()
    assert_same_cache(host_cache(gc, og), oc)

    ws = kivi.Workspace(kg)
    out = torch.empty(B, H * QPK, 128, device="cuda")
    q = None
    for t in range(S0, S0 + N):
        kn, vn = kb[:, :, t].copy(), vb[:, :, t].copy()
        q = synth.bits_u16(synth.query(w, seed, step=t))
        out.fill_(float("nan"))
        _, f = kivi.decode_step(kg, gc, bits_to_dev(kn), bits_to_dev(vn), bits_to_dev(q), out=out,
                                ws=ws, softmax_scale=scale)
        oracle.append(oc, kn, vn)
        assert oracle.flush(oc) == f, t
    torch.cuda.synchronize()
    assert (gc.n_q, gc.n_res, gc.res_start) == (oc.n_q, oc.n_res, oc.res_start)
    assert_same_cache(host_cache(gc, og), oc)
    if q is not None:
        o = to_np(out)
        assert np.isfinite(o).all(), "unwritten output"
        err = row_rel_err(o, oracle.attention(oc, q, scale))
        assert err <= ATTN_TOL, f"last step: row-relative error {err:.3e}"

    q = synth.bits_u16(synth.query(w, seed, step=S0 + N + 1))
    out.fill_(float("nan"))
    kivi.decode_attention(kg, gc, bits_to_dev(q), out=out, ws=ws, softmax_scale=scale)
    torch.cuda.synchronize()
    o = to_np(out)
    assert np.isfinite(o).all(), "unwritten output"
    err = row_rel_err(o, oracle.attention(oc, q, scale))
    assert err <= ATTN_TOL, f"row-relative error {err:.3e}"
