"""GPU parity of the fused decode step (kivi_decode_step).

One call appends the new token, flushes the G oldest residual tokens when the
ring fills and attends.  The check runs the same token stream through the
three separate calls (append, flush, attend) on a second cache and through
the CPU oracle:

* the fused and separate paths agree bit for bit in the flush flags, the
  counters and the cache bytes (the new token's ring slot is written by the
  attention kernel in the fused path), and in every output when launched with
  the deterministic flag (in the default launch, whose waves may merge in the
  order they finish, to within REPEAT_TOL (2e-4) row-relative);
* outputs agree with the oracle within the attention tolerance, and the
  final cache equals the oracle's byte for byte.

Cases cover GQA and MHA (one query head per kv head), both bit widths, a ring
of R = 32, R = 0 (where a flush step runs as three launches), prefill lengths
that start with an empty history, and several flushes per run.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from kivi_testutil import ATTN_TOL, REPEAT_TOL, assert_same_cache, bits_to_dev, host_cache, row_rel_err, to_np

kivi = pytest.importorskip("decode_attention_channel_amd.kivi")

pytestmark = pytest.mark.gpu

DET = kivi.FLAG_DETERMINISTIC
CASES = [
    # B, H, QPK, bits, R, S0, N, flags
    (2, 2, 4, 2, 128, 150, 45, 0),
    (2, 2, 4, 2, 128, 150, 45, DET),
    (2, 2, 4, 4, 128, 300, 40, 0),
    (2, 2, 1, 2, 128, 150, 45, 0),
    (1, 3, 1, 4, 128, 1000, 40, 0),
    (1, 3, 1, 4, 128, 1000, 40, DET),
    (1, 2, 3, 2, 32, 70, 80, 0),
    (1, 2, 8, 4, 0, 100, 70, 0),
    (1, 2, 8, 4, 0, 100, 70, DET),
    (1, 1, 1, 2, 0, 40, 40, 0),
    (2, 1, 16, 2, 128, 1, 165, 0),
]


@pytest.mark.parametrize("B,H,QPK,bits,R,S0,N,flags", CASES)
def test_decode_step_matches_separate_calls_and_oracle(B, H, QPK, bits, R, S0, N, flags):
    print(f"decode_step B={B} H={H} QPK={QPK} bits={bits} R={R} S0={S0} N={N} flags={flags}",
          flush=True)
    w = synth.Workload("case", B, H, QPK, S0 + N, bits, 1, 3, 8.0)
    seed = 1000 + 7 * QPK + bits + R
    k, v = synth.prefill_kv(w, seed)
    kb, vb = synth.bits_u16(k), synth.bits_u16(v)
    T = 32 * ((S0 + N) // 32 + 1)
    kg = kivi.Geom(B, H, QPK, bits=bits, residual=R, max_tokens=T, flags=flags)
    og = oracle.Geom(B, H, QPK, bits=bits, residual=R, max_tokens=T)
    sep, fus = kivi.Cache(kg), kivi.Cache(kg)
    k0, v0 = bits_to_dev(kb[:, :, :S0].copy()), bits_to_dev(vb[:, :, :S0].copy())
    kivi.quantize_prefill(kg, sep, k0, v0)
    kivi.quantize_prefill(kg, fus, k0, v0)
    oc = oracle.prefill(og, kb[:, :, :S0].copy(), vb[:, :, :S0].copy())
    ws_s, ws_f = kivi.Workspace(kg), kivi.Workspace(kg)
    shape = (B, H * QPK, 128)
    out_s = torch.empty(shape, device="cuda")
    out_f = torch.empty(shape, device="cuda")
    scale = 1.0 / math.sqrt(128)
    flushes = 0
    worst = 0.0
    for t in range(S0, S0 + N):
        kn, vn = kb[:, :, t].copy(), vb[:, :, t].copy()
        kn_d, vn_d = bits_to_dev(kn), bits_to_dev(vn)
        q = synth.bits_u16(synth.query(w, seed, step=t))
        q_d = bits_to_dev(q)
        out_s.fill_(float("nan"))
        out_f.fill_(float("nan"))
        kivi.append_token(kg, sep, kn_d, vn_d)
        f_sep = kivi.flush_residual(kg, sep)
        kivi.decode_attention(kg, sep, q_d, out=out_s, ws=ws_s)
        _, f_fus = kivi.decode_step(kg, fus, kn_d, vn_d, q_d, out=out_f, ws=ws_f)
        oracle.append(oc, kn, vn)
        f_ref = oracle.flush(oc)
        assert f_sep == f_fus == f_ref, t
        flushes += f_fus
        assert (fus.n_q, fus.n_res, fus.res_start) == (sep.n_q, sep.n_res, sep.res_start)
        assert (fus.n_q, fus.n_res, fus.res_start) == (oc.n_q, oc.n_res, oc.res_start)
        torch.cuda.synchronize()
        o_s, o_f = to_np(out_s), to_np(out_f)
        assert np.isfinite(o_f).all(), f"step {t}: unwritten output"
        if flags & DET:
            assert np.array_equal(o_s.view(np.uint32), o_f.view(np.uint32)), f"step {t}"
        else:
            assert row_rel_err(o_f, o_s) <= REPEAT_TOL, f"step {t}"
        if f_fus or t % 9 == 0 or t == S0 + N - 1:
            err = row_rel_err(o_f, oracle.attention(oc, q, scale))
            assert err <= ATTN_TOL, f"step {t}: row-relative error {err:.3e}"
            worst = max(worst, err)
    assert flushes >= 1
    torch.cuda.synchronize()
    hf = host_cache(fus, og)
    assert_same_cache(hf, oc)
    assert_same_cache(hf, host_cache(sep, og))
    print(f"  flushes {flushes}, worst row error {worst:.2e}", flush=True)


def test_decode_step_then_separate_calls_interleave():
    """The fused step leaves a cache that the separate calls continue from
    (and the other way round), with the same results as the oracle."""
    B, H, QPK, bits, S0 = 1, 2, 4, 2, 140
    w = synth.Workload("case", B, H, QPK, S0 + 60, bits, 1, 3, 8.0)
    k, v = synth.prefill_kv(w, 4242)
    kb, vb = synth.bits_u16(k), synth.bits_u16(v)
    T = 32 * ((S0 + 60) // 32 + 1)
    kg = kivi.Geom(B, H, QPK, bits=bits, max_tokens=T)
    og = oracle.Geom(B, H, QPK, bits=bits, max_tokens=T)
    gc = kivi.Cache(kg)
    kivi.quantize_prefill(kg, gc, bits_to_dev(kb[:, :, :S0].copy()), bits_to_dev(vb[:, :, :S0].copy()))
    oc = oracle.prefill(og, kb[:, :, :S0].copy(), vb[:, :, :S0].copy())
    ws = kivi.Workspace(kg)
    out = torch.empty(B, H * QPK, 128, device="cuda")
    for t in range(S0, S0 + 60):
        kn, vn = kb[:, :, t].copy(), vb[:, :, t].copy()
        q = synth.bits_u16(synth.query(w, 4242, step=t))
        out.fill_(float("nan"))
        if (t // 7) % 2:
            kivi.decode_step(kg, gc, bits_to_dev(kn), bits_to_dev(vn), bits_to_dev(q), out=out, ws=ws)
        else:
            kivi.append_token(kg, gc, bits_to_dev(kn), bits_to_dev(vn))
            kivi.flush_residual(kg, gc)
            kivi.decode_attention(kg, gc, bits_to_dev(q), out=out, ws=ws)
        oracle.append(oc, kn, vn)
        oracle.flush(oc)
        torch.cuda.synchronize()
        err = row_rel_err(to_np(out), oracle.attention(oc, q, 1.0 / math.sqrt(128)))
        assert err <= ATTN_TOL, f"step {t}: {err:.3e}"
    assert_same_cache(host_cache(gc, og), oc)
