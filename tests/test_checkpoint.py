"""Checkpoint and resume of a cache (Cache.state_dict / load_state_dict).

The cache is three buffers and three host counters, so a snapshot is host
copies of the live group records, the residual ring and the counters.

* CPU: a snapshot survives torch.save / torch.load(weights_only=True) into a
  cache with a larger max_tokens; the live bytes and the counters come back;
  a snapshot of another geometry, or with counters that do not fit, is
  refused.
* GPU: a stream snapshotted after some decode steps, restored into a fresh
  cache and continued through a flush gives the same outputs (bit for bit,
  deterministic launch) and the same cache bytes as the uninterrupted stream.
"""
import io
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from kivi_testutil import assert_same_cache, bits_to_dev, host_cache, to_np

kivi = pytest.importorskip("decode_attention_channel_amd.kivi")


def _roundtrip(sd: dict) -> dict:
    buf = io.BytesIO()
    torch.save(sd, buf)
    buf.seek(0)
    return torch.load(buf, weights_only=True)


def test_snapshot_roundtrip_on_host():
    g = kivi.Geom(2, 3, 4, bits=4, max_tokens=256)
    c = kivi.Cache(g, device="cpu")
    gen = torch.Generator().manual_seed(5)
    for name in kivi.BUFFERS:
        t = getattr(c, name)
        t.view(torch.uint8).copy_(torch.randint(0, 256, t.view(torch.uint8).shape,
                                                dtype=torch.uint8, generator=gen))
    c.set_counters(96, 140, 32)
    sd = _roundtrip(c.state_dict())
    assert sd["records"].shape[2] == 3   # the live groups only

    big = kivi.Geom(2, 3, 4, bits=4, max_tokens=512)
    r = kivi.Cache(big, device="cpu")
    r.load_state_dict(sd)
    assert (r.n_q, r.n_res, r.res_start) == (96, 140, 32)
    assert torch.equal(r.records[:, :, :3], c.records[:, :, :3])
    assert torch.equal(r.k_res.view(torch.int16), c.k_res.view(torch.int16))
    assert torch.equal(r.v_res.view(torch.int16), c.v_res.view(torch.int16))

    with pytest.raises(ValueError):   # other bit width
        kivi.Cache(kivi.Geom(2, 3, 4, bits=2, max_tokens=256), device="cpu").load_state_dict(sd)
    with pytest.raises(ValueError):   # history longer than the target holds
        kivi.Cache(kivi.Geom(2, 3, 4, bits=4, max_tokens=64), device="cpu").load_state_dict(sd)
    bad = dict(sd, res_start=16)      # not a multiple of G
    with pytest.raises(ValueError):
        kivi.Cache(g, device="cpu").load_state_dict(bad)


@pytest.mark.gpu
@pytest.mark.parametrize("bits,QPK", [(2, 4), (4, 1)])
def test_resumed_stream_equals_uninterrupted(bits, QPK):
    B, H, S0, N1, N2 = 2, 2, 300, 10, 30
    print(f"checkpoint resume bits={bits} QPK={QPK} S0={S0} N1={N1} N2={N2}", flush=True)
    w = synth.Workload("case", B, H, QPK, S0 + N1 + N2, bits, 1, 3, 8.0)
    seed = 77 + bits + QPK
    k, v = synth.prefill_kv(w, seed)
    kb, vb = synth.bits_u16(k), synth.bits_u16(v)
    T = 32 * ((S0 + N1 + N2) // 32 + 1)
    g = kivi.Geom(B, H, QPK, bits=bits, max_tokens=T, flags=kivi.FLAG_DETERMINISTIC)
    og = oracle.Geom(B, H, QPK, bits=bits, max_tokens=T)
    full = kivi.Cache(g)
    kivi.quantize_prefill(g, full, bits_to_dev(kb[:, :, :S0].copy()), bits_to_dev(vb[:, :, :S0].copy()))
    ws = kivi.Workspace(g)
    scale = 1.0 / math.sqrt(128)

    def run(cache, t0, t1):
        outs, flushes = [], 0
        for t in range(t0, t1):
            q = bits_to_dev(synth.bits_u16(synth.query(w, seed, step=t)))
            out = torch.full((B, H * QPK, 128), float("nan"), device="cuda")
            _, f = kivi.decode_step(g, cache, bits_to_dev(kb[:, :, t].copy()),
                                    bits_to_dev(vb[:, :, t].copy()), q, out=out, ws=ws,
                                    softmax_scale=scale)
            flushes += f
            outs.append(out)
        torch.cuda.synchronize()
        return [to_np(o) for o in outs], flushes

    run(full, S0, S0 + N1)
    snap = _roundtrip(full.state_dict())
    ref_outs, ref_flushes = run(full, S0 + N1, S0 + N1 + N2)
    assert ref_flushes >= 1   # the resumed part crosses a flush

    resumed = kivi.Cache(g)
    resumed.load_state_dict(snap)
    outs, flushes = run(resumed, S0 + N1, S0 + N1 + N2)
    assert flushes == ref_flushes
    for i, (a, b) in enumerate(zip(outs, ref_outs)):
        assert np.isfinite(a).all(), f"step {i}: unwritten output"
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"step {i}"
    assert (resumed.n_q, resumed.n_res, resumed.res_start) == (full.n_q, full.n_res, full.res_start)
    assert_same_cache(host_cache(resumed, og), host_cache(full, og))
