"""GPU parity at the full sizes of the workloads (the launch configuration
that bench.py times), checked on sampled (sequence, kv head) units that the
oracle recomputes one by one:

* Llama-3-8B GQA, batch 16, 8 kv / 32 q heads, 8192 tokens, 2-bit: prefill
  bytes and decode attention on sampled units, with fp32 and with 16-bit
  (fp16 scale, bf16 zero) scale/zero;
* Llama-2-7B-shaped MHA layer, batch 8, 32 heads, 4096 tokens, 2-bit:
  prefill, then 128 decode steps (append, flush, attend) with 4 flushes;
* long-context 4-bit GQA, batch 4, 8 kv / 32 q heads, 32768 tokens: prefill,
  then 1024 streamed tokens with a flush every 32, attention checked along
  the way;
* Llama-2-13B-shaped MHA, 40 heads, 4096 tokens, at batch 8 (the memory-wall
  sweep of that workload is a benchmark, not a test);
* the timed call itself, kivi_decode_step, at the 8K GQA and 32K 4-bit
  sizes across flushes, against the oracle and against separate calls;
* one workspace reused by back-to-back launches (every unit checked);
* bitwise repeatability of the deterministic launch at the 8K GQA size.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from kivi_testutil import ATTN_TOL, REPEAT_TOL, bits_to_dev, row_rel_err, to_np

kivi = pytest.importorskip("decode_attention_channel_amd.kivi")

pytestmark = pytest.mark.gpu


def _unit_geoms(w, T, meta=0):
    return oracle.Geom(1, 1, w.q_per_kv, bits=w.bits, max_tokens=T, meta=meta)


def _check_unit_cache(gc, oc1, b, h):
    """Device cache unit (b, h) against a one-unit oracle cache."""
    nq, ng = oc1.n_q, oc1.n_q // 32
    assert (gc.n_q, gc.n_res) == (oc1.n_q, oc1.n_res)
    hist = gc.history()
    np.testing.assert_array_equal(hist["k_codes"][b, h, :nq], oc1.k_codes[0, 0, :nq])
    np.testing.assert_array_equal(hist["v_codes"][b, h, :ng], oc1.v_codes[0, 0, :ng])
    for name in ("k_scale", "k_zero", "v_scale", "v_zero"):
        np.testing.assert_array_equal(np.ascontiguousarray(hist[name][b, h, :ng]).view(np.uint8),
                                      getattr(oc1, name)[0, 0, :ng].view(np.uint8), name)
    slots = 160
    go = [(gc.res_start + i) % slots for i in range(gc.n_res)]
    ro = [(oc1.res_start + i) % slots for i in range(oc1.n_res)]
    np.testing.assert_array_equal(to_np(gc.k_res[b, h])[go], oc1.k_res[0, 0, ro])
    np.testing.assert_array_equal(to_np(gc.v_res[b, h])[go], oc1.v_res[0, 0, ro])


def _check_unit_attention(out_np, oc1, q_bits, b, h, qpk, scale):
    qrows = q_bits[b:b + 1, h * qpk:(h + 1) * qpk].copy()
    ref = oracle.attention(oc1, qrows, scale)[0]
    err = row_rel_err(out_np[b, h * qpk:(h + 1) * qpk], ref)
    assert err <= ATTN_TOL, f"unit (b={b}, h={h}): row-relative error {err:.3e}"
    return err


def _sample_units(w, k, seed):
    rng = np.random.default_rng(seed)
    units = {(0, 0), (w.batch - 1, w.kv_heads - 1)}
    while len(units) < k:
        units.add((int(rng.integers(w.batch)), int(rng.integers(w.kv_heads))))
    return sorted(units)


@pytest.mark.parametrize("name,meta", [("llama3-8b-gqa-8k", 0), ("llama2-13b-mha-wall", 0),
                                       ("llama3-8b-gqa-8k", 1)])
def test_prefill_and_decode_full_size(name, meta):
    w = synth.WORKLOADS[name]
    batch = 8 if name == "llama2-13b-mha-wall" else w.batch
    print(f"workload {name} batch {batch} meta {meta}", flush=True)
    k, v = synth.prefill_kv(w, 11, batch=batch)
    q = synth.query(w, 11, batch=batch)
    T = 32 * math.ceil((w.seq_len - 128 + 32) / 32)
    g = kivi.Geom(batch, w.kv_heads, w.q_per_kv, bits=w.bits, max_tokens=T, meta_format=meta)
    gc = kivi.Cache(g)
    kivi.quantize_prefill(g, gc, k.cuda(), v.cuda())
    out = torch.full((batch, w.q_heads, 128), float("nan"), device="cuda")
    kivi.decode_attention(g, gc, q.cuda(), out=out)
    torch.cuda.synchronize()
    out_np = to_np(out)
    assert np.isfinite(out_np).all()
    kb, vb, qb = synth.bits_u16(k), synth.bits_u16(v), synth.bits_u16(q)
    og = _unit_geoms(w, T, meta)
    scale = 1.0 / math.sqrt(128)
    for b, h in _sample_units(synth.Workload(name, batch, w.kv_heads, w.q_per_kv, w.seq_len,
                                             w.bits, 1, 3, 8.0), 4, 1):
        oc1 = oracle.prefill(og, kb[b:b + 1, h:h + 1].copy(), vb[b:b + 1, h:h + 1].copy())
        _check_unit_cache(gc, oc1, b, h)
        _check_unit_attention(out_np, oc1, qb, b, h, w.q_per_kv, scale)


@pytest.mark.parametrize("name,steps,check_every", [("llama2-7b-mha-4k", 128, 16),
                                                    ("llama3-8b-gqa-32k-4bit", 1024, 128)])
def test_streaming_decode_full_size(name, steps, check_every):
    w = synth.WORKLOADS[name]
    print(f"workload {name} steps {steps}", flush=True)
    k, v = synth.prefill_kv(w, 21)
    T = 32 * math.ceil((w.seq_len - 128 + steps + 32) / 32)
    g = kivi.Geom(w.batch, w.kv_heads, w.q_per_kv, bits=w.bits, max_tokens=T)
    gc = kivi.Cache(g)
    kivi.quantize_prefill(g, gc, k.cuda(), v.cuda())
    units = _sample_units(w, 3, 2)
    og = _unit_geoms(w, T)
    kb, vb = synth.bits_u16(k), synth.bits_u16(v)
    ocs = {(b, h): oracle.prefill(og, kb[b:b + 1, h:h + 1].copy(), vb[b:b + 1, h:h + 1].copy())
           for b, h in units}
    del k, v, kb, vb
    ws = kivi.Workspace(g)
    out = torch.empty(w.batch, w.q_heads, 128, device="cuda")
    scale = 1.0 / math.sqrt(128)
    flushes = 0
    for step in range(steps):
        kn, vn = synth.new_token(w, 21, 0, step)
        kivi.append_token(g, gc, kn.cuda(), vn.cuda())
        f = kivi.flush_residual(g, gc)
        flushes += f
        knb, vnb = synth.bits_u16(kn), synth.bits_u16(vn)
        for (b, h), oc1 in ocs.items():
            oracle.append(oc1, knb[b:b + 1, h:h + 1].copy(), vnb[b:b + 1, h:h + 1].copy())
            assert oracle.flush(oc1) == f
        if step % check_every == check_every - 1 or step == steps - 1:
            q = synth.query(w, 21, 0, step)
            out.fill_(float("nan"))
            kivi.decode_attention(g, gc, q.cuda(), out=out, ws=ws)
            torch.cuda.synchronize()
            out_np, qb = to_np(out), synth.bits_u16(q)
            assert np.isfinite(out_np).all()
            for (b, h), oc1 in ocs.items():
                _check_unit_attention(out_np, oc1, qb, b, h, w.q_per_kv, scale)
            print(f"step {step}: n_q {gc.n_q} n_res {gc.n_res} ok", flush=True)
    assert flushes == steps // 32
    torch.cuda.synchronize()
    for (b, h), oc1 in ocs.items():
        _check_unit_cache(gc, oc1, b, h)


@pytest.mark.parametrize("name,steps", [("llama3-8b-gqa-8k", 40), ("llama3-8b-gqa-32k-4bit", 64)])
def test_fused_decode_step_full_size(name, steps):
    """The timed call (kivi_decode_step through LayerStepper.step: append and,
    when the ring fills, the flush folded into the attention launch) at
    the full workload size, across flushes: sampled units against the
    oracle at every flush step and at the end (cache bytes exact, attention
    within the bound), and every output against the same steps made of the
    three separate calls on a second cache, both sharing one workspace."""
    w = synth.WORKLOADS[name]
    print(f"fused step {name} steps {steps}", flush=True)
    k, v = synth.prefill_kv(w, 31)
    T = 32 * math.ceil((w.seq_len - 128 + steps + 32) / 32)
    g = kivi.Geom(w.batch, w.kv_heads, w.q_per_kv, bits=w.bits, max_tokens=T)
    fused, sep = kivi.Cache(g), kivi.Cache(g)
    kd, vd = k.cuda(), v.cuda()
    kivi.quantize_prefill(g, fused, kd, vd)
    kivi.quantize_prefill(g, sep, kd, vd)
    del kd, vd
    units = _sample_units(w, 4, 3)
    og = _unit_geoms(w, T)
    kb, vb = synth.bits_u16(k), synth.bits_u16(v)
    ocs = {(b, h): oracle.prefill(og, kb[b:b + 1, h:h + 1].copy(), vb[b:b + 1, h:h + 1].copy())
           for b, h in units}
    del k, v, kb, vb
    ws = kivi.Workspace(g)
    q_dev = torch.empty(w.batch, w.q_heads, 128, dtype=torch.bfloat16, device="cuda")
    out_f = torch.empty(w.batch, w.q_heads, 128, device="cuda")
    out_s = torch.empty_like(out_f)
    stepper = kivi.LayerStepper(g, fused, ws, q_dev, out_f)
    separate = kivi.LayerStepper(g, sep, ws, q_dev, out_s)
    scale = 1.0 / math.sqrt(128)
    flush_steps = []
    for step in range(steps):
        kn, vn = synth.new_token(w, 31, 0, step)
        q = synth.query(w, 31, 0, step)
        q_dev.copy_(q)
        kn_d, vn_d = kn.cuda(), vn.cuda()
        out_f.fill_(float("nan"))
        out_s.fill_(float("nan"))
        f = stepper.step(kn_d, vn_d)
        separate.append(kn_d, vn_d)
        assert separate.flush() == f
        separate.attend()
        knb, vnb = synth.bits_u16(kn), synth.bits_u16(vn)
        for (b, h), oc1 in ocs.items():
            oracle.append(oc1, knb[b:b + 1, h:h + 1].copy(), vnb[b:b + 1, h:h + 1].copy())
            assert oracle.flush(oc1) == f
        torch.cuda.synchronize()
        of, os_ = to_np(out_f), to_np(out_s)
        assert np.isfinite(of).all() and np.isfinite(os_).all()
        assert row_rel_err(of, os_) <= REPEAT_TOL, f"step {step}: fused vs separate calls"
        assert (fused.n_q, fused.n_res, fused.res_start) == (sep.n_q, sep.n_res, sep.res_start)
        if f or step == steps - 1:
            flush_steps += [step] if f else []
            qb = synth.bits_u16(q)
            errs = [_check_unit_attention(of, oc1, qb, b, h, w.q_per_kv, scale)
                    for (b, h), oc1 in ocs.items()]
            for (b, h), oc1 in ocs.items():
                _check_unit_cache(fused, oc1, b, h)
                _check_unit_cache(sep, oc1, b, h)
            print(f"step {step}: flushed {f} n_q {fused.n_q} n_res {fused.n_res} "
                  f"max err {max(errs):.2e}", flush=True)
    assert len(flush_steps) == steps // 32
    # the two caches hold the same bytes everywhere the cache is in use
    torch.cuda.synchronize()
    ng = fused.n_q // 32
    assert torch.equal(fused.records[:, :, :ng], sep.records[:, :, :ng])


def test_workspace_reuse_back_to_back():
    """One workspace, many back-to-back decode launches over different caches
    and queries with no synchronisation in between: every unit of every
    launch against the oracle.  A launch whose combine read a partial still
    in flight, or left by the previous launch, would fail here."""
    B, H, QPK, S, layers = 4, 8, 4, 4096, 6
    w = synth.Workload("reuse", B, H, QPK, S, 2, layers, 3, 8.0)
    T = 32 * ((S - 128) // 32)
    g = kivi.Geom(B, H, QPK, max_tokens=T)
    ws = kivi.Workspace(g)
    caches, qs, refs = [], [], []
    for layer in range(layers):
        k, v = synth.prefill_kv(w, 41, layer)
        c = kivi.Cache(g)
        kivi.quantize_prefill(g, c, k.cuda(), v.cuda())
        q = synth.query(w, 41, layer)
        oc = oracle.prefill(oracle.Geom(B, H, QPK, max_tokens=T), synth.bits_u16(k),
                            synth.bits_u16(v))
        refs.append(oracle.attention(oc, synth.bits_u16(q), 1 / math.sqrt(128)))
        caches.append(c)
        qs.append(q.cuda())
    outs = [torch.full((B, H * QPK, 128), float("nan"), device="cuda") for _ in range(layers)]
    torch.cuda.synchronize()
    for rep in range(3):
        for layer in range(layers):
            kivi.decode_attention(g, caches[layer], qs[layer], out=outs[layer], ws=ws)
        torch.cuda.synchronize()
        for layer in range(layers):
            o = to_np(outs[layer])
            assert np.isfinite(o).all()
            err = row_rel_err(o, refs[layer])
            assert err <= ATTN_TOL, f"rep {rep} layer {layer}: {err:.3e}"
            outs[layer].fill_(float("nan"))


def test_deterministic_launch_repeats_bitwise_full_size():
    """With KIVI_FLAG_DETERMINISTIC the 8K GQA launch is bitwise repeatable;
    the default launch (dynamic claims) stays within REPEAT_TOL of it."""
    w = synth.WORKLOADS["llama3-8b-gqa-8k"]
    k, v = synth.prefill_kv(w, 51)
    q = synth.query(w, 51).cuda()
    T = 32 * ((w.seq_len - 128) // 32)
    outs = {}
    for flags in (kivi.FLAG_DETERMINISTIC, 0):
        g = kivi.Geom(w.batch, w.kv_heads, w.q_per_kv, bits=w.bits, max_tokens=T, flags=flags)
        c = kivi.Cache(g)
        kivi.quantize_prefill(g, c, k.cuda(), v.cuda())
        ws = kivi.Workspace(g)
        runs = []
        for _ in range(4):
            out = torch.full((w.batch, w.q_heads, 128), float("nan"), device="cuda")
            kivi.decode_attention(g, c, q, out=out, ws=ws)
            runs.append(out)
        torch.cuda.synchronize()
        runs = [to_np(o) for o in runs]
        if flags:
            for o in runs[1:]:
                np.testing.assert_array_equal(o, runs[0])
        else:
            for o in runs[1:]:
                assert row_rel_err(o, runs[0]) <= REPEAT_TOL
        outs[flags] = runs[0]
        del c, ws
    assert row_rel_err(outs[0], outs[kivi.FLAG_DETERMINISTIC]) <= REPEAT_TOL
