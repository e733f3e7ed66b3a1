"""GPU parity of mixed-length and paged batches over seeded random shapes.

Each case draws kv heads, query heads per kv head (1-16), bit width,
scale/zero format, launch flag, softmax scale, 1-6 sequence lengths (1-2000,
so residual-only, group-aligned and ragged histories mix in one batch), a
number of decode steps (crossing each sequence's flushes at different steps)
and, for the paged form, the page size (1-16 groups) and a shuffled page
pool, from numpy's default_rng(4048).  Every sequence is checked against the
oracle run on it alone: the caches byte for byte after the prefill and after
the steps, the per-sequence device state after every step, and the outputs
within the attention tolerance every eighth step and at the last one."""
import math

import numpy as np
import pytest
import torch

import oracle
from kivi_testutil import ATTN_TOL, assert_same_cache, bits_to_dev, row_rel_err, to_np
from test_gpu_paged import _assign, _gather
from test_gpu_paged import _inputs as _paged_inputs
from test_gpu_paged import _padded as _paged_padded
from test_gpu_ragged import _check_seq_cache, _inputs, _oracle_seq, _ragged_cache

import synth

kivi = pytest.importorskip("decode_attention_channel_amd.kivi")

pytestmark = pytest.mark.gpu


def _cases(n, seed, paged):
    rng = np.random.default_rng(seed + paged)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 7))
        H = int(rng.integers(1, 5))
        QPK = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16]))
        bits = int(rng.choice([2, 4]))
        meta = int(rng.integers(0, 2))
        flags = int(rng.integers(0, 2))
        scale = float(rng.choice([0.25, 1.0, 4.0])) / math.sqrt(128)
        lens = [int(np.exp(rng.uniform(0, math.log(2000)))) if rng.random() < 0.5
                else int(rng.integers(1, 2001)) for _ in range(B)]
        steps = int(rng.integers(1, 41))
        P = int(rng.choice([1, 2, 4, 8, 16]))
        out.append((i, H, QPK, bits, meta, flags, scale, lens, steps, P))
    return out


def _check_step(t, steps, o, q, ocs, scale):
    if t % 8 != 7 and t != steps - 1:
        return
    for b, oc in enumerate(ocs):
        err = row_rel_err(o[b], oracle.attention(oc, q[b:b + 1].copy(), scale)[0])
        assert err <= ATTN_TOL, f"step {t} sequence {b}: {err:.3e}"


@pytest.mark.parametrize("i,H,QPK,bits,meta,flags,scale,lens,steps,P", _cases(32, 4048, 0))
def test_random_ragged(i, H, QPK, bits, meta, flags, scale, lens, steps, P):
    B = len(lens)
    print(f"random ragged {i}: H={H} QPK={QPK} bits={bits} meta={meta} flags={flags} "
          f"lens={lens} steps={steps}", flush=True)
    stride = max(lens)
    w, kb, vb = _inputs(B, H, QPK, stride, bits, 6000 + i, steps)
    T = 32 * ((stride + steps) // 32 + 1)
    kg, gc, st_a = _ragged_cache(B, H, QPK, bits, meta, T, lens, kb, vb, stride, flags=flags)
    torch.cuda.synchronize()
    ocs = [_oracle_seq(b, H, QPK, bits, meta, T, kb, vb, n)[1] for b, n in enumerate(lens)]
    st = to_np(st_a)
    for b, oc in enumerate(ocs):
        assert tuple(st[b]) == (oc.n_q, oc.n_res, 0, 0)
        _check_seq_cache(gc, kg, b, oc)
    st_b = torch.empty_like(st_a)
    ws = kivi.Workspace(kg)
    out = torch.empty(B, H * QPK, 128, device="cuda")
    for t in range(steps):
        kn = np.stack([kb[b, :, n + t] for b, n in enumerate(lens)])
        vn = np.stack([vb[b, :, n + t] for b, n in enumerate(lens)])
        q = synth.bits_u16(synth.query(w, 6000 + i, step=t))
        out.fill_(float("nan"))
        kivi.ragged_decode_step(kg, gc, st_a, st_b, bits_to_dev(kn), bits_to_dev(vn),
                                bits_to_dev(q), out=out, ws=ws, softmax_scale=scale)
        st_a, st_b = st_b, st_a
        torch.cuda.synchronize()
        o, st = to_np(out), to_np(st_a)
        assert np.isfinite(o).all(), f"step {t}: unwritten output"
        for b, oc in enumerate(ocs):
            oracle.append(oc, kn[b:b + 1], vn[b:b + 1])
            oracle.flush(oc)
            assert tuple(st[b]) == (oc.n_q, oc.n_res, oc.res_start, 0), (t, b)
        _check_step(t, steps, o, q, ocs, scale)
    for b, oc in enumerate(ocs):
        _check_seq_cache(gc, kg, b, oc)


@pytest.mark.parametrize("i,H,QPK,bits,meta,flags,scale,lens,steps,P", _cases(32, 4048, 1))
def test_random_paged(i, H, QPK, bits, meta, flags, scale, lens, steps, P):
    B = len(lens)
    print(f"random paged {i}: H={H} QPK={QPK} bits={bits} meta={meta} flags={flags} P={P} "
          f"lens={lens} steps={steps}", flush=True)
    stride = max(lens)
    w, kb, vb = _paged_inputs(B, H, QPK, stride + steps, bits, 7000 + i)
    T = 32 * ((stride + steps) // 32 + 1)
    g = kivi.Geom(B, H, QPK, bits=bits, max_tokens=T, meta_format=meta, flags=flags)
    NG = T // 32
    pc = kivi.PagedCache(g, P, B * ((NG + P - 1) // P) + 2)
    table = _assign(pc, [NG] * B, np.random.default_rng(7000 + i))
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    st_a = kivi.paged_prefill(g, pc, bits_to_dev(_paged_padded(kb, lens, stride)),
                              bits_to_dev(_paged_padded(vb, lens, stride)), seq)
    torch.cuda.synchronize()
    og1 = oracle.Geom(1, H, QPK, bits=bits, max_tokens=T, meta=meta)
    ocs = [oracle.prefill(og1, kb[b:b + 1, :, :n].copy(), vb[b:b + 1, :, :n].copy())
           for b, n in enumerate(lens)]
    st = to_np(st_a)
    for b, oc in enumerate(ocs):
        assert tuple(st[b]) == (oc.n_q, oc.n_res, 0, 0)
        assert_same_cache(_gather(pc, b, table, og1, oc.n_q, oc.n_res, oc.res_start), oc)
    st_b = torch.empty_like(st_a)
    ws = kivi.Workspace(g)
    out = torch.empty(B, H * QPK, 128, device="cuda")
    for t in range(steps):
        kn = np.stack([kb[b, :, n + t] for b, n in enumerate(lens)])
        vn = np.stack([vb[b, :, n + t] for b, n in enumerate(lens)])
        q = synth.bits_u16(synth.query(w, 7000 + i, step=t))
        out.fill_(float("nan"))
        kivi.paged_decode_step(g, pc, st_a, st_b, bits_to_dev(kn), bits_to_dev(vn),
                               bits_to_dev(q), out=out, ws=ws, softmax_scale=scale)
        st_a, st_b = st_b, st_a
        torch.cuda.synchronize()
        o, st = to_np(out), to_np(st_a)
        assert np.isfinite(o).all(), f"step {t}: unwritten output"
        for b, oc in enumerate(ocs):
            oracle.append(oc, kn[b:b + 1], vn[b:b + 1])
            oracle.flush(oc)
            assert tuple(st[b]) == (oc.n_q, oc.n_res, oc.res_start, 0), (t, b)
        _check_step(t, steps, o, q, ocs, scale)
    for b, oc in enumerate(ocs):
        assert_same_cache(_gather(pc, b, table, og1, oc.n_q, oc.n_res, oc.res_start), oc)
