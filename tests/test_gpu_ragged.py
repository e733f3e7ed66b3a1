"""GPU parity of mixed-length batches (kivi_ragged_prefill and
kivi_ragged_decode_step) against the oracle run on each sequence alone.

* Prefill: every sequence's quantised history, scale/zero and residual equal,
  byte for byte, the oracle's prefill of that sequence as a batch of one; the
  padding past each length holds Inf/NaN and must not be read.
* Decode steps: sequences of different lengths flush at different steps;
  every step's output rows of a sequence match the oracle's attention over
  that sequence's own cache, the device state matches the oracle's
  counters, and the final caches are byte-identical.
* Flags: a sequence with an out-of-range length is empty (output rows 0);
  one whose history is full stops taking tokens and keeps its cache.
* The two launches of a step take the same arguments every step, so a HIP
  graph of two steps (state buffers swapped) replays them; replays are
  checked against the same steps run eagerly, bitwise with the deterministic
  flag and to within REPEAT_TOL (2e-4) row-relative in the default launch (whose waves may
  merge in the order they finish).
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

SCALE = 1.0 / math.sqrt(128)


def _inputs(B, H, QPK, stride, bits, seed, steps=0):
    w = synth.Workload("ragged", B, H, QPK, stride + steps, bits, 1, 3, 8.0)
    k, v = synth.prefill_kv(w, seed)
    return w, synth.bits_u16(k), synth.bits_u16(v)


def _padded(x, lens, stride):
    """Copy of x[:, :, :stride] with Inf/NaN past each sequence's length."""
    y = x[:, :, :stride].copy()
    for b, n in enumerate(lens):
        y[b, :, n:] = 0x7FC0          # NaN
        y[b, :, n::3] = 0xFF80        # -Inf
    return y


def _ragged_cache(B, H, QPK, bits, meta, T, lens, kb, vb, stride, flags=0):
    kg = kivi.Geom(B, H, QPK, bits=bits, max_tokens=T, meta_format=meta, flags=flags)
    gc = kivi.Cache(kg)
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    state = kivi.ragged_prefill(kg, gc, bits_to_dev(_padded(kb, lens, stride)),
                                bits_to_dev(_padded(vb, lens, stride)), seq)
    return kg, gc, state


def _oracle_seq(b, H, QPK, bits, meta, T, kb, vb, n):
    og = oracle.Geom(1, H, QPK, bits=bits, max_tokens=T, meta=meta)
    return og, oracle.prefill(og, kb[b:b + 1, :, :n].copy(), vb[b:b + 1, :, :n].copy())


def _check_seq_cache(gc, kg, b, oc):
    og_full = oracle.Geom(kg.batch, kg.kv_heads, kg.q_per_kv, bits=kg.bits,
                          max_tokens=kg.max_tokens, meta=kg.meta_format)
    hc = host_cache(gc, og_full)
    hc.n_q, hc.n_res, hc.res_start = oc.n_q, oc.n_res, oc.res_start
    H = kg.kv_heads
    assert_same_cache(hc, oc, units=[(b, h) for h in range(H)], ref_units=[(0, h) for h in range(H)])


CASES = [
    # H, QPK, bits, meta, lengths
    (2, 4, 2, 0, [150, 700, 1509, 33]),
    (2, 1, 2, 0, [1509, 129, 160, 1000]),
    (1, 4, 4, 1, [300, 1, 1200]),
    (3, 2, 4, 0, [161, 991]),
]


@pytest.mark.parametrize("H,QPK,bits,meta,lens", CASES)
def test_ragged_prefill_and_steps_match_each_sequence_alone(H, QPK, bits, meta, lens):
    B, steps = len(lens), 70
    print(f"ragged H={H} QPK={QPK} bits={bits} meta={meta} lens={lens}", flush=True)
    stride = max(lens)
    w, kb, vb = _inputs(B, H, QPK, stride, bits, 900 + sum(lens), steps)
    T = 32 * ((stride + steps) // 32 + 1)
    kg, gc, st_a = _ragged_cache(B, H, QPK, bits, meta, T, lens, kb, vb, stride)
    torch.cuda.synchronize()
    ocs = [_oracle_seq(b, H, QPK, bits, meta, T, kb, vb, n)[1] for b, n in enumerate(lens)]
    st = to_np(st_a)
    for b, oc in enumerate(ocs):
        assert tuple(st[b]) == (oc.n_q, oc.n_res, 0, 0)
        _check_seq_cache(gc, kg, b, oc)
    # decode steps: token t of sequence b is its row lens[b] + t of the inputs
    st_b = torch.empty_like(st_a)
    ws = kivi.Workspace(kg)
    out = torch.empty(B, H * QPK, 128, device="cuda")
    for t in range(steps):
        kn = np.stack([kb[b, :, n + t] for b, n in enumerate(lens)])
        vn = np.stack([vb[b, :, n + t] for b, n in enumerate(lens)])
        q = synth.bits_u16(synth.query(w, 900 + t))
        out.fill_(float("nan"))
        kivi.ragged_decode_step(kg, gc, st_a, st_b, bits_to_dev(kn), bits_to_dev(vn),
                                bits_to_dev(q), out=out, ws=ws, softmax_scale=SCALE)
        st_a, st_b = st_b, st_a
        torch.cuda.synchronize()
        o, st = to_np(out), to_np(st_a)
        for b, oc in enumerate(ocs):
            oracle.append(oc, kn[b:b + 1], vn[b:b + 1])
            oracle.flush(oc)
            assert tuple(st[b]) == (oc.n_q, oc.n_res, oc.res_start, 0), (t, b)
            ref = oracle.attention(oc, q[b:b + 1].copy(), SCALE)
            err = row_rel_err(o[b], ref[0])
            assert err <= ATTN_TOL, f"step {t} sequence {b}: {err:.3e}"
    for b, oc in enumerate(ocs):
        _check_seq_cache(gc, kg, b, oc)


def test_ragged_flags():
    """Sequence 0: length 0 (bad); sequence 1: a history of one group fills up
    and the sequence stops; sequence 2: unaffected."""
    B, H, QPK, bits = 3, 2, 4, 2
    lens = [0, 180, 140]
    stride = 200
    w, kb, vb = _inputs(B, H, QPK, stride, bits, 77, 60)
    T = 64   # two groups of history
    kg, gc, st_a = _ragged_cache(B, H, QPK, bits, 0, T, lens, kb, vb, stride)
    st_b = torch.empty_like(st_a)
    ws = kivi.Workspace(kg)
    out = torch.empty(B, H * QPK, 128, device="cuda")
    oc2 = _oracle_seq(2, H, QPK, bits, 0, T, kb, vb, lens[2])[1]
    oc1 = _oracle_seq(1, H, QPK, bits, 0, T, kb, vb, lens[1])[1]
    full_at = None
    for t in range(60):   # sequence 1 flushes at step 11 and is full from step 43
        kn = np.stack([kb[b, :, max(n, 1) + t] for b, n in enumerate(lens)])
        vn = np.stack([vb[b, :, max(n, 1) + t] for b, n in enumerate(lens)])
        q = synth.bits_u16(synth.query(w, 77 + t))
        kivi.ragged_decode_step(kg, gc, st_a, st_b, bits_to_dev(kn), bits_to_dev(vn),
                                bits_to_dev(q), out=out, ws=ws, softmax_scale=SCALE)
        st_a, st_b = st_b, st_a
        torch.cuda.synchronize()
        st, o = to_np(st_a), to_np(out)
        assert st[0][3] == kivi.SEQ_BAD_LENGTH and np.all(o[0] == 0)
        oracle.append(oc2, kn[2:3], vn[2:3])
        oracle.flush(oc2)
        assert tuple(st[2]) == (oc2.n_q, oc2.n_res, oc2.res_start, 0)
        assert row_rel_err(o[2], oracle.attention(oc2, q[2:3].copy(), SCALE)[0]) <= ATTN_TOL
        if full_at is None:
            if oc1.n_res + 1 == oc1.geom.slots and oc1.n_q + 32 > T:
                full_at = t   # the oracle cannot flush: the sequence is full
            else:
                oracle.append(oc1, kn[1:2], vn[1:2])
                oracle.flush(oc1)
        if full_at is not None:
            assert st[1][3] == kivi.SEQ_FULL
            assert tuple(st[1][:3]) == (oc1.n_q, oc1.n_res, oc1.res_start)
        else:
            assert tuple(st[1]) == (oc1.n_q, oc1.n_res, oc1.res_start, 0)
        assert row_rel_err(o[1], oracle.attention(oc1, q[1:2].copy(), SCALE)[0]) <= ATTN_TOL
    assert full_at is not None
    _check_seq_cache(gc, kg, 1, oc1)


@pytest.mark.parametrize("flags", [0, 1])
def test_ragged_steps_in_a_graph_replay_like_eager(flags):
    assert kivi.FLAG_DETERMINISTIC == 1
    B, H, QPK, bits = 3, 2, 4, 2
    lens = [155, 412, 1000]   # sequences 0 and 1 flush inside the replays (steps 4 and 3)
    stride = max(lens)
    reps = 6
    w, kb, vb = _inputs(B, H, QPK, stride, bits, 55, 2 * reps + 2)
    T = 32 * ((stride + 2 * reps + 2) // 32 + 1)
    kg, g_cache, ga = _ragged_cache(B, H, QPK, bits, 0, T, lens, kb, vb, stride, flags)
    _, e_cache, ea = _ragged_cache(B, H, QPK, bits, 0, T, lens, kb, vb, stride, flags)
    gb, eb = torch.empty_like(ga), torch.empty_like(ea)
    g_ws, e_ws = kivi.Workspace(kg), kivi.Workspace(kg)
    kn = torch.empty(2, B, H, 128, dtype=torch.bfloat16, device="cuda")
    vn = torch.empty_like(kn)
    q = torch.empty(2, B, H * QPK, 128, dtype=torch.bfloat16, device="cuda")
    g_out = torch.zeros(2, B, H * QPK, 128, device="cuda")
    e_out = torch.zeros_like(g_out)

    def inputs(i):
        toks = []
        for j in range(2):
            t = 2 * i + j
            k1 = np.stack([kb[b, :, n + t] for b, n in enumerate(lens)])
            v1 = np.stack([vb[b, :, n + t] for b, n in enumerate(lens)])
            q1 = synth.bits_u16(synth.query(w, 55 + t))
            toks.append((k1, v1, q1))
        return toks

    def load(toks):
        for j, (k1, v1, q1) in enumerate(toks):
            kn[j].copy_(bits_to_dev(k1))
            vn[j].copy_(bits_to_dev(v1))
            q[j].copy_(bits_to_dev(q1))

    def two_steps(cache, sa, sb, ws, out):
        kivi.ragged_decode_step(kg, cache, sa, sb, kn[0], vn[0], q[0], out=out[0], ws=ws,
                                softmax_scale=SCALE)
        kivi.ragged_decode_step(kg, cache, sb, sa, kn[1], vn[1], q[1], out=out[1], ws=ws,
                                softmax_scale=SCALE)

    # warm-up outside the capture (launch shapes are cached per device), on a
    # scratch cache so that the compared caches stay in step
    _, w_cache, wa = _ragged_cache(B, H, QPK, bits, 0, T, lens, kb, vb, stride)
    load(inputs(0))
    two_steps(w_cache, wa, torch.empty_like(wa), kivi.Workspace(kg), torch.empty_like(g_out))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        two_steps(g_cache, ga, gb, g_ws, g_out)
    for i in range(reps):
        toks = inputs(i)
        load(toks)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        g_res = to_np(g_out).copy()
        e_out.fill_(float("nan"))            # eager work between replays
        two_steps(e_cache, ea, eb, e_ws, e_out)
        torch.cuda.synchronize()
        if flags:
            assert np.array_equal(g_res.view(np.uint32), to_np(e_out).view(np.uint32)), i
        else:
            assert row_rel_err(g_res, to_np(e_out)) <= REPEAT_TOL, i
        assert np.array_equal(to_np(ga), to_np(ea)), i
    # the used part of each sequence's cache (the rest was never written)
    og = oracle.Geom(B, H, QPK, bits=bits, max_tokens=T)
    hg, he = host_cache(g_cache, og), host_cache(e_cache, og)
    for b, row in enumerate(to_np(ea)):
        for c in (hg, he):
            c.n_q, c.n_res, c.res_start = int(row[0]), int(row[1]), int(row[2])
        assert_same_cache(hg, he, units=[(b, h) for h in range(H)])


def test_ragged_state_rows_out_of_range_become_empty_sequences():
    """State rows that no call wrote: each is an empty bad sequence (output 0,
    state {0,0,0,BAD}); the other sequences step as usual."""
    B, H, QPK, bits = 6, 1, 4, 2
    lens = [300] * B
    w, kb, vb = _inputs(B, H, QPK, 300, bits, 91, 1)
    T = 320
    kg, gc, st_a = _ragged_cache(B, H, QPK, bits, 0, T, lens, kb, vb, 300)
    oc = _oracle_seq(0, H, QPK, bits, 0, T, kb, vb, 300)[1]
    bad_rows = {1: (1 << 20, 0, 0, 0),      # history beyond capacity
                2: (33, 4, 0, 0),           # history not whole groups
                3: (160, 160, 0, 0),        # ring count >= slots
                4: (160, 10, 7, 0),         # ring start off a group boundary
                5: (160, 140, 0, 8)}        # unknown flag bit
    for b, row in bad_rows.items():
        st_a[b] = torch.tensor(row, dtype=torch.int32)
    st_b = torch.empty_like(st_a)
    kn = np.stack([kb[b, :, 300] for b in range(B)])
    vn = np.stack([vb[b, :, 300] for b in range(B)])
    q = synth.bits_u16(synth.query(w, 91))
    out = kivi.ragged_decode_step(kg, gc, st_a, st_b, bits_to_dev(kn), bits_to_dev(vn),
                                  bits_to_dev(q), softmax_scale=SCALE)
    torch.cuda.synchronize()
    st, o = to_np(st_b), to_np(out)
    for b in bad_rows:
        assert tuple(st[b]) == (0, 0, 0, kivi.SEQ_BAD_LENGTH) and np.all(o[b] == 0), b
    oracle.append(oc, kn[0:1], vn[0:1])
    oracle.flush(oc)
    assert tuple(st[0]) == (oc.n_q, oc.n_res, oc.res_start, 0)
    assert row_rel_err(o[0], oracle.attention(oc, q[0:1].copy(), SCALE)[0]) <= ATTN_TOL
