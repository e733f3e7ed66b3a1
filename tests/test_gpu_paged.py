"""GPU parity of the paged history (kivi_paged_prefill, kivi_paged_decode_step)
against the oracle run on each sequence alone.

Pages are handed out from a shuffled pool, so that the sequences' groups are
interleaved in the pools.  The device pools are gathered back, page by page,
into the oracle's per-sequence layout and compared byte for byte; outputs and
per-sequence state are checked at every step.  Also: a sequence whose next
page is not assigned stops at the flush that needs it (KIVI_SEQ_FULL) while
the others go on; a prefill whose history lacks a page gives
KIVI_SEQ_BAD_LENGTH; graph replays of paged steps equal eager steps (bitwise
with the deterministic flag, to within REPEAT_TOL (2e-4) row-relative in the default
launch, whose waves may merge in the order they finish).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from kivi_testutil import ATTN_TOL, REPEAT_TOL, assert_same_cache, bits_to_dev, row_rel_err, to_np

kivi = pytest.importorskip("decode_attention_channel_amd.kivi")

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(128)


def _inputs(B, H, QPK, rows, bits, seed):
    w = synth.Workload("paged", B, H, QPK, rows, bits, 1, 3, 8.0)
    k, v = synth.prefill_kv(w, seed)
    return w, synth.bits_u16(k), synth.bits_u16(v)


def _assign(pc, lens_groups, rng, skip=None):
    """Pages for the first lens_groups[b] groups of each sequence (ceil),
    drawn from a shuffled pool; skip = {b: page index left unassigned}."""
    P = pc.page_groups
    free = list(rng.permutation(pc.num_pages))
    table = np.full((pc.geom.batch, pc.max_pages), -1, np.int32)
    for b, ng in enumerate(lens_groups):
        for i in range(min((ng + P - 1) // P, pc.max_pages)):
            if skip and skip.get(b) == i:
                continue
            table[b, i] = free.pop()
    pc.block_table.copy_(torch.from_numpy(table))
    return table


def _gather(pc, b, table, og1, n_q, n_res, res_start):
    """oracle.Cache (batch 1) of sequence b read out of the device pools."""
    hc = oracle.Cache(og1)
    G, H = og1.group, og1.kv_heads
    pools = pc.pool_history()   # per-array layout, from the group records
    res = {n: to_np(getattr(pc, n)) for n in ("k_res", "v_res")}
    for h in range(H):
        for g in range(n_q // G):
            s = pc.slot(b, h, g, table)
            assert s >= 0
            hc.k_codes[0, h, g * G:(g + 1) * G] = pools["k_codes"][s]
            for n in ("k_scale", "k_zero", "v_codes", "v_scale", "v_zero"):
                getattr(hc, n)[0, h, g] = np.ascontiguousarray(pools[n][s]).view(
                    getattr(hc, n).dtype).reshape(getattr(hc, n)[0, h, g].shape)
        hc.k_res[0, h] = res["k_res"][b, h]
        hc.v_res[0, h] = res["v_res"][b, h]
    hc.n_q, hc.n_res, hc.res_start = n_q, n_res, res_start
    return hc


def _padded(x, lens, stride):
    y = x[:, :, :stride].copy()
    for b, n in enumerate(lens):
        y[b, :, n:] = 0x7FC0
    return y


CASES = [
    # H, QPK, bits, meta, page_groups, lengths
    (2, 4, 2, 0, 4, [150, 700, 1509]),
    (2, 1, 2, 0, 2, [1509, 300, 161]),
    (1, 4, 4, 1, 1, [700, 129, 1000]),
    (2, 2, 4, 0, 8, [400, 1200]),
]


@pytest.mark.parametrize("H,QPK,bits,meta,P,lens", CASES)
def test_paged_prefill_and_steps_match_each_sequence_alone(H, QPK, bits, meta, P, lens):
    B, steps = len(lens), 70
    print(f"paged H={H} QPK={QPK} bits={bits} meta={meta} P={P} lens={lens}", flush=True)
    stride = max(lens)
    w, kb, vb = _inputs(B, H, QPK, stride + steps, bits, 1300 + sum(lens) + P)
    T = 32 * ((stride + steps) // 32 + 1)
    g = kivi.Geom(B, H, QPK, bits=bits, max_tokens=T, meta_format=meta)
    NG = T // 32
    num_pages = B * ((NG + P - 1) // P) + 3
    pc = kivi.PagedCache(g, P, num_pages)
    rng = np.random.default_rng(len(lens) * 7 + P)
    table = _assign(pc, [NG] * B, rng)
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    st_a = kivi.paged_prefill(g, pc, bits_to_dev(_padded(kb, lens, stride)),
                              bits_to_dev(_padded(vb, lens, stride)), seq)
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
        q = synth.bits_u16(synth.query(w, 1300 + t))
        out.fill_(float("nan"))
        kivi.paged_decode_step(g, pc, st_a, st_b, bits_to_dev(kn), bits_to_dev(vn),
                               bits_to_dev(q), out=out, ws=ws, softmax_scale=SCALE)
        st_a, st_b = st_b, st_a
        torch.cuda.synchronize()
        o, st = to_np(out), to_np(st_a)
        for b, oc in enumerate(ocs):
            oracle.append(oc, kn[b:b + 1], vn[b:b + 1])
            oracle.flush(oc)
            assert tuple(st[b]) == (oc.n_q, oc.n_res, oc.res_start, 0), (t, b)
            err = row_rel_err(o[b], oracle.attention(oc, q[b:b + 1].copy(), SCALE)[0])
            assert err <= ATTN_TOL, f"step {t} sequence {b}: {err:.3e}"
    for b, oc in enumerate(ocs):
        assert_same_cache(_gather(pc, b, table, og1, oc.n_q, oc.n_res, oc.res_start), oc)


def test_paged_missing_pages():
    """Sequence 0 lacks the page of its first flushed group: it stops there
    (KIVI_SEQ_FULL, cache and output as before the token); sequence 1 lacks a
    page of its prefilled history: KIVI_SEQ_BAD_LENGTH, output 0; sequence 2
    is unaffected."""
    B, H, QPK, bits, P = 3, 2, 4, 2, 2
    lens = [150, 600, 400]
    steps = 24
    w, kb, vb = _inputs(B, H, QPK, 700, bits, 808)
    T = 1024
    g = kivi.Geom(B, H, QPK, bits=bits, max_tokens=T)
    pc = kivi.PagedCache(g, P, 60)
    rng = np.random.default_rng(5)
    # sequence 0 (150 tokens: n_q 0) flushes its group 0 at step 9: page 0
    # missing; sequence 1 (600: n_q 448 = 14 groups): page 3 missing
    table = _assign(pc, [16, 16, 16], rng, skip={0: 0, 1: 3})
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    st_a = kivi.paged_prefill(g, pc, bits_to_dev(_padded(kb, lens, 700)),
                              bits_to_dev(_padded(vb, lens, 700)), seq)
    st_b = torch.empty_like(st_a)
    ws = kivi.Workspace(g)
    og1 = oracle.Geom(1, H, QPK, bits=bits, max_tokens=T)
    oc0 = oracle.prefill(og1, kb[0:1, :, :150].copy(), vb[0:1, :, :150].copy())
    oc2 = oracle.prefill(og1, kb[2:3, :, :400].copy(), vb[2:3, :, :400].copy())
    full_at = None
    for t in range(steps):
        kn = np.stack([kb[b, :, n + t] for b, n in enumerate(lens)])
        vn = np.stack([vb[b, :, n + t] for b, n in enumerate(lens)])
        q = synth.bits_u16(synth.query(w, 808 + t))
        out = kivi.paged_decode_step(g, pc, st_a, st_b, bits_to_dev(kn), bits_to_dev(vn),
                                     bits_to_dev(q), ws=ws, softmax_scale=SCALE)
        st_a, st_b = st_b, st_a
        torch.cuda.synchronize()
        st, o = to_np(st_a), to_np(out)
        assert st[1][3] == kivi.SEQ_BAD_LENGTH and np.all(o[1] == 0)
        oracle.append(oc2, kn[2:3], vn[2:3])
        oracle.flush(oc2)
        assert tuple(st[2]) == (oc2.n_q, oc2.n_res, oc2.res_start, 0)
        assert row_rel_err(o[2], oracle.attention(oc2, q[2:3].copy(), SCALE)[0]) <= ATTN_TOL
        if full_at is None and oc0.n_res + 1 == og1.slots:
            full_at = t          # the flush would need the missing page
        if full_at is None:
            oracle.append(oc0, kn[0:1], vn[0:1])
            oracle.flush(oc0)
            assert tuple(st[0]) == (oc0.n_q, oc0.n_res, oc0.res_start, 0)
        else:
            assert st[0][3] == kivi.SEQ_FULL
            assert tuple(st[0][:3]) == (oc0.n_q, oc0.n_res, oc0.res_start)
        assert row_rel_err(o[0], oracle.attention(oc0, q[0:1].copy(), SCALE)[0]) <= ATTN_TOL
    assert full_at == 9
    assert_same_cache(_gather(pc, 0, table, og1, oc0.n_q, oc0.n_res, oc0.res_start), oc0)


@pytest.mark.parametrize("flags", [0, 1])
def test_paged_steps_in_a_graph_replay_like_eager(flags):
    assert kivi.FLAG_DETERMINISTIC == 1
    B, H, QPK, bits, P = 3, 2, 4, 2, 4
    lens = [155, 412, 1000]   # sequences 0 and 1 flush inside the replays
    reps = 6
    w, kb, vb = _inputs(B, H, QPK, 1000 + 2 * reps + 2, bits, 66)
    T = 32 * ((1000 + 2 * reps + 2) // 32 + 1)
    g = kivi.Geom(B, H, QPK, bits=bits, max_tokens=T, flags=flags)
    NG = T // 32
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    caches, states = [], []
    for i in range(3):   # graph, eager, warm-up
        pc = kivi.PagedCache(g, P, B * ((NG + P - 1) // P))
        _assign(pc, [NG] * B, np.random.default_rng(9))
        st = kivi.paged_prefill(g, pc, bits_to_dev(_padded(kb, lens, 1000)),
                                bits_to_dev(_padded(vb, lens, 1000)), seq)
        caches.append(pc)
        states.append((st, torch.empty_like(st)))
    kn = torch.empty(2, B, H, 128, dtype=torch.bfloat16, device="cuda")
    vn = torch.empty_like(kn)
    q = torch.empty(2, B, H * QPK, 128, dtype=torch.bfloat16, device="cuda")
    outs = [torch.zeros(2, B, H * QPK, 128, device="cuda") for _ in range(3)]
    steppers = [[kivi.RaggedStepper(g, caches[i], kivi.Workspace(g), *states[i], kn[j], vn[j],
                                    q[j], outs[i][j], softmax_scale=SCALE) for j in range(2)]
                for i in range(3)]

    def load(i):
        for j in range(2):
            t = 2 * i + j
            kn[j].copy_(bits_to_dev(np.stack([kb[b, :, n + t] for b, n in enumerate(lens)])))
            vn[j].copy_(bits_to_dev(np.stack([vb[b, :, n + t] for b, n in enumerate(lens)])))
            q[j].copy_(bits_to_dev(synth.bits_u16(synth.query(w, 66 + t))))

    def two_steps(i):
        steppers[i][0].step(0)
        steppers[i][1].step(1)

    load(0)
    two_steps(2)          # warm-up on its own cache
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        two_steps(0)
    for i in range(reps):
        load(i)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        g_res = to_np(outs[0]).copy()
        outs[1].fill_(float("nan"))
        two_steps(1)
        torch.cuda.synchronize()
        if flags:
            assert np.array_equal(g_res.view(np.uint32), to_np(outs[1]).view(np.uint32)), i
        else:
            assert row_rel_err(g_res, to_np(outs[1])) <= REPEAT_TOL, i
        assert np.array_equal(to_np(states[0][0]), to_np(states[1][0])), i
    og1 = oracle.Geom(1, H, QPK, bits=bits, max_tokens=T)
    ta, tb = caches[0].block_table.cpu().numpy(), caches[1].block_table.cpu().numpy()
    for b, row in enumerate(to_np(states[1][0])):
        n_q, n_res, rs = int(row[0]), int(row[1]), int(row[2])
        assert_same_cache(_gather(caches[0], b, ta, og1, n_q, n_res, rs),
                          _gather(caches[1], b, tb, og1, n_q, n_res, rs))
