"""kivi_decode_step_noalloc (the decode workspace in the library's static
device array) against kivi_decode_step with a caller workspace, through the
C ABI: two calls in a row, the second on a smaller input, each compared with
kivi_decode_step on identical inputs (cache bytes exact; outputs bitwise
equal for deterministic launches, within REPEAT_TOL otherwise) and with the oracle
(1e-3).  The first call flushes a group, which the attention launch
quantises itself before attending with the fused append."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from kivi_testutil import ATTN_TOL, REPEAT_TOL, row_rel_err, to_np

kivi = pytest.importorskip("decode_attention_channel_amd.kivi")

pytestmark = pytest.mark.gpu

# (batch, kv heads, query heads per kv head, prefill length, bits); the
# first leaves R + G - 1 tokens in the ring (its step flushes), the second is
# smaller in every dimension that sizes the workspace
CALLS = [(4, 8, 4, 4031, 2), (2, 2, 4, 1000, 4)]


def _one_call(B, H, QPK, S, bits, flags, seed):
    w = synth.Workload("noalloc", B, H, QPK, S, bits, 1, 3, 8.0)
    k, v = synth.prefill_kv(w, seed)
    kn, vn = synth.new_token(w, seed, 0, 0)
    q = synth.query(w, seed, 0, 0)
    T = 32 * math.ceil((S - 128 + 64) / 32)
    g = kivi.Geom(B, H, QPK, bits=bits, max_tokens=T, flags=flags)
    ref_c, got_c = kivi.Cache(g), kivi.Cache(g)
    for c in (ref_c, got_c):
        kivi.quantize_prefill(g, c, k.cuda(), v.cuda())
    kn_d, vn_d, q_d = kn.cuda(), vn.cuda(), q.cuda()
    ref_out = torch.full((B, H * QPK, 128), float("nan"), device="cuda")
    got_out = torch.full_like(ref_out, float("nan"))
    _, f_ref = kivi.decode_step(g, ref_c, kn_d, vn_d, q_d, out=ref_out, ws=kivi.Workspace(g))
    f_got = kivi.decode_step_noalloc(g, got_c, kn_d, vn_d, q_d, got_out)
    torch.cuda.synchronize()
    assert f_ref == f_got
    assert (got_c.n_q, got_c.n_res, got_c.res_start) == (ref_c.n_q, ref_c.n_res, ref_c.res_start)
    # the used part of the caches: the history's groups and the ring in
    # logical order (the rest is whatever the allocator left there)
    ng = got_c.n_q // 32
    assert torch.equal(got_c.records[:, :, :ng], ref_c.records[:, :, :ng])
    slots = [(got_c.res_start + i) % g.slots for i in range(got_c.n_res)]
    for a, b in ((got_c.k_res, ref_c.k_res), (got_c.v_res, ref_c.v_res)):
        assert torch.equal(a[:, :, slots], b[:, :, slots])
    go, ro = to_np(got_out), to_np(ref_out)
    assert np.isfinite(go).all()
    if flags & kivi.FLAG_DETERMINISTIC:
        np.testing.assert_array_equal(go, ro)
    else:
        assert row_rel_err(go, ro) <= REPEAT_TOL
    og = oracle.Geom(B, H, QPK, bits=bits, max_tokens=T)
    oc = oracle.prefill(og, synth.bits_u16(k), synth.bits_u16(v))
    oracle.append(oc, synth.bits_u16(kn), synth.bits_u16(vn))
    assert oracle.flush(oc) == f_got
    ref = oracle.attention(oc, synth.bits_u16(q), 1 / math.sqrt(128))
    err = row_rel_err(go, ref)
    assert err <= ATTN_TOL, err
    return f_got


@pytest.mark.parametrize("flags", [0, 1])
def test_noalloc_step_matches_decode_step(flags):
    flushed = []
    for i, (B, H, QPK, S, bits) in enumerate(CALLS):
        print(f"noalloc call {i}: B={B} H={H} QPK={QPK} S={S} bits={bits} flags={flags}",
              flush=True)
        flushed.append(_one_call(B, H, QPK, S, bits, flags, 61 + i))
    assert flushed == [1, 0]


def test_noalloc_rejects_a_step_beyond_the_array():
    # 512 units x 4 heads at 24K tokens need ~100 MB of partials: refused on
    # the host, nothing enqueued, counters unchanged
    g = kivi.Geom(64, 8, 4, max_tokens=32768)
    c = kivi.Cache(g)
    c.set_counters(24576, 140, 0)
    tok = torch.zeros(64, 8, 128, dtype=torch.bfloat16, device="cuda")
    q = torch.zeros(64, 32, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.zeros(64, 32, 128, device="cuda")
    with pytest.raises(kivi.KiviError) as e:
        kivi.decode_step_noalloc(g, c, tok, tok, q, out)
    assert e.value.status == 7
    assert (c.n_q, c.n_res, c.res_start) == (24576, 140, 0)
