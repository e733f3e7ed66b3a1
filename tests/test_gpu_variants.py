"""GPU parity of both launches of the decode kernel against the oracle when
every (sequence, kv head) fits on its own compute unit (one workgroup per
compute unit): by default its waves take groups from an LDS counter; with
KIVI_FLAG_DETERMINISTIC they take them round-robin.  Two shapes: few units at
a long context (many workgroups per unit) and 256 units (one workgroup per
unit, so that its waves claim groups to the end of the unit).  The
round-robin launch must also repeat bitwise.  (The four-wave static launch,
used when the units outnumber the compute units, is covered by the
many-unit cases of test_gpu_parity.py.)"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from kivi_testutil import ATTN_TOL, REPEAT_TOL, bits_to_dev, row_rel_err, to_np

kivi = pytest.importorskip("decode_attention_channel_amd.kivi")

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,H,S", [(2, 2, 8192), (64, 4, 2048)])
@pytest.mark.parametrize("bits,meta", [(2, 0), (4, 0), (2, 1), (4, 1)])
def test_static_and_dynamic_launches_match_the_oracle(B, H, S, bits, meta):
    QPK = 4
    print(f"variants B={B} H={H} S={S} bits={bits} meta={meta}", flush=True)
    w = synth.Workload("var", B, H, QPK, S, bits, 1, 3, 8.0)
    k, v = synth.prefill_kv(w, 70 + bits + meta)
    kb, vb = synth.bits_u16(k), synth.bits_u16(v)
    T = 32 * ((S - 128) // 32)
    oc = oracle.prefill(oracle.Geom(B, H, QPK, bits=bits, max_tokens=T, meta=meta), kb, vb)
    q = synth.bits_u16(synth.query(w, 71))
    scale = 1 / math.sqrt(128)
    ref = oracle.attention(oc, q, scale)
    outs = {}
    for flags in (0, kivi.FLAG_DETERMINISTIC):
        g = kivi.Geom(B, H, QPK, bits=bits, max_tokens=T, meta_format=meta, flags=flags)
        c = kivi.Cache(g)
        kivi.quantize_prefill(g, c, bits_to_dev(kb), bits_to_dev(vb))
        ws = kivi.Workspace(g)
        runs = []
        for _ in range(3):
            out = torch.full((B, H * QPK, 128), float("nan"), device="cuda")
            kivi.decode_attention(g, c, bits_to_dev(q), out=out, softmax_scale=scale, ws=ws)
            torch.cuda.synchronize()
            o = to_np(out)
            assert np.isfinite(o).all()
            err = row_rel_err(o, ref)
            assert err <= ATTN_TOL, f"flags={flags}: {err:.3e}"
            runs.append(o)
        if flags:
            for o in runs[1:]:
                np.testing.assert_array_equal(o, runs[0])
        outs[flags] = runs[0]
    # the variants differ only in how fp32 partial sums are grouped
    assert row_rel_err(outs[0], outs[kivi.FLAG_DETERMINISTIC]) <= REPEAT_TOL
