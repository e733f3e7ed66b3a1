"""GPU parity of every launch variant of the GQA decode kernel at a long
context, against the oracle: the static one (four waves per workgroup,
fixed shares) and the dynamic one (one workgroup per compute unit whose
waves take groups from an LDS counter), each with one workgroup per unit
(so that a workgroup holds 252 groups and the dynamic claims run to the end
of the unit) and with the launcher's own split count.  The library reads
KIVI_DYN and KIVI_WPU at every launch; they only choose how the same work is
distributed."""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from kivi_testutil import ATTN_TOL, bits_to_dev, row_rel_err, to_np

kivi = pytest.importorskip("decode_attention_channel_amd.kivi")

pytestmark = pytest.mark.gpu


@pytest.fixture
def env():
    saved = {k: os.environ.get(k) for k in ("KIVI_DYN", "KIVI_WPU")}
    yield os.environ
    for k, v in saved.items():
        if v is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = v


@pytest.mark.parametrize("bits,meta", [(2, 0), (4, 0), (2, 1), (4, 1)])
def test_static_and_dynamic_launches_match_the_oracle(env, bits, meta):
    B, H, QPK, S = 2, 2, 4, 8192
    print(f"variants bits={bits} meta={meta}", flush=True)
    w = synth.Workload("var", B, H, QPK, S, bits, 1, 3, 8.0)
    k, v = synth.prefill_kv(w, 70 + bits + meta)
    kb, vb = synth.bits_u16(k), synth.bits_u16(v)
    T = 32 * ((S - 128) // 32)
    g = kivi.Geom(B, H, QPK, bits=bits, max_tokens=T, meta_format=meta)
    c = kivi.Cache(g)
    kivi.quantize_prefill(g, c, bits_to_dev(kb), bits_to_dev(vb))
    oc = oracle.prefill(oracle.Geom(B, H, QPK, bits=bits, max_tokens=T, meta=meta), kb, vb)
    q = synth.bits_u16(synth.query(w, 71))
    scale = 1 / math.sqrt(128)
    ref = oracle.attention(oc, q, scale)
    ws = kivi.Workspace(g)
    outs = {}
    for dyn in ("0", "1"):
        for wpu in ("1", None):
            env["KIVI_DYN"] = dyn
            if wpu is None:
                env.pop("KIVI_WPU", None)
            else:
                env["KIVI_WPU"] = wpu
            out = torch.full((B, H * QPK, 128), float("nan"), device="cuda")
            kivi.decode_attention(g, c, bits_to_dev(q), out=out, softmax_scale=scale, ws=ws)
            torch.cuda.synchronize()
            o = to_np(out)
            assert np.isfinite(o).all()
            err = row_rel_err(o, ref)
            assert err <= ATTN_TOL, f"dyn={dyn} wpu={wpu}: {err:.3e}"
            outs[(dyn, wpu)] = o
    # the distributions differ only in how fp32 partial sums are grouped:
    # each is ~1e-5 from the exact result, so two of them are within 1e-4
    base = outs[("0", None)]
    for key, o in outs.items():
        assert row_rel_err(o, base) <= 1e-4, key
