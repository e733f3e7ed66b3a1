"""GPU parity of the uncompressed bf16 baseline (kivi_dense_decode_attention)
against the oracle's dense attention: GQA and MHA, ragged lengths that end
inside a 32-token chunk, one token, a length below the capacity (the tail
must not be read: it is filled with Inf/NaN), and sampled checks at the
Llama-2-13B-shaped memory-wall geometry (40 heads, 4096 tokens): batch 8
(more units than compute units: static shares) and batch 2 (one workgroup
per compute unit, each with more 32-token chunks than waves)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from kivi_testutil import ATTN_TOL, row_rel_err, to_np

kivi = pytest.importorskip("decode_attention_channel_amd.kivi")

pytestmark = pytest.mark.gpu

CASES = [
    # B, H, QPK, T, seq_len
    (2, 2, 4, 256, 256),
    (2, 2, 4, 256, 201),
    (1, 3, 1, 512, 509),
    (2, 2, 1, 128, 1),
    (1, 1, 8, 1024, 1000),
    (1, 2, 3, 96, 64),
    (3, 1, 16, 160, 33),
]


def _kv(B, H, T, seed):
    w = synth.Workload("dense", B, H, 1, T, 2, 1, 3, 8.0)
    k, v = synth.prefill_kv(w, seed)
    return synth.bits_u16(k), synth.bits_u16(v)


@pytest.mark.parametrize("B,H,QPK,T,S", CASES)
def test_dense_attention_matches_oracle(B, H, QPK, T, S):
    print(f"dense B={B} H={H} QPK={QPK} T={T} S={S}", flush=True)
    kb, vb = _kv(B, H, T, 500 + S)
    # the tail past seq_len holds +Inf keys and NaN values: never read
    kb[:, :, S:] = 0x7F80
    vb[:, :, S:] = 0x7FC0
    w = synth.Workload("dense", B, H, QPK, T, 2, 1, 3, 8.0)
    qb = synth.bits_u16(synth.query(w, 600 + S))
    g = kivi.Geom(B, H, QPK, max_tokens=T)
    dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    out = torch.full((B, H * QPK, 128), float("nan"), device="cuda")
    kivi.dense_decode_attention(g, dev(kb), dev(vb), S, dev(qb), out=out)
    torch.cuda.synchronize()
    o = to_np(out)
    assert np.isfinite(o).all()
    ref = oracle.attention_dense(oracle.Geom(B, H, QPK), kb, vb, S, qb, 1 / math.sqrt(128))
    err = row_rel_err(o, ref)
    assert err <= ATTN_TOL, f"row-relative error {err:.3e}"


@pytest.mark.parametrize("B", [8, 2])
def test_dense_attention_memory_wall_geometry_sampled(B):
    """40 heads x 4096 tokens; a few (sequence, head) units recomputed by the
    oracle."""
    print(f"dense wall B={B}", flush=True)
    H, T = 40, 4096
    w = synth.WORKLOADS["llama2-13b-mha-wall"]
    k, v = synth.prefill_kv(w, 77, batch=B)
    q = synth.query(w, 77, batch=B)
    g = kivi.Geom(B, H, 1, max_tokens=T)
    out = kivi.dense_decode_attention(g, k.cuda(), v.cuda(), T, q.cuda())
    torch.cuda.synchronize()
    o = to_np(out)
    kb, vb, qb = synth.bits_u16(k), synth.bits_u16(v), synth.bits_u16(q)
    rng = np.random.default_rng(5)
    units = sorted({0, B * H - 1, *map(int, rng.integers(0, B * H, 4))})
    ref = oracle.attention_dense(oracle.Geom(B, H, 1), kb, vb, T, qb, 1 / math.sqrt(128),
                                 units=units)
    rows = [(u // H, u % H) for u in units]
    err = row_rel_err(np.stack([o[b, h] for b, h in rows]), np.stack([ref[b, h] for b, h in rows]))
    assert err <= ATTN_TOL, f"row-relative error {err:.3e}"
