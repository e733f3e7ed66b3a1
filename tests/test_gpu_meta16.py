"""GPU parity of the 16-bit scale/zero format (fp16 scale, bf16 zero) against
the oracle: byte-exact quantised history (codes, fp16 scale bits, bf16 zero
bits) and decode attention within the tolerance, for GQA and MHA (one query
head per kv head), both bit widths, ragged lengths, streaming with flushes
through the separate calls and through kivi_decode_step, groups whose
scales are fp16 subnormals, and a saturated scale."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from kivi_testutil import ATTN_TOL, assert_same_cache, bits_to_dev, host_cache, row_rel_err, to_np

kivi = pytest.importorskip("decode_attention_channel_amd.kivi")

pytestmark = pytest.mark.gpu

META = 1


def _geoms(B, H, QPK, bits, T):
    return (kivi.Geom(B, H, QPK, bits=bits, max_tokens=T, meta_format=META),
            oracle.Geom(B, H, QPK, bits=bits, max_tokens=T, meta=META))


def _attend(kg, gc, oc, qb):
    scale = 1.0 / math.sqrt(128)
    out = torch.full((kg.batch, kg.q_heads, 128), float("nan"), device="cuda")
    kivi.decode_attention(kg, gc, bits_to_dev(qb), out=out, softmax_scale=scale)
    torch.cuda.synchronize()
    o = to_np(out)
    assert np.isfinite(o).all()
    err = row_rel_err(o, oracle.attention(oc, qb, scale))
    assert err <= ATTN_TOL, f"row-relative error {err:.3e}"


@pytest.mark.parametrize("B,H,QPK,S,bits", [
    (2, 2, 4, 1509, 2), (2, 1, 4, 1509, 4), (1, 2, 3, 500, 2), (2, 2, 1, 1509, 2),
    (2, 2, 1, 700, 4), (1, 1, 8, 293, 2),
])
def test_prefill_and_attention_16bit(B, H, QPK, S, bits):
    print(f"meta16 B={B} H={H} QPK={QPK} S={S} bits={bits}", flush=True)
    w = synth.Workload("m16", B, H, QPK, S, bits, 1, 3, 8.0)
    k, v = synth.prefill_kv(w, 300 + S)
    kb, vb = synth.bits_u16(k), synth.bits_u16(v)
    T = 32 * ((S - 128) // 32 + 1)
    kg, og = _geoms(B, H, QPK, bits, T)
    gc = kivi.Cache(kg)
    assert gc.records.shape[-1] == 1024 * (bits + 1)   # codes plus one 16-bit meta plane
    kivi.quantize_prefill(kg, gc, bits_to_dev(kb), bits_to_dev(vb))
    oc = oracle.prefill(og, kb, vb)
    torch.cuda.synchronize()
    assert_same_cache(host_cache(gc, og), oc)
    _attend(kg, gc, oc, synth.bits_u16(synth.query(w, 300 + S)))


@pytest.mark.parametrize("bits,QPK", [(2, 4), (4, 1)])
def test_streaming_16bit_separate_and_fused(bits, QPK):
    B, H, S0, N = 2, 2, 150, 80
    w = synth.Workload("m16", B, H, QPK, S0 + N, bits, 1, 3, 8.0)
    k, v = synth.prefill_kv(w, 400 + bits)
    kb, vb = synth.bits_u16(k), synth.bits_u16(v)
    T = 32 * ((S0 + N) // 32 + 1)
    kg, og = _geoms(B, H, QPK, bits, T)
    sep, fus = kivi.Cache(kg), kivi.Cache(kg)
    for c in (sep, fus):
        kivi.quantize_prefill(kg, c, bits_to_dev(kb[:, :, :S0].copy()), bits_to_dev(vb[:, :, :S0].copy()))
    oc = oracle.prefill(og, kb[:, :, :S0].copy(), vb[:, :, :S0].copy())
    ws = kivi.Workspace(kg)
    out = torch.empty(B, H * QPK, 128, device="cuda")
    flushes = 0
    for t in range(S0, S0 + N):
        kn, vn = kb[:, :, t].copy(), vb[:, :, t].copy()
        kivi.append_token(kg, sep, bits_to_dev(kn), bits_to_dev(vn))
        kivi.flush_residual(kg, sep)
        q = synth.bits_u16(synth.query(w, 400 + bits, step=t))
        _, f = kivi.decode_step(kg, fus, bits_to_dev(kn), bits_to_dev(vn), bits_to_dev(q), out=out, ws=ws)
        oracle.append(oc, kn, vn)
        assert oracle.flush(oc) == f
        flushes += f
        if f or t % 17 == 0:
            torch.cuda.synchronize()
            err = row_rel_err(to_np(out), oracle.attention(oc, q, 1 / math.sqrt(128)))
            assert err <= ATTN_TOL, f"step {t}: {err:.3e}"
    assert flushes == 3   # at 160 tokens, then every 32: steps 159, 191, 223
    torch.cuda.synchronize()
    assert_same_cache(host_cache(sep, og), oc)
    assert_same_cache(host_cache(fus, og), oc)


def test_fp16_subnormal_and_saturated_scales():
    """Tiny groups (fp16-subnormal scales, including ones that round to zero)
    and a group whose range saturates the fp16 scale: byte-exact."""
    B, H, S = 1, 2, 160 + 128
    rng = np.random.default_rng(17)
    x = rng.standard_normal((2, B, H, S, 128)).astype(np.float32)
    x[:, :, 0, 0:32] *= 1e-6          # group 0 of unit 0: subnormal scales
    x[:, :, 0, 32:64] *= 1e-9         # scales that round to zero in fp16
    x[0, :, 1, 64:96, 7] *= 1e5       # a key channel with a saturated scale
    x[1, :, 1, 70, :] *= 1e5          # a value token with saturated scales
    b = (x.view(np.uint32) >> 16).astype(np.uint16)
    kb, vb = b[0].copy(), b[1].copy()
    kg, og = _geoms(B, H, 4, 2, 192)
    gc = kivi.Cache(kg)
    kivi.quantize_prefill(kg, gc, bits_to_dev(kb), bits_to_dev(vb))
    oc = oracle.prefill(og, kb, vb)
    torch.cuda.synchronize()
    hc = host_cache(gc, og)
    assert_same_cache(hc, oc)
    assert (oc.k_scale[0, 1, 2, 7] == 0x7BFF)
    assert 0 < oc.k_scale[0, 0, 0, 0] < 0x0400   # an fp16 subnormal
