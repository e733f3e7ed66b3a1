"""Pins of the oracle's KV-bytes-per-token arithmetic against the figures the
pages print (tests/golden/kv_bytes_per_token.txt: catalog record
kivi-2bit-llama3-8b-gqa-8k, KV bytes basis and notes; paper card, headline
claims; news article, memory-math paragraph), and of the bytes this layout
stores (scale and zero included) against an explicit count of its buffers."""
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "kv_bytes_per_token.txt")


def _rows():
    for line in open(GOLD):
        line = line.split("#")[0].strip()
        if line:
            p = line.split()
            yield [int(x) for x in p[:7]], p[7], float(p[8])


def test_golden_byte_figures():
    seen = set()
    for (L, H, D, b, G, R, ctx), what, want in _rows():
        bf16, conv, exact, stored, stored16 = oracle.bytes_per_token(L, H, D, b, G, R, ctx)
        grouped = conv - R * bf16 / ctx
        got = {
            "grouped_term": grouped,
            "residual_amortized": conv - grouped,
            "convention_total": conv,
            "bf16_total": bf16,
            "convention_ratio": round(bf16 / conv, 2),
            "exact_total": exact,
            "exact_ratio": round(bf16 / exact, 2),
            "convention_ratio_limit": round(bf16 / conv, 3),
            # half precision, no quantisation: the bf16 column times the tokens
            "fp16_cache_gb_approx": round(bf16 * ctx / 1e9),
        }[what]
        assert got == pytest.approx(want, abs=1e-9), (what, got, want)
        seen.add(what)
    assert len(seen) >= 9


def test_llama2_7b_cache_is_about_a_third_of_its_weights():
    bf16, *_ = oracle.bytes_per_token(32, 32, 128, 2, 32, 128, 10_000)
    cache = bf16 * 10_000
    assert 5.0e9 < cache < 5.5e9
    assert 0.3 < cache / (7e9 * 2) < 0.4


def test_stored_bytes_count_every_buffer():
    # Llama-3-8B geometry at 8192 tokens: n_q = 8064 quantised tokens and a
    # 128-token bf16 residual per layer and kv head.  Count the buffers of the
    # documented layout directly.
    L, H, D, G, R, S = 32, 8, 128, 32, 128, 8192
    for b in (2, 4):
        n_q = oracle.prefill_split(S, G, R)
        k_codes = n_q * D * b / 8
        v_codes = n_q * D * b / 8
        k_meta = (n_q // G) * D * 4 * 2
        v_meta = n_q * (D // G) * 4 * 2
        resid = (S - n_q) * D * 2 * 2
        total = (k_codes + v_codes + k_meta + v_meta + resid) * L * H / S
        assert oracle.bytes_per_token(L, H, D, b, G, R, S)[3] == pytest.approx(total)
    assert oracle.bytes_per_token(L, H, D, 2, G, R, S)[3] == 34304.0


def test_stored_bytes_with_16bit_scale_and_zero():
    """Same count with fp16 scale and bf16 zero: 2 bytes each instead of 4."""
    L, H, D, G, R, S = 32, 8, 128, 32, 128, 8192
    for b in (2, 4):
        n_q = oracle.prefill_split(S, G, R)
        meta = ((n_q // G) * D + n_q * (D // G)) * 2 * 2
        codes = 2 * n_q * D * b / 8
        resid = (S - n_q) * D * 2 * 2
        total = (codes + meta + resid) * L * H / S
        assert oracle.bytes_per_token(L, H, D, b, G, R, S)[4] == pytest.approx(total)
    bf16, _, _, stored, stored16 = oracle.bytes_per_token(L, H, D, 2, G, R, S)
    assert stored16 == 26240.0
    assert round(bf16 / stored16, 2) == 5.0 and round(bf16 / stored, 2) == 3.82
