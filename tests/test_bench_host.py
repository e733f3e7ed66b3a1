"""Host-side arithmetic of bench.py (no GPU).

* Algorithmic bytes: the decode-attention and prefill byte counts that the
  roofline divides by are closed forms of the cache layout (KV bytes basis of
  the catalog record kivi-2bit-llama3-8b-gqa-8k: grouped history of codes
  plus scale/zero, bf16 residual of R tokens); the values below are those
  closed forms evaluated by hand for the measured workloads, at the cache
  state right after prefill (n_q = G * floor((S - R) / G), r = S - n_q).
* Traffic validity: the committed counter figures are tied to the kernel's
  code by a hash that ignores comments; a code change must void them.
"""
import os

import pytest

import bench
import synth


def _w(name):
    return synth.WORKLOADS[name]


@pytest.mark.parametrize("name,n_q,r,expected", [
    # B*H * [n_q*(2*D*b/8 + 16*D/G) + r*4*D] + B*Hq*D*(2+4), fp32 scale/zero
    ("llama3-8b-gqa-8k", 8064, 128, 128 * (8064 * 128 + 128 * 512) + 16 * 32 * 128 * 6),
    ("llama2-7b-mha-4k", 3968, 128, 256 * (3968 * 128 + 128 * 512) + 8 * 32 * 128 * 6),
    ("llama3-8b-gqa-32k-4bit", 32640, 128, 32 * (32640 * 192 + 128 * 512) + 4 * 32 * 128 * 6),
])
def test_attention_bytes_closed_form(name, n_q, r, expected):
    assert bench.attn_bytes(_w(name), n_q, r) == expected


def test_attention_bytes_headline_values():
    # 140.9 MB per layer at 8192 tokens; 147.0 MB for the MHA layer at 4096;
    # 202.7 MB for the 32K 4-bit layer
    assert bench.attn_bytes(_w("llama3-8b-gqa-8k"), 8064, 128) == 140_902_400
    assert bench.attn_bytes(_w("llama2-7b-mha-4k"), 3968, 128) == 146_997_248
    assert bench.attn_bytes(_w("llama3-8b-gqa-32k-4bit"), 32640, 128) == 202_735_616


def test_attention_bytes_terms():
    w = _w("llama3-8b-gqa-8k")
    base = bench.attn_bytes(w, 8064, 128)
    # one more residual token: 4*D bytes (bf16 K and V) per (sequence, kv head)
    assert bench.attn_bytes(w, 8064, 129) - base == 128 * 4 * 128
    # one more group: its codes (2*D*b/8 per token) and fp32 scale/zero (16*D/G per token)
    assert bench.attn_bytes(w, 8096, 128) - base == 128 * 32 * (64 + 64)
    # the fused append's ring write: 4*D per (sequence, kv head)
    assert bench.attn_bytes(w, 8064, 128, fused_append=True) - base == 128 * 512
    # 16-bit scale/zero halve the metadata term
    assert base - bench.attn_bytes(w, 8064, 128, meta_bytes=2) == 128 * 8064 * 32


def test_prefill_bytes_closed_form():
    # B*H * [4*S*D (bf16 K, V in) + n_q*(codes + scale/zero) + 4*r*D (residual copy)]
    w = _w("llama3-8b-gqa-8k")
    assert bench.prefill_bytes(w, 8192, 8064) == 128 * (4 * 8192 * 128 + 8064 * 128 + 4 * 128 * 128)
    assert bench.prefill_bytes(w, 8192, 8064) == 677_380_096


def test_code_hash_ignores_comments_only(tmp_path):
    src = tmp_path / "k.hip"
    src.write_text("int f(int x) {\n  return x + 1;   // add one\n}\n")
    h0 = bench.code_hash(str(src))
    src.write_text("// a new header comment\n\nint f(int x) {\n  return x + 1;   // adds one\n\n}\n")
    assert bench.code_hash(str(src)) == h0
    src.write_text("int f(int x) {\n  return x + 2;   // add one\n}\n")
    assert bench.code_hash(str(src)) != h0


def test_traffic_voided_by_a_code_change(tmp_path, monkeypatch):
    """read_traffic returns the committed figure only while the file's hash
    equals the current code hash of the decode kernel's sources (a change to
    either voids it)."""
    csrc = os.path.join(bench.ROOT, "decode_attention_channel_amd", "csrc")
    root = tmp_path / "repo"
    (root / "profiles").mkdir(parents=True)
    (root / "decode_attention_channel_amd" / "csrc").mkdir(parents=True)
    srcs = [root / "decode_attention_channel_amd" / "csrc" / f for f in bench.DECODE_SOURCES]
    orig = [open(os.path.join(csrc, f)).read() for f in bench.DECODE_SOURCES]
    for p, text in zip(srcs, orig):
        p.write_text(text)
    h = bench.code_hash(*[str(p) for p in srcs])
    prof = root / "profiles" / "k_traffic.txt"
    prof.write_text(f"# comment: 1\nkernel_code_sha256_16: {h}\nhbm_bytes_per_launch: 12345\n")
    monkeypatch.setattr(bench, "ROOT", str(root))
    assert bench.read_traffic("k") == 12345.0
    for p, text in zip(srcs, orig):
        p.write_text(text + "\n// a comment at the end\n")
        assert bench.read_traffic("k") == 12345.0
        p.write_text(text + "\nstatic int unused_marker = 0;\n")
        assert bench.read_traffic("k") is None
        p.write_text(text)
    assert bench.read_traffic("k") == 12345.0


def test_cpu_flush_baseline_runs_the_oracle_flush():
    """The flush timing of cpu_baseline at a small sample: every timed flush
    quantises one group per (sequence, kv head) of the 32K 4-bit geometry."""
    r = bench.cpu_flush_baseline(seed=5, threads=2, layers=2, steps=1)
    assert r["workload"] == "llama3-8b-gqa-32k-4bit" and r["cores"] == 2
    assert r["ms_per_step"] > 0 and r["ms_per_step_1thread"] > 0 and r["gelem_s"] > 0
