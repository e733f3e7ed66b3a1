"""Benchmark: KIVI decode step on one MI355X.

Workload (Llama-3-8B GQA geometry of the catalog record kivi-2bit-llama3-8b-gqa-8k:
32 layers, 8 kv heads, 32 query heads, head_dim 128, 8K context), batch 16,
2-bit, G = 32, R = 128, seeded synthetic K/V/q with outlier key channels.

* prefill leg: every layer's 8192-token K/V is quantised into its own cache
  (all layers' inputs generated first, then the prefills run back to back,
  each timed with a HIP event pair; reported as quantise Gelem/s and HBM
  GB/s);
* decode leg (the timed "step"): for each of the 32 layers, one
  kivi_decode_step call -- append one token per sequence, flush a group when
  the residual is full, and decode attention over the whole mixed cache, in
  one launch (a due flush is quantised inside it).  value = tokens/s (batch / step
  time).  The same number of steps is then timed with the three separate
  calls (append, flush, attend) for comparison.  The 32 layer caches (4.5 GB)
  rotate, so the 256 MB MALL cannot serve them;
* roofline of the dominant kernel (decode attention with the fused append,
  one launch per layer): algorithmic bytes per launch / its duration, from
  one HIP event pair around a block of 10 further flush-free decode steps
  (320 back-to-back launches), against 8 TB/s;
* mixed-length leg (reported beside, not in, value): per-sequence counters
  in device memory -- paged copies of the caches (pages of 4 groups from a
  shuffled pool) through kivi_paged_decode_step at the lockstep length, then
  the caches themselves through kivi_ragged_decode_step at the lockstep
  length and with lengths drawn uniformly from [S/2, S]; eager launches and
  HIP graph replays of all layers (one launch per layer) are timed;
* flush-amortised rate: a further window of 32 fused steps, in which every
  layer flushes exactly once (value's window of `steps` steps holds
  floor or ceil of steps/32 flushes);
* copy bandwidth: a plain 1 GiB device-to-device copy (torch copy_), timed
  with HIP events; the decode kernel's rate is also reported as a fraction of
  it;
* --deterministic times the same legs with KIVI_FLAG_DETERMINISTIC (the
  bitwise-repeatable launch); its line carries no traffic figure, which was
  counted for the default launch;
* cpu_baseline: the CPU oracle (plain C) on a bounded sample of the same
  workload (eight layers' worth of (sequence, kv head) units), threads over
  units, plus a single-thread rate on a smaller sample, and one residual
  flush per layer at the 32K 4-bit geometry (4 sequences x 8 kv heads).

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import concurrent.futures
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "KIVI decode-attention achieved HBM GB/s + tokens/sec; quantize Gelem/s"


def attn_bytes(w, n_q, n_res, fused_append=False, meta_bytes=4):
    """Algorithmic bytes of one decode-attention launch: the packed history
    (codes + scale/zero of meta_bytes each), the bf16 residual (the appended
    token included, read from its input in a fused step), q (bf16) and out
    (fp32); a fused step also writes the appended K and V rows into the ring."""
    D, G, b = w.head_dim, w.group, w.bits
    per_unit = (n_q * (2 * D * b / 8 + 4 * meta_bytes * D / G) + n_res * 4 * D +
                (4 * D if fused_append else 0))
    return w.batch * w.kv_heads * per_unit + w.batch * w.q_heads * D * (2 + 4)


def prefill_bytes(w, S, n_q, meta_bytes=4):
    D, G, b = w.head_dim, w.group, w.bits
    r = S - n_q
    return w.batch * w.kv_heads * (4 * S * D + n_q * (2 * D * b / 8 + 4 * meta_bytes * D / G) +
                                   4 * r * D)


def code_hash(*paths: str) -> str:
    """sha256 prefix of source files' code, in order: '//' comments, trailing
    blanks and empty lines removed, so that editing a comment keeps the hash."""
    import hashlib
    import re
    lines = []
    for path in paths:
        for line in open(path).read().splitlines():
            line = re.sub(r"//.*$", "", line).rstrip()
            if line:
                lines.append(line)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


# the sources of the decode kernel's device code (it folds the per-wave group
# quantiser in for flushes)
DECODE_SOURCES = ("decode_attn.hip", "quantize_group.h")


def read_traffic(kernel_tag: str):
    """HBM traffic per launch measured with rocprofv3 counters (committed
    summary), valid only while the kernel's code is unchanged."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_traffic.txt")
    srcs = [os.path.join(ROOT, "decode_attention_channel_amd", "csrc", f) for f in DECODE_SOURCES]
    if not os.path.exists(path) or not all(os.path.exists(f) for f in srcs):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            vals[key.strip()] = val.strip()
    if vals.get("kernel_code_sha256_16") != code_hash(*srcs):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_bandwidth(nbytes=1 << 30, reps=10):
    """GB/s of a plain device-to-device copy (bytes read + bytes written per
    second), HIP events around `reps` back-to-back copies."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / t / 1e9


def cpu_baseline(w, seed, units_wanted=1024, meta=0, units_1thread=64):
    import numpy as np

    import oracle
    import synth
    # the machine's CPU share for one GPU is 16 threads, whatever the host has
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    og = oracle.Geom(1, 1, w.q_per_kv, bits=w.bits, max_tokens=w.seq_len, meta=meta)
    per_layer = w.batch * w.kv_heads
    jobs = []
    for layer in range(math.ceil(units_wanted / per_layer)):
        for bi in range(w.batch):
            if len(jobs) >= units_wanted:
                break
            jobs.append((layer, bi))
    # inputs: one sequence (all kv heads) at a time, same recipe as the GPU run
    inputs = {}
    for layer, bi in jobs:
        k, v = synth.prefill_kv(w, seed + 7919 + 131 * bi, layer, batch=1)
        q = synth.query(w, seed + 7919 + 131 * bi, layer, batch=1)
        inputs[(layer, bi)] = (synth.bits_u16(k), synth.bits_u16(v), synth.bits_u16(q))
    units = [(key, h) for key in inputs for h in range(w.kv_heads)][:units_wanted]
    scale = 1.0 / math.sqrt(w.head_dim)

    def prefill_one(item):
        key, h = item
        kb, vb, _ = inputs[key]
        return oracle.prefill(og, kb[:, h:h + 1].copy(), vb[:, h:h + 1].copy())

    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        t0 = time.perf_counter()
        caches = list(ex.map(prefill_one, units))
        t_prefill = time.perf_counter() - t0

        def attend_one(i):
            (key, h), c = units[i], caches[i]
            q = inputs[key][2][:, h * w.q_per_kv:(h + 1) * w.q_per_kv].copy()
            return oracle.attention(c, q, scale)

        t0 = time.perf_counter()
        outs = list(ex.map(attend_one, range(len(units))))
        t_attn = time.perf_counter() - t0
    # one thread, on the first units_1thread units
    n1 = min(units_1thread, len(units))
    t0 = time.perf_counter()
    for i in range(n1):
        attend_one(i)
    t_attn1 = time.perf_counter() - t0
    assert all(np.isfinite(o).all() for o in outs)
    n = len(units)
    n_q = caches[0].n_q
    units_per_step = w.layers * w.batch * w.kv_heads
    step_s = t_attn / n * units_per_step
    step_s1 = t_attn1 / n1 * units_per_step
    return {
        "value": w.batch / step_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
        "sample": (f"{n} (sequence, kv head) units at {w.seq_len} tokens ({n / per_layer:.0f} "
                   f"layers' worth): oracle prefill + one decode-attention step per unit; "
                   f"decode time scaled to {units_per_step} units per 32-layer step"),
        "value_1thread": w.batch / step_s1,
        "sample_1thread": f"decode attention of {n1} of those units on one thread",
        "nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
        "cpu_model": _cpu_model(),
        "quantize_gelem_s": 2 * n * n_q * w.head_dim / t_prefill / 1e9,
        "attn_wall_s": t_attn, "prefill_wall_s": t_prefill, "attn_wall_s_1thread": t_attn1,
        "flush": cpu_flush_baseline(seed, threads, meta),
    }


def cpu_flush_baseline(seed, threads, meta=0, name="llama3-8b-gqa-32k-4bit", layers=32,
                       steps=4):
    """Oracle residual flush timed at the 32K 4-bit workload, one flush per
    layer per decode step: a flush quantises the oldest G ring tokens of every
    (sequence, kv head) unit into a new group, and its cost does not depend on
    the history length, so each layer's cache is built from a prefill of
    R+G-1 tokens and one appended token (n_res = R+G).  `steps` steps' worth
    of layer caches are flushed threaded over layers, one step's worth on one
    thread, after one untimed flush."""
    import oracle
    import synth
    w = synth.WORKLOADS[name]
    og = oracle.Geom(w.batch, w.kv_heads, w.q_per_kv, bits=w.bits, max_tokens=192, meta=meta)
    S = og.residual + og.group - 1

    def ready(layer):
        k, v = synth.prefill_kv(w, seed + 4099, layer, seq_len=S)
        c = oracle.prefill(og, synth.bits_u16(k), synth.bits_u16(v))
        kn, vn = synth.new_token(w, seed + 4099, layer, 0)
        oracle.append(c, synth.bits_u16(kn), synth.bits_u16(vn))
        return c

    base = [ready(layer) for layer in range(layers)]
    oracle.flush(base[0].copy())
    caches = [base[i % layers].copy() for i in range(steps * layers)]
    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        t0 = time.perf_counter()
        flushed = list(ex.map(oracle.flush, caches))
        t_thr = (time.perf_counter() - t0) / steps
    t0 = time.perf_counter()
    flushed += [oracle.flush(c) for c in base]
    t_one = time.perf_counter() - t0
    assert all(f == 1 for f in flushed) and all(c.n_q == og.group for c in caches + base)
    elems = 2 * layers * w.batch * w.kv_heads * og.group * w.head_dim
    return {
        "workload": name, "cores": threads,
        "ms_per_step": t_thr * 1e3, "ms_per_step_1thread": t_one * 1e3,
        "gelem_s": elems / t_thr / 1e9,
        "sample": (f"one flush in each of {layers} layers ({w.batch} sequences x {w.kv_heads} "
                   f"kv heads, {og.group} tokens of K and V each) per step, {steps} steps "
                   f"threaded over layers, one step on one thread"),
    }


def _fill_random_cache(cache, n_q, n_res, gen):
    """Seeded synthetic cache contents for timing: uniform codes, positive
    scales, normal zeros and residual, placed in the record planes."""
    import torch

    from decode_attention_channel_amd import kivi

    g = cache.geom
    rec = cache.records.view(-1, kivi.record_bytes(g) // 1024, 1024)
    rec[:, :g.bits].random_(0, 256, generator=gen)
    meta = rec[:, g.bits:].contiguous()
    if g.meta_format == kivi.META_FP16_BF16:   # per lane: ks, kz, vs, vz pairs
        m = meta.view(torch.int16).view(-1, 64, 4, 2)
        sc = torch.empty(m[:, :, 0::2].shape, device=m.device).uniform_(0.01, 0.5, generator=gen)
        zr = torch.empty(m[:, :, 1::2].shape, device=m.device).normal_(generator=gen)
        m[:, :, 0::2] = sc.to(torch.float16).view(torch.int16)
        m[:, :, 1::2] = zr.to(torch.bfloat16).view(torch.int16)
    else:                                      # per lane: scale pair, zero pair
        m = meta.view(torch.float32).view(-1, 64, 2, 2)
        m[:, :, 0].uniform_(0.01, 0.5, generator=gen)
        m[:, :, 1].normal_(generator=gen)
    rec[:, g.bits:] = meta
    for t in (cache.k_res, cache.v_res):
        t.normal_(generator=gen)
    cache.set_counters(n_q, n_res, 0)


def _time_launches(fns, reps):
    """Mean duration of each launch from HIP event pairs, the GPU kept busy
    ahead of the timed launches."""
    import torch
    for f in fns:
        f()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps * len(fns))]
    for f in fns[:2]:
        f()
    for i, (e0, e1) in enumerate(ev):
        e0.record()
        fns[i % len(fns)]()
        e1.record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / len(ev) / 1e3


def batch_sweep(args):
    """Memory-wall sweep (Llama-2-13B-shaped MHA: 40 layers x 40 heads, 4096
    tokens): decode-attention time per layer vs batch for the 2-bit KIVI cache
    and for the uncompressed bf16 baseline, each up to the largest batch whose
    40-layer cache fits in free HBM.  Every batch allocates all 40 layer caches
    (so the largest one shows that it fits) and times launches rotating over
    them."""
    import torch

    import synth
    from decode_attention_channel_amd import kivi

    w = synth.WORKLOADS[args.workload if args.workload != "llama3-8b-gqa-8k"
                        else "llama2-13b-mha-wall"]
    dev = torch.device("cuda", 0)
    D, G, R, S, L = w.head_dim, w.group, w.residual, w.seq_len, w.layers
    n_q = G * ((S - R) // G)
    n_res = S - n_q
    T = n_q   # the quantised history holds exactly the prefill's groups
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)

    def kivi_geom(B):
        return kivi.Geom(B, w.kv_heads, w.q_per_kv, bits=w.bits, max_tokens=T)

    def dense_geom(B):
        return kivi.Geom(B, w.kv_heads, w.q_per_kv, bits=w.bits, max_tokens=S)

    per_seq_kivi = sum(kivi.cache_layout(kivi_geom(1))) * L
    per_seq_bf16 = w.kv_heads * S * D * 2 * 2 * L
    torch.zeros(1, device=dev).add_(1)   # runtime and context set up before measuring
    torch.cuda.synchronize()
    free0, total = torch.cuda.mem_get_info()
    headroom = 8 << 30   # workspace, q/out, allocator slack
    bmax_kivi = int((free0 - headroom) // per_seq_kivi)
    bmax_bf16 = int((free0 - headroom) // per_seq_bf16)

    def batches(bmax):
        out, b = [], 1
        while b < bmax:
            out.append(b)
            b *= 2
        return out + [bmax]

    rows = {}
    for B in batches(bmax_kivi):
        g = kivi_geom(B)
        n_layers = L
        caches = [kivi.Cache(g, dev) for _ in range(n_layers)]
        for c in caches:
            _fill_random_cache(c, n_q, n_res, gen)
        ws = kivi.Workspace(g, dev)
        q = torch.randn(B, w.q_heads, D, device=dev, generator=gen).to(torch.bfloat16)
        out = torch.empty(B, w.q_heads, D, device=dev)
        st = [kivi.LayerStepper(g, c, ws, q, out) for c in caches]
        t = _time_launches([x.attend for x in st], max(2, 40 // n_layers))
        byt = attn_bytes(synth.Workload(w.name, B, w.kv_heads, w.q_per_kv, S, w.bits, L, 3, 8.0),
                         n_q, n_res)
        rows.setdefault(B, {})["kivi"] = {"us_per_layer": t * 1e6, "tokens_s": B / (t * L),
                                          "hbm_gbps": byt / t / 1e9, "layers_resident": n_layers}
        print(f"batch sweep: KIVI batch {B}: {t * 1e6:.1f} us per layer", file=sys.stderr, flush=True)
        del st, caches, ws, q, out
        torch.cuda.empty_cache()
    for B in batches(bmax_bf16):
        g = dense_geom(B)
        n_layers = L
        kv = []
        for _ in range(n_layers):
            k = torch.empty(B, w.kv_heads, S, D, dtype=torch.bfloat16, device=dev)
            v = torch.empty_like(k)
            k.normal_(generator=gen)
            v.normal_(generator=gen)
            kv.append((k, v))
        ws = kivi.Workspace(g, dev, n_q=0, n_res=S)
        q = torch.randn(B, w.q_heads, D, device=dev, generator=gen).to(torch.bfloat16)
        out = torch.empty(B, w.q_heads, D, device=dev)
        fns = [lambda k=k, v=v: kivi.dense_decode_attention(g, k, v, S, q, out=out, ws=ws)
               for k, v in kv]
        t = _time_launches(fns, max(2, 40 // n_layers))
        byt = B * w.kv_heads * S * D * 4 + B * w.q_heads * D * 6
        rows.setdefault(B, {})["bf16"] = {"us_per_layer": t * 1e6, "tokens_s": B / (t * L),
                                          "hbm_gbps": byt / t / 1e9, "layers_resident": n_layers}
        print(f"batch sweep: bf16 batch {B}: {t * 1e6:.1f} us per layer", file=sys.stderr, flush=True)
        del fns, kv, ws, q, out
        torch.cuda.empty_cache()
    best_kivi = max(r["kivi"]["tokens_s"] for r in rows.values() if "kivi" in r)
    best_bf16 = max(r["bf16"]["tokens_s"] for r in rows.values() if "bf16" in r)
    res = {
        "metric": "decode-attention tokens/s vs batch at the memory wall", "unit": "tokens/s",
        "workload": w.name, "layers": L, "kv_heads": w.kv_heads, "context": S, "bits": w.bits,
        "hbm_free_bytes": free0, "hbm_total_bytes": total,
        "bytes_per_sequence": {"kivi": per_seq_kivi, "bf16": per_seq_bf16},
        "max_batch": {"kivi": bmax_kivi, "bf16": bmax_bf16,
                      "ratio": bmax_kivi / max(bmax_bf16, 1)},
        "best_tokens_s": {"kivi": best_kivi, "bf16": best_bf16, "ratio": best_kivi / best_bf16},
        "rows": [{"batch": B, **rows[B]} for B in sorted(rows)],
        "data": "synthetic (seeded random cache contents; timing only)",
        "paper_context": "up to 4x batch and 2.35x-3.47x throughput vs FP16 (Llama-2-7B, one "
                         "A100 80GB, whole model; not comparable, quoted as context)",
    }
    print(json.dumps(res))


def _advance(counters, steps, slots, group):
    """Per-sequence (n_q, n_res) after `steps` mixed-length steps (a flush
    when the ring would fill, then the append)."""
    out = [list(x) for x in counters]
    for _ in range(steps):
        for x in out:
            if x[1] + 1 == slots:
                x[0] += group
                x[1] -= group
            x[1] += 1
    return out


def _ragged_bytes(w, counters, steps, slots, meta_bytes):
    """Algorithmic attention bytes of `steps` mixed-length steps from the
    given per-sequence (n_q, n_res) counters (each step attends over the
    cache after its flush and append, and writes the appended rows)."""
    D, G, b = w.head_dim, w.group, w.bits
    total = 0.0
    for i in range(steps):
        for n_q, n_res in _advance(counters, i + 1, slots, G):
            total += w.kv_heads * (n_q * (2 * D * b / 8 + 4 * meta_bytes * D / G) +
                                   n_res * 4 * D + 4 * D)
        total += w.batch * w.q_heads * D * (2 + 4)
    return total


RAGGED_EXTRA_STEPS = 4   # untimed steps per case: two eager, two graph replays


PAGE_GROUPS = 4   # groups per page of the paged case (128 tokens)


def _paged_copy(geom, cache, page_groups, rng):
    """A kivi.PagedCache holding the same quantised history and rings as a
    lockstep cache, its pages drawn from a shuffled pool."""
    import numpy as np
    import torch

    from decode_attention_channel_amd import kivi

    B, H, G, T = geom.batch, geom.kv_heads, geom.group, geom.max_tokens
    NG = T // G
    per_seq = -(-NG // page_groups)
    pc = kivi.PagedCache(geom, page_groups, B * per_seq)
    table = rng.permutation(B * per_seq).astype(np.int32).reshape(B, per_seq)
    pc.block_table.copy_(torch.from_numpy(table))
    tb = pc.block_table.long()
    g = torch.arange(NG, device=tb.device)
    h = torch.arange(H, device=tb.device)
    slot = ((tb[:, g // page_groups][:, None, :] * H + h[None, :, None]) * page_groups +
            (g % page_groups)[None, None, :]).reshape(-1)
    pc.records[slot] = cache.records.reshape(B * H * NG, -1)   # the group records
    pc.k_res.copy_(cache.k_res)
    pc.v_res.copy_(cache.v_res)
    return pc


def ragged_leg(w, geom, caches, ws, qs, outs, tok, steps, seed, meta_bytes):
    """Mixed-length decode steps (per-sequence counters in device memory):
    first on paged copies of the caches (kivi_paged_decode_step, pages of
    PAGE_GROUPS groups from a shuffled pool) at the lockstep length, then
    (kivi_ragged_decode_step) on the caches themselves at the lockstep
    length and with lengths drawn uniformly from [S/2, S] per sequence (the
    cache bytes beyond a sequence's length are not read).  Each case is timed
    as eager launches and as HIP graph replays (one graph per state parity,
    all layers, one launch per layer).  `steps` is even."""
    import numpy as np
    import torch

    from decode_attention_channel_amd import kivi

    assert steps % 2 == 0
    dev = caches[0].records.device
    G, R = w.group, w.residual
    slots = R + G
    layers = len(caches)
    rng = np.random.default_rng(seed)
    lens = rng.integers(w.seq_len // 2, w.seq_len + 1, size=w.batch)
    mixed = []
    for L in lens:
        n_q = G * ((int(L) - R) // G)
        mixed.append((n_q, int(L) - n_q))
    c0 = caches[0]
    uniform = [(c0.n_q, c0.n_res)] * w.batch
    cases = {"paged_uniform": uniform, "uniform": uniform, "mixed": mixed}
    res = {"lengths_mixed": "uniform integers in [%d, %d] per sequence, numpy default_rng(%d); "
                            "min %d, mean %.0f, max %d" % (w.seq_len // 2, w.seq_len, seed,
                                                          lens.min(), lens.mean(), lens.max())}
    for name, counters in cases.items():
        # the uniform cases continue the lockstep caches' rings; the mixed
        # case starts its rings at slot 0 (the ring contents are valid bf16)
        rs = 0 if name == "mixed" else c0.res_start
        store = caches
        if name == "paged_uniform":
            prng = np.random.default_rng(seed + 1)
            store = [_paged_copy(geom, c, PAGE_GROUPS, prng) for c in caches]
            torch.cuda.synchronize()
        st_rows = torch.tensor([(n_q, n_res, rs, 0) for n_q, n_res in counters],
                               dtype=torch.int32)
        states, steppers = [], []
        for layer in range(layers):
            a = st_rows.to(dev)
            b = torch.empty_like(a)
            states.append((a, b))
            kn, vn = tok[layer]
            steppers.append(kivi.RaggedStepper(geom, store[layer], ws, a, b, kn, vn, qs[layer],
                                               outs[layer]))

        def eager(parity):
            for sp in steppers:
                sp.step(parity)

        eager(0)
        eager(1)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            eager(i & 1)
        torch.cuda.synchronize()
        t_eager = (time.perf_counter() - t0) / steps
        # one graph per parity; capturing enqueues nothing, so the replays
        # continue from the state the eager steps left (parity 0 next)
        graphs = []
        for parity in (0, 1):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                eager(parity)
            graphs.append(g)
        graphs[0].replay()
        graphs[1].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            graphs[i & 1].replay()
        torch.cuda.synchronize()
        t_graph = (time.perf_counter() - t0) / steps
        # the device counters must be where the host model says
        done = _advance(counters, 2 * steps + RAGGED_EXTRA_STEPS, slots, G)
        for layer in (0, layers - 1):
            got = [list(r[:2]) for r in states[layer][0].cpu().tolist()]
            if got != done:
                raise RuntimeError(f"mixed-length state of layer {layer} off the host model")
        start = _advance(counters, steps + RAGGED_EXTRA_STEPS, slots, G)
        gbytes = _ragged_bytes(w, start, steps, slots, meta_bytes) * layers / steps
        res[name] = {"ms_per_step_eager": t_eager * 1e3, "ms_per_step_graph": t_graph * 1e3,
                     "tokens_s_eager": w.batch / t_eager, "tokens_s_graph": w.batch / t_graph,
                     "attn_bytes_per_step": gbytes,
                     "step_hbm_gbps_graph": gbytes / t_graph / 1e9}
        if name == "paged_uniform":
            res[name]["page_groups"] = PAGE_GROUPS
        del graphs, steppers, states, store
    return res


OTHER_WORKLOADS = ("llama2-7b-mha-4k", "llama3-8b-gqa-32k-4bit")


def other_workload(name, seed, steps=20, warmup=3):
    """Whole decode steps of another workload at its full size (all layers),
    measured like the headline's timed steps: per layer one kivi_decode_step
    (append, flush when the ring is full, decode attention), `steps` steps
    between two synchronisations, after `warmup` untimed ones."""
    import torch

    import synth
    from decode_attention_channel_amd import kivi

    w = synth.WORKLOADS[name]
    dev = torch.device("cuda", 0)
    G, R, layers = w.group, w.residual, w.layers
    total = warmup + steps
    geom = kivi.Geom(w.batch, w.kv_heads, w.q_per_kv, bits=w.bits,
                     max_tokens=G * math.ceil((w.seq_len - R + total + G) / G))
    caches, qs, outs = [], [], []
    for layer in range(layers):       # one layer's bf16 K/V at a time
        k, v = synth.prefill_kv(w, seed, layer, device=dev)
        c = kivi.Cache(geom, dev)
        kivi.quantize_prefill(geom, c, k, v)
        caches.append(c)
        del k, v
        qs.append(synth.query(w, seed, layer, device=dev))
        outs.append(torch.empty(w.batch, w.q_heads, w.head_dim, dtype=torch.float32, device=dev))
    ws = kivi.Workspace(geom, dev)
    steppers = [kivi.LayerStepper(geom, caches[layer], ws, qs[layer], outs[layer])
                for layer in range(layers)]
    new_tok = [[synth.new_token(w, seed, layer, i, device=dev) for layer in range(layers)]
               for i in range(total)]
    n_q0, n_res0 = caches[0].n_q, caches[0].n_res
    for i in range(warmup):
        for layer in range(layers):
            steppers[layer].step(*new_tok[i][layer])
    torch.cuda.synchronize()
    nq_w, nres_w = caches[0].n_q, caches[0].n_res
    t0 = time.perf_counter()
    for i in range(warmup, total):
        for layer in range(layers):
            steppers[layer].step(*new_tok[i][layer])
    torch.cuda.synchronize()
    t = time.perf_counter() - t0
    # attention bytes of the timed steps: the cache grows by one token a step
    # (a flush only moves G tokens from the residual into the history)
    nbytes = 0.0
    nq, nres = nq_w, nres_w
    for _ in range(steps):
        if nres + 1 >= R + G:
            nq, nres = nq + G, nres - G
        nres += 1
        nbytes += attn_bytes(w, nq, nres, fused_append=True) * layers
    res = {"workload": name, "batch": w.batch, "kv_heads": w.kv_heads, "q_heads": w.q_heads,
           "context": w.seq_len, "bits": w.bits, "layers": layers, "scale_zero": "fp32",
           "steps": steps, "warmup": warmup, "ms_per_step": t / steps * 1e3,
           "tokens_s": w.batch * steps / t, "step_attn_hbm_gbps": nbytes / t / 1e9,
           "flushes_in_timed_steps": (caches[0].n_q - nq_w) // G}
    del steppers, caches, ws
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama3-8b-gqa-8k")
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--seed", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="run only N decode steps after warmup, no reporting (profilers)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (scales HBM byte counters)")
    ap.add_argument("--meta", choices=("fp32", "fp16"), default="fp32",
                    help="scale/zero format: fp32 scale + zero (default), or fp16 scale + "
                         "bf16 zero")
    ap.add_argument("--deterministic", action="store_true",
                    help="time the bitwise-repeatable launch (KIVI_FLAG_DETERMINISTIC)")
    ap.add_argument("--no-other", action="store_true",
                    help="skip the whole-step measurement of the other workloads")
    ap.add_argument("--no-ragged", action="store_true",
                    help="skip the mixed-length (per-sequence state) step timing")
    ap.add_argument("--batch-sweep", action="store_true",
                    help="memory-wall sweep: KIVI 2-bit vs bf16 decode attention vs batch "
                         "(Llama-2-13B-shaped MHA); prints its own JSON line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the library "
              "runs on one GPU, and sharding across GPUs is described, not built",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    from decode_attention_channel_amd import kivi

    torch.cuda.set_device(0)
    if args.batch_sweep:
        batch_sweep(args)
        return
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4,
                          "launches": 5}))
        return
    w = synth.WORKLOADS[args.workload]
    layers = args.layers or w.layers
    dev = torch.device("cuda", 0)
    D, G, R = w.head_dim, w.group, w.residual
    kernel_steps = 10   # flush-free fused steps timed as one block
    amort_steps = G     # a window in which every layer flushes exactly once
    ragged_steps = args.steps + (args.steps & 1)
    # timed steps (fused, then separate calls), the flush-amortised window, then
    # up to R+G steps to a flush-free block, a lead-in and the block
    total_steps = args.warmup + (args.profile_steps or
                                 2 * args.steps + amort_steps + R + G + kernel_steps + 1)
    # the mixed-length leg continues the caches for 2 * (2 * steps + 4) more tokens
    cap_steps = total_steps + 2 * (2 * ragged_steps + RAGGED_EXTRA_STEPS)
    max_tokens = G * math.ceil((w.seq_len - R + cap_steps + G) / G)
    meta = kivi.META_FP16_BF16 if args.meta == "fp16" else kivi.META_FP32
    geom = kivi.Geom(w.batch, w.kv_heads, w.q_per_kv, bits=w.bits, max_tokens=max_tokens,
                     meta_format=meta,
                     flags=kivi.FLAG_DETERMINISTIC if args.deterministic else 0)
    default_launch = args.meta == "fp32" and not args.deterministic

    caches = [kivi.Cache(geom, dev) for _ in range(layers)]
    ws = kivi.Workspace(geom, dev)
    # ---- prefill leg: every layer's K/V generated first (17 GB at the 8K GQA
    # workload), then quantised layer by layer in generation order with a HIP
    # event pair around each prefill; a layer's 537 MB of input was written 31
    # layers earlier, so none of it sits in the 256 MB MALL when it is read
    kv = [synth.prefill_kv(w, args.seed, layer, device=dev) for layer in range(layers)]
    torch.cuda.synchronize()
    pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(layers)]
    # untimed lead-in (the last layer, whose input is the most recently
    # written anyway) keeps the GPU busy while the timed launches are queued
    kivi.quantize_prefill(geom, caches[layers - 1], *kv[layers - 1])
    for layer in range(layers):
        e0, e1 = pev[layer]
        e0.record()
        kivi.quantize_prefill(geom, caches[layer], *kv[layer])
        e1.record()
    torch.cuda.synchronize()
    pre_ms = [a.elapsed_time(b) for a, b in pev]
    n_q0 = caches[0].n_q
    del kv
    torch.cuda.empty_cache()
    pre_t = sum(pre_ms) / 1e3
    quant_gelem_s = 2 * w.batch * w.kv_heads * n_q0 * D * layers / pre_t / 1e9
    mbytes = 2 if meta == kivi.META_FP16_BF16 else 4
    pre_gbps = prefill_bytes(w, w.seq_len, n_q0, mbytes) * layers / pre_t / 1e9

    # ---- decode inputs (resident before timing)
    qs = [synth.query(w, args.seed, layer, device=dev) for layer in range(layers)]
    outs = [torch.empty(w.batch, w.q_heads, D, dtype=torch.float32, device=dev)
            for _ in range(layers)]
    new_tok = [[synth.new_token(w, args.seed, layer, step, device=dev) for layer in range(layers)]
               for step in range(total_steps)]
    steppers = [kivi.LayerStepper(geom, caches[layer], ws, qs[layer], outs[layer])
                for layer in range(layers)]

    def step(i):
        for layer in range(layers):
            kn, vn = new_tok[i][layer]
            steppers[layer].step(kn, vn)

    def step_separate(i):
        for layer in range(layers):
            st = steppers[layer]
            kn, vn = new_tok[i][layer]
            st.append(kn, vn)
            st.flush()
            st.attend()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if args.profile_steps:
        for i in range(args.warmup, total_steps):
            step(i)
        torch.cuda.synchronize()
        print(json.dumps({"profile_steps": args.profile_steps}))
        return

    # step timing: exactly `steps` decode steps of all layers
    n_timed = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, args.warmup + n_timed):
        step(i)
    torch.cuda.synchronize()
    t_steps = time.perf_counter() - t0
    # the same number of steps through the three separate calls
    t0 = time.perf_counter()
    for i in range(args.warmup + n_timed, args.warmup + 2 * n_timed):
        step_separate(i)
    torch.cuda.synchronize()
    t_steps_sep = time.perf_counter() - t0
    # flush-amortised: G consecutive fused steps hold exactly one flush per layer
    i0 = args.warmup + 2 * n_timed
    nq_before = caches[0].n_q
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(i0, i0 + amort_steps):
        step(i)
    torch.cuda.synchronize()
    t_amort = time.perf_counter() - t0
    if caches[0].n_q != nq_before + G:
        raise RuntimeError("the flush-amortised window does not hold one flush per layer")

    # kernel timing: a block of further fused steps in which no layer flushes
    # (all layers flush on the same steps: their counters move in lockstep),
    # between one HIP event pair on the stream the library launches on.  The
    # launches run back to back as in the timed steps; the block's time over
    # its launch count is the per-launch time.  A step flushes iff n_res + 1
    # == R + G before it, so the block starts after the next flush if one
    # would fall inside it.
    slots = R + G
    c0 = caches[0]
    i = args.warmup + 2 * n_timed + amort_steps
    while c0.n_res + kernel_steps + 1 >= slots:
        step(i)
        i += 1
    n_q0 = c0.n_q
    # after the lead-in step, timed step j attends over n_res + 2 + j tokens
    kern_bytes = [attn_bytes(w, n_q0, c0.n_res + 2 + j, fused_append=True, meta_bytes=mbytes)
                  for j in range(kernel_steps)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    step(i)           # lead-in: keeps the GPU busy while the block is enqueued
    e0.record()
    for j in range(kernel_steps):
        step(i + 1 + j)
    e1.record()
    torch.cuda.synchronize()
    if any(c.n_q != n_q0 for c in caches):
        raise RuntimeError("a layer flushed inside the kernel-timing block")
    kern_us = [e0.elapsed_time(e1) * 1e3 / (kernel_steps * layers)]
    avg_kern_s = sum(kern_us) / len(kern_us) / 1e6
    avg_bytes = sum(kern_bytes) / len(kern_bytes)
    achieved = avg_bytes / avg_kern_s / 1e9

    copy_gbps = copy_bandwidth()

    ragged = None
    if not args.no_ragged:
        tok = new_tok[0]
        ragged = ragged_leg(w, geom, caches, ws, qs, outs, tok, ragged_steps, args.seed, mbytes)

    ms_per_step = t_steps / n_timed * 1e3
    tokens_s = w.batch / (t_steps / n_timed)
    res = {
        "metric": METRIC, "value": tokens_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": n_timed, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "kv_heads": w.kv_heads,
                   "q_heads": w.q_heads, "head_dim": D, "context": w.seq_len, "bits": w.bits,
                   "group": G, "residual": R, "layers": layers,
                   "scale_zero": "fp16 scale + bf16 zero" if args.meta == "fp16" else "fp32",
                   "launch": "deterministic" if args.deterministic else "default",
                   "step": "per layer: kivi_decode_step (append + flush-if-full + decode "
                           "attention, the flush quantised inside the launch; one launch)"},
        "ms_per_step_separate_calls": t_steps_sep / n_timed * 1e3,
        "tokens_s_flush_amortised": w.batch * amort_steps / t_amort,
        "ms_per_step_flush_amortised": t_amort / amort_steps * 1e3,
        "copy_gbps": copy_gbps,
        "attn_frac_of_copy": achieved / copy_gbps,
        "attn_hbm_gbps": achieved,
        "attn_bytes_per_launch": avg_bytes,
        "attn_kernel_us": avg_kern_s * 1e6,
        "attn_kernel_launches_timed": kernel_steps * layers,
        "attn_tokens_s_kernel_only": w.batch / (avg_kern_s * layers),
        "quantize_gelem_s": quant_gelem_s,
        "quantize_hbm_gbps": pre_gbps,
        "quantize_prefill_ms_per_layer": pre_t / layers * 1e3,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": (read_traffic(f"decode_attn_{w.name}") if default_launch
                                 else None)},
        "mixed_length_steps": ragged,
        "paper_context": "2.35x-3.47x decode throughput vs FP16 and 2.6x less peak memory "
                         "(Llama-2-7B, one A100 80GB; not comparable, quoted as context)",
    }
    if not args.no_other and args.workload == "llama3-8b-gqa-8k" and default_launch:
        # the headline's caches first give way to the others'
        del steppers, caches, ws, new_tok
        torch.cuda.empty_cache()
        others = {}
        for name in OTHER_WORKLOADS:
            try:
                others[name] = other_workload(name, args.seed)
            except Exception as e:   # reported, so that the headline line still prints
                others[name] = {"error": f"{type(e).__name__}: {e}"}
        res["other_workloads"] = others
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.seed, meta=meta)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
