"""Seeded synthetic inputs and workload shapes.

This module holds no arithmetic of the method.  It only draws inputs, shared
by the oracle side and the HIP side of every comparison:

* K, V ~ N(0, 1) drawn in fp32 and rounded to bf16, with a few key channels
  per kv head multiplied by a constant to mimic the outlier channels that the
  pages describe for real keys (news article "KV cache quantization squeezes
  5GB ...", asymmetry paragraph: keys carry large magnitudes in certain
  channels, values do not).  Outlier channels are a property of a (layer,
  kv head) and are reused by every appended token.
* q ~ N(0, 1) in bf16.

The shapes stand in for the models the pages name (catalog record
kivi-2bit-llama3-8b-gqa-8k, Model: Llama-3-8B, 32 layers, 8 kv heads, 32 query
heads, head_dim 128, 8K context; paper card: LLaMA / Falcon / Mistral; news
article: Llama-2-7B).  No dataset, prompt or trained weight is involved.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    kv_heads: int
    q_per_kv: int
    seq_len: int
    bits: int
    layers: int
    outlier_count: int            # key channels per kv head scaled by outlier_factor
    outlier_factor: float
    fixed_outliers: tuple = ()    # explicit channel list (same for every head)
    decode_steps: int = 0
    head_dim: int = 128
    group: int = 32
    residual: int = 128

    @property
    def q_heads(self) -> int:
        return self.kv_heads * self.q_per_kv


# round(0.02 * 128) = 3 outlier channels per head for the "2% of channels" recipe
WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 1, 256, 2, 1, 4, 10.0, fixed_outliers=(3, 42, 85, 126)),
    "llama2-7b-mha-4k": Workload("llama2-7b-mha-4k", 8, 32, 1, 4096, 2, 32, 3, 8.0,
                                 decode_steps=128),
    "llama3-8b-gqa-8k": Workload("llama3-8b-gqa-8k", 16, 8, 4, 8192, 2, 32, 3, 8.0),
    "llama2-13b-mha-wall": Workload("llama2-13b-mha-wall", 1, 40, 1, 4096, 2, 40, 3, 8.0),
    "llama3-8b-gqa-32k-4bit": Workload("llama3-8b-gqa-32k-4bit", 4, 8, 4, 32768, 4, 32, 3,
                                       8.0, decode_steps=1024),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def _stream_seed(seed: int, *ids: int) -> int:
    """Distinct, reproducible seed for one tensor of one (layer, step)."""
    mask = (1 << 64) - 1
    h = (0x9E3779B97F4A7C15 * (int(seed) + 1)) & mask
    for i in ids:
        h ^= (int(i) + 0x632BE59BD9B4E019 + (h << 6) + (h >> 2)) & mask
    return h & 0x7FFF_FFFF_FFFF_FFFF


def outlier_channels(w: Workload, seed: int, layer: int) -> np.ndarray:
    """int64 [kv_heads][outlier_count]: outlier key channels of each kv head."""
    if w.fixed_outliers:
        return np.tile(np.asarray(w.fixed_outliers, np.int64), (w.kv_heads, 1))
    rng = np.random.default_rng(_stream_seed(seed, 5, layer))
    return np.stack([rng.choice(w.head_dim, size=w.outlier_count, replace=False)
                     for _ in range(w.kv_heads)]).astype(np.int64)


def _normal(shape, seed: int, device) -> torch.Tensor:
    return torch.randn(*shape, dtype=torch.float32, device=device,
                       generator=_gen(seed, device))


def _key_scale(w: Workload, seed: int, layer: int, device) -> torch.Tensor:
    """fp32 [kv_heads][head_dim]: 1, or outlier_factor on outlier channels."""
    scale = torch.ones(w.kv_heads, w.head_dim, dtype=torch.float32)
    ch = outlier_channels(w, seed, layer)
    for h in range(w.kv_heads):
        scale[h, torch.from_numpy(ch[h])] = w.outlier_factor
    return scale.to(device)


def prefill_kv(w: Workload, seed: int, layer: int = 0, seq_len: int | None = None,
               batch: int | None = None, device="cpu"):
    """(k, v) bf16 [B][H][S][D]."""
    S = w.seq_len if seq_len is None else seq_len
    B = w.batch if batch is None else batch
    shape = (B, w.kv_heads, S, w.head_dim)
    k = _normal(shape, _stream_seed(seed, 0, layer), device)
    k.mul_(_key_scale(w, seed, layer, device)[None, :, None, :])
    v = _normal(shape, _stream_seed(seed, 1, layer), device)
    return k.to(torch.bfloat16), v.to(torch.bfloat16)


def query(w: Workload, seed: int, layer: int = 0, step: int = 0, batch: int | None = None,
          device="cpu") -> torch.Tensor:
    """q bf16 [B][Hq][D]."""
    B = w.batch if batch is None else batch
    q = _normal((B, w.q_heads, w.head_dim), _stream_seed(seed, 2, layer, step), device)
    return q.to(torch.bfloat16)


def new_token(w: Workload, seed: int, layer: int, step: int, batch: int | None = None,
              device="cpu"):
    """(k_new, v_new) bf16 [B][H][D] for decode step `step` (same outlier channels)."""
    B = w.batch if batch is None else batch
    shape = (B, w.kv_heads, w.head_dim)
    k = _normal(shape, _stream_seed(seed, 3, layer, step), device)
    k.mul_(_key_scale(w, seed, layer, device)[None, :, :])
    v = _normal(shape, _stream_seed(seed, 4, layer, step), device)
    return k.to(torch.bfloat16), v.to(torch.bfloat16)


def bits_u16(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
