"""KIVI asymmetric low-bit KV cache and decode attention for MI355X (gfx950).

The product is libkivi.so (C ABI in include/kivi.h, HIP kernels in csrc/);
``decode_attention_channel_amd.kivi`` is its thin ctypes binding.
"""
from . import kivi  # noqa: F401  (raises if libkivi.so is missing)
from .kivi import (Cache, Geom, KiviError, PagedCache, RaggedStepper, Workspace,  # noqa: F401
                   append_token, cache_layout, decode_attention, decode_step,
                   dense_decode_attention, flush_residual, paged_decode_step, paged_layout,
                   paged_prefill, quantize_prefill, ragged_decode_step, ragged_prefill,
                   workspace_bytes)
