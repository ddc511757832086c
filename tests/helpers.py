"""Test-side plumbing: hand workload inputs to the CPU oracle as NumPy bit
patterns, and lay the GPU pool out in the oracle's order for comparison."""
from __future__ import annotations

import numpy as np
import torch

from oracle import OracleCache


def dtype_name(t: torch.Tensor) -> str:
    return {torch.bfloat16: "bf16", torch.float32: "f32"}[t.dtype]


def np_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensors as uint16 bit patterns, f32 tensors as float32 arrays."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(t.dtype)


def oracle_for(w, fill_bits=None) -> OracleCache:
    return OracleCache(w.n_layers, w.n_pages, w.page_size, w.n_kv_heads, w.head_dim,
                       w.kv_format, fill_bits=fill_bits)


def oracle_write_rounds(cache: OracleCache, w, rounds, layer=0):
    for r in rounds:
        cache.write(layer, w.tables, r.start_pos, r.cu_new, np_bits(r.k), np_bits(r.v),
                    dtype_name(r.k))
