"""Oracle decode attention over a paged cache, in float64.  Test
infrastructure only (see the package docstring).

What it computes (one query token per sequence):
  * K/V of sequence b are its first lens[b] tokens, gathered by the block
    table (tiny-llm paged_kv.py: the toy gathers each sequence's blocks into a
    contiguous view before attention; here the gather is the oracle's own).
  * Query head h attends with KV head h // G, G = n_q_heads / n_kv_heads
    (query heads outnumbering KV heads, as in metrale_storage
    high_speed_swap/impl_more.rs attend_layer; contiguous groups).
  * Scores s_t = scale * <q_h, k_t>; weights softmax(s) over t < lens[b]
    (the length mask of tiny-llm paged_kv.py begin_step, which includes the
    token written in the same step); output sum_t p_t v_t.  A sequence with
    no tokens gives zeros.

Several queries per sequence (a chunk of new tokens, ``attend_multi``):
  * sequence b's T_b = cu_q[b+1] - cu_q[b] query rows stand for its last T_b
    tokens (the rows a chunked write just stored, AstrAI cache.py
    PagedCache.write with seq_len > 1): query i sits at position
    lens[b] - T_b + i;
  * it sees the tokens t <= its position and no later ones: the valid-slot
    rule of metrale_storage high_speed_swap/impl_more.rs (a query at q_pos
    reads only the first q_pos % page_size + 1 slots of its own block), and
    the decode rule above when T_b = 1.  A position below 0 sees nothing
    (zeros).
"""
from __future__ import annotations

import numpy as np

from .paged_cache import OracleCache, bf16_bits_to_f32


def _kv_group(h: int, group: int) -> int:
    return h // group


def _q_f64(q: np.ndarray, q_dtype: str) -> np.ndarray:
    if q_dtype == "bf16":
        return bf16_bits_to_f32(q).astype(np.float64)
    return np.asarray(q).view(np.float32).astype(np.float64)


def attend_one(K: np.ndarray, V: np.ndarray, qh: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of one query row over K, V [n, D] (float64)."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], np.float64)
    s = float(scale) * (K @ qh)
    p = np.exp(s - s.max())
    return (p @ V) / p.sum()


def attend(cache: OracleCache, layer: int, q: np.ndarray, q_dtype: str, tables, lens,
           scale: float, seqs=None, heads=None) -> np.ndarray:
    """Decode attention for every (sequence, query head), or for the chosen
    ``seqs``/``heads`` only; returns float64 [B, Hq, D] (unchosen rows zero).

    q is [B, Hq, D] (bf16 bit patterns as uint16, or float32)."""
    B, Hq, D = q.shape
    G = Hq // cache.n_kv_heads
    if G * cache.n_kv_heads != Hq:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    qf = _q_f64(q, q_dtype)
    out = np.zeros((B, Hq, D), np.float64)
    sc = float(np.float32(scale))
    for b in (range(B) if seqs is None else seqs):
        K, V = cache.gather_f64(layer, tables[b], int(lens[b]))
        for h in (range(Hq) if heads is None else heads):
            g = _kv_group(h, G)
            out[b, h] = attend_one(K[:, g, :], V[:, g, :], qf[b, h], sc)
    return out


def query_positions(lens, cu_q) -> np.ndarray:
    """Absolute position of every query row (int64 [total_q]): the T_b rows
    of sequence b are its last T_b tokens, row cu_q[b] + i at lens[b] - T_b + i."""
    cu = np.asarray(cu_q, np.int64)
    pos = np.zeros(int(cu[-1]), np.int64)
    for b in range(len(cu) - 1):
        T = int(cu[b + 1] - cu[b])
        pos[cu[b]:cu[b + 1]] = int(lens[b]) - T + np.arange(T)
    return pos


def _visible(pos: int) -> int:
    """Tokens a query at position pos sees: 0 .. pos."""
    return max(pos + 1, 0)


def attend_multi(cache: OracleCache, layer: int, q: np.ndarray, q_dtype: str, tables, lens,
                 cu_q, scale: float, rows=None) -> np.ndarray:
    """Causal attention of several query rows per sequence; returns float64
    [total_q, Hq, D] (rows not in ``rows`` are zero when it is given).

    q is [total_q, Hq, D]; row r of sequence b attends to tokens
    0 .. query_positions(lens, cu_q)[r] of that sequence."""
    total_q, Hq, D = q.shape
    G = Hq // cache.n_kv_heads
    if G * cache.n_kv_heads != Hq:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    cu = np.asarray(cu_q, np.int64)
    if int(cu[-1]) != total_q:
        raise ValueError("cu_q[-1] must equal the number of query rows")
    pos = query_positions(lens, cu)
    qf = _q_f64(q, q_dtype)
    out = np.zeros((total_q, Hq, D), np.float64)
    sc = float(np.float32(scale))
    want = None if rows is None else set(int(r) for r in rows)
    for b in range(len(cu) - 1):
        mine = [r for r in range(int(cu[b]), int(cu[b + 1])) if want is None or r in want]
        if not mine:
            continue
        K, V = cache.gather_f64(layer, tables[b], int(lens[b]))
        for r in mine:
            n_vis = _visible(int(pos[r]))
            for h in range(Hq):
                g = _kv_group(h, G)
                out[r, h] = attend_one(K[:n_vis, g, :], V[:n_vis, g, :], qf[r, h], sc)
    return out
