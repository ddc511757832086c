"""Oracle page store: block-table addressing, page write, int8 quantization
and gather.  Test infrastructure only (see the package docstring).

Citations name the page and the part of it that defines the step:
  * tiny-llm paged_kv.py, module docstring: logical block j of a sequence maps
    to a physical block through the sequence's block table, token t lives at
    (table[t // block_size], t % block_size), and only real tokens are stored.
  * AstrAI astrai/inference/cache.py, PagedCache.write / PagedCache.gather /
    CacheView.gather: the page-by-page chunked write from an unaligned
    start position, and the gather that concatenates pages and truncates to
    the bound length.
  * libmir-metal src/engine/kv/paged/mod.rs, PagedStore (Arena with separate
    key/value scale arrays; KvPageFormat::Int8PerTokenHead, one scale per
    token and KV head) and PagedStore::context (take pages by the table, slice
    to the context length, refuse lengths past the stored pages).
"""
from __future__ import annotations

import numpy as np

_STORE_DTYPE = {"f32": np.uint32, "bf16": np.uint16}


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 values (exact: bf16 is the top half)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _as_f32(x: np.ndarray, in_dtype: str) -> np.ndarray:
    if in_dtype == "bf16":
        return bf16_bits_to_f32(x)
    if in_dtype == "f32":
        return np.asarray(x).view(np.float32) if x.dtype != np.float32 else x
    raise ValueError(in_dtype)


def quantize_int8_rows(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Symmetric int8 quantization, one scale per row (the last axis is one
    (token, KV head) row of head_dim values).

    Format: libmir-metal paged/mod.rs, KvPageFormat::Int8PerTokenHead names the
    per-(token, KV head) int8 layout but prints no formula; the rule used here
    is scale = max|x| / 127 with codes round(x / scale) clamped to [-127, 127].
    Every operation is a single IEEE float32 operation with round-to-nearest-
    even: the maximum is exact, the scale is one float32 division, each code is
    one float32 division followed by rint (ties to even).  A row of zeros gets
    scale 0 and codes 0.
    """
    x = np.asarray(x, np.float32)
    m = np.max(np.abs(x), axis=-1)  # exact
    s = (m / np.float32(127.0)).astype(np.float32)  # one IEEE division
    safe = np.where(s == 0, np.float32(1.0), s).astype(np.float32)
    q = np.rint((x / safe[..., None]).astype(np.float32))  # IEEE division, ties to even
    q = np.clip(q, -127, 127)
    q = np.where((s == 0)[..., None], 0, q)
    return q.astype(np.int8), s.astype(np.float32)


class OracleCache:
    """Page store of one cache: ``n_layers`` x ``n_pages`` pages of
    ``page_size`` token slots, each slot holding ``n_kv_heads`` x ``head_dim``
    K and V values.

    fmt "f32"/"bf16": slots hold the raw bit patterns of the written values
    (a native write is a bit copy).  fmt "int8": slots hold int8 codes, and a
    separate float32 array holds one scale per (slot, KV head) for K and for V.
    """

    def __init__(self, n_layers, n_pages, page_size, n_kv_heads, head_dim, fmt,
                 fill_bits: int | None = None):
        self.n_layers, self.n_pages, self.page_size = n_layers, n_pages, page_size
        self.n_kv_heads, self.head_dim, self.fmt = n_kv_heads, head_dim, fmt
        shape = (n_layers, n_pages, page_size, n_kv_heads, head_dim)
        if fmt == "int8":
            self.k = np.zeros(shape, np.int8)
            self.v = np.zeros(shape, np.int8)
            self.k_scale = np.zeros(shape[:-1], np.float32)
            self.v_scale = np.zeros(shape[:-1], np.float32)
        else:
            self.k = np.zeros(shape, _STORE_DTYPE[fmt])
            self.v = np.zeros(shape, _STORE_DTYPE[fmt])
            self.k_scale = self.v_scale = None
        if fill_bits is not None:
            self.k[...] = fill_bits
            self.v[...] = fill_bits
            if fmt == "int8":
                self.k_scale[...] = np.float32(fill_bits)
                self.v_scale[...] = np.float32(fill_bits)

    # -- addressing: tiny-llm paged_kv.py, module docstring ----------------------
    def address(self, table_row: np.ndarray, t: int) -> tuple[int, int]:
        """Physical (page, slot) of token t of the sequence with this table row."""
        return int(table_row[t // self.page_size]), t % self.page_size

    def _store_row(self, layer, page, slot, krow, vrow, in_dtype):
        if not (0 <= page < self.n_pages):
            raise IndexError(f"physical page {page} outside the pool")
        if self.fmt == "int8":
            kc, ks = quantize_int8_rows(_as_f32(krow, in_dtype))
            vc, vs = quantize_int8_rows(_as_f32(vrow, in_dtype))
            self.k[layer, page, slot] = kc
            self.v[layer, page, slot] = vc
            self.k_scale[layer, page, slot] = ks
            self.v_scale[layer, page, slot] = vs
        else:
            want = "bf16" if self.fmt == "bf16" else "f32"
            if in_dtype != want:
                raise TypeError(f"{self.fmt} pages take {want} rows, not {in_dtype}")
            self.k[layer, page, slot] = np.asarray(krow).view(self.k.dtype)
            self.v[layer, page, slot] = np.asarray(vrow).view(self.v.dtype)

    # -- write, one token at a time ---------------------------------------------
    def write(self, layer, tables, start_pos, cu_new, k, v, in_dtype):
        """Store row i of sequence b at position start_pos[b] + i.

        ``k``/``v`` are [total_new, Hkv, D] (bit patterns for bf16 as uint16,
        float32 for f32); rows cu_new[b]:cu_new[b+1] belong to sequence b.
        AstrAI cache.py PagedCache.write fixes what is stored and where; one
        start position per sequence generalises its single batch start_pos
        (tiny-llm paged_kv.py writes each slot at its own length).
        """
        start_pos = np.asarray(start_pos, np.int64)
        cu_new = np.asarray(cu_new, np.int64)
        counts = np.diff(cu_new)
        seq = np.repeat(np.arange(len(start_pos)), counts)  # sequence of each row
        if seq.size == 0:
            return
        t = start_pos[seq] + (np.arange(seq.size) - cu_new[seq])  # token position of each row
        page = np.asarray(tables, np.int64)[seq, t // self.page_size]
        slot = t % self.page_size
        if np.any((page < 0) | (page >= self.n_pages)):
            raise IndexError("physical page outside the pool")
        if self.fmt == "int8":
            kc, ks = quantize_int8_rows(_as_f32(np.asarray(k), in_dtype))
            vc, vs = quantize_int8_rows(_as_f32(np.asarray(v), in_dtype))
            self.k[layer, page, slot] = kc
            self.v[layer, page, slot] = vc
            self.k_scale[layer, page, slot] = ks
            self.v_scale[layer, page, slot] = vs
        else:
            want = "bf16" if self.fmt == "bf16" else "f32"
            if in_dtype != want:
                raise TypeError(f"{self.fmt} pages take {want} rows, not {in_dtype}")
            self.k[layer, page, slot] = np.asarray(k).view(self.k.dtype)
            self.v[layer, page, slot] = np.asarray(v).view(self.v.dtype)

    # -- write, page by page --------------------------------------------------
    def write_by_pages(self, layer, tables, start_pos: int, k, v, in_dtype):
        """The chunked form of AstrAI cache.py PagedCache.write: one scalar start
        position for the whole batch, k/v shaped [B, n, Hkv, D]; for every
        logical page the write overlaps, the overlapping run of rows is copied
        into that page at its in-page offset.  Used only to cross-check
        ``write``: both must leave byte-identical pages."""
        n = k.shape[1]
        if n == 0:
            return
        ps = self.page_size
        end = start_pos + n
        j = start_pos // ps
        while j * ps < end:
            lo = max(j * ps, start_pos)
            hi = min((j + 1) * ps, end)
            for b in range(k.shape[0]):
                page = int(tables[b][j])
                for t in range(lo, hi):
                    self._store_row(layer, page, t - j * ps, k[b, t - start_pos],
                                    v[b, t - start_pos], in_dtype)
            j += 1

    # -- gather -----------------------------------------------------------------
    def gather(self, layer, table_row, length):
        """Rows 0..length-1 of one sequence, in token order, [length, Hkv, D]
        (bit patterns / int8 codes), plus [length, Hkv] scales for int8.

        Only the first ceil(length / page_size) table entries are read; a
        length past the pages the table row lists is an error (libmir-metal
        paged/mod.rs, PagedStore::context)."""
        ps = self.page_size
        npages = -(-length // ps)
        if npages > len(table_row):
            raise IndexError("context exceeds the pages of the table")
        ks, vs, kss, vss = [], [], [], []
        for j in range(npages):
            page = int(table_row[j])
            if not (0 <= page < self.n_pages):
                raise IndexError(f"physical page {page} outside the pool")
            n = min(ps, length - j * ps)
            ks.append(self.k[layer, page, :n])
            vs.append(self.v[layer, page, :n])
            if self.fmt == "int8":
                kss.append(self.k_scale[layer, page, :n])
                vss.append(self.v_scale[layer, page, :n])
        shape = (0, self.n_kv_heads, self.head_dim)
        K = np.concatenate(ks) if ks else np.zeros(shape, self.k.dtype)
        V = np.concatenate(vs) if vs else np.zeros(shape, self.v.dtype)
        if self.fmt != "int8":
            return K, V, None, None
        KS = np.concatenate(kss) if kss else np.zeros(shape[:2], np.float32)
        VS = np.concatenate(vss) if vss else np.zeros(shape[:2], np.float32)
        return K, V, KS, VS

    def gather_f64(self, layer, table_row, length):
        """Gathered K/V upcast to float64 values: bf16/f32 bits converted exactly,
        int8 codes multiplied by their per-(token, KV head) scale."""
        K, V, KS, VS = self.gather(layer, table_row, length)
        if self.fmt == "int8":
            return (K.astype(np.float64) * KS.astype(np.float64)[..., None],
                    V.astype(np.float64) * VS.astype(np.float64)[..., None])
        if self.fmt == "bf16":
            return bf16_bits_to_f32(K).astype(np.float64), bf16_bits_to_f32(V).astype(np.float64)
        return K.view(np.float32).astype(np.float64), V.view(np.float32).astype(np.float64)
