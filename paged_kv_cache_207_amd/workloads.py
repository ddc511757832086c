"""Seeded synthetic inputs for the paged KV cache workloads.

This module only draws random numbers and lays out inputs: sequence lengths,
physical-page permutations, block tables, write rounds (start positions and
ragged row offsets) and N(0, 1) K/V/Q values.  It holds no part of the page
write, the int8 quantization or the attention arithmetic.  The HIP library's
tests and benchmark and the CPU reference both consume what it produces, so a
test can hand the very same inputs to each side.

Recipe (the same for every workload):
  * ``numpy.random.default_rng(1000 + c)`` draws lengths, page permutations
    and the unaligned head chunk of the int8 prefill;
  * ``torch.Generator().manual_seed(...)`` draws N(0, 1) values in float32,
    which are then cast to the input dtype with round-to-nearest-even
    (``Tensor.to(torch.bfloat16)``).  K/V values are drawn per sequence from a
    seed derived from (workload seed, sequence index), so any one sequence can
    be regenerated on its own.
  * Block tables hold physical page ids taken, in order, from a random
    permutation of the pool; unused table entries are -1 (never read).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

# Page-format and dtype names shared with the binding (plain labels only).
FORMATS = ("f32", "bf16", "int8")


@dataclass
class WriteRound:
    """One ``paged_write`` call: rows ``cu_new[b]:cu_new[b+1]`` of k/v go to
    positions ``start_pos[b] + i`` of sequence b."""

    start_pos: np.ndarray  # int32 [B]
    cu_new: np.ndarray  # int32 [B + 1]
    k: torch.Tensor  # [total_new, Hkv, D] (input dtype)
    v: torch.Tensor

    @property
    def total_new(self) -> int:
        return int(self.cu_new[-1])


@dataclass
class Workload:
    name: str
    n_pages: int
    page_size: int
    n_kv_heads: int
    head_dim: int
    n_q_heads: int
    kv_format: str  # "f32" | "bf16" | "int8"
    in_dtype: torch.dtype  # dtype of the K/V rows handed to paged_write
    q_dtype: torch.dtype
    scale: float  # softmax scale, an exact float32 value
    tables: np.ndarray  # int32 [B, table_stride]; entries past ceil(len/bs) are -1
    lens: np.ndarray  # int32 [B]: tokens stored once every write round ran
    seed: int
    n_layers: int = 1
    # int8 prefill: per-sequence size of the unaligned first chunk (0 = one chunk)
    head_chunk: np.ndarray | None = None
    chunk: int = 0  # rows per sequence per later round (0 = single round)
    meta: dict = field(default_factory=dict)

    # ---- shapes -------------------------------------------------------
    @property
    def batch(self) -> int:
        return int(self.lens.shape[0])

    @property
    def table_stride(self) -> int:
        return int(self.tables.shape[1])

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def max_len(self) -> int:
        return int(self.lens.max()) if self.batch else 0

    # ---- values -------------------------------------------------------
    def seq_kv(self, b: int) -> tuple[torch.Tensor, torch.Tensor]:
        """K and V rows [len_b, Hkv, D] of sequence b, regenerated from its seed."""
        g = torch.Generator().manual_seed(self.seed * 100003 + b)
        shape = (int(self.lens[b]), self.n_kv_heads, self.head_dim)
        k = torch.randn(shape, generator=g, dtype=torch.float32)
        v = torch.randn(shape, generator=g, dtype=torch.float32)
        return k.to(self.in_dtype), v.to(self.in_dtype)

    def query(self, step: int = 0) -> torch.Tensor:
        g = torch.Generator().manual_seed(self.seed * 7919 + 17 + step)
        q = torch.randn((self.batch, self.n_q_heads, self.head_dim), generator=g)
        return q.to(self.q_dtype)

    def rounds(self, seqs: list[int] | None = None, kv: dict | None = None) -> list[WriteRound]:
        """The write rounds that fill every sequence to ``lens``.

        Single-round workloads write all rows from position 0 in one call.
        The int8 prefill first writes ``head_chunk[b]`` rows, then rounds of
        ``chunk`` rows, so every later round starts off a page boundary.
        """
        seqs = list(range(self.batch)) if seqs is None else seqs
        if kv is None:
            kv = {b: self.seq_kv(b) for b in seqs}
        bounds: list[list[tuple[int, int]]] = []
        for b in range(self.batch):
            L = int(self.lens[b])
            if self.chunk <= 0:
                spans = [(0, L)]
            else:
                h = min(int(self.head_chunk[b]), L)
                spans = [(0, h)]
                s = h
                while s < L:
                    spans.append((s, min(s + self.chunk, L)))
                    s += self.chunk
            bounds.append(spans)
        n_rounds = max(len(s) for s in bounds) if bounds else 0
        out = []
        for r in range(n_rounds):
            start = np.zeros(self.batch, np.int32)
            cu = np.zeros(self.batch + 1, np.int32)
            ks, vs = [], []
            for b in range(self.batch):
                if b in kv and r < len(bounds[b]):
                    t0, t1 = bounds[b][r]
                else:
                    t0 = t1 = int(self.lens[b])
                start[b] = t0
                cu[b + 1] = cu[b] + (t1 - t0)
                if t1 > t0:
                    ks.append(kv[b][0][t0:t1])
                    vs.append(kv[b][1][t0:t1])
            empty = torch.empty((0, self.n_kv_heads, self.head_dim), dtype=self.in_dtype)
            k = torch.cat(ks) if ks else empty
            v = torch.cat(vs) if vs else empty
            out.append(WriteRound(start, cu, k.contiguous(), v.contiguous()))
        return out


def _tables_from_perm(perm: np.ndarray, pages_per_seq: list[int], stride: int) -> np.ndarray:
    t = np.full((len(pages_per_seq), max(stride, 1)), -1, np.int32)
    o = 0
    for b, n in enumerate(pages_per_seq):
        t[b, :n] = perm[o:o + n]
        o += n
    return t


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def tiny_f32(seed: int = 1) -> Workload:
    """Two sequences of 37 and 50 fp32 tokens, 16-token pages, a 16-page pool
    whose ids are a seeded permutation; 4 query heads over 2 KV heads, D=64."""
    rng = np.random.default_rng(1000 + seed)
    perm = rng.permutation(16).astype(np.int32)
    lens = np.array([37, 50], np.int32)
    tables = _tables_from_perm(perm, [3, 4], 4)
    return Workload("tiny_f32", 16, 16, 2, 64, 4, "f32", torch.float32, torch.float32,
                    float(np.float32(1.0 / math.sqrt(64))), tables, lens, 2000 + seed)


def _random_pool(rng, lens, bs, slack=1.25, stride_pages=None):
    pages = [_cdiv(int(n), bs) for n in lens]
    total = sum(pages)
    P = max(int(math.ceil(slack * total)), 1)
    perm = rng.permutation(P).astype(np.int32)
    stride = stride_pages if stride_pages is not None else max(pages + [1])
    return P, _tables_from_perm(perm, pages, stride)


def decode_bf16(batch=32, lo=512, hi=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
                page_size=16, seed: int = 2) -> Workload:
    """bf16 decode: lengths uniform in [lo, hi], pool 1.25x the pages needed,
    shuffled page ids."""
    rng = np.random.default_rng(1000 + seed)
    lens = rng.integers(lo, hi + 1, size=batch).astype(np.int32)
    P, tables = _random_pool(rng, lens, page_size)
    return Workload("decode_bf16", P, page_size, n_kv_heads, head_dim, n_q_heads, "bf16",
                    torch.bfloat16, torch.bfloat16,
                    float(np.float32(1.0 / math.sqrt(head_dim))), tables, lens, 2000 + seed)


def long_bf16(batch=8, seq_len=32768, n_q_heads=64, n_kv_heads=8, head_dim=128,
              page_size=16, seed: int = 3) -> Workload:
    """bf16 long context: every sequence ``seq_len`` tokens, one random
    permutation over exactly the pages needed (fully fragmented table)."""
    rng = np.random.default_rng(1000 + seed)
    lens = np.full(batch, seq_len, np.int32)
    npg = _cdiv(seq_len, page_size)
    P = batch * npg
    perm = rng.permutation(P).astype(np.int32)
    tables = perm.reshape(batch, npg).copy()
    return Workload("long_bf16", P, page_size, n_kv_heads, head_dim, n_q_heads, "bf16",
                    torch.bfloat16, torch.bfloat16,
                    float(np.float32(1.0 / math.sqrt(head_dim))), tables, lens, 2000 + seed)


def int8_kv(batch=64, lo=128, hi=16384, n_q_heads=64, n_kv_heads=8, head_dim=128,
            page_size=32, chunk=512, seed: int = 4) -> Workload:
    """int8 per-(token, KV head) pages: log-uniform lengths in [lo, hi]; the
    prefill writes a seeded 1..page_size-1 row head chunk, then ``chunk``-row
    rounds, so no round after the first starts on a page boundary."""
    rng = np.random.default_rng(1000 + seed)
    lens = np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), size=batch)))
    lens = np.clip(lens, lo, hi).astype(np.int32)
    P, tables = _random_pool(rng, lens, page_size)
    head = rng.integers(1, page_size, size=batch).astype(np.int32)
    return Workload("int8_kv", P, page_size, n_kv_heads, head_dim, n_q_heads, "int8",
                    torch.bfloat16, torch.bfloat16,
                    float(np.float32(1.0 / math.sqrt(head_dim))), tables, lens, 2000 + seed,
                    head_chunk=head, chunk=chunk)


@dataclass
class SharedPrefix:
    """Decode steps over sequences that share their first ``prefix_pages``
    pages (same physical ids in every table) and own private suffixes.

    ``base`` holds the state before step 0: its tables already list every
    page the steps will grow into (entries are read only below the length).
    Step s writes one row per sequence at position ``lens0 + s`` and attends
    over ``lens0 + s + 1`` tokens.
    """

    base: Workload
    prefix_pages: int
    suffix: np.ndarray  # int32 [B]
    n_steps: int

    @property
    def prefix_tokens(self) -> int:
        return self.prefix_pages * self.base.page_size

    def prefix_kv(self) -> tuple[torch.Tensor, torch.Tensor]:
        w = self.base
        g = torch.Generator().manual_seed(w.seed * 100003 + 999_983)
        shape = (self.prefix_tokens, w.n_kv_heads, w.head_dim)
        k = torch.randn(shape, generator=g)
        v = torch.randn(shape, generator=g)
        return k.to(w.in_dtype), v.to(w.in_dtype)

    def private_kv(self, b: int) -> tuple[torch.Tensor, torch.Tensor]:
        """Rows of sequence b after the prefix: the suffix, then one row per step."""
        w = self.base
        g = torch.Generator().manual_seed(w.seed * 100003 + b)
        shape = (int(self.suffix[b]) + self.n_steps, w.n_kv_heads, w.head_dim)
        k = torch.randn(shape, generator=g)
        v = torch.randn(shape, generator=g)
        return k.to(w.in_dtype), v.to(w.in_dtype)

    def fill_rounds(self) -> list[WriteRound]:
        """Prefix once (through sequence 0's table), then every suffix."""
        w = self.base
        B = w.batch
        pk, pv = self.prefix_kv()
        start = np.zeros(B, np.int32)
        cu = np.zeros(B + 1, np.int32)
        cu[1:] = self.prefix_tokens
        r0 = WriteRound(start, cu, pk, pv)
        ks, vs = [], []
        cu1 = np.zeros(B + 1, np.int32)
        for b in range(B):
            k, v = self.private_kv(b)
            n = int(self.suffix[b])
            ks.append(k[:n])
            vs.append(v[:n])
            cu1[b + 1] = cu1[b] + n
        r1 = WriteRound(np.full(B, self.prefix_tokens, np.int32), cu1,
                        torch.cat(ks).contiguous(), torch.cat(vs).contiguous())
        return [r0, r1]

    def step_round(self, s: int) -> WriteRound:
        w = self.base
        B = w.batch
        ks, vs = [], []
        for b in range(B):
            k, v = self.private_kv(b)
            n = int(self.suffix[b]) + s
            ks.append(k[n:n + 1])
            vs.append(v[n:n + 1])
        return WriteRound((w.lens + s).astype(np.int32), np.arange(B + 1, dtype=np.int32),
                          torch.cat(ks).contiguous(), torch.cat(vs).contiguous())

    def step_lens(self, s: int) -> np.ndarray:
        return (self.base.lens + s + 1).astype(np.int32)

    def step_rows_all(self) -> tuple[torch.Tensor, torch.Tensor]:
        """K/V rows of every step, [n_steps, B, Hkv, D]."""
        w = self.base
        ks = torch.empty((self.n_steps, w.batch, w.n_kv_heads, w.head_dim), dtype=w.in_dtype)
        vs = torch.empty_like(ks)
        for b in range(w.batch):
            k, v = self.private_kv(b)
            n = int(self.suffix[b])
            ks[:, b] = k[n:n + self.n_steps]
            vs[:, b] = v[n:n + self.n_steps]
        return ks, vs


def shared_prefix(batch=256, prefix_pages=64, lo=16, hi=2048, n_steps=32, n_q_heads=32,
                  n_kv_heads=4, head_dim=64, page_size=16, seed: int = 5) -> SharedPrefix:
    rng = np.random.default_rng(1000 + seed)
    suffix = rng.integers(lo, hi + 1, size=batch).astype(np.int32)
    prefix_tokens = prefix_pages * page_size
    final = suffix + n_steps  # private tokens once every step ran
    priv_pages = [_cdiv(int(n), page_size) for n in final]
    P = int(math.ceil(1.25 * (prefix_pages + sum(priv_pages))))
    perm = rng.permutation(P).astype(np.int32)
    stride = prefix_pages + max(priv_pages)
    tables = np.full((batch, stride), -1, np.int32)
    tables[:, :prefix_pages] = perm[:prefix_pages]
    o = prefix_pages
    for b, n in enumerate(priv_pages):
        tables[b, prefix_pages:prefix_pages + n] = perm[o:o + n]
        o += n
    lens0 = (prefix_tokens + suffix).astype(np.int32)
    base = Workload("shared_prefix", P, page_size, n_kv_heads, head_dim, n_q_heads, "bf16",
                    torch.bfloat16, torch.bfloat16,
                    float(np.float32(1.0 / math.sqrt(head_dim))), tables, lens0, 2000 + seed)
    return SharedPrefix(base, prefix_pages, suffix, n_steps)


@dataclass
class ChunkedPrefill:
    """Several new tokens per sequence at once (a prefill chunk).

    ``base`` holds the sequences at their final length (context + chunk);
    its write rounds are the context (from position 0), then the chunk (from
    position context[b]).  The chunk's queries are rows cu_q[b] .. cu_q[b+1]
    of ``queries()``, one per new token, in position order.
    """

    base: Workload
    context: np.ndarray  # int32 [B]: tokens already stored before the chunk
    chunk: np.ndarray  # int32 [B]: new tokens (and queries) per sequence

    @property
    def cu_q(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.chunk)]).astype(np.int32)

    @property
    def total_q(self) -> int:
        return int(self.chunk.sum())

    @property
    def max_q(self) -> int:
        return int(self.chunk.max()) if len(self.chunk) else 0

    def context_round(self, kv: dict | None = None) -> WriteRound:
        return self.base.rounds(kv=kv)[0]

    def chunk_round(self, kv: dict | None = None) -> WriteRound:
        r = self.base.rounds(kv=kv)
        if len(r) > 1:
            return r[1]
        B = self.base.batch  # every chunk empty
        empty = torch.empty((0, self.base.n_kv_heads, self.base.head_dim),
                            dtype=self.base.in_dtype)
        return WriteRound(self.base.lens.copy(), np.zeros(B + 1, np.int32), empty, empty)

    def queries(self) -> torch.Tensor:
        w = self.base
        g = torch.Generator().manual_seed(w.seed * 7919 + 29)
        q = torch.randn((self.total_q, w.n_q_heads, w.head_dim), generator=g)
        return q.to(w.q_dtype)


def chunked_prefill(batch=4, context=(4096, 4096), chunk=(512, 512), n_q_heads=32,
                    n_kv_heads=8, head_dim=128, page_size=16, kv_format="bf16",
                    seed: int = 6) -> ChunkedPrefill:
    """Chunked prefill: per sequence a context length uniform in ``context``
    and a chunk length uniform in ``chunk`` (inclusive ranges), pool 1.25x the
    pages needed, shuffled page ids."""
    rng = np.random.default_rng(1000 + seed)
    ctx = rng.integers(context[0], context[1] + 1, size=batch).astype(np.int32)
    ch = rng.integers(chunk[0], chunk[1] + 1, size=batch).astype(np.int32)
    lens = (ctx + ch).astype(np.int32)
    P, tables = _random_pool(rng, lens, page_size)
    in_dtype = torch.float32 if kv_format == "f32" else torch.bfloat16
    base = Workload("chunked_prefill", P, page_size, n_kv_heads, head_dim, n_q_heads, kv_format,
                    in_dtype, in_dtype if kv_format == "f32" else torch.bfloat16,
                    float(np.float32(1.0 / math.sqrt(head_dim))), tables, lens, 2000 + seed,
                    head_chunk=ctx.copy(), chunk=max(int(ch.max()), 1))
    return ChunkedPrefill(base, ctx, ch)


def by_name(name: str, **kw):
    return {"tiny_f32": tiny_f32, "decode_bf16": decode_bf16, "long_bf16": long_bf16,
            "int8_kv": int8_kv, "shared_prefix": shared_prefix,
            "chunked_prefill": chunked_prefill}[name](**kw)
