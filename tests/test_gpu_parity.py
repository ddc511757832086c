"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Writes and int8 quantization are compared bit for bit on whole page arrays
(sentinel-filled first, so untouched slots are checked too); attention is
compared with the float64 oracle at 1e-5 (f32), 2e-2 (bf16) and 5e-2 (int8
pages, against attention on the dequantized pages).  Reduced workloads keep
the oracle to seconds while still spanning several splits, tiles and a
ragged last page; the full-size workloads are checked on sampled sequences.
"""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

from oracle import OracleCache, attend
from paged_kv_cache_207_amd import pkv
from paged_kv_cache_207_amd import workloads as W
from tests.gpu_helpers import (TOL, dev, gpu_write, make_cache, max_err, pages_in_oracle_order,
                               require_gpu, say, sentinel_oracle)
from tests.helpers import dtype_name, np_bits, oracle_write_rounds

pytestmark = pytest.mark.gpu


def reduced(name):
    return {
        "tiny_f32": lambda: W.tiny_f32(),
        "decode_bf16": lambda: W.decode_bf16(batch=6, lo=100, hi=700),
        "long_bf16": lambda: W.long_bf16(batch=2, seq_len=3000),
        "int8_kv": lambda: W.int8_kv(batch=6, lo=40, hi=2000),
    }[name]()


NAMES = ["tiny_f32", "decode_bf16", "long_bf16", "int8_kv"]


def _run_fill(w, rounds=None):
    c = make_cache(w)
    tdev = dev(w.tables)
    gpu_write(c, tdev, w.rounds() if rounds is None else rounds)
    return c, tdev


# ------------------------------------------------------------------- write --

@pytest.mark.parametrize("name", NAMES)
def test_write_bit_exact(name):
    require_gpu()
    w = reduced(name)
    say(f"write {name}: B={w.batch} P={w.n_pages} fmt={w.kv_format}")
    rounds = w.rounds()
    c, _ = _run_fill(w, rounds)
    o = sentinel_oracle(w)
    oracle_write_rounds(o, w, rounds)
    K, V, KS, VS = pages_in_oracle_order(c)
    assert np.array_equal(K, o.k), "K pages differ"
    assert np.array_equal(V, o.v), "V pages differ"
    if w.kv_format == "int8":
        assert np.array_equal(KS.view(np.uint32), o.k_scale.view(np.uint32))
        assert np.array_equal(VS.view(np.uint32), o.v_scale.view(np.uint32))
    assert c.status() == 0


@pytest.mark.parametrize("fmt", ["f32", "int8"])
def test_int8_and_f32_rows_with_ties_and_zero_rows(fmt):
    """Rows planted with exact .5 ties after division, all-zero rows and a
    single spike; int8 pages fed with f32 and bf16 rows."""
    require_gpu()
    Hkv, D, bs = 2, 64, 16
    n = 40
    g = torch.Generator().manual_seed(12)
    k = torch.randn(n, Hkv, D, generator=g)
    v = torch.randn(n, Hkv, D, generator=g) * 5
    k[3, 0] = 0.0
    k[4, 1] = 0.0
    k[4, 1, 7] = -3.0
    k[5, 0] = torch.tensor([127.0, 0.5, 1.5, 2.5, -0.5, -2.5] + [0.0] * (D - 6))
    v[6] = 0.0
    table = np.array([[5, 2, 7, 0]], np.int32)
    P = 8
    w = W.Workload("rows", P, bs, Hkv, D, 2 * Hkv, fmt, torch.float32, torch.float32, 0.125,
                   table, np.array([n], np.int32), 0)
    for in_dt in ([torch.float32, torch.bfloat16] if fmt == "int8" else [torch.float32]):
        kk, vv = k.to(in_dt), v.to(in_dt)
        r = W.WriteRound(np.array([3], np.int32), np.array([0, n - 3], np.int32),
                         kk[:n - 3].contiguous(), vv[:n - 3].contiguous())
        c, _ = _run_fill(w, [r])
        o = sentinel_oracle(w)
        o.write(0, table, r.start_pos, r.cu_new, np_bits(r.k), np_bits(r.v), dtype_name(r.k))
        K, V, KS, VS = pages_in_oracle_order(c)
        assert np.array_equal(K, o.k) and np.array_equal(V, o.v)
        if fmt == "int8":
            assert np.array_equal(KS.view(np.uint32), o.k_scale.view(np.uint32))
            assert np.array_equal(VS.view(np.uint32), o.v_scale.view(np.uint32))


@pytest.mark.parametrize("fmt", ["f32", "bf16", "int8"])
@pytest.mark.parametrize("bs", [4, 8, 16, 32])
def test_write_aligned_runs_and_stragglers(fmt, bs):
    """Blocks of rows that fill whole aligned runs of a page's slots (stored
    as vectors along each V dim row) next to blocks that straddle sequences,
    pages or an unaligned start (stored slot by slot), over two rounds."""
    require_gpu()
    Hkv, D = 2, 64
    lens = np.array([80, 37, 64, 21], np.int32)
    npg = [-(-int(n) // bs) for n in lens]
    P = sum(npg) + 3
    perm = np.random.default_rng(bs).permutation(P).astype(np.int32)
    table = np.full((len(lens), max(npg)), -1, np.int32)
    o_ = 0
    for b, n in enumerate(npg):
        table[b, :n] = perm[o_:o_ + n]
        o_ += n
    in_dt = torch.bfloat16 if fmt == "bf16" else torch.float32
    w = W.Workload("runs", P, bs, Hkv, D, 2 * Hkv, fmt, in_dt, in_dt, 0.125, table, lens, 0)
    g = torch.Generator().manual_seed(bs)
    # round 1 writes 48 / 16 / 32 / 5 rows from position 0, round 2 the rest
    first = np.array([48, 16, 32, 5], np.int32)
    rounds = []
    for start, n in ((np.zeros(4, np.int32), first), (first, lens - first)):
        cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
        k = (torch.randn(int(cu[-1]), Hkv, D, generator=g) * 3).to(in_dt)
        v = (torch.randn(int(cu[-1]), Hkv, D, generator=g) * 3).to(in_dt)
        rounds.append(W.WriteRound(start.astype(np.int32), cu, k, v))
    c, _ = _run_fill(w, rounds)
    o = sentinel_oracle(w)
    oracle_write_rounds(o, w, rounds)
    K, V, KS, VS = pages_in_oracle_order(c)
    assert np.array_equal(K, o.k), "K pages differ"
    assert np.array_equal(V, o.v), "V pages differ"
    if fmt == "int8":
        assert np.array_equal(KS.view(np.uint32), o.k_scale.view(np.uint32))
        assert np.array_equal(VS.view(np.uint32), o.v_scale.view(np.uint32))
    assert c.status() == 0


@pytest.mark.parametrize("fmt", ["f32", "bf16", "int8"])
@pytest.mark.parametrize("bs", [5, 16, 32])
def test_write_ragged_starts_and_empty_sequences(fmt, bs):
    """Forty sequences with seeded start positions and row counts (zero, one,
    a few, a hundred) in one call: every position-aligned window of the
    write, full or partly used, against the oracle bit for bit."""
    require_gpu()
    rng = np.random.default_rng(77 + bs)
    Hkv, D, B = 2, 64, 40
    start = rng.integers(0, 300, size=B).astype(np.int32)
    n = rng.choice([0, 1, 2, 7, 15, 16, 17, 33, 100], size=B).astype(np.int32)
    lens = start + n
    npg = [-(-int(x) // bs) for x in lens]
    P = sum(npg) + 2
    perm = rng.permutation(P).astype(np.int32)
    table = np.full((B, max(npg)), -1, np.int32)
    o_ = 0
    for b_, k_ in enumerate(npg):
        table[b_, :k_] = perm[o_:o_ + k_]
        o_ += k_
    in_dt = torch.bfloat16 if fmt == "bf16" else torch.float32
    w = W.Workload("ragged", P, bs, Hkv, D, 2 * Hkv, fmt, in_dt, in_dt, 0.125, table, lens, 0)
    g = torch.Generator().manual_seed(bs)
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    k = (torch.randn(int(cu[-1]), Hkv, D, generator=g) * 2).to(in_dt)
    v = (torch.randn(int(cu[-1]), Hkv, D, generator=g) * 2).to(in_dt)
    r = W.WriteRound(start, cu, k, v)
    c, _ = _run_fill(w, [r])
    o = sentinel_oracle(w)
    oracle_write_rounds(o, w, [r])
    K, V, KS, VS = pages_in_oracle_order(c)
    assert np.array_equal(K, o.k), "K pages differ"
    assert np.array_equal(V, o.v), "V pages differ"
    if fmt == "int8":
        assert np.array_equal(KS.view(np.uint32), o.k_scale.view(np.uint32))
        assert np.array_equal(VS.view(np.uint32), o.v_scale.view(np.uint32))
    assert c.status() == 0


def test_int8_quotients_next_to_half_integers():
    """Rows whose quotients x / scale sit a few float32 ulps either side of
    k + 0.5 (and on it), for scales that are not powers of two: the codes
    must follow the correctly rounded division exactly."""
    require_gpu()
    Hkv, D, bs = 1, 64, 16
    rows = []
    for mx in (100.0, 3.7, 0.011, 2.0e-30):
        s = np.float32(np.float32(mx) / np.float32(127.0))
        for j in range(4):
            row = np.zeros(D, np.float32)
            row[0] = np.float32(mx)
            for i in range(1, D):
                kk = (i * 7 + j * 13) % 126 - 63
                x = np.float32(np.float32(kk + 0.5) * s)
                row[i] = np.nextafter(x, np.float32(np.inf if (i + j) % 2 else -np.inf),
                                      dtype=np.float32) if (i % 5) else x
                for _ in range((i // 5) % 3):
                    row[i] = np.nextafter(row[i], np.float32(np.inf), dtype=np.float32)
            rows.append(row)
    x = torch.from_numpy(np.stack(rows)).reshape(-1, Hkv, D)
    n = x.shape[0]
    table = np.arange(-(-n // bs), dtype=np.int32)[None]
    w = W.Workload("ties", table.shape[1], bs, Hkv, D, Hkv, "int8", torch.float32, torch.float32,
                   0.125, table, np.array([n], np.int32), 0)
    r = W.WriteRound(np.array([0], np.int32), np.array([0, n], np.int32), x, -x)
    c, _ = _run_fill(w, [r])
    o = sentinel_oracle(w)
    oracle_write_rounds(o, w, [r])
    K, V, KS, VS = pages_in_oracle_order(c)
    assert np.array_equal(K, o.k) and np.array_equal(V, o.v)
    assert np.array_equal(KS.view(np.uint32), o.k_scale.view(np.uint32))


# ------------------------------------------------------------------ gather --

@pytest.mark.parametrize("name", NAMES)
def test_gather_round_trip(name):
    require_gpu()
    w = reduced(name)
    say(f"gather {name}")
    c, tdev = _run_fill(w)
    o = sentinel_oracle(w)
    oracle_write_rounds(o, w, w.rounds())
    for b in range(w.batch):
        L = int(w.lens[b])
        k, v, ks, vs = c.gather(tdev[b], L)
        K, V, KS, VS = o.gather(0, w.tables[b], L)
        if w.kv_format == "int8":
            assert np.array_equal(k.cpu().numpy(), K) and np.array_equal(v.cpu().numpy(), V)
            assert np.array_equal(ks.cpu().numpy(), KS) and np.array_equal(vs.cpu().numpy(), VS)
        else:
            kin, vin = w.seq_kv(b)  # gather(write(x)) == x
            assert torch.equal(k.cpu(), kin) and torch.equal(v.cpu(), vin)


# --------------------------------------------------------------- attention --

@pytest.mark.parametrize("flags", [0, pkv.ATTEND_VALU, pkv.ATTEND_COMBINE_KERNEL,
                                   pkv.ATTEND_COMBINE_FUSED],
                         ids=["auto", "valu", "combine_kernel", "combine_fused"])
@pytest.mark.parametrize("split", [0, "unit"])
@pytest.mark.parametrize("name", NAMES)
def test_attend_parity(name, split, flags):
    require_gpu()
    w = reduced(name)
    split_tokens = 0 if split == 0 else int(64 // np.gcd(64, w.page_size) * w.page_size)
    say(f"attend {name} split={split_tokens} flags={flags}")
    c, tdev = _run_fill(w)
    o = sentinel_oracle(w)
    oracle_write_rounds(o, w, w.rounds())
    q = w.query()
    out = c.attend(q.cuda(), tdev, dev(w.lens), w.max_len, w.scale, split_tokens=split_tokens,
                   flags=flags)
    ref = attend(o, 0, np_bits(q), dtype_name(q), w.tables, w.lens, w.scale)
    err = max_err(out, ref)
    say(f"  max err {err:.3e} (tol {TOL[w.kv_format]})")
    assert err <= TOL[w.kv_format]
    assert c.status() == 0


DECODE_SHAPES = [
    # fmt, Hq, Hkv, D, bs: every group size class and page-size path of the
    # matrix-core kernel (16- and 32-token pages and the general multiple of 32)
    ("bf16", 8, 8, 128, 16),    # G = 1
    ("bf16", 12, 4, 64, 32),    # G = 3
    ("bf16", 32, 2, 128, 64),   # G = 16, 64-token pages
    ("bf16", 16, 8, 64, 128),   # G = 2, 128-token pages
    ("int8", 8, 8, 64, 16),     # G = 1
    ("int8", 20, 4, 128, 64),   # G = 5
    ("int8", 32, 2, 64, 32),    # G = 16
]


@pytest.mark.parametrize("case", DECODE_SHAPES,
                         ids=lambda c: f"{c[0]}-G{c[1] // c[2]}-D{c[3]}-bs{c[4]}")
def test_attend_group_and_page_shapes(case):
    """Decode attention over seeded ragged lengths for group sizes 1 to 16,
    head dims 64 and 128 and pages of 16, 32, 64 and 128 tokens, with the
    planned split and with one-unit splits (many partials to combine)."""
    require_gpu()
    fmt, Hq, Hkv, D, bs = case
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    lens = rng.integers(1, 900, size=5).astype(np.int32)
    lens[0] = 1
    npg = [-(-int(n) // bs) for n in lens]
    P = sum(npg) + 3
    perm = rng.permutation(P).astype(np.int32)
    tables = np.full((len(lens), max(npg)), -1, np.int32)
    o_ = 0
    for b, n in enumerate(npg):
        tables[b, :n] = perm[o_:o_ + n]
        o_ += n
    w = W.Workload("shapes", P, bs, Hkv, D, Hq, fmt, torch.bfloat16, torch.bfloat16,
                   float(np.float32(D ** -0.5)), tables, lens, 91)
    say(f"decode {fmt} G={Hq // Hkv} D={D} bs={bs} lens={lens.tolist()}")
    c = make_cache(w, sentinel=0xFF)
    tdev = dev(w.tables)
    gpu_write(c, tdev, w.rounds())
    o = sentinel_oracle(w, 0xFF)
    oracle_write_rounds(o, w, w.rounds())
    q = w.query()
    ref = attend(o, 0, np_bits(q), dtype_name(q), tables, lens, w.scale)
    unit = int(64 // np.gcd(64, bs) * bs)
    for split in (0, unit):
        out = c.attend(q.cuda(), tdev, dev(lens), int(lens.max()), w.scale, split_tokens=split)
        e = max_err(out, ref)
        say(f"  split {split}: max err {e:.3e}")
        assert e <= TOL[fmt], split
    assert c.status() == 0


@pytest.mark.parametrize("fill", [0x5A, 0xFF], ids=["finite", "nan"])
@pytest.mark.parametrize("fmt,D", [("f32", 64), ("bf16", 128), ("bf16", 64), ("int8", 128)])
def test_attend_edge_lengths(fmt, D, fill):
    """Lengths 0, 1, one short of / exactly / one past a page, a tile and a
    split; max_len larger than every length.  With fill 0xFF every slot no
    write reached holds NaN (f32/bf16) or a NaN scale (int8): slots past a
    length must never reach the result."""
    require_gpu()
    bs, Hkv, Hq = 16, 2, 16
    lens = np.array([0, 1, 15, 16, 17, 63, 64, 65, 255, 256, 257, 700], np.int32)
    rng = np.random.default_rng(21)
    npg = [-(-int(n) // bs) for n in lens]
    P = sum(npg) + 5
    perm = rng.permutation(P).astype(np.int32)
    stride = 48
    tables = np.full((len(lens), stride), -1, np.int32)
    o_ = 0
    for b, n in enumerate(npg):
        tables[b, :n] = perm[o_:o_ + n]
        o_ += n
    dt = torch.float32 if fmt == "f32" else torch.bfloat16
    w = W.Workload("edge", P, bs, Hkv, D, Hq, fmt, dt, dt, float(np.float32(D ** -0.5)), tables,
                   lens, 77)
    c = make_cache(w, sentinel=fill)
    tdev = dev(w.tables)
    gpu_write(c, tdev, w.rounds())
    o = sentinel_oracle(w)
    oracle_write_rounds(o, w, w.rounds())
    q = w.query()
    max_len = stride * bs
    for flags in (0, pkv.ATTEND_VALU, pkv.ATTEND_COMBINE_KERNEL, pkv.ATTEND_COMBINE_FUSED):
        for split in (0, 64, 256):
            out = c.attend(q.cuda(), tdev, dev(lens), max_len, w.scale, split_tokens=split,
                           flags=flags)
            ref = attend(o, 0, np_bits(q), dtype_name(q), tables, lens, w.scale)
            assert max_err(out, ref) <= TOL[fmt], (flags, split)
            oc = out.cpu()
            assert not oc[0].float().any(), "empty sequence must give zeros"
            if fmt != "int8":
                k1, v1 = w.seq_kv(1)
                for h in range(Hq):  # one token: exactly its V row
                    assert torch.equal(oc[1, h], v1[0, h // (Hq // Hkv)].to(dt))
    assert c.status() == 0


def test_split_and_kernel_agreement_and_determinism():
    require_gpu()
    w = W.decode_bf16(batch=8, lo=300, hi=2500, seed=31)
    c, tdev = _run_fill(w)
    q = w.query().cuda()
    lens = dev(w.lens)
    outs = {}
    for flags in (0, pkv.ATTEND_VALU, pkv.ATTEND_COMBINE_KERNEL, pkv.ATTEND_COMBINE_FUSED):
        for split in (64, 256, 1024, 0):
            outs[flags, split] = c.attend(q, tdev, lens, w.max_len, w.scale, split_tokens=split,
                                          flags=flags).float()
    base = outs[0, 0]
    for key, o in outs.items():
        assert (o - base).abs().max().item() <= 2 * TOL["bf16"], key
    again = c.attend(q, tdev, lens, w.max_len, w.scale).float()
    assert torch.equal(again, base)


@pytest.mark.parametrize("fmt", ["bf16", "int8"])
def test_page_permutation_bit_identical(fmt):
    """Relabelling the physical pages (moving each page's slabs and remapping
    the tables) leaves every GPU output bit-identical."""
    require_gpu()
    w = reduced("int8_kv") if fmt == "int8" else reduced("decode_bf16")
    c, tdev = _run_fill(w)
    q = w.query().cuda()
    out = c.attend(q, tdev, dev(w.lens), w.max_len, w.scale)
    pi = np.random.default_rng(3).permutation(w.n_pages)
    c2 = make_cache(w)
    pit = torch.as_tensor(pi).cuda()
    c2.k_view()[:, pit] = c.k_view()
    c2.v_view()[:, pit] = c.v_view()
    if fmt == "int8":
        for dst, src in zip(c2.scale_views(), c.scale_views()):
            dst[:, pit] = src
    t2 = np.where(w.tables >= 0, pi[np.maximum(w.tables, 0)], -1)
    out2 = c2.attend(q, dev(t2), dev(w.lens), w.max_len, w.scale)
    assert torch.equal(out, out2)


def test_shared_prefix_steps_and_bit_identity():
    """Shared-prefix decode: each step appends one row per sequence and attends;
    outputs match the oracle, and sharing tables give bit-identical outputs
    to tables with private copies of the prefix."""
    require_gpu()
    sp = W.shared_prefix(batch=12, prefix_pages=8, lo=16, hi=300, n_steps=4)
    w = sp.base
    c = make_cache(w)
    tdev = dev(w.tables)
    fill = sp.fill_rounds()
    gpu_write(c, tdev, fill)
    o = sentinel_oracle(w)
    oracle_write_rounds(o, w, fill)
    # a second cache whose tables hold private copies of the prefix
    P2 = w.n_pages + w.batch * sp.prefix_pages
    w2 = W.Workload("private", P2, w.page_size, w.n_kv_heads, w.head_dim, w.n_q_heads, "bf16",
                    w.in_dtype, w.q_dtype, w.scale, w.tables.copy(), w.lens, 0)
    for b in range(w.batch):
        w2.tables[b, :sp.prefix_pages] = w.n_pages + b * sp.prefix_pages + np.arange(sp.prefix_pages)
    c2 = make_cache(w2)
    t2 = dev(w2.tables)
    pk, pv = sp.prefix_kv()
    B = w.batch
    r0 = W.WriteRound(np.zeros(B, np.int32), np.arange(B + 1, dtype=np.int32) * sp.prefix_tokens,
                      pk.repeat(B, 1, 1).contiguous(), pv.repeat(B, 1, 1).contiguous())
    gpu_write(c2, t2, [r0, fill[1]])
    for s in range(sp.n_steps):
        r = sp.step_round(s)
        gpu_write(c, tdev, [r])
        gpu_write(c2, t2, [r])
        oracle_write_rounds(o, w, [r])
        q = w.query(step=s)
        lens = sp.step_lens(s)
        out = c.attend(q.cuda(), tdev, dev(lens), int(lens.max()), w.scale)
        out2 = c2.attend(q.cuda(), t2, dev(lens), int(lens.max()), w.scale)
        ref = attend(o, 0, np_bits(q), "bf16", w.tables, lens, w.scale)
        assert max_err(out, ref) <= TOL["bf16"], s
        assert torch.equal(out, out2), s
    assert c.status() == 0 and c2.status() == 0


# ------------------------------------------------------- device-side checks --

def test_device_status_flags_without_fault():
    """Bad table entries and positions are skipped and reported, never
    dereferenced; the good rows are still written."""
    require_gpu()
    w = W.tiny_f32()
    bad = w.tables.copy()
    bad[1, 1] = w.n_pages + 9  # rows 16..31 of sequence 1 point outside the pool
    c = make_cache(w)
    tdev = dev(bad)
    r = w.rounds()[0]
    gpu_write(c, tdev, [r])
    assert c.status() & pkv.DEV_WRITE_PAGE
    o = sentinel_oracle(w)
    good = r.cu_new.copy()
    # the oracle writes everything except sequence 1's second page
    o.write(0, w.tables, r.start_pos[:1], good[:2], np_bits(r.k)[:37], np_bits(r.v)[:37], "f32")
    k1 = np_bits(r.k)[37:]
    v1 = np_bits(r.v)[37:]
    keep = [i for i in range(50) if not 16 <= i < 32]
    o.write(0, w.tables[1:], np.array([0]), np.array([0, 16]), k1[:16], v1[:16], "f32")
    o.write(0, w.tables[1:], np.array([32]), np.array([0, 18]), k1[32:], v1[32:], "f32")
    assert len(keep) == 34
    K, V, _, _ = pages_in_oracle_order(c)
    assert np.array_equal(K, o.k) and np.array_equal(V, o.v)
    # a position past the table row
    c2 = make_cache(w)
    short = np.ascontiguousarray(w.tables[:, :2])
    c2.write(dev(short), dev(np.array([0, 0], np.int32)), dev(r.cu_new), r.k.cuda(), r.v.cuda())
    assert c2.status() & pkv.DEV_WRITE_TABLE
    # decreasing row offsets: the malformed sequence is skipped and reported
    c5 = make_cache(w)
    badcu = np.array([0, 40, 30], np.int32)
    c5.write(tdev, dev(r.start_pos), dev(badcu), r.k[:30].cuda(), r.v[:30].cuda())
    torch.cuda.synchronize()
    assert c5.status() & pkv.DEV_WRITE_ROWS
    # attention over a bad entry and a length past the bound
    c3, t3 = _run_fill(w)
    q = w.query().cuda()
    badt = w.tables.copy()
    badt[0, 1] = -7
    c3.attend(q, dev(badt), dev(w.lens), 50, w.scale)
    torch.cuda.synchronize()
    assert c3.status() & pkv.DEV_READ_PAGE
    c4, t4 = _run_fill(w)
    c4.attend(q, t4, dev(np.array([37, 50], np.int32)), 40, w.scale)
    torch.cuda.synchronize()
    assert c4.status() & pkv.DEV_LEN


def test_table_apply_and_seq_tables():
    require_gpu()
    pool = pkv.PagePool(64)
    s = pkv.SeqTables(pool, 3, 8, 16)
    s.append(0, 40)
    s.share(1, 0, 2)
    s.append(1, 9)
    s.append(2, 100)
    table = dev(np.full((3, 8), -1, np.int32))
    upd = s.take_updates()
    pkv.table_apply(table, upd.cuda())
    assert table.cpu().tolist() == s.table()
    s.release(2)
    pkv.table_apply(table, s.take_updates().cuda())
    assert table.cpu().tolist() == s.table()


def test_workspace_reuse_across_calls():
    """One workspace, many calls: lengths, batch subsets and split sizes change
    from call to call; every call must match a fresh-workspace call bit for
    bit (the split counters are left at zero by each call)."""
    require_gpu()
    w = W.decode_bf16(batch=12, lo=50, hi=3000, seed=41)
    c, tdev = _run_fill(w)
    q = w.query().cuda()
    rng = np.random.default_rng(5)
    ws = c.workspace(w.batch, w.n_q_heads, w.max_len, 64)  # largest need: the smallest split
    for it in range(40):
        lens = np.minimum(w.lens, rng.integers(0, w.max_len + 1, size=w.batch)).astype(np.int32)
        lens[rng.integers(0, w.batch)] = w.lens.max() if it % 3 == 0 else lens[0]
        lens = np.minimum(lens, w.lens)
        split = [0, 64, 128, 256, 1024][it % 5]
        B = w.batch if it % 4 else 7
        fl = [0, pkv.ATTEND_COMBINE_FUSED, pkv.ATTEND_COMBINE_KERNEL][it % 3]
        ld = dev(lens[:B])
        out = c.attend(q[:B].contiguous(), tdev[:B].contiguous(), ld, w.max_len, w.scale,
                       workspace=ws, split_tokens=split, flags=fl)
        ref = c.attend(q[:B].contiguous(), tdev[:B].contiguous(), ld, w.max_len, w.scale,
                       split_tokens=split, flags=fl)
        assert torch.equal(out, ref), it
    assert c.status() == 0
