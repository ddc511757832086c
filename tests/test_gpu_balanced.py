"""The balanced schedule of the matrix-core decode pass (bf16 pages, planned
split): each wave takes an equal share of all (sequence, KV head) units'
32-token steps, so a unit may be cut anywhere and its pieces merged by the
combine kernel from the record its first piece leaves in the workspace.

Checked against the float64 oracle at the bf16 tolerance on batches that
stress the partition: many short sequences beside a few long ones, empty
sequences, one sequence cut into more than 64 pieces (the combine's path for
many pieces), a workspace reused by calls whose lengths cut the units
differently (equal lengths take fixed splits inside the same kernel), and the
decode step.  Fixed splits of the same call agree within
tolerance; the same call repeated is bit-identical.
"""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

from oracle import attend
from paged_kv_cache_207_amd import workloads as W
from tests.gpu_helpers import (TOL, dev, gpu_write, make_cache, max_err, require_gpu, say,
                               sentinel_oracle)
from tests.helpers import dtype_name, np_bits, oracle_write_rounds

pytestmark = pytest.mark.gpu


def _workload(name, lens, Hq, Hkv, D, bs, seed):
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, np.int32)
    npg = [-(-int(n) // bs) for n in lens]
    P = sum(npg) + 4
    perm = rng.permutation(P).astype(np.int32)
    tables = np.full((len(lens), max(max(npg), 1)), -1, np.int32)
    o_ = 0
    for b, n in enumerate(npg):
        tables[b, :n] = perm[o_:o_ + n]
        o_ += n
    return W.Workload(name, P, bs, Hkv, D, Hq, "bf16", torch.bfloat16, torch.bfloat16,
                      float(np.float32(D ** -0.5)), tables, lens, seed)


def _filled(w):
    c = make_cache(w)
    tdev = dev(w.tables)
    gpu_write(c, tdev, w.rounds())
    o = sentinel_oracle(w)
    oracle_write_rounds(o, w, w.rounds())
    return c, tdev, o


CASES = {
    # many short sequences (a wave covers several units) beside long ones
    "skewed": dict(lens=[3000, 7, 40, 1, 2500, 33, 64, 65, 0, 18, 900, 5, 31, 32, 2],
                   Hq=32, Hkv=8, D=128, bs=16),
    # G = 1 and 32-token pages
    "mha_bs32": dict(lens=[1200, 3, 0, 450, 77, 1999], Hq=4, Hkv=4, D=64, bs=32),
    # 64-token pages: pieces may start inside a page
    "bs64": dict(lens=[1500, 100, 31, 1024, 6], Hq=16, Hkv=2, D=128, bs=64),
}


@pytest.mark.parametrize("case", list(CASES))
def test_balanced_against_oracle_and_fixed_splits(case):
    require_gpu()
    k = CASES[case]
    w = _workload(case, k["lens"], k["Hq"], k["Hkv"], k["D"], k["bs"],
                  zlib.crc32(case.encode()))
    say(f"balanced {case}: lens={w.lens.tolist()}")
    c, tdev, o = _filled(w)
    q = w.query()
    ref = attend(o, 0, np_bits(q), dtype_name(q), w.tables, w.lens, w.scale)
    lens = dev(w.lens)
    planned = c.attend(q.cuda(), tdev, lens, w.max_len, w.scale)
    e = max_err(planned, ref)
    say(f"  planned: max err {e:.3e}")
    assert e <= TOL["bf16"]
    unit = int(64 // np.gcd(64, w.page_size) * w.page_size)
    fixed = c.attend(q.cuda(), tdev, lens, w.max_len, w.scale, split_tokens=unit)
    assert max_err(fixed, ref) <= TOL["bf16"]
    assert float((planned.float() - fixed.float()).abs().max()) <= TOL["bf16"]
    again = c.attend(q.cuda(), tdev, lens, w.max_len, w.scale)
    assert torch.equal(planned, again)
    zero = np.flatnonzero(w.lens == 0)
    assert not planned[zero].float().abs().any()
    assert c.status() == 0


def test_balanced_one_sequence_many_pieces():
    """One (sequence, KV head) unit long enough to be cut into more than 64
    pieces, so the combine weighs them through LDS."""
    require_gpu()
    w = _workload("one_long", [70000], Hq=8, Hkv=1, D=64, bs=16, seed=5)
    c, tdev, o = _filled(w)
    q = w.query()
    ref = attend(o, 0, np_bits(q), dtype_name(q), w.tables, w.lens, w.scale)
    out = c.attend(q.cuda(), tdev, dev(w.lens), w.max_len, w.scale)
    e = max_err(out, ref)
    say(f"one sequence of 70000 tokens: max err {e:.3e}")
    assert e <= TOL["bf16"]
    assert c.status() == 0


def test_balanced_workspace_reused_across_lengths():
    """One workspace, calls whose lengths cut the units differently (units
    that had several pieces now have one, and the reverse): stale records
    from the earlier call must not leak into the later one."""
    require_gpu()
    w = _workload("reuse", [2000, 1500, 900, 40, 3000, 10], Hq=16, Hkv=4, D=128, bs=16, seed=9)
    c, tdev, o = _filled(w)
    q = w.query()
    ws = c.workspace(w.batch, w.n_q_heads, w.max_len)
    # equal non-empty lengths take fixed splits inside the same kernel; the
    # combine must follow that choice, and the next uneven call switch back
    for lens in ([2000, 1500, 900, 40, 3000, 10], [5, 1500, 1, 40, 100, 10],
                 [2000, 0, 900, 39, 3000, 9], [1, 1, 1, 1, 1, 1],
                 [900, 0, 900, 0, 900, 0], [2000, 1500, 900, 40, 3000, 10]):
        lens = np.asarray(lens, np.int32)
        ref = attend(o, 0, np_bits(q), dtype_name(q), w.tables, lens, w.scale)
        out = c.attend(q.cuda(), tdev, dev(lens), w.max_len, w.scale, workspace=ws)
        e = max_err(out, ref)
        say(f"  lens {lens.tolist()}: max err {e:.3e}")
        assert e <= TOL["bf16"]
    assert c.status() == 0


def test_balanced_decode_step_matches_write_then_attend():
    """The decode step under the balanced schedule: the piece holding a
    unit's last step writes the new row; pages and outputs equal a page write
    followed by attention, bit for bit."""
    require_gpu()
    w = _workload("step", [700, 1, 33, 2100, 15, 64, 0, 500], Hq=32, Hkv=8, D=128, bs=16, seed=13)
    lens_new = np.where(w.lens > 0, w.lens, 0).astype(np.int32)
    # room for one more token: the tables already cover ceil(len / bs) pages;
    # sequences whose next token opens a page get one of the spare pages
    tables = np.concatenate([w.tables, np.full((w.batch, 1), -1, np.int32)], axis=1)
    used = set(int(x) for x in w.tables.ravel() if x >= 0)
    spare = iter([p for p in range(w.n_pages) if p not in used])
    for b, n in enumerate(lens_new):
        if n > 0 and n % w.page_size == 0:
            tables[b, n // w.page_size] = next(spare)
    w2 = W.Workload("step", w.n_pages, w.page_size, w.n_kv_heads, w.head_dim, w.n_q_heads,
                    "bf16", torch.bfloat16, torch.bfloat16, w.scale, tables, w.lens, w.seed)
    step_lens = np.where(w.lens > 0, w.lens + 1, 0).astype(np.int32)
    gen = torch.Generator().manual_seed(77)
    k_new = torch.randn(w.batch, w.n_kv_heads, w.head_dim, generator=gen).to(torch.bfloat16).cuda()
    v_new = torch.randn(w.batch, w.n_kv_heads, w.head_dim, generator=gen).to(torch.bfloat16).cuda()
    q = w.query().cuda()
    tdev = dev(tables)
    max_len = int(step_lens.max())
    outs, pages = [], []
    for fused in (True, False):
        c = make_cache(w2)
        gpu_write(c, tdev, w2.rounds())
        if fused:
            out = c.decode_step(tdev, dev(step_lens), max_len, k_new, v_new, q, w.scale)
        else:
            live = np.flatnonzero(step_lens > 0)
            start = np.maximum(step_lens - 1, 0).astype(np.int32)
            cu = np.concatenate([[0], np.cumsum(step_lens > 0)]).astype(np.int32)
            c.write(tdev, dev(start), dev(cu), k_new[live].contiguous(), v_new[live].contiguous())
            out = c.attend(q, tdev, dev(step_lens), max_len, w.scale)
        outs.append(out)
        pages.append((c.k_pages.clone(), c.v_pages.clone()))
        assert c.status() == 0
    assert torch.equal(outs[0], outs[1])
    assert torch.equal(pages[0][0], pages[1][0]) and torch.equal(pages[0][1], pages[1][1])


@pytest.mark.parametrize("fmt,n_seq", [("bf16", 700), ("int8", 700), ("bf16", 65),
                                       ("int8", 65), ("bf16", 4096), ("int8", 4096)])
def test_many_sequences_scan_blocks(fmt, n_seq):
    """Many short sequences, some empty, for the balanced schedule (bf16)
    and fixed splits (int8).  The schedule's prefix sums give each of the 64
    lanes a run of ceil(n / 64) consecutive sequences: 700 leaves the last
    lane a shorter run, 65 one lane a run of 1 and the rest none, and 4096
    (the most a call takes) fills every lane with 64."""
    require_gpu()
    rng = np.random.default_rng(700 + n_seq)
    lens = rng.integers(0, 90 if n_seq < 4096 else 40, size=n_seq).astype(np.int32)
    lens[::37] = 0
    lens[5] = 400
    bs = 16
    npg = [-(-int(n) // bs) for n in lens]
    P = sum(npg) + 4
    perm = rng.permutation(P).astype(np.int32)
    tables = np.full((len(lens), max(npg)), -1, np.int32)
    o_ = 0
    for b, n in enumerate(npg):
        tables[b, :n] = perm[o_:o_ + n]
        o_ += n
    w = W.Workload("many", P, bs, 2, 64, 8, fmt, torch.bfloat16, torch.bfloat16,
                   float(np.float32(64 ** -0.5)), tables, lens, 77)
    c, tdev, o = _filled(w)
    q = w.query()
    ref = attend(o, 0, np_bits(q), dtype_name(q), w.tables, w.lens, w.scale)
    out = c.attend(q.cuda(), tdev, dev(w.lens), w.max_len, w.scale)
    e = max_err(out, ref)
    say(f"{n_seq} sequences ({fmt}): max err {e:.3e}")
    assert e <= TOL[fmt]
    assert not out[np.flatnonzero(w.lens == 0)].float().abs().any()
    assert c.status() == 0


def test_max_len_zero_after_balanced_call():
    """A call with max_len 0 (every length 0) on a workspace that a balanced
    call used before: no split pass runs, and the combine must still write
    the zero outputs rather than follow the earlier call's schedule record."""
    require_gpu()
    w = _workload("zero", [900, 20, 1700, 5], Hq=16, Hkv=4, D=128, bs=16, seed=21)
    c, tdev, o = _filled(w)
    q = w.query().cuda()
    ws = c.workspace(w.batch, w.n_q_heads, w.max_len)
    first = c.attend(q, tdev, dev(w.lens), w.max_len, w.scale, workspace=ws)
    assert first.float().abs().sum() > 0
    zeros = np.zeros(w.batch, np.int32)
    out = torch.full_like(q, 7.0)
    c.attend(q, tdev, dev(zeros), 0, w.scale, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert not out.float().abs().any()
    assert c.status() == 0
