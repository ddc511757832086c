"""The fused decode step (write one row per sequence at lens - 1, then attend)
against the two separate calls it replaces, and against the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import attend
from paged_kv_cache_207_amd import pkv
from paged_kv_cache_207_amd import workloads as W
from tests.gpu_helpers import (TOL, dev, make_cache, max_err, pages_in_oracle_order, require_gpu,
                               say, sentinel_oracle)
from tests.helpers import dtype_name, np_bits

pytestmark = pytest.mark.gpu


def workload(name):
    return {
        "tiny_f32": lambda: W.tiny_f32(),
        "decode_bf16": lambda: W.decode_bf16(batch=6, lo=1, hi=700, seed=13),
        "long_bf16": lambda: W.long_bf16(batch=2, seq_len=2999),
        "int8_kv": lambda: W.int8_kv(batch=6, lo=1, hi=2000, seed=14),
        "d64": lambda: W.decode_bf16(batch=5, lo=1, hi=900, n_q_heads=16, n_kv_heads=4,
                                      head_dim=64, seed=15),
    }[name]()


def fill_all_but_last(c, w, tdev, kv):
    """Every sequence's rows except its newest token, one write per sequence."""
    for b in range(w.batch):
        L = int(w.lens[b])
        if L > 1:
            k, v = kv[b]
            c.write(tdev[b:b + 1].contiguous(), dev(np.zeros(1, np.int32)),
                    dev(np.array([0, L - 1], np.int32)), k[:L - 1].cuda(), v[:L - 1].cuda())


def newest_rows(w, kv):
    k = torch.stack([kv[b][0][int(w.lens[b]) - 1] for b in range(w.batch)])
    v = torch.stack([kv[b][1][int(w.lens[b]) - 1] for b in range(w.batch)])
    return k.contiguous(), v.contiguous()


@pytest.mark.parametrize("flags", [0, pkv.ATTEND_VALU, pkv.ATTEND_COMBINE_FUSED],
                         ids=["auto", "valu", "combine_fused"])
@pytest.mark.parametrize("name", ["tiny_f32", "decode_bf16", "long_bf16", "int8_kv", "d64"])
def test_decode_step_equals_write_then_attend(name, flags):
    require_gpu()
    w = workload(name)
    say(f"decode step {name} flags={flags}")
    kv = {b: w.seq_kv(b) for b in range(w.batch)}
    kn, vn = newest_rows(w, kv)
    tdev = dev(w.tables)
    lens = dev(w.lens)
    q = w.query().cuda()
    a = make_cache(w)
    fill_all_but_last(a, w, tdev, kv)
    out_a = a.decode_step(tdev, lens, w.max_len, kn.cuda(), vn.cuda(), q, w.scale, flags=flags)
    b_ = make_cache(w)
    fill_all_but_last(b_, w, tdev, kv)
    b_.write(tdev, dev(w.lens - 1), dev(np.arange(w.batch + 1, dtype=np.int32)), kn.cuda(),
             vn.cuda())
    out_b = b_.attend(q, tdev, lens, w.max_len, w.scale, flags=flags)
    assert torch.equal(out_a, out_b)
    for x, y in zip(pages_in_oracle_order(a), pages_in_oracle_order(b_)):
        if x is not None:
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8))
    # and against the oracle
    o = sentinel_oracle(w)
    o.write(0, w.tables, np.zeros(w.batch, np.int32),
            np.concatenate([[0], np.cumsum(w.lens)]).astype(np.int32),
            np.concatenate([np_bits(kv[b][0]) for b in range(w.batch)]),
            np.concatenate([np_bits(kv[b][1]) for b in range(w.batch)]), dtype_name(kn))
    ref = attend(o, 0, np_bits(q.cpu()), dtype_name(q), w.tables, w.lens, w.scale)
    assert max_err(out_a, ref) <= TOL[w.kv_format]
    assert a.status() == 0


def test_decode_step_edge_lengths_and_loop():
    """Lengths 0 (no row, zero output) and 1 (the first token); then 40 steps
    of a growing batch, each checked against write + attend bit for bit."""
    require_gpu()
    bs, Hkv, Hq, D = 16, 2, 8, 128
    B, steps = 5, 40
    start = np.array([0, 0, 15, 16, 70], np.int32)
    final = start + steps
    npg = [-(-int(n) // bs) for n in final]
    P = sum(npg) + 3
    perm = np.random.default_rng(9).permutation(P).astype(np.int32)
    stride = max(npg)
    tables = np.full((B, stride), -1, np.int32)
    o_ = 0
    for b, n in enumerate(npg):
        tables[b, :n] = perm[o_:o_ + n]
        o_ += n
    w = W.Workload("loop", P, bs, Hkv, D, Hq, "bf16", torch.bfloat16, torch.bfloat16,
                   float(np.float32(D ** -0.5)), tables, final, 3)
    kv = {b: w.seq_kv(b) for b in range(B)}
    tdev = dev(tables)
    a, c = make_cache(w), make_cache(w)
    for cache in (a, c):
        for b in range(B):
            if start[b] > 0:
                cache.write(tdev[b:b + 1].contiguous(), dev(np.zeros(1, np.int32)),
                            dev(np.array([0, start[b]], np.int32)), kv[b][0][:start[b]].cuda(),
                            kv[b][1][:start[b]].cuda())
    zero_len = np.array([0, 1, 1, 1, 1], np.int32)  # sequence 0 stays empty in step 0
    for s in range(steps):
        lens = start + s + 1
        if s == 0:
            lens = np.where(zero_len == 0, 0, lens).astype(np.int32)
        idx = np.maximum(lens - 1, 0)
        kn = torch.stack([kv[b][0][idx[b]] for b in range(B)]).contiguous().cuda()
        vn = torch.stack([kv[b][1][idx[b]] for b in range(B)]).contiguous().cuda()
        q = w.query(step=s).cuda()
        ld = dev(lens)
        max_len = int(final.max())
        out_a = a.decode_step(tdev, ld, max_len, kn, vn, q, w.scale)
        if s == 0:
            assert not out_a[0].float().any()  # empty sequence: zero output
        keep = lens > 0
        cu = np.concatenate([[0], np.cumsum(keep)]).astype(np.int32)
        mask = torch.as_tensor(keep).cuda()
        c.write(tdev, dev(np.where(keep, lens - 1, 0)), dev(cu), kn[mask].contiguous(),
                vn[mask].contiguous())
        out_c = c.attend(q, tdev, ld, max_len, w.scale)
        assert torch.equal(out_a, out_c), s
        if s == 0:
            start = np.where(zero_len == 0, start - 1, start)  # sequence 0 starts one step late
    for x, y in zip(pages_in_oracle_order(a), pages_in_oracle_order(c)):
        if x is not None:
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8))
    assert a.status() == 0 and c.status() == 0
