"""The allocation-free attend (static scratch, no workspace argument) against
pkv_paged_attend on the same inputs: two calls in a row on one device, the
second with a smaller batch, each bit for bit equal to the workspace call and
within tolerance of the oracle; plus its host-side refusals."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import attend
from paged_kv_cache_207_amd import pkv
from paged_kv_cache_207_amd import workloads as W
from tests.gpu_helpers import TOL, dev, gpu_write, make_cache, max_err, require_gpu, say
from tests.helpers import dtype_name, np_bits, oracle_write_rounds
from tests.gpu_helpers import sentinel_oracle

pytestmark = pytest.mark.gpu


def _check_pair(c, o, w, seqs, split_tokens=0, flags=0):
    """Attend over sequences `seqs` of workload w both ways; compare."""
    q = w.query()[seqs].contiguous()
    tables = np.ascontiguousarray(w.tables[seqs])
    lens = np.ascontiguousarray(w.lens[seqs])
    max_len = int(lens.max())
    tdev, ldev, qdev = dev(tables), dev(lens), q.cuda()
    ref_gpu = c.attend(qdev, tdev, ldev, max_len, w.scale, split_tokens=split_tokens, flags=flags)
    out = torch.full_like(qdev, float("nan"))
    c.attend_noalloc(qdev, tdev, ldev, max_len, w.scale, out, split_tokens=split_tokens,
                     flags=flags)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_gpu)
    ref = attend(o, 0, np_bits(q), dtype_name(q), tables, lens, w.scale)
    e = max_err(out, ref)
    say(f"  {len(seqs)} sequences, max_len {max_len}, split {split_tokens}, flags {flags}: "
        f"max err {e:.3e}")
    assert e <= TOL[w.kv_format]
    assert c.status() == 0


def test_noalloc_matches_workspace_attend():
    require_gpu()
    # bf16 pages, uneven lengths: the balanced schedule with its piece records
    w = W.decode_bf16(batch=24, lo=100, hi=3000, n_q_heads=16, n_kv_heads=4, head_dim=128,
                      seed=31)
    c = make_cache(w)
    gpu_write(c, dev(w.tables), w.rounds())
    o = sentinel_oracle(w)
    oracle_write_rounds(o, w, w.rounds())
    say("bf16 workload, full batch then a smaller one")
    _check_pair(c, o, w, list(range(24)))
    _check_pair(c, o, w, [3, 7, 11])  # smaller: the scratch keeps the first call's data
    _check_pair(c, o, w, list(range(10)), split_tokens=64)
    _check_pair(c, o, w, [5], flags=pkv.ATTEND_VALU)

    # int8 pages (fixed splits), again a big call then a small one
    wi = W.int8_kv(batch=16, lo=64, hi=4000, n_q_heads=16, n_kv_heads=2, head_dim=64,
                   page_size=32, chunk=100, seed=32)
    ci = make_cache(wi)
    gpu_write(ci, dev(wi.tables), wi.rounds())
    oi = sentinel_oracle(wi)
    oracle_write_rounds(oi, wi, wi.rounds())
    say("int8 workload, full batch then a smaller one")
    _check_pair(ci, oi, wi, list(range(16)))
    _check_pair(ci, oi, wi, [0, 9])


def test_noalloc_refusals():
    require_gpu()
    w = W.decode_bf16(batch=2, lo=10, hi=40, n_q_heads=8, n_kv_heads=2, head_dim=64, seed=33)
    c = make_cache(w)
    q = w.query().cuda()
    out = torch.empty_like(q)
    t, L = dev(w.tables), dev(w.lens)
    with pytest.raises(pkv.PkvError) as e:
        c.attend_noalloc(q, t, L, w.max_len, w.scale, out, flags=pkv.ATTEND_COMBINE_FUSED)
    assert e.value.code == pkv.EINVAL
    # sizes whose workspace exceeds the static array are refused before any launch
    big = pkv.PagedKVCache(16, 16, 8, 256, "int8")
    qb = torch.zeros(4096, 128, 256, dtype=torch.bfloat16, device="cuda")
    tb = torch.zeros(4096, 1, dtype=torch.int32, device="cuda")
    lb = torch.zeros(4096, dtype=torch.int32, device="cuda")
    need = big.workspace_size(4096, 128, 16, 64)
    assert need > 64 << 20
    with pytest.raises(pkv.PkvError) as e:
        big.attend_noalloc(qb, tb, lb, 16, 0.1, torch.empty_like(qb), split_tokens=64)
    assert e.value.code == pkv.ENOMEM
    assert c.status() == 0 and big.status() == 0
