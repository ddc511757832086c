#!/usr/bin/env python3
"""Paged KV cache decode steps on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload all]

A step is one pass of the hot path over the batch: one pkv_decode_step call
that writes one new K/V row per sequence (at position len-1, the newest
token) and runs paged attention (split-K partial pass + combine) of one query
per sequence over all len tokens, read in place through a fully fragmented
block table.  The K/V pages are filled once before timing.  Prints one JSON
line (stdout); details go to stderr.

The default run measures the headline (the 32k-token bf16 workload: 8
sequences x 32 768 tokens, 64 query / 8 KV heads, head_dim 128, 16-token
pages) and, under "configs", the other four workloads: the tiny f32 one, the
uneven bf16 decode batch, the int8 batch and the shared-prefix job (32 steps
of host table growth + decode step with the shared pages read once).  Each
carries its own timing, roofline fraction and CPU-oracle baseline.

Timing: W warmup steps, then K steps back to back between two
synchronisations (the timed region: value, ms_per_step); then the same K
steps again with the library's kernel events, whose dispatch-stamped
durations give the split-K kernel's average (roofline.achieved); for the
headline also K steps each after a 512 MiB read-only sweep of the caches
(cold_cache).

value = KV bytes the attention reads per step / step time (GB/s);
roofline = the split-K partial kernel (the dominant one): its algorithmic
bytes (K/V pages + table entries + queries + the new rows) / its average
duration.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from paged_kv_cache_207_amd import pkv  # noqa: E402
from paged_kv_cache_207_amd import workloads as W  # noqa: E402

HBM_PEAK_GBPS = 8000.0
METRIC = "paged decode attention KV GB/s (% of HBM peak) and decode tokens/s"
# calibrated rocprofv3 traffic of the split pass, one file per workload
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attend_split_{}_traffic.json")
# the split kernel and what decides its launch: its sources, its argument
# struct and the split planner (the traffic counters are kept only while
# these are unchanged)
KERNEL_SOURCES = ["paged_kv_cache_207_amd/csrc/attend_mfma.hip",
                  "paged_kv_cache_207_amd/csrc/mfma_step.h",
                  "paged_kv_cache_207_amd/csrc/prefix_wave.h",
                  "paged_kv_cache_207_amd/csrc/pkv_device.h"]
KERNEL_PARTS = [("paged_kv_cache_207_amd/csrc/pkv_internal.h", "struct AttendArgs {", "};"),
                ("paged_kv_cache_207_amd/csrc/pkv_host.hip", "int plan_split(", "\n}\n"),
                ("paged_kv_cache_207_amd/csrc/pkv_host.hip", "constexpr int kMaxBalWavesPerCu",
                 "\n\n"),
                ("paged_kv_cache_207_amd/csrc/pkv_host.hip", "constexpr int kPrefixChunkTarget",
                 "\n")]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    for p, start, end in KERNEL_PARTS:
        with open(os.path.join(ROOT, p)) as f:
            text = f.read()
        i = text.index(start)
        h.update(text[i:text.index(end, i) + len(end)].encode())
    return h.hexdigest()[:16]


def schedule_name(cache, w, max_len: int, split: int) -> str:
    """How the decode pass divides its work: the library plans bf16 pages on
    the matrix-core path with the balanced schedule (equal shares of all
    sequences' steps per wave) unless every non-empty length is equal, and
    other formats with fixed splits."""
    if split:
        return f"fixed splits of {split} tokens"
    live = w.lens[w.lens > 0]
    if w.kv_format == "bf16" and live.size and live.min() < live.max():
        return "balanced (equal shares of the batch's 32-token steps per wave)"
    why = "equal lengths" if w.kv_format == "bf16" else "planned"
    return f"fixed splits of {cache.split_for(w.batch, w.n_q_heads, max_len)} tokens ({why})"


def kv_bytes(w) -> int:
    elem = {"f32": 4, "bf16": 2, "int8": 1}[w.kv_format]
    per_tok = w.n_kv_heads * w.head_dim * elem * 2
    if w.kv_format == "int8":
        per_tok += w.n_kv_heads * 4 * 2
    return int(w.lens.astype(np.int64).sum()) * per_tok


def split_kernel_bytes(w, fused_write: bool = True) -> int:
    """Algorithmic bytes of one split-pass launch: K/V pages of every token,
    the table entries that map them, and the queries; in a fused decode step
    also the new K/V rows it reads and stores in their pages."""
    npages = sum(-(-int(n) // w.page_size) for n in w.lens)
    qb = w.batch * w.n_q_heads * w.head_dim * (2 if w.q_dtype == torch.bfloat16 else 4)
    rows = 0
    if fused_write:
        in_elem = 2 if w.in_dtype == torch.bfloat16 else 4
        elem = {"f32": 4, "bf16": 2, "int8": 1}[w.kv_format]
        rows = w.batch * w.n_kv_heads * w.head_dim * 2 * (in_elem + elem)
    return kv_bytes(w) + 4 * npages + qb + rows


def fill(w, cache, device):
    """Write every row of every sequence through the workload's write rounds
    (one round from position 0, or the unaligned head chunk then 512-row
    rounds for int8 pages); a second pass over the same rounds is timed by the
    library's events.  Returns the table, the host rows and that timing."""
    table = torch.as_tensor(w.tables).to(device)
    kv = {b: w.seq_kv(b) for b in range(w.batch)}
    rounds = [(torch.as_tensor(r.start_pos).to(device), torch.as_tensor(r.cu_new).to(device),
               r.k.to(device), r.v.to(device)) for r in w.rounds(kv=kv)]
    # the fill, then the same rounds again (they store the same bits) timed
    # warm, with every kernel's first-launch costs already paid
    for timed in (False, True):
        torch.cuda.synchronize()
        cache.timing_read()
        cache.timing(timed)
        for sp, cu, k, v in rounds:
            cache.write(table, sp, cu, k, v)
        cache.timing(False)
        torch.cuda.synchronize()
    ms, n = cache.timing_read()["write"]
    n_rounds = len(rounds)
    del rounds
    in_elem = 2 if w.in_dtype == torch.bfloat16 else 4
    rows = int(w.lens.astype(np.int64).sum())
    moved = rows * w.n_kv_heads * w.head_dim * 2 * in_elem + kv_bytes(w)  # rows in + pages out
    info = {"rounds": n_rounds, "write_us": round(ms * 1e3, 1),
            "write_GBps_in_plus_out": round(moved / (ms / 1e3) / 1e9, 1)}
    return table, [kv[b][0] for b in range(w.batch)], [kv[b][1] for b in range(w.batch)], info


def read_probe(device, nbytes=4 << 30, reps=10, scrambled=False) -> float:
    """Achievable streaming-read rate: the probe kernel (16-byte non-temporal
    loads, 4 KiB blocks, 16 blocks per wave) over 4 GiB, 10 launches back to
    back; in order, or with the blocks in a scrambled order (the page slabs
    of a fragmented pool)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=device)
    src.fill_(1)
    sink = torch.empty(pkv.lib().pkv_probe_blocks(nbytes), dtype=torch.float32, device=device)
    pkv.probe_stream(src, sink=sink, scrambled=scrambled)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        pkv.probe_stream(src, sink=sink, scrambled=scrambled)
    e1.record()
    torch.cuda.synchronize()
    gbps = nbytes * reps / (e0.elapsed_time(e1) / 1e3) / 1e9
    del src
    return gbps


def calibration_copy(device, nbytes=256 << 20) -> float:
    """A plain copy of known size (read nbytes, write nbytes): the reference
    dispatch for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=device)
    dst = torch.empty_like(src)
    src.fill_(3)
    pkv.probe_stream(src, dst)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    pkv.probe_stream(src, dst)
    e1.record()
    torch.cuda.synchronize()
    return 2 * nbytes / (e0.elapsed_time(e1) / 1e3) / 1e9


def load_traffic(workload: str):
    try:
        with open(TRAFFIC_FILE.format(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sources_sha256_16") != kernel_hash():
        return None  # the kernel changed since the counters were taken
    return t.get("traffic_bytes_per_launch")


def host_threads():
    """(cores this process may run on, BLAS threads NumPy uses)."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        blas = int(os.environ.get("OMP_NUM_THREADS", "1") or 1)
    return len(os.sched_getaffinity(0)), int(blas)


def cpu_baseline(w, ks, vs, q, budget_s: float, lens=None, note=""):
    """The oracle, as it stands, on a bounded sample of the same workload:
    decode steps of whole sequences (the oracle page write of the step's row,
    then its float64 gather and attention over every query head), sequence
    after sequence, until about budget_s of CPU time has been spent.  ks[b] /
    vs[b] hold sequence b's rows, lens[b] (default w.lens) its length after
    the step; each sequence's other rows are written untimed first."""
    from oracle import OracleCache, attend
    cores, blas = host_threads()

    def bits(t):
        t = t.contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()
    in_dt = "bf16" if w.in_dtype == torch.bfloat16 else "f32"
    q_dt = "bf16" if w.q_dtype == torch.bfloat16 else "f32"
    qb = bits(q)
    lens = w.lens if lens is None else lens
    elem = {"f32": 4, "bf16": 2, "int8": 1}[w.kv_format]
    per_tok = w.n_kv_heads * w.head_dim * elem * 2 + (w.n_kv_heads * 8 if w.kv_format == "int8"
                                                     else 0)
    caches = {}

    def state(b):  # untimed: the pages as the GPU holds them before the step
        if b not in caches:
            L = int(lens[b])
            npg = -(-L // w.page_size)
            oc = OracleCache(1, npg, w.page_size, w.n_kv_heads, w.head_dim, w.kv_format)
            table = np.arange(npg, dtype=np.int32)[None]
            kb, vb = bits(ks[b]), bits(vs[b])
            oc.write(0, table, [0], [0, L - 1], kb[:L - 1], vb[:L - 1], in_dt)
            caches[b] = (oc, table, kb[L - 1:L], vb[L - 1:L], L)
        return caches[b]
    live = [b for b in range(w.batch) if int(lens[b]) > 0]
    elapsed, steps, kv_done, i = 0.0, 0, 0, 0
    while elapsed < budget_s:
        b = live[i % len(live)]
        i += 1
        oc, table, kr, vr, L = state(b)
        t0 = time.perf_counter()
        oc.write(0, table, [L - 1], [0, 1], kr, vr, in_dt)
        attend(oc, 0, qb[b:b + 1], q_dt, table, np.array([L]), w.scale)
        elapsed += time.perf_counter() - t0
        steps += 1
        kv_done += L * per_tok
    lo, hi = int(min(lens[b] for b in live)), int(max(lens[b] for b in live))
    return {"value": round(kv_done / elapsed / 1e9, 4), "unit": "GB/s",
            "tokens_per_s": round(steps / elapsed, 3), "cores": blas, "kind": "oracle",
            "host_cores": cores, "blas_threads": blas,
            "sample": f"{steps} sequence decode steps over the {len(live)} non-empty sequences "
                      f"of the workload ({lo}..{hi} tokens, all {w.n_q_heads} query heads "
                      f"each): oracle page write of the step's row + float64 gather and "
                      f"attention; {elapsed:.1f} s of CPU time" + note}


def gather_compare(w, cache, table, device, reps=5):
    """Time the gather-first alternative's extra copy: every sequence's K/V
    copied out of its pages into a contiguous buffer (one pkv_gather per
    sequence), the copy an in-place read avoids."""
    outs = []
    for b in range(w.batch):
        L = int(w.lens[b])
        kb = torch.empty((L, w.n_kv_heads, w.head_dim), dtype=pkv.PAGE_DTYPE[w.kv_format],
                         device=device)
        sc = (torch.empty((L, w.n_kv_heads), dtype=torch.float32, device=device)
              if w.kv_format == "int8" else None)
        outs.append((kb, torch.empty_like(kb), sc, None if sc is None else torch.empty_like(sc)))

    def run():
        for b in range(w.batch):
            k, v, ks, vs = outs[b]
            pkv._check(pkv.lib().pkv_gather(cache._h, 0, pkv._dev(table[b]), int(w.lens[b]),
                                            pkv._dev(k), pkv._dev(v), pkv._dev(ks), pkv._dev(vs),
                                            pkv._stream(device)))
    run()
    torch.cuda.synchronize()
    cache.timing_read()
    cache.timing(True)
    for _ in range(reps):
        run()
    cache.timing(False)
    ms, n = cache.timing_read()["gather"]
    per_batch_ms = ms / reps
    moved = 2 * kv_bytes(w)  # read the pages, write the copy
    del outs
    return {"gather_us_per_batch": round(per_batch_ms * 1e3, 2),
            "gather_GBps_read_plus_write": round(moved / (per_batch_ms / 1e3) / 1e9, 1)}


def shared_prefix_bytes(sp) -> dict:
    """Byte counts of the shared-prefix job, per step on average: logical KV
    bytes (the prefix counted once per sequence), unique KV bytes (the prefix
    once), and the split launch's algorithmic bytes (the private K/V and their
    table entries, the shared pages once with their table entries, the
    queries, and the new rows it reads and stores)."""
    w = sp.base
    B, bs, P0 = w.batch, w.page_size, sp.prefix_tokens
    lens_steps = [sp.step_lens(s).astype(np.int64) for s in range(sp.n_steps)]
    per_tok = w.n_kv_heads * w.head_dim * 2 * 2
    logical = sum(int(l.sum()) for l in lens_steps) * per_tok
    private = sum(int((l - P0).sum()) for l in lens_steps) * per_tok
    unique = private + sp.n_steps * P0 * per_tok
    priv_pages = sum(int((-(-(l) // bs)).sum()) - B * sp.prefix_pages for l in lens_steps)
    qb = B * w.n_q_heads * w.head_dim * 2
    rows = B * w.n_kv_heads * w.head_dim * 2 * (2 + 2)
    split = ((private + 4 * priv_pages) / sp.n_steps + P0 * per_tok + 4 * sp.prefix_pages
             + qb + rows)
    n = sp.n_steps
    return {"logical": logical / n, "unique": unique / n, "split_launch": int(split)}


def run_shared_prefix(args, device, cpu_seconds: float = 0.0):
    """The shared-prefix workload as one job of n_steps decode steps after the
    fill.  Each step = host table growth (pool-backed block tables: a sequence
    whose length reaches a page boundary gets the lowest free page; the new
    entries go to the device as update triples) + paged_write of one row per
    sequence at its length + paged_attend over length + 1 tokens.  The
    attention reads the 64 shared prefix pages once for all sequences
    (pkv_decode_step_prefix: a prefix pass over the shared pages, the split
    pass over the private suffixes, the combine), and the host grows its
    tables one step ahead, so each step's launch also writes the next step's
    table entries; the same job through pkv_decode_step, which streams the
    prefix once per sequence and applies each step's entries with a table
    update launch, is timed beside it.  Every timed job starts from the same rebuilt pool state
    (untimed)."""
    sp = W.shared_prefix()
    w = sp.base
    B, bs = w.batch, w.page_size
    P0 = sp.prefix_tokens
    calibration_copy(device)  # the reference dispatch for scaling HBM counters

    def build_tables():
        pool = pkv.PagePool(w.n_pages)
        seqs = pkv.SeqTables(pool, B, w.table_stride, bs)
        seqs.append(0, P0)
        for b in range(1, B):
            seqs.share(b, 0, sp.prefix_pages)
        for b in range(B):
            seqs.append(b, int(sp.suffix[b]))
        return pool, seqs

    table = torch.full((B, w.table_stride), -1, dtype=torch.int32, device=device)
    pool, seqs = build_tables()
    pkv.table_apply(table, seqs.take_updates().to(device))
    prefix_refs = pool.refcount(seqs.table()[0][0])
    seqs.close()
    pool.close()
    cache = pkv.PagedKVCache(w.n_pages, bs, w.n_kv_heads, w.head_dim, w.kv_format, device=device)
    for r in sp.fill_rounds():
        cache.write(table, torch.as_tensor(r.start_pos).to(device),
                    torch.as_tensor(r.cu_new).to(device), r.k.to(device), r.v.to(device))
    ks, vs = sp.step_rows_all()
    ks, vs = ks.to(device), vs.to(device)
    qs = torch.stack([w.query(step=s) for s in range(sp.n_steps)]).to(device)
    lens_all = torch.stack([torch.as_tensor(sp.step_lens(s)) for s in range(sp.n_steps)]).to(device)
    max_len = int(sp.step_lens(sp.n_steps - 1).max())
    # every table row lists the shared pages first: row 0's entries are the list
    prefix_pages = table[0, :sp.prefix_pages]
    ws_pre = cache.prefix_workspace(B, w.n_q_heads, max_len, P0)
    ws_seq = cache.workspace(B, w.n_q_heads, max_len)
    out = torch.empty_like(qs[0])
    upd_host = [torch.empty((B + 8, 3), dtype=torch.int32).pin_memory()
                for _ in range(sp.n_steps)]
    torch.cuda.synchronize()
    ones = np.ones(B, np.int32)

    def step(s, shared, next_updates=None):
        if shared:
            cache.decode_step_prefix(table, lens_all[s], max_len, prefix_pages, P0, qs[s],
                                     w.scale, k_new=ks[s], v_new=vs[s], out=out,
                                     workspace=ws_pre, next_updates=next_updates)
        else:
            cache.decode_step(table, lens_all[s], max_len, ks[s], vs[s], qs[s], w.scale,
                              out=out, workspace=ws_seq)

    def fresh():
        pool, seqs = build_tables()
        table.fill_(-1)
        pkv.table_apply(table, seqs.take_updates().to(device))
        torch.cuda.synchronize()
        return pool, seqs

    def grow(seqs, s):  # every sequence grows by its new token: step s's new entries
        seqs.append_all(ones)
        n = seqs.take_updates(upd_host[s]).shape[0]
        return upd_host[s][:n] if n else None

    def job(seqs, shared):
        if not shared:
            for s in range(sp.n_steps):
                u = grow(seqs, s)
                if u is not None:  # the kernel reads the step's pinned list in place
                    pkv.table_apply(table, u)
                step(s, False)
            return
        # the host grows its tables one step ahead: step s's launch writes the
        # entries step s + 1 adds (no table-update launch inside the loop)
        u = grow(seqs, 0)
        if u is not None:
            pkv.table_apply(table, u)
        for s in range(sp.n_steps):
            step(s, True, grow(seqs, s + 1) if s + 1 < sp.n_steps else None)

    jobs = max(1, args.steps)
    res = {}
    for shared in (True, False):
        times = []
        # warmup jobs, the timed jobs, then one more job with the library's
        # kernel events on (for the kernel durations only)
        for rep in range(args.warmup + jobs + 1):
            pool, seqs = fresh()
            timed = args.warmup <= rep < args.warmup + jobs
            if rep == args.warmup + jobs:
                cache.timing_read()
                cache.timing(True)
            t0 = time.perf_counter()
            job(seqs, shared)
            torch.cuda.synchronize()
            if timed:
                times.append(time.perf_counter() - t0)
            if rep == 0:
                assert seqs.lens() == [int(x) for x in sp.step_lens(sp.n_steps - 1)]
                assert cache.status() == 0
            seqs.close()
            pool.close()
        cache.timing(False)
        t = cache.timing_read()
        res[shared] = {"job_s": float(np.mean(times)),
                       "kern": {k: (v[0] / max(v[1], 1)) for k, v in t.items()},
                       "last_out": out.clone()}
    assert cache.status() == 0
    # the two paths compute the same attention: agreement within the bf16 tolerance
    diff = float((res[True]["last_out"].float() - res[False]["last_out"].float()).abs().max())
    assert diff <= 2e-2, diff

    # The shared-prefix job with each step's device work replayed from a HIP
    # graph captured once (padded update lists of fixed size: padding rows
    # name no sequence and are skipped), the host table growth still per step,
    # one step ahead: step s's graph writes the entries of step s + 1 from
    # its pinned list, which the host fills before replaying it.
    cap = B + 8
    g_upd_host = [torch.full((cap, 3), -1, dtype=torch.int32).pin_memory()
                  for _ in range(sp.n_steps)]
    g_stream = torch.cuda.Stream(device=device)
    graphs = []
    with torch.cuda.stream(g_stream):
        for s in range(sp.n_steps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=g_stream):
                step(s, True, g_upd_host[s + 1] if s + 1 < sp.n_steps else None)
            graphs.append(g)
    torch.cuda.synchronize()

    g_upd_np = [u.numpy() for u in g_upd_host]  # views of the pinned lists

    def graph_job(seqs):
        def fill(s):
            seqs.append_all(ones)
            seqs.take_updates_padded(g_upd_np[s])
        fill(0)
        pkv.table_apply(table, g_upd_host[0])
        for s in range(sp.n_steps):
            if s + 1 < sp.n_steps:
                fill(s + 1)
            graphs[s].replay()

    g_times = []
    for rep in range(args.warmup + jobs):
        pool, seqs = fresh()
        t0 = time.perf_counter()
        graph_job(seqs)
        torch.cuda.synchronize()
        if rep >= args.warmup:
            g_times.append(time.perf_counter() - t0)
        # the replayed job leaves the tables the host grew and the eager
        # job's last output, bit for bit
        assert table.cpu().tolist() == seqs.table()
        assert torch.equal(out, res[True]["last_out"])
        seqs.close()
        pool.close()
    assert cache.status() == 0
    graph_job_s = float(np.mean(g_times))
    nb = shared_prefix_bytes(sp)
    logical, unique = nb["logical"] * sp.n_steps, nb["unique"] * sp.n_steps
    split_bytes = nb["split_launch"]
    kp, ks_ = res[True]["kern"], res[False]["kern"]
    split_s, comb_s = kp["attend_split"] / 1e3, kp["attend_combine"] / 1e3
    attn_s = split_s + comb_s
    log(f"shared_prefix: job {graph_job_s * 1e3:.3f} ms (graphs), eager "
        f"{res[True]['job_s'] * 1e3:.3f} ms; per step: split pass with prefix waves "
        f"{split_s * 1e6:.1f} us, combine {comb_s * 1e6:.1f} us; per-sequence path: split "
        f"{ks_['attend_split'] * 1e3:.1f} us, combine {ks_['attend_combine'] * 1e3:.1f} us, job "
        f"{res[False]['job_s'] * 1e3:.3f} ms eager; prefix refcount {prefix_refs}")
    line = {
        "metric": METRIC, "value": round(unique / graph_job_s / 1e9, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": jobs, "warmup": args.warmup,
        "ms_per_step": round(graph_job_s * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "page_size": bs,
                   "prefix_pages": sp.prefix_pages, "suffix": "uniform [16, 2048]",
                   "step": f"one job = {sp.n_steps} decode steps (host table growth + "
                           "decode_step_prefix: paged_write 1 row/seq + paged_attend with the "
                           "shared prefix read once, one call)",
                   "value_bytes": "unique KV bytes (shared prefix once)"},
        "tokens_per_s": round(B * sp.n_steps / graph_job_s, 1),
        "logical_kv_GBps": round(logical / graph_job_s / 1e9, 2),
        "job": "the host grows its tables one step ahead (append_all, take_updates into a "
               "padded pinned list); each step's decode_step_prefix, replayed from a HIP "
               "graph captured once, also writes the next step's table entries from that "
               "list (one table_apply before the first step)",
        "eager": {"ms_per_job": round(res[True]["job_s"] * 1e3, 5),
                  "GBps_unique": round(unique / res[True]["job_s"] / 1e9, 2),
                  "note": "the same job with every library call launched from Python"},
        "pct_hbm_peak": round(100 * unique / graph_job_s / 1e9 / HBM_PEAK_GBPS, 2),
        "attention_per_step_us": {"split_pass_with_prefix_waves": round(split_s * 1e6, 2),
                                  "combine": round(comb_s * 1e6, 2),
                                  "total": round(attn_s * 1e6, 2),
                                  "unique_GBps": round(unique / sp.n_steps / attn_s / 1e9, 2)},
        "per_sequence_path": {
            "ms_per_job_eager": round(res[False]["job_s"] * 1e3, 5),
            "split_pass_us": round(ks_["attend_split"] * 1e3, 2),
            "combine_us": round(ks_["attend_combine"] * 1e3, 2),
            "note": "pkv_decode_step over the same tables: every sequence streams the shared "
                    "prefix itself"},
        "roofline": {"bound": "hbm", "achieved": round(split_bytes / split_s / 1e9, 2),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(split_bytes / split_s / 1e9 / HBM_PEAK_GBPS, 4),
                     "traffic": load_traffic(w.name),
                     "kernel": "attend_mfma (split-K partial pass over the private suffixes, "
                               "with the shared-prefix waves in the same launch)",
                     "avg_launch_us": round(split_s * 1e6, 2),
                     "bytes_per_launch": int(split_bytes),
                     "note": "the dominant kernel: the private K/V of a step and their table "
                             "entries, the shared pages once, the queries and the new rows, over "
                             "its mean launch time"},
    }
    if cpu_seconds > 0:
        pk, pv = sp.prefix_kv()
        kl, vl = [], []
        for b in range(B):
            k, v = sp.private_kv(b)
            n = int(sp.suffix[b]) + 1
            kl.append(torch.cat([pk, k[:n]]))
            vl.append(torch.cat([pv, v[:n]]))
        line["cpu_baseline"] = cpu_baseline(w, kl, vl, qs[0].cpu(), cpu_seconds,
                                            lens=sp.step_lens(0),
                                            note="; the shared prefix is part of every "
                                                 "sequence's own oracle copy")
    else:
        line["cpu_baseline"] = None
    return line


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


def multi_layer_write(cp, device, kc, vc, start, cu_new, n_layers=32, reps=5):
    """The chunk's rows stored in every layer of a 32-layer store: one
    pkv_paged_write_layers launch against one pkv_paged_write per layer."""
    w = cp.base
    cache = pkv.PagedKVCache(w.n_pages, w.page_size, w.n_kv_heads, w.head_dim, w.kv_format,
                             n_layers, device=device)
    table = torch.as_tensor(w.tables).to(device)
    k = kc.unsqueeze(0).expand(n_layers, *kc.shape).contiguous()
    v = vc.unsqueeze(0).expand(n_layers, *vc.shape).contiguous()

    def one_launch():
        cache.write_layers(table, start, cu_new, k, v)

    def per_layer():
        for layer in range(n_layers):
            cache.write(table, start, cu_new, k[layer], v[layer], layer=layer)

    out = {"layers": n_layers, "rows_per_layer": int(kc.shape[0])}
    moved = 2 * k.numel() * k.element_size() * 2  # K and V rows read, pages written
    for name, fn in (("one_launch", one_launch), ("launch_per_layer", per_layer)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name + "_us"] = round(ms * 1e3, 1)
        out[name + "_GBps_in_plus_out"] = round(moved / (ms / 1e3) / 1e9, 1)
    assert cache.status() == 0
    del cache
    return out


def run_fork_copy(args, device, n_layers=32, n_forks=256):
    """Copy-on-write page copies: after forks share every page, the first
    append of each fork into the shared, partly filled last page copies that
    page (every layer) to a fresh one.  One step = pkv_copy_pages of n_forks
    (source, fresh page) pairs over a 32-layer bf16 store (Hkv 8, D 128, bs 16)."""
    P, bs, Hkv, D = 4096, 16, 8, 128
    cache = pkv.PagedKVCache(P, bs, Hkv, D, "bf16", n_layers, device=device)
    cache.k_pages.fill_(3)
    cache.v_pages.fill_(5)
    rng = np.random.default_rng(9)
    ids = rng.permutation(P)[:2 * n_forks].astype(np.int32)
    pairs = torch.as_tensor(ids.reshape(n_forks, 2)).to(device)
    for _ in range(args.warmup):
        cache.copy_pages(pairs)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        cache.copy_pages(pairs)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    cache.timing_read()
    cache.timing(True)
    for _ in range(args.steps):
        cache.copy_pages(pairs)
    cache.timing(False)
    t = cache.timing_read()
    k_ms = t["copy_pages"][0] / max(t["copy_pages"][1], 1)
    assert cache.status() == 0
    page_bytes = Hkv * bs * D * 2 * 2  # K and V slabs of one page of one layer
    moved = 2 * n_forks * n_layers * page_bytes  # read + write
    log(f"fork copy: {n_forks} pages x {n_layers} layers: {ms * 1e3:.1f} us per call, kernel "
        f"{k_ms * 1e3:.1f} us = {moved / (k_ms / 1e3) / 1e9:.0f} GB/s read + write")
    return {
        "metric": "copy-on-write page copy GB/s (read + write)", "unit": "GB/s",
        "value": round(moved / (ms / 1e3) / 1e9, 2), "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "fork_copy", "pairs": n_forks, "layers": n_layers,
                   "n_kv_heads": Hkv, "head_dim": D, "page_size": bs},
        "roofline": {"bound": "hbm", "achieved": round(moved / (k_ms / 1e3) / 1e9, 2),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(moved / (k_ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "traffic": None, "kernel": "copy_pages", "avg_launch_us": round(k_ms * 1e3, 2)},
        "cpu_baseline": None,
    }


def run_chunked_prefill(args, device, kv_format="bf16"):
    """Several queries per sequence: each step writes every sequence's chunk
    of new rows (paged_write at position context[b]) and runs causal
    multi-query attention of the chunk over context + chunk tokens.  The
    context is written once before timing; each step rewrites the same chunk."""
    cp = W.chunked_prefill(kv_format=kv_format)
    w = cp.base
    B = w.batch
    log(f"workload chunked_prefill ({kv_format} pages): B={B} context={cp.context.tolist()} "
        f"chunk={cp.chunk.tolist()} Hq={w.n_q_heads} Hkv={w.n_kv_heads} D={w.head_dim} "
        f"bs={w.page_size}")
    cache = pkv.PagedKVCache(w.n_pages, w.page_size, w.n_kv_heads, w.head_dim, w.kv_format,
                             device=device)
    table = torch.as_tensor(w.tables).to(device)
    kv = {b: w.seq_kv(b) for b in range(B)}
    r0, r1 = cp.context_round(kv), cp.chunk_round(kv)
    cache.write(table, torch.as_tensor(r0.start_pos).to(device),
                torch.as_tensor(r0.cu_new).to(device), r0.k.to(device), r0.v.to(device))
    start = torch.as_tensor(r1.start_pos).to(device)
    cu_new = torch.as_tensor(r1.cu_new).to(device)
    kc, vc = r1.k.to(device), r1.v.to(device)
    lens = torch.as_tensor(w.lens).to(device)
    cu_q = torch.as_tensor(cp.cu_q).to(device)
    q = cp.queries().to(device)
    out = torch.empty_like(q)

    def step():
        cache.write(table, start, cu_new, kc, vc)
        cache.attend_multi(q, table, lens, cu_q, cp.max_q, w.max_len, w.scale, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert cache.status() == 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    cache.timing_read()
    cache.timing(True)
    for _ in range(args.steps):
        step()
    cache.timing(False)
    t = cache.timing_read()
    attn_ms = t["attend_multi"][0] / max(t["attend_multi"][1], 1)
    wr_ms = t["write"][0] / max(t["write"][1], 1)
    # the same K steps once more, now that the chip has run this compute-heavy
    # loop for a while: the first timed pass (value) runs slower
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(args.steps):
        step()
    s1.record()
    torch.cuda.synchronize()
    steady_ms = s0.elapsed_time(s1) / args.steps
    # algorithmic work: every query row scores and weights its visible tokens
    pos = (w.lens.astype(np.int64) - cp.chunk)[:, None]
    visible = sum(int((pos[b, 0] + np.arange(1, int(cp.chunk[b]) + 1)).sum()) for b in range(B))
    flops = 4 * w.n_q_heads * w.head_dim * visible
    kvb = kv_bytes(w)
    tflops = flops / (attn_ms / 1e3) / 1e12
    log(f"chunked prefill step {ms_per_step * 1e3:.1f} us (steady state {steady_ms * 1e3:.1f} us): "
        f"write {wr_ms * 1e3:.1f} us, multi-query attention {attn_ms * 1e3:.1f} us = "
        f"{tflops:.1f} TFLOP/s")
    layers_info = multi_layer_write(cp, device, kc, vc, start, cu_new) if kv_format == "bf16" else None
    if layers_info:
        log(f"multi-layer write: {layers_info}")
    return {
        "metric": METRIC, "value": round(kvb / (ms_per_step / 1e3) / 1e9, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.kv_format, "data": "synthetic",
        "steady_state_ms_per_step": round(steady_ms, 5),
        "multi_layer_write": layers_info,
        "config": {"workload": "chunked_prefill" + ("" if kv_format == "bf16" else "_" + kv_format),
                   "pages": kv_format, "batch": B,
                   "context": cp.context.tolist(), "chunk": cp.chunk.tolist(),
                   "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "page_size": w.page_size,
                   "step": "paged_write of each chunk + causal multi-query paged attention"},
        "tokens_per_s": round(cp.total_q / (ms_per_step / 1e3), 1),
        "attention_TFLOPs": round(tflops, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "attend_multi (causal, several queries per sequence)",
                     "avg_launch_us": round(attn_ms * 1e3, 2),
                     "flops_per_launch": flops,
                     "timing": "library kernel events over a second run of the K steps "
                               "(their durations match the steady-state step, not the first "
                               "timed pass)"},
        "cpu_baseline": None,
    }


def run_decode(args, device, name: str, headline: bool, cpu_seconds: float):
    """One decode workload: fill its pages, then W warmup steps and K timed
    steps of pkv_decode_step (one row written per sequence, one query per
    sequence attending over all its tokens).  The headline run also measures
    the streaming probes, cold-cache steps and the gather comparison."""
    w = W.by_name(name)
    log(f"workload {w.name}: B={w.batch} lens={int(w.lens.min())}..{int(w.lens.max())} "
        f"Hq={w.n_q_heads} Hkv={w.n_kv_heads} D={w.head_dim} bs={w.page_size} P={w.n_pages}")

    if headline:
        read_gbps = read_probe(device)
        read_pages_gbps = read_probe(device, scrambled=True)
        copy_gbps = calibration_copy(device)
        log(f"probe: streaming read {read_gbps:.0f} GB/s in order, {read_pages_gbps:.0f} GB/s "
            f"as 4 KiB blocks in a scrambled order; copy {copy_gbps:.0f} GB/s")

    cache = pkv.PagedKVCache(w.n_pages, w.page_size, w.n_kv_heads, w.head_dim, w.kv_format,
                             device=device)
    t0 = time.perf_counter()
    table, ks, vs, fill_info = fill(w, cache, device)
    log(f"filled {kv_bytes(w) / 2**30:.2f} GiB of pages in {time.perf_counter() - t0:.1f} s: "
        f"{fill_info}")

    B = w.batch
    lens = torch.as_tensor(w.lens).to(device)
    start = (lens - 1).contiguous()
    cu = torch.arange(B + 1, dtype=torch.int32, device=device)
    k_new = torch.stack([ks[b][int(w.lens[b]) - 1] for b in range(B)]).to(device)
    v_new = torch.stack([vs[b][int(w.lens[b]) - 1] for b in range(B)]).to(device)
    q_host = w.query()
    q = q_host.to(device)
    out = torch.empty_like(q)
    max_len = w.max_len
    split = args.split  # 0: the library's plan
    schedule = schedule_name(cache, w, max_len, split)
    ws = cache.workspace(B, w.n_q_heads, max_len, split)
    if headline:  # the read-only sweep that flushes the caches between cold steps
        sweep_buf = torch.empty(512 << 20, dtype=torch.uint8, device=device)
        sweep_buf.fill_(7)
        sweep_sink = torch.empty(pkv.lib().pkv_probe_blocks(sweep_buf.numel()),
                                 dtype=torch.float32, device=device)

    def step():
        if args.separate_write:
            cache.write(table, start, cu, k_new, v_new)
            cache.attend(q, table, lens, max_len, w.scale, out=out, workspace=ws,
                         split_tokens=split)
        else:  # one call: the decode step writes each sequence's row and attends
            cache.decode_step(table, lens, max_len, k_new, v_new, q, w.scale, out=out,
                              workspace=ws, split_tokens=split)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    cache.status() == 0 or sys.exit("device status flags set during warmup")

    # (1) the timed region: K steps back to back between two synchronisations
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - wall0) * 1e3 / args.steps
    ms_per_step = e0.elapsed_time(e1) / args.steps

    def kernel_times():
        t = cache.timing_read()
        return {k: v[0] / max(v[1], 1) for k, v in t.items()}

    # (2) the same K steps with the library's kernel events (each kernel's
    # dispatch stamps its own start and end): the per-kernel durations
    cache.timing_read()
    cache.timing(True)
    for _ in range(args.steps):
        step()
    cache.timing(False)
    kt = kernel_times()
    split_avg = kt["attend_split"]

    if headline:
        # (3) cold caches: each step after a 512 MiB read-only sweep (which leaves
        # no dirty lines behind), kernels timed by the library's events: whether
        # the back-to-back steps gain anything from data left in the caches
        cache.timing(True)
        for i in range(args.steps):
            pkv.probe_stream(sweep_buf, sink=sweep_sink)
            step()
        torch.cuda.synchronize()
        cache.timing(False)
        kt_cold = kernel_times()

        # (4) the same cold steps timed one by one with events on the stream (no
        # library timing): median and minimum step time with flushed caches
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for ea, eb in evs:
            pkv.probe_stream(sweep_buf, sink=sweep_sink)
            ea.record()
            step()
            eb.record()
        torch.cuda.synchronize()
        cold_steps = sorted(ea.elapsed_time(eb) * 1e3 for ea, eb in evs)
    assert cache.status() == 0
    comb_avg, wr_avg = kt["attend_combine"], kt["write"]
    log(f"{w.name} step: {ms_per_step * 1e3:.1f} us back to back (wall {wall_ms * 1e3:.1f} us); "
        f"split pass {split_avg * 1e3:.1f} us, combine {comb_avg * 1e3:.1f} us, write "
        f"{wr_avg * 1e3:.1f} us; {schedule}")

    kvb = kv_bytes(w)
    value = kvb / (ms_per_step / 1e3) / 1e9
    achieved = split_kernel_bytes(w, not args.separate_write) / (split_avg / 1e3) / 1e9
    traffic = load_traffic(w.name)
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.kv_format,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "seq_len": int(w.lens.max()),
                   "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "page_size": w.page_size, "n_pages": w.n_pages,
                   "table": "seeded random permutation of the pool",
                   "step": ("paged_write 1 row/seq + paged_attend" if args.separate_write else
                            "decode_step: paged_write 1 row/seq + paged_attend, one call"),
                   "split_tokens": split, "schedule": schedule},
        "tokens_per_s": round(B / (ms_per_step / 1e3), 1),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "kv_bytes_per_step": kvb,
        "wall_ms_per_step": round(wall_ms, 5),
        "fill_write": fill_info,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "kernel": "attend_mfma (split-K partial pass)",
                     "avg_launch_us": round(split_avg * 1e3, 2),
                     "timing": "library kernel events over a second run of the K steps"},
    }
    if headline:
        line["achievable_read_GBps"] = round(read_gbps, 1)
        line["split_pass_frac_of_achievable_read"] = round(achieved / read_gbps, 4)
        # the pages of this workload are 4 KiB slabs in a shuffled order
        line["achievable_read_4k_scrambled_GBps"] = round(read_pages_gbps, 1)
        line["split_pass_frac_of_scrambled_read"] = round(achieved / read_pages_gbps, 4)
        line["cold_cache"] = {
            "split_pass_us": round(kt_cold["attend_split"] * 1e3, 2),
            "combine_us": round(kt_cold["attend_combine"] * 1e3, 2),
            "step_us_median": round(float(np.median(cold_steps)), 2),
            "step_us_min": round(cold_steps[0], 2),
            "note": "each step follows a 512 MiB read-only sweep of the caches: kernel "
                    "durations from the library's events, step median and minimum from events "
                    "on the stream around each step"}
        log(f"after a cache sweep: split pass {kt_cold['attend_split'] * 1e3:.1f} us, combine "
            f"{kt_cold['attend_combine'] * 1e3:.1f} us")
        if args.gather_compare:
            line["gather_compare"] = gather_compare(w, cache, table, device)
            line["gather_compare"]["inplace_attend_us"] = round((split_avg + comb_avg) * 1e3, 2)
            log(f"gather compare: {line['gather_compare']}")
    line["cpu_baseline"] = (cpu_baseline(w, ks, vs, q_host, cpu_seconds) if cpu_seconds > 0
                            else None)
    del cache, table, ks, vs
    torch.cuda.empty_cache()
    return line


def compact(line: dict) -> dict:
    """The fields a config keeps inside the headline line."""
    keep = ("value", "unit", "ms_per_step", "tokens_per_s", "pct_hbm_peak", "dtype", "config",
            "kv_bytes_per_step", "roofline", "cpu_baseline", "logical_kv_GBps",
            "attention_per_step_us", "per_sequence_path", "eager")
    return {k: line[k] for k in keep if k in line}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all",
                    help="all (the 32k-token headline plus the other four configs), or one of "
                         "long_bf16, tiny_f32, decode_bf16, int8_kv, shared_prefix, "
                         "chunked_prefill, chunked_prefill_int8, fork_copy")
    ap.add_argument("--split", type=int, default=0, help="split tokens (0 = library plan)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle time for the headline's CPU baseline")
    ap.add_argument("--config-cpu-seconds", type=float, default=4.0,
                    help="oracle time for each other config's CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--separate-write", action="store_true",
                    help="run the step as pkv_paged_write + pkv_paged_attend instead of one "
                         "pkv_decode_step call")
    ap.add_argument("--gather-compare", type=int, default=1,
                    help="1: also time gathering every sequence into a contiguous copy")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); this library has no "
              "multi-GPU path: run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    device = torch.device("cuda:0")
    cpu_main = 0.0 if args.no_cpu_baseline else args.cpu_seconds
    cpu_cfg = 0.0 if args.no_cpu_baseline else args.config_cpu_seconds
    if args.workload == "shared_prefix":
        print(json.dumps(run_shared_prefix(args, device, cpu_main)), flush=True)
        return
    if args.workload in ("chunked_prefill", "chunked_prefill_int8"):
        fmt = "int8" if args.workload.endswith("int8") else "bf16"
        print(json.dumps(run_chunked_prefill(args, device, fmt)), flush=True)
        return
    if args.workload == "fork_copy":
        print(json.dumps(run_fork_copy(args, device)), flush=True)
        return
    if args.workload != "all":
        print(json.dumps(run_decode(args, device, args.workload, True, cpu_main)), flush=True)
        return
    # the headline: the 32k-token workload; the other four configs beside it
    line = run_decode(args, device, "long_bf16", True, cpu_main)
    configs = {}
    for name in ("tiny_f32", "decode_bf16", "int8_kv"):
        configs[name] = compact(run_decode(args, device, name, False, cpu_cfg))
    configs["shared_prefix"] = compact(run_shared_prefix(args, device, cpu_cfg))
    line["configs"] = configs
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
