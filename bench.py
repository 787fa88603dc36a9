#!/usr/bin/env python3
"""Benchmark of content-selected block-sparse attention on one MI355X.

Headline: the mixed variable-length batch at sparsity 0.95 (16 sequences of 4096..131072 tokens,
32 query / 8 KV heads, d 128, 64-token blocks, per-head top ceil((c+1)/20) + current block, log-gate).
One step = its prefill half (8 sequences, their last 4096 rows: representatives of the new blocks,
block scores, top-k, sparse prefill) then its decode half (8 sequences, one row each: fused scores +
top-k, sparse decode); earlier representatives are resident, like the KV cache itself.
`value` = decode GB/s: the decode half's algorithmic bytes / its time; the prefill half's TFLOP/s
(algorithmic FLOP / time) sits beside it, and each half has its roofline object (`roofline`: the
decode attention kernel against HBM; `roofline_prefill`: the prefill kernel against bf16 MFMA).
The L2s and the 256 MB MALL are flushed (1 GiB read) before every timed interval, outside it, so
bytes come from HBM.  extra.* holds the other workloads: the 32K decode batch, the 32K causal
prefill and both backwards, the SSA-style gist decode and its two-level variant, paged decode, reps.
The CPU baseline (the oracle) runs first, before the GPU is touched.

Usage: python bench.py [--steps K] [--warmup W] [--only NAME,...] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
FLUSH_BYTES = 1 << 30


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------------------------------------------
# timing helpers
# ------------------------------------------------------------------------------------------------
class Timer:
    """HIP event timing on the stream the library launches on.

    Each timed call is preceded by a 1 GiB read (outside the timed interval) that evicts the
    L2s and the MALL, so the bytes of the timed call come from HBM.
    """

    def __init__(self, torch):
        self.torch = torch
        self.flush_f32 = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        self.sink = None

    def flush(self):
        # read 1 GiB: evicts the L2s and the MALL with clean lines (a write-based flush would leave
        # dirty lines whose write-back would be charged to the timed kernels)
        self.sink = self.flush_f32.sum()

    def graph(self, fn):
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    def time(self, fn, steps, warmup, use_graph=False):
        """Median device ms of fn over `steps` calls, and the wall seconds of the whole timed loop
        (flushes included).  The median keeps a rare host-side stall (which lets the GPU run
        dry inside one interval) out of the figure.

        Each call is bracketed by two events on the current stream (the stream the library
        launches on).  The call is queued behind the ~270 us flush, so host launch latency is
        hidden and the interval is the device time of the call's kernels and the gaps between
        them.  use_graph replays a HIP graph of fn instead; for steps of a few tens of us the
        graph launch itself adds several us on this runtime, so it is reported as a secondary
        figure."""
        torch = self.torch
        run = fn
        if use_graph:
            g = self.graph(fn)
            run = g.replay
        for _ in range(warmup):
            self.flush()
            run()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        evs = []
        t0 = time.perf_counter()
        for _ in range(steps):
            self.flush()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            run()
            b.record(stream)
            evs.append((a, b))
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ts = sorted(a.elapsed_time(b) for a, b in evs)
        return _median(ts), wall

    def time_halves(self, fa, fb, steps, warmup):
        """One step = fa then fb (the two halves of a mixed batch), each queued behind its own flush and
        bracketed by its own events; (median ms of fa, median ms of fb) and the wall seconds of the loop."""
        torch = self.torch
        for _ in range(warmup):
            self.flush()
            fa()
            self.flush()
            fb()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        evs = []
        t0 = time.perf_counter()
        for _ in range(steps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            self.flush()
            e[0].record(stream)
            fa()
            e[1].record(stream)
            self.flush()
            e[2].record(stream)
            fb()
            e[3].record(stream)
            evs.append(e)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ta = sorted(e[0].elapsed_time(e[1]) for e in evs)
        tb = sorted(e[2].elapsed_time(e[3]) for e in evs)
        return (_median(ta), _median(tb)), wall


def _median(ts):
    n = len(ts)
    return ts[n // 2] if n % 2 else 0.5 * (ts[n // 2 - 1] + ts[n // 2])


# ------------------------------------------------------------------------------------------------
# workloads
# ------------------------------------------------------------------------------------------------
def decode_step_setup(sas, w, inp, gist=False):
    """Preallocated buffers + a step closure for scores -> top-k -> decode (reps resident)."""
    import torch
    lens = inp.seq_lens
    Lmax = inp.K.shape[2]
    dt = sas.SAS_BF16
    budget = sas.Budget(k_fixed=w.k_fixed, frac_num=w.frac_num, frac_den=w.frac_den,
                        count_current=w.count_current, sink=w.sink, gate=w.gate)
    reps = inp.gist_k if gist else sas.block_reps(inp.K, lens, w.block)
    sel_ws = torch.zeros(sas.select_decode_workspace_bytes(len(lens), w.hq, w.hkv, w.d, w.block, dt, Lmax, lens),
                         dtype=torch.uint8, device="cuda")
    scores, idx, nsel, gate = sas.select_decode(inp.Q, reps, lens, w.block, w.hkv, Lmax, budget, sel_mode=w.sel,
                                                gist=gist, workspace=sel_ws)
    O = torch.empty_like(inp.Q)
    ws = torch.zeros(sas.decode_workspace_bytes(len(lens), w.hq, w.hkv, w.d, w.block, dt, Lmax, lens, w.sel,
                                                idx.shape[1], gist), dtype=torch.uint8, device="cuda")
    gk = inp.gist_k if gist else None
    gv = inp.gist_v if gist else None

    def attend():
        sas.sparse_decode(inp.Q, inp.K, inp.V, lens, w.block, idx, nsel, gate, sel_mode=w.sel, gist_k=gk,
                          gist_v=gv, O=O, workspace=ws)

    def select():
        sas.select_decode(inp.Q, reps, lens, w.block, w.hkv, Lmax, budget, sel_mode=w.sel, gist=gist,
                          kcap=idx.shape[1], scores=scores, idx=idx, nsel=nsel, gate=gate, workspace=sel_ws)

    idx2, nsel2 = torch.empty_like(idx), torch.empty_like(nsel)
    gate2 = torch.empty_like(gate) if gate is not None else None

    def select_two_calls():
        # the same selection as two launches: block scores, then the top-k
        sas.block_scores(inp.Q, reps, lens, w.block, w.hkv, Lmax, sel_mode=w.sel, gist=gist, scores=scores)
        sas.topk_select(scores, lens, w.block, w.hq, w.hkv, w.d, dt, Lmax, budget, sel_mode=w.sel,
                        kcap=idx.shape[1], idx=idx2, nsel=nsel2, gate=gate2)

    def step():
        select()
        attend()

    fns = dict(step=step, attend=attend, select=select, select_two_calls=select_two_calls)
    return fns, dict(reps=reps, scores=scores, idx=idx, nsel=nsel, gate=gate, O=O)


def hssa_step_setup(sas, w, inp):
    """Two-level gist selection + its attention (gist and meta-gist keys resident)."""
    import torch
    lens = inp.seq_lens
    Lmax = inp.K.shape[2]
    M, k1, k2 = w.spec["group_chunks"], w.spec["k_groups"], w.k_fixed
    idx, nsel, gidx, gsel = sas.hssa_select_decode(inp.Q, inp.gist_k, inp.meta_k, lens, w.block, w.hkv, Lmax, M,
                                                   k1, k2, sel_mode=w.sel)
    O = torch.empty_like(inp.Q)
    B = len(lens)
    dec_ws = torch.zeros(sas.hssa_decode_workspace_bytes(B, w.hq, w.hkv, w.d, w.block, Lmax, lens, w.sel,
                                                         idx.shape[1], gidx.shape[1], M),
                         dtype=torch.uint8, device="cuda")
    sel_ws = torch.empty(max(16, sas.hssa_select_workspace_bytes(B, w.hq, w.hkv, w.d, w.block, Lmax, lens, w.sel, M,
                                                                 k1)), dtype=torch.uint8, device="cuda")

    def attend():
        sas.hssa_decode(inp.Q, inp.K, inp.V, lens, w.block, inp.gist_k, inp.gist_v, inp.meta_k, inp.meta_v, M,
                        idx, nsel, gidx, sel_mode=w.sel, O=O, workspace=dec_ws)

    def step():
        sas.hssa_select_decode(inp.Q, inp.gist_k, inp.meta_k, lens, w.block, w.hkv, Lmax, M, k1, k2,
                               sel_mode=w.sel, kcap=idx.shape[1], gcap=gidx.shape[1], idx=idx, nsel=nsel, gidx=gidx,
                               gsel=gsel, workspace=sel_ws)
        attend()

    return dict(step=step, attend=attend), dict(idx=idx, nsel=nsel, gidx=gidx, gsel=gsel, O=O)


def hssa_bytes(w, inp, bufs):
    """Bytes the two-level step must move, per (sequence, KV group): the meta-gist keys of the
    complete groups and the gist keys of the open groups' chunks (read once for scoring), the K/V
    rows of the expanded chunks and of the current chunk, the gist values of the open groups'
    unexpanded chunks, the meta-gist values of the closed groups, Q and O."""
    idx = bufs["idx"].cpu().numpy()
    nsel = bufs["nsel"].cpu().numpy()
    gidx = bufs["gidx"].cpu().numpy()
    gsel = bufs["gsel"].cpu().numpy()
    M = w.spec["group_chunks"]
    e, d = 2, w.d
    assert w.sel == "group"
    total = 0
    for bi, L in enumerate(inp.seq_lens):
        c = (L - 1) // w.block
        nm = c // M
        for g in range(w.hkv):
            u = bi * w.hkv + g
            groups = [int(x) for x in gidx[u, :gsel[u]]]
            cand = [j for j in range(c) if j // M in set(groups)]
            sel = [int(x) for x in idx[u, :nsel[u]]]
            rows = sum(min((j + 1) * w.block, L) - j * w.block for j in sel)
            total += nm * d * e + len(cand) * d * e                     # scoring reads
            total += rows * d * e * 2                                   # raw K and V
            total += (len(cand) - (len(sel) - 1)) * d * e               # gist V of open, unexpanded chunks
            total += (nm - (len(groups) - 1)) * d * e                   # meta-gist V of closed groups
            total += w.group * d * e * 2                                # Q and O
    return total


def prefill_step_setup(sas, w, inp):
    """Preallocated buffers + closures for the prefill step: representatives of the blocks the new rows
    touch (earlier blocks are resident, pooled once with the cached context), block scores, top-k,
    sparse prefill."""
    import torch
    lens = inp.seq_lens
    Lmax = inp.K.shape[2]
    dt = sas.SAS_BF16
    budget = sas.Budget(k_fixed=w.k_fixed, frac_num=w.frac_num, frac_den=w.frac_den,
                        count_current=w.count_current, sink=w.sink, gate=w.gate,
                        sqrt_num=w.sqrt_num, sqrt_den=w.sqrt_den)
    reps = sas.block_reps(inp.K, lens, w.block)
    first = [q0 // w.block for q0 in inp.q_start]
    scores = sas.block_scores(inp.Q, reps, lens, w.block, w.hkv, Lmax, q_start=inp.q_start, sel_mode=w.sel)
    ws = torch.empty(max(1, len(lens) * (w.hq if w.sel == "head" else w.hkv) * sas.num_qblocks(w.tq, w.block)
                         * w.d * 4), dtype=torch.uint8, device="cuda")
    idx, nsel, gate = sas.topk_select(scores, lens, w.block, w.hq, w.hkv, w.d, dt, Lmax, budget, tq=w.tq,
                                      q_start=inp.q_start, sel_mode=w.sel)
    O = torch.empty_like(inp.Q)

    def make_reps():
        sas.block_reps(inp.K, lens, w.block, reps=reps, first_block=first)

    def attend():
        sas.sparse_prefill(inp.Q, inp.K, inp.V, lens, w.block, inp.q_start, idx, nsel, gate, sel_mode=w.sel, O=O)

    def select():
        make_reps()
        sas.block_scores(inp.Q, reps, lens, w.block, w.hkv, Lmax, q_start=inp.q_start, sel_mode=w.sel,
                         scores=scores, workspace=ws)
        sas.topk_select(scores, lens, w.block, w.hq, w.hkv, w.d, dt, Lmax, budget, tq=w.tq, q_start=inp.q_start,
                        sel_mode=w.sel, idx=idx, nsel=nsel, gate=gate)

    def step():
        select()
        attend()

    return (dict(step=step, attend=attend, reps=make_reps, select=select),
            dict(reps=reps, idx=idx, nsel=nsel, gate=gate, O=O))


# ------------------------------------------------------------------------------------------------
# algorithmic work (from the selected lists, copied to the host once)
# ------------------------------------------------------------------------------------------------
def decode_bytes(w, inp, bufs, gist=False):
    """Bytes the decode step must move: representatives of the candidate blocks (once per KV
    head), the union over a KV group's query heads of the selected K/V rows, Q and O."""
    import numpy as np
    idx = bufs["idx"].cpu().numpy()
    nsel = bufs["nsel"].cpu().numpy()
    B = len(inp.seq_lens)
    S = w.hq if w.sel == "head" else w.hkv
    G = w.hq // w.hkv
    e = 2
    total = 0
    kv_bytes = 0
    rep_bytes = 0
    for bi, L in enumerate(inp.seq_lens):
        c = (L - 1) // w.block
        for g in range(w.hkv):
            heads = range(g * G, (g + 1) * G) if w.sel == "head" else [g]
            union = set()
            for s in heads:
                u = bi * S + s
                union |= set(int(x) for x in idx[u, : nsel[u]])
            rows = sum(min((j + 1) * w.block, L) - j * w.block for j in union)
            kv_bytes += rows * w.d * e * 2
            if gist:
                ncand = c
                rep_bytes += ncand * w.d * e                               # gist K, scored once
                kv_bytes += (c - len([j for j in union if j < c])) * w.d * e  # gist V of the others
            else:
                rep_bytes += c * w.d * 4                                   # fp32 reps j < c
    qo = 2 * B * w.hq * w.d * e
    total = kv_bytes + rep_bytes + qo
    return dict(total=total, kv=kv_bytes, reps=rep_bytes, qo=qo)


def prefill_flops(w, inp, bufs):
    """4*d per visible (row, head, key) pair of the selected blocks (QK^T and PV)."""
    import numpy as np
    idx = bufs["idx"].cpu().numpy()
    nsel = bufs["nsel"].cpu().numpy()
    S = w.hq if w.sel == "head" else w.hkv
    nh = 1 if w.sel == "head" else w.hq // w.hkv
    QB = (w.tq - 1 + w.block - 1) // w.block + 1 if w.tq > 1 else 1
    pairs = 0
    for bi, L in enumerate(inp.seq_lens):
        q0 = inp.q_start[bi]
        c0 = q0 // w.block
        for s in range(S):
            for i in range(QB):
                u = (bi * S + s) * QB + i
                n = int(nsel[u])
                if n == 0:
                    continue
                c = c0 + i
                p_lo = max(q0, c * w.block)
                p_hi = min(q0 + w.tq, (c + 1) * w.block) - 1
                pos = np.arange(p_lo, p_hi + 1)
                for j in idx[u, :n]:
                    j = int(j)
                    hi = np.minimum(min((j + 1) * w.block, L), pos + 1)
                    pairs += int(np.clip(hi - j * w.block, 0, None).sum()) * nh
    full = sum(sum(q0 + t + 1 for t in range(w.tq)) for q0 in inp.q_start) * w.hq
    return dict(flops=4.0 * w.d * pairs, pairs=pairs, sparsity=1.0 - pairs / full)


# ------------------------------------------------------------------------------------------------
# HBM traffic from the committed rocprofv3 counter summary
# ------------------------------------------------------------------------------------------------
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def kernel_source_hash(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """Calibrated HBM bytes per launch of `kernel` (FETCH_SIZE and WRITE_SIZE, each scaled by what
    the same counter reads for a copy of known size), or None when there is no record or the
    kernel's sources have changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)["kernels"][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if kernel_source_hash(rec["sources"]) != rec["source_sha256_16"]:
        return None
    cal = rec["calibration"]
    fetch = rec["fetch_kib_per_launch"] * 1024 * cal["fetch_factor"]
    write = rec["write_kib_per_launch"] * 1024 * cal["write_factor"]
    return {"bytes": int(round(fetch + write)), "fetch_bytes": int(round(fetch)), "write_bytes": int(round(write))}


# ------------------------------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on bounded samples of the mixed batch, one single-threaded
# process per host core.  It runs before anything touches the GPU, in a fork pool that shares the
# generated inputs.
# ------------------------------------------------------------------------------------------------
_CPU = {}


def _cpu_init():
    from threadpoolctl import threadpool_limits
    _CPU["limit"] = threadpool_limits(1)


def _cpu_decode_task(task):
    """Oracle decode (scores, top-k, gate, attention) of the per-head units of one (sequence, KV group)
    of the mixed batch's decode half; the representatives are resident, as on the GPU."""
    from oracle import sas_oracle as orc
    b, g = task
    w = _CPU["w"]
    q, K, V = _CPU["host"][b]
    t0 = time.perf_counter()
    orc.run_sequence(q, K, V, w.seq_lens[b], w.q_start[b], w.block, w.sel, k_fixed=w.k_fixed, frac_num=w.frac_num,
                     frac_den=w.frac_den, count_current=w.count_current, sink=w.sink, gate=w.gate,
                     reps=_CPU["reps"][b], unit_filter=lambda u: u.sel_head // w.group == g)
    return time.perf_counter() - t0, w.group


def _cpu_prefill_task(task):
    """Oracle prefill (scores, top-k, gate, attention) of a few sampled per-head units of one sequence."""
    from oracle import sas_oracle as orc
    b, keys = task
    w = _CPU["w"]
    q, K, V = _CPU["host"][b]
    keyset = set(keys)
    t0 = time.perf_counter()
    orc.run_sequence(q, K, V, w.seq_lens[b], w.q_start[b], w.block, w.sel, k_fixed=w.k_fixed, frac_num=w.frac_num,
                     frac_den=w.frac_den, count_current=w.count_current, sink=w.sink, gate=w.gate,
                     reps=_CPU["reps"][b], unit_filter=lambda u: (u.sel_head, u.c) in keyset)
    return time.perf_counter() - t0, len(keys)


def cpu_baseline_mixed(w, host, decode_seqs, prefill_seqs, seconds):
    """Time the oracle on the mixed batch: every decode unit (repeated until ~seconds/2 of wall time)
    and a seeded sample of prefill units (~seconds/2), in a pool of one single-threaded process per core of
    the affinity mask; also the decode units in one single-threaded process.  Returns seconds per decode
    step (all 8 x 32 units), seconds per prefill half (extrapolated from the sample), and the details."""
    import multiprocessing as mp

    import numpy as np
    from oracle import sas_oracle as orc
    from threadpoolctl import threadpool_limits
    cores = len(os.sched_getaffinity(0))
    _CPU["w"] = w
    _CPU["host"] = host
    # representatives are resident in both paths (pooled once per context): not timed
    _CPU["reps"] = {b: np.stack([orc.block_reps(host[b][1][g], w.seq_lens[b], w.block) for g in range(w.hkv)])
                    for b in list(decode_seqs) + list(prefill_seqs)}
    dec_tasks = [(b, g) for b in decode_seqs for g in range(w.hkv)]
    units_per_step = len(decode_seqs) * w.hq
    rng = np.random.default_rng(99)
    ctx = mp.get_context("fork")
    with ctx.Pool(cores, initializer=_cpu_init) as pool:
        n_dec, t_dec = 0, 0.0
        while t_dec < seconds / 2:
            t0 = time.perf_counter()
            res = pool.map(_cpu_decode_task, dec_tasks, chunksize=1)
            t_dec += time.perf_counter() - t0
            n_dec += sum(r[1] for r in res)
        # prefill: per-head units of the sampled sequences, ~seconds/2 of wall time in rounds
        qb = {b: orc.query_blocks(w.q_start[b], w.rows[b], w.block) for b in prefill_seqs}
        n_pf, t_pf = 0, 0.0
        while t_pf < seconds / 2:
            tasks = []
            for _ in range(cores):
                b = int(rng.choice(list(prefill_seqs)))
                keys = [(int(rng.integers(w.hq)), int(qb[b][int(rng.integers(len(qb[b])))][0])) for _ in range(4)]
                tasks.append((b, keys))
            t0 = time.perf_counter()
            res = pool.map(_cpu_prefill_task, tasks, chunksize=1)
            t_pf += time.perf_counter() - t0
            n_pf += sum(r[1] for r in res)
    # one single-threaded process, the same decode units
    with threadpool_limits(1):
        n1, t1 = 0, 0.0
        while t1 < seconds / 4:
            for task in dec_tasks:
                dt, n = _cpu_decode_task(task)
                t1 += dt
                n1 += n
    pf_units = sum(len(qb[b]) for b in qb) * w.hq * (w.spec["n_prefill"] / len(prefill_seqs))
    return dict(cores=cores, step_s=t_dec / n_dec * units_per_step, step_s_1proc=t1 / n1 * units_per_step,
                prefill_s=t_pf / n_pf * pf_units, n_dec=n_dec, t_dec=t_dec, n_pf=n_pf, t_pf=t_pf, n1=n1, t1=t1,
                pf_units=int(pf_units), units_per_step=units_per_step)


# ------------------------------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", default="mixed,decode,paged,reps,prefill,backward,gist,hssa",
                    help="comma list of measurements: mixed,decode,paged,reps,prefill,backward,gist,hssa,copy")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=16.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (each GPU would run the same "
              "kernels on its own share of sequences / KV heads); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    only = set(x for x in args.only.split(",") if x)

    import numpy as np
    import torch
    from workloads import Workload
    from workloads.device import upload

    K_, W_ = args.steps, args.warmup
    k_small = max(5, args.steps // 5)
    extra = {}
    result = {"metric": "decode GB/s (%HBM peak) + prefill TFLOP/s (%MFMA peak) at sparsity 0.95",
              "value": None, "unit": "GB/s", "n_gpus": 1, "steps": K_, "warmup": W_, "ms_per_step": None,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
              "data": "synthetic (seeded; needle blocks planted)"}

    # ---------------------------------------------------------------- inputs of the headline workload
    w5 = Workload(5)
    dseq, pseq = w5.decode_seqs(), w5.prefill_seqs()
    pre5 = {}
    cpu = None
    if "mixed" in only:
        log("[bench] generating the mixed batch (16 sequences, 4096..131072 tokens)")
        pre5 = {b: (w5.q(b), *w5.kv(b)) for b in dseq + pseq}
        if not args.no_cpu_baseline:
            log("[bench] cpu baseline (oracle, before the GPU is touched)")
            cpu = cpu_baseline_mixed(w5, pre5, dseq, pseq[:2], args.cpu_seconds)
            log(f"[bench] cpu: decode step {cpu['step_s'] * 1e3:.1f} ms on {cpu['cores']} processes "
                f"({cpu['step_s_1proc'] * 1e3:.1f} ms in one), prefill half {cpu['prefill_s']:.1f} s (extrapolated)")

    import top_block_sparse_gist_amd as sas
    sas.load()
    torch.cuda.init()
    timer = Timer(torch)

    # ---------------------------------------------------------------- headline: the mixed batch at 0.95
    if "mixed" in only:
        inp_p = upload(w5, pseq, pre=pre5)
        inp_d = upload(w5, dseq, pre=pre5)
        pre5.clear()
        pf_fns, pf_bufs = prefill_step_setup(sas, w5, inp_p)
        dc_fns, dc_bufs = decode_step_setup(sas, w5, inp_d)
        torch.cuda.synchronize()
        fl = prefill_flops(w5, inp_p, pf_bufs)
        by = decode_bytes(w5, inp_d, dc_bufs)
        log("[bench] timing the mixed batch (prefill half, then decode half, per step)")
        (t_pf, t_dc), wall = timer.time_halves(pf_fns["step"], dc_fns["step"], K_, W_)
        t_pf_att, _ = timer.time(pf_fns["attend"], k_small, 2)
        t_pf_sel, _ = timer.time(pf_fns["select"], k_small, 2)
        t_dc_att, _ = timer.time(dc_fns["attend"], K_, W_)
        t_dc_sel, _ = timer.time(dc_fns["select"], K_, W_)
        t_dc_sel2, _ = timer.time(dc_fns["select_two_calls"], K_, W_)
        t_dc_graph, _ = timer.time(dc_fns["step"], K_, W_, use_graph=True)
        value = by["total"] / (t_dc * 1e-3) / 1e9
        tf_half = fl["flops"] / (t_pf * 1e-3) / 1e12
        tf_att = fl["flops"] / (t_pf_att * 1e-3) / 1e12
        dec_bytes = by["kv"] + by["qo"]
        ach = dec_bytes / (t_dc_att * 1e-3) / 1e9
        tr_d = measured_traffic("decode_bf16_kernel<128, 4, 1, unsigned short, false, 32>")
        tr_p = measured_traffic("prefill_bf16_kernel<128, 2, 64>")
        result.update({
            "value": round(value, 2), "ms_per_step": round(t_pf + t_dc, 5),
            "config": {"workload": "mixed_varlen_16seq_h32x8_d128_blk64_perhead_top5pct+current_gate",
                       "sequences": 16, "seq_lens": w5.seq_lens, "prefill": "8 sequences, their last 4096 rows",
                       "decode": "8 sequences, one row each", "hq": w5.hq, "hkv": w5.hkv, "d": w5.d,
                       "block": w5.block, "budget": "ceil((c+1)/20) + current, per query head, log-gate",
                       "step": "prefill half (reps of the new blocks, block scores, top-k, sparse prefill) then decode "
                               "half (fused scores + top-k, sparse decode); earlier reps resident",
                       "timing": "HIP events around each half on the launch stream, each queued behind a 1 GiB "
                                 "cache flush; medians over the steps",
                       "value_is": "decode half: algorithmic bytes / decode-half time",
                       "decode_half_ms": round(t_dc, 5), "decode_bytes_per_step": by["total"],
                       "decode_pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
                       "decode_graph_replay_ms": round(t_dc_graph, 5),
                       "decode_selection_ms": round(t_dc_sel, 5),
                       "decode_selection_two_calls_ms": round(t_dc_sel2, 5),
                       "prefill_half_ms": round(t_pf, 5), "prefill_half_TFLOP/s": round(tf_half, 1),
                       "prefill_half_pct_mfma_peak": round(100 * tf_half / BF16_PEAK_TFLOPS, 2),
                       "prefill_selection_ms": round(t_pf_sel, 5),
                       "prefill_flops": fl["flops"], "prefill_sparsity": round(fl["sparsity"], 4),
                       "wall_ms_per_step_incl_cache_flushes": round(wall / K_ * 1e3, 4)},
            "roofline": {"bound": "hbm", "kernel": "decode_bf16_kernel (sas_sparse_decode, mixed batch decode half)",
                         "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": tr_d["bytes"] if tr_d else None,
                         "bytes_per_launch": dec_bytes, "avg_launch_ms": round(t_dc_att, 5),
                         "traffic_detail": tr_d},
            "roofline_prefill": {"bound": "mfma", "kernel": "prefill_bf16_kernel (sas_sparse_prefill, mixed batch "
                                                            "prefill half)",
                                 "achieved": round(tf_att, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                 "frac": round(tf_att / BF16_PEAK_TFLOPS, 4), "traffic": tr_p["bytes"] if tr_p else None,
                                 "flops_per_launch": fl["flops"], "avg_launch_ms": round(t_pf_att, 5),
                                 "traffic_detail": tr_p,
                                 # the bandwidth roof that the kernel's measured traffic implies (its FLOP per
                                 # HBM byte x 8 TB/s), and the fraction of that roof reached
                                 "traffic_roof": ({"flop_per_byte": round(fl["flops"] / tr_p["bytes"], 2),
                                                   "roof_TFLOP/s": round(fl["flops"] / tr_p["bytes"] * HBM_PEAK_GBS / 1e3, 1),
                                                   "frac": round(tf_att / (fl["flops"] / tr_p["bytes"] * HBM_PEAK_GBS / 1e3), 4)}
                                                  if tr_p else None)},
        })
        if cpu is not None:
            result["cpu_baseline"] = {
                "value": round(by["total"] / cpu["step_s"] / 1e9, 4), "unit": "GB/s", "cores": cpu["cores"],
                "kind": "oracle",
                "sample": (f"every decode unit of the mixed batch ({cpu['units_per_step']} per step) run "
                           f"{cpu['n_dec'] // cpu['units_per_step']} times in {cpu['t_dec']:.1f} s by a pool of "
                           f"{cpu['cores']} single-threaded processes (one per core of the affinity mask), reps "
                           f"resident: {cpu['step_s'] * 1e3:.1f} ms per decode step"),
                "one_process": {"value": round(by["total"] / cpu["step_s_1proc"] / 1e9, 4), "unit": "GB/s",
                                "step_ms": round(cpu["step_s_1proc"] * 1e3, 2)},
                "prefill": {"value": round(fl["flops"] / cpu["prefill_s"] / 1e12, 6), "unit": "TFLOP/s",
                            "half_s_extrapolated": round(cpu["prefill_s"], 2),
                            "sample": (f"{cpu['n_pf']} sampled per-head units of 2 of the 8 prefill sequences in "
                                       f"{cpu['t_pf']:.1f} s on the same pool, extrapolated to the "
                                       f"{cpu['pf_units']} units of the prefill half")}}
        log(f"[bench] mixed: decode half {t_dc * 1e3:.1f} us -> {value:.0f} GB/s ({100 * value / HBM_PEAK_GBS:.1f} %); "
            f"attention {t_dc_att * 1e3:.1f} us -> {ach:.0f} GB/s; graph {t_dc_graph * 1e3:.1f} us; selection {t_dc_sel * 1e3:.1f} us "
            f"(two calls {t_dc_sel2 * 1e3:.1f} us)")
        log(f"[bench] mixed: prefill half {t_pf:.3f} ms -> {tf_half:.0f} TFLOP/s; attention {t_pf_att:.3f} ms -> "
            f"{tf_att:.0f} TFLOP/s ({100 * tf_att / BF16_PEAK_TFLOPS:.1f} %); selection {t_pf_sel:.3f} ms")
        if "backward" in only:
            backward_measure(sas, torch, timer, extra, "mixed_prefill_backward", w5, inp_p,
                             "backward of the mixed batch's prefill half", pf_fns, pf_bufs, fl, k_small)
        del inp_p, inp_d, pf_fns, pf_bufs, dc_fns, dc_bufs
        torch.cuda.empty_cache()

    # ---------------------------------------------------------------- the 32K decode batch
    if only & {"decode", "paged", "reps"}:
        w2 = Workload(2)
        log("[bench] generating the 32K decode workload")
        inp2 = upload(w2, list(range(w2.batch)))
        fns, bufs = decode_step_setup(sas, w2, inp2)
        torch.cuda.synchronize()
        by2 = decode_bytes(w2, inp2, bufs)
        if "decode" in only:
            ms, _ = timer.time(fns["step"], K_, W_)
            ms_graph, _ = timer.time(fns["step"], K_, W_, use_graph=True)
            ms_att, _ = timer.time(fns["attend"], K_, W_)
            gbs = by2["total"] / (ms * 1e-3) / 1e9
            att = (by2["kv"] + by2["qo"]) / (ms_att * 1e-3) / 1e9
            tr = measured_traffic("decode_bf16_kernel<128, 4, 1, unsigned short, false, 64>")
            extra["decode_32k"] = {"workload": "decode_b8_h32x8_d128_ctx32768_blk64_top16+current (sparsity 0.967)",
                                   "step_us": round(ms * 1e3, 2), "GB/s": round(gbs, 1),
                                   "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                                   "graph_replay_us": round(ms_graph * 1e3, 2), "attend_us": round(ms_att * 1e3, 2),
                                   "attend_GB/s": round(att, 1), "attend_pct_hbm_peak": round(100 * att / HBM_PEAK_GBS, 2),
                                   "bytes_per_step": by2["total"], "attend_traffic_bytes": tr["bytes"] if tr else None}
            log(f"[bench] decode 32K: step {ms * 1e3:.1f} us (graph {ms_graph * 1e3:.1f}) -> {gbs:.0f} GB/s; "
                f"attention {ms_att * 1e3:.1f} us -> {att:.0f} GB/s")
        if "decode" in only:
            # the same step with the lengths in device memory (what a graph-replayed decode loop uses):
            # the current blocks pooled again, fused selection, attention
            lens_dev = torch.tensor(inp2.seq_lens, dtype=torch.int32, device="cuda")
            Lm2 = inp2.K.shape[2]
            bud2 = sas.Budget(k_fixed=w2.k_fixed)
            O_dev = torch.empty_like(inp2.Q)
            ws_sel = torch.zeros(sas.select_decode_workspace_bytes(w2.batch, w2.hq, w2.hkv, w2.d, w2.block,
                                                                   sas.SAS_BF16, Lm2, inp2.seq_lens),
                                 dtype=torch.uint8, device="cuda")
            ws_dec = torch.zeros(sas.decode_workspace_bytes(w2.batch, w2.hq, w2.hkv, w2.d, w2.block, sas.SAS_BF16, Lm2,
                                                            inp2.seq_lens, w2.sel, bufs["idx"].shape[1], False),
                                 dtype=torch.uint8, device="cuda")

            def step_dev():
                sas.block_reps(inp2.K, lens_dev, w2.block, reps=bufs["reps"], current_block=True)
                sas.select_decode(inp2.Q, bufs["reps"], lens_dev, w2.block, w2.hkv, Lm2, bud2, kcap=bufs["idx"].shape[1],
                                  scores=bufs["scores"], idx=bufs["idx"], nsel=bufs["nsel"], workspace=ws_sel)
                sas.sparse_decode(inp2.Q, inp2.K, inp2.V, lens_dev, w2.block, bufs["idx"], bufs["nsel"], None, O=O_dev,
                                  workspace=ws_dec)
            t_dev, _ = timer.time(step_dev, K_, W_)
            t_dev_g, _ = timer.time(step_dev, K_, W_, use_graph=True)
            extra["decode_32k_device_lengths"] = {
                "step_us": round(t_dev * 1e3, 2), "graph_replay_us": round(t_dev_g * 1e3, 2),
                "what": "lengths read from device memory: current blocks pooled again, fused selection, attention"}
            log(f"[bench] decode 32K with device lengths (reps update + selection + attention): {t_dev * 1e3:.1f} us, "
                f"graph {t_dev_g * 1e3:.1f} us")
        if "paged" in only:
            paged_measure(sas, torch, np, timer, extra, w2, inp2, bufs, K_, W_)
        if "reps" in only:
            K = inp2.K
            reps = bufs["reps"]
            t, _ = timer.time(lambda: sas.block_reps(K, inp2.seq_lens, w2.block, reps=reps), k_small, 2)
            rb = K.numel() * 2 + reps.numel() * 4
            extra["reps_32k"] = {"us": round(t * 1e3, 2), "GB/s": round(rb / (t * 1e-3) / 1e9, 1), "bytes": rb,
                                 "pct_hbm_peak": round(100 * rb / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}
            log(f"[bench] reps 32K: {t * 1e3:.1f} us -> {rb / (t * 1e-3) / 1e9:.0f} GB/s")
            first = [(L - 1) // w2.block for L in inp2.seq_lens]
            tu, _ = timer.time(lambda: sas.block_reps(K, inp2.seq_lens, w2.block, reps=reps, first_block=first), K_, W_)
            extra["reps_update_32k"] = {"us": round(tu * 1e3, 2), "blocks": len(inp2.seq_lens) * w2.hkv,
                                        "what": "the current block of every (sequence, KV head) pooled again"}
        del inp2, bufs, fns
        torch.cuda.empty_cache()

    if "prefill" in only:
        w3 = Workload(3)
        log("[bench] generating the 32K prefill workload")
        inp3 = upload(w3, [0])
        fns, bufs = prefill_step_setup(sas, w3, inp3)
        torch.cuda.synchronize()
        fl3 = prefill_flops(w3, inp3, bufs)
        t_step, _ = timer.time(fns["step"], k_small, 2)
        t_att, _ = timer.time(fns["attend"], k_small, 2)
        t_sel, _ = timer.time(fns["select"], k_small, 2)
        tf = fl3["flops"] / (t_att * 1e-3) / 1e12
        tr = measured_traffic("prefill_bf16_kernel<128, 4, 128>")
        extra["prefill_32k"] = {"workload": "prefill_b1_h28x4_d128_32768_blk128_top1/8+sink+current_gate",
                                "step_ms": round(t_step, 4), "prefill_ms": round(t_att, 4),
                                "selection_ms": round(t_sel, 4), "TFLOP/s": round(tf, 1),
                                "pct_mfma_peak": round(100 * tf / BF16_PEAK_TFLOPS, 2),
                                "step_TFLOP/s": round(fl3["flops"] / (t_step * 1e-3) / 1e12, 1),
                                "flops": fl3["flops"], "sparsity": round(fl3["sparsity"], 4),
                                "traffic_bytes": tr["bytes"] if tr else None}
        log(f"[bench] prefill 32K: {t_att:.3f} ms -> {tf:.0f} TFLOP/s ({100 * tf / BF16_PEAK_TFLOPS:.1f} %); "
            f"step {t_step:.3f} ms, selection {t_sel:.3f} ms")
        if "backward" in only:
            backward_measure(sas, torch, timer, extra, "prefill_backward_32k", w3, inp3,
                             "backward of prefill_b1_h28x4_d128_32768_blk128_top1/8+sink+current_gate", fns, bufs,
                             fl3, k_small)
        del inp3, fns, bufs
        torch.cuda.empty_cache()

    if "gist" in only:
        w4 = Workload(4)
        log("[bench] generating the 128K gist decode workload")
        inp4 = upload(w4, list(range(w4.batch)), gist=True)
        fns, bufs = decode_step_setup(sas, w4, inp4, gist=True)
        torch.cuda.synchronize()
        byw = decode_bytes(w4, inp4, bufs, gist=True)
        t_step, _ = timer.time(fns["step"], K_, W_)
        t_att, _ = timer.time(fns["attend"], K_, W_)
        gbs = byw["total"] / (t_step * 1e-3) / 1e9
        extra["gist_decode_128k"] = {"workload": "gist_decode_b4_h64x8_d128_ctx131073_chunk64_top104",
                                     "step_us": round(t_step * 1e3, 2), "attend_us": round(t_att * 1e3, 2),
                                     "GB/s": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                                     "bytes_per_step": byw["total"]}
        log(f"[bench] gist decode 128K: step {t_step * 1e3:.1f} us -> {gbs:.0f} GB/s; attend {t_att * 1e3:.1f} us")
        del inp4, fns, bufs
        torch.cuda.empty_cache()

    if "hssa" in only:
        w6 = Workload(6)
        log("[bench] generating the 128K two-level gist decode workload")
        inp6 = upload(w6, list(range(w6.batch)), gist=True, meta=True)
        fns, bufs = hssa_step_setup(sas, w6, inp6)
        torch.cuda.synchronize()
        hb = hssa_bytes(w6, inp6, bufs)
        t_step, _ = timer.time(fns["step"], K_, W_)
        t_att, _ = timer.time(fns["attend"], K_, W_)
        gbs = hb / (t_step * 1e-3) / 1e9
        extra["hssa_decode_128k"] = {
            "workload": "hssa_decode_b4_h64x8_d128_ctx131073_chunk64_groups32_open8_top104",
            "step_us": round(t_step * 1e3, 2), "attend_us": round(t_att * 1e3, 2), "GB/s": round(gbs, 1),
            "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2), "bytes_per_step": hb}
        log(f"[bench] hssa decode 128K: step {t_step * 1e3:.1f} us -> {gbs:.0f} GB/s; attend {t_att * 1e3:.1f} us")
        del inp6, fns, bufs
        torch.cuda.empty_cache()

    if "copy" in only:
        # plain copy of known size: calibrates the profiler's HBM byte counters
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        b_ = torch.empty_like(a)
        for _ in range(3):
            b_.copy_(a)
        torch.cuda.synchronize()
        extra["copy_calibration_bytes"] = {"read": a.numel(), "write": a.numel()}

    result["extra"] = extra
    print(json.dumps(result), flush=True)


def backward_measure(sas, torch, timer, extra, name, w, inp, desc, fns, bufs, fl, k_small):
    """Gradients of the sparse prefill (loss sum(O * dO)) for the step's own lists and O."""
    # the training forward keeps each row's log-sum-exp for the backward
    lse = torch.empty(inp.Q.shape[:3], dtype=torch.float32, device=inp.Q.device)
    sas.sparse_prefill(inp.Q, inp.K, inp.V, inp.seq_lens, w.block, inp.q_start, bufs["idx"], bufs["nsel"],
                       bufs["gate"], sel_mode=w.sel, O=bufs["O"], lse=lse)
    dO = torch.zeros_like(inp.Q)
    for bi, b in enumerate(inp.seqs):
        dO[bi] = torch.from_numpy(w.grad_out(b)).to(torch.bfloat16).to(dO.device)
    f32 = dict(dtype=torch.float32, device=inp.Q.device)
    B, hq, tq, d = inp.Q.shape
    _, hkv, lmax, _ = inp.K.shape
    has_gate = bufs["gate"] is not None
    grads = (torch.empty(B, hq, tq, d, **f32), torch.zeros(B, hkv, lmax, d, **f32),
             torch.zeros(B, hkv, lmax, d, **f32), torch.empty(bufs["idx"].shape, **f32) if has_gate else None,
             torch.empty(bufs["idx"].shape, **f32) if has_gate else None)
    need = sas.prefill_backward_workspace_bytes(B, hq, hkv, d, w.block, lmax, inp.seq_lens, tq, w.sel,
                                                bufs["idx"].shape[1], has_gate)
    ws = torch.empty(max(1, need), dtype=torch.uint8, device=inp.Q.device)

    def backward():
        sas.sparse_prefill_backward(inp.Q, inp.K, inp.V, bufs["O"], dO, inp.seq_lens, w.block, inp.q_start,
                                    bufs["idx"], bufs["nsel"], bufs["gate"], sel_mode=w.sel, workspace=ws,
                                    grads=grads, lse=lse)
    t_bwd, _ = timer.time(backward, k_small, 2)
    bflops = 2.5 * fl["flops"]  # 10 d per visible pair: S, dP, dQ, dK, dV (the forward's 4 d x 2.5)
    tf = bflops / (t_bwd * 1e-3) / 1e12
    extra[name] = {"workload": desc, "backward_ms": round(t_bwd, 4), "TFLOP/s": round(tf, 1),
                   "pct_mfma_peak": round(100 * tf / BF16_PEAK_TFLOPS, 2), "flops": bflops, "workspace_bytes": need}
    log(f"[bench] {name}: backward {t_bwd:.3f} ms -> {tf:.0f} TFLOP/s")
    del grads, ws, dO


def paged_measure(sas, torch, np, timer, extra, w2, inp2, bufs, K_, W_):
    """The 32K decode over a paged cache: K/V blocks scattered into shuffled pages of one block each,
    read through a block table."""
    blk, lens2 = w2.block, inp2.seq_lens
    nbs = [-(-L // blk) for L in lens2]
    perm = np.random.default_rng(5).permutation(sum(nbs))
    Kp = torch.zeros((sum(nbs), w2.hkv, blk, w2.d), dtype=inp2.K.dtype, device="cuda")
    Vp = torch.zeros_like(Kp)
    table = torch.empty((len(lens2), max(nbs)), dtype=torch.int32)
    n = 0
    for b, L in enumerate(lens2):
        pages = torch.from_numpy(perm[n:n + nbs[b]]).cuda()
        Kp[pages] = inp2.K[b, :, :nbs[b] * blk].reshape(w2.hkv, nbs[b], blk, w2.d).transpose(0, 1)
        Vp[pages] = inp2.V[b, :, :nbs[b] * blk].reshape(w2.hkv, nbs[b], blk, w2.d).transpose(0, 1)
        table[b, :nbs[b]] = torch.from_numpy(perm[n:n + nbs[b]].astype(np.int32))
        n += nbs[b]
    table = table.cuda()
    Op = torch.empty_like(inp2.Q)
    ws_p = torch.zeros(sas.decode_workspace_bytes(len(lens2), w2.hq, w2.hkv, w2.d, blk, sas.SAS_BF16,
                                                  inp2.K.shape[2], lens2, w2.sel, bufs["idx"].shape[1], False),
                       dtype=torch.uint8, device="cuda")
    Lm = inp2.K.shape[2]

    def attend_paged():
        sas.sparse_decode_paged(inp2.Q, Kp, Vp, table, lens2, blk, Lm, bufs["idx"], bufs["nsel"], bufs["gate"],
                                sel_mode=w2.sel, O=Op, workspace=ws_p)
    tp, _ = timer.time(attend_paged, K_, W_)
    extra["decode_paged_32k"] = {"attend_us": round(tp * 1e3, 2),
                                 "what": "sas_sparse_decode_paged on the 32K decode batch, shuffled pages"}
    log(f"[bench] paged decode attention: {tp * 1e3:.1f} us")
    del Kp, Vp, table, Op, ws_p
    torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
