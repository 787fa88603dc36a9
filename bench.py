#!/usr/bin/env python3
"""Benchmark of content-selected block-sparse attention on one MI355X.

Headline (`value`): decode GB/s on the 32K decode workload (batch 8, 32 query / 8 KV heads,
d 128, 64-token blocks, top-16 + current block).  One step = block scores + top-k + sparse
decode for the whole batch; the block representatives are resident (computed once per
context, like the KV cache itself) and are timed separately under extra.reps.
Throughput = algorithmic bytes of the step / step time; the L2s and the 256 MB MALL are
flushed (1 GiB read) before every timed step, outside the timed interval, so bytes come
from HBM.  extra.* holds the other workloads: causal prefill (TFLOP/s) and its backward, the SSA-style gist
decode, and the mixed variable-length batch at sparsity 0.95 (prefill TFLOP/s, decode GB/s).

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
        n = len(ts)
        med = ts[n // 2] if n % 2 else 0.5 * (ts[n // 2 - 1] + ts[n // 2])
        return med, wall


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

    def step():
        sas.select_decode(inp.Q, reps, lens, w.block, w.hkv, Lmax, budget, sel_mode=w.sel, gist=gist,
                          kcap=idx.shape[1], scores=scores, idx=idx, nsel=nsel, gate=gate, workspace=sel_ws)
        attend()

    fns = dict(step=step, attend=attend)
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
    import torch
    lens = inp.seq_lens
    Lmax = inp.K.shape[2]
    dt = sas.SAS_BF16
    budget = sas.Budget(k_fixed=w.k_fixed, frac_num=w.frac_num, frac_den=w.frac_den,
                        count_current=w.count_current, sink=w.sink, gate=w.gate)
    reps = sas.block_reps(inp.K, lens, w.block)
    scores = sas.block_scores(inp.Q, reps, lens, w.block, w.hkv, Lmax, q_start=inp.q_start, sel_mode=w.sel)
    ws = torch.empty(max(1, len(lens) * (w.hq if w.sel == "head" else w.hkv) * sas.num_qblocks(w.tq, w.block)
                         * w.d * 4), dtype=torch.uint8, device="cuda")
    idx, nsel, gate = sas.topk_select(scores, lens, w.block, w.hq, w.hkv, w.d, dt, Lmax, budget, tq=w.tq,
                                      q_start=inp.q_start, sel_mode=w.sel)
    O = torch.empty_like(inp.Q)

    def make_reps():
        sas.block_reps(inp.K, lens, w.block, reps=reps)

    def attend():
        sas.sparse_prefill(inp.Q, inp.K, inp.V, lens, w.block, inp.q_start, idx, nsel, gate, sel_mode=w.sel, O=O)

    def step():
        make_reps()
        sas.block_scores(inp.Q, reps, lens, w.block, w.hkv, Lmax, q_start=inp.q_start, sel_mode=w.sel,
                         scores=scores, workspace=ws)
        sas.topk_select(scores, lens, w.block, w.hq, w.hkv, w.d, dt, Lmax, budget, tq=w.tq, q_start=inp.q_start,
                        sel_mode=w.sel, idx=idx, nsel=nsel, gate=gate)
        attend()

    return dict(step=step, attend=attend, reps=make_reps), dict(reps=reps, idx=idx, nsel=nsel, gate=gate, O=O)


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
# CPU baseline: the oracle as it stands, on a bounded sample of the decode workload
# ------------------------------------------------------------------------------------------------
def cpu_baseline_decode(w, host, bytes_per_step, seconds):
    import numpy as np
    from oracle import sas_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    seqs = sorted(host)
    reps = {b: np.stack([orc.block_reps(host[b]["k"][g], w.seq_lens[b], w.block) for g in range(w.hkv)])
            for b in seqs}
    units = 0
    t0 = time.perf_counter()
    while True:
        for b in seqs:
            h = host[b]
            orc.run_sequence(h["q"], h["k"], h["v"], w.seq_lens[b], w.q_start[b], w.block, w.sel,
                             k_fixed=w.k_fixed, reps=reps[b])
            units += w.hkv
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    units_per_step = w.batch * w.hkv
    step_s = dt / units * units_per_step
    return {"value": round(bytes_per_step / step_s / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{units} (sequence, KV group) decode units of the 32K decode workload "
                      f"({len(seqs)} sequences repeated for {dt:.1f} s; reps precomputed), scaled to the "
                      f"{units_per_step}-unit step: {step_s * 1e3:.1f} ms/step"}


# ------------------------------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", default="decode,paged,reps,prefill,backward,gist,hssa,mixed",
                    help="comma list of measurements: decode,reps,prefill,gist,mixed,copy")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (each GPU would run the same "
              "kernels on its own share of sequences / KV heads); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    only = set(x for x in args.only.split(",") if x)

    import numpy as np
    import torch
    import top_block_sparse_gist_amd as sas
    from workloads import Workload
    from workloads.device import upload

    sas.load()
    torch.cuda.init()
    timer = Timer(torch)
    extra = {}
    result = None
    K_, W_ = args.steps, args.warmup
    k_small = max(3, args.steps // 10)

    # ---------------------------------------------------------------- headline: 32K decode
    w2 = Workload(2)
    need_decode = bool(only & {"decode", "reps", "paged"}) or not args.no_cpu_baseline
    if not need_decode:
        log("[bench] skipping the 32K decode workload")
    log("[bench] generating the 32K decode workload") if need_decode else None
    keep = {0, 1} if not args.no_cpu_baseline else set()
    inp2 = upload(w2, list(range(w2.batch)), keep_host=keep) if need_decode else None
    fns, bufs = decode_step_setup(sas, w2, inp2) if need_decode else (None, None)
    torch.cuda.synchronize()
    by = decode_bytes(w2, inp2, bufs) if need_decode else None
    if "decode" in only:
        log("[bench] timing decode")
        ms, wall = timer.time(fns["step"], K_, W_)
        ms_graph, _ = timer.time(fns["step"], K_, W_, use_graph=True)
        ms_att, _ = timer.time(fns["attend"], K_, W_)
        value = by["total"] / (ms * 1e-3) / 1e9
        dec_bytes = by["kv"] + by["qo"]
        ach = dec_bytes / (ms_att * 1e-3) / 1e9
        tr = measured_traffic("decode_bf16_kernel<128, 4, 1, unsigned short, false>")
        result = {
            "metric": "decode GB/s (%HBM peak) + prefill TFLOP/s (%MFMA peak) at sparsity 0.95",
            "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K_, "warmup": W_,
            "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic (seeded; needle blocks planted)",
            "config": {"workload": "decode_b8_h32x8_d128_ctx32768_blk64_top16+current",
                       "batch": w2.batch, "hq": w2.hq, "hkv": w2.hkv, "d": w2.d, "context": w2.seq_lens[0],
                       "block": w2.block, "k": w2.k_fixed, "selection": "per KV group",
                       "step": "fused block scores + top-k, then sparse decode (2 launches); block reps resident",
                       "timing": "HIP events around each step on the launch stream, queued behind a 1 GiB cache flush",
                       "bytes_per_step": by["total"], "sparsity": round(1 - 17 / 512, 4),
                       "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
                       "graph_replay_ms_per_step": round(ms_graph, 5),
                       "wall_ms_per_step_incl_cache_flush": round(wall / K_ * 1e3, 4)},
            "roofline": {"bound": "hbm", "kernel": "sas_sparse_decode (decode_bf16_kernel, split-K with in-kernel merge)",
                         "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": tr["bytes"] if tr else None,
                         "bytes_per_launch": dec_bytes, "avg_launch_ms": round(ms_att, 5),
                         "traffic_detail": tr},
        }
        log(f"[bench] decode step {ms * 1e3:.1f} us (graph replay {ms_graph * 1e3:.1f}) -> {value:.0f} GB/s; "
            f"attention {ms_att * 1e3:.1f} us -> {ach:.0f} GB/s")
    if "paged" in only and inp2 is not None:
        # the same 32K decode over a paged cache: the K/V blocks scattered into shuffled pages of one
        # block each, read through a block table
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
    if "reps" in only:
        K = inp2.K
        reps = bufs["reps"]
        t, _ = timer.time(lambda: sas.block_reps(K, inp2.seq_lens, w2.block, reps=reps), k_small, 2)
        rb = K.numel() * 2 + reps.numel() * 4
        extra["reps_32k"] = {"us": round(t * 1e3, 2), "GB/s": round(rb / (t * 1e-3) / 1e9, 1), "bytes": rb}
        log(f"[bench] reps 32K: {t * 1e3:.1f} us -> {rb / (t * 1e-3) / 1e9:.0f} GB/s")
        # a decode loop pools again only the block its new token lands in (one per sequence and KV head)
        first = [(L - 1) // w2.block for L in inp2.seq_lens]
        tu, _ = timer.time(lambda: sas.block_reps(K, inp2.seq_lens, w2.block, reps=reps, first_block=first), K_, W_)
        extra["reps_update_32k"] = {"us": round(tu * 1e3, 2), "blocks": len(inp2.seq_lens) * w2.hkv,
                                    "what": "the current block of every (sequence, KV head) pooled again"}
        log(f"[bench] reps update (current block only): {tu * 1e3:.1f} us")
    if not args.no_cpu_baseline and result is not None:
        log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline_decode(w2, inp2.host, by["total"], args.cpu_seconds)
    del inp2, bufs, fns
    torch.cuda.empty_cache()

    def prefill_measure(name, w, inp, desc):
        fns, bufs = prefill_step_setup(sas, w, inp)
        torch.cuda.synchronize()
        fl = prefill_flops(w, inp, bufs)
        t_step, _ = timer.time(fns["step"], k_small, 2)
        t_att, _ = timer.time(fns["attend"], k_small, 2)
        t_rep, _ = timer.time(fns["reps"], k_small, 2)
        tf = fl["flops"] / (t_att * 1e-3) / 1e12
        extra[name] = {"workload": desc, "step_ms": round(t_step, 4), "prefill_ms": round(t_att, 4),
                       "reps_ms": round(t_rep, 4), "TFLOP/s": round(tf, 1),
                       "pct_mfma_peak": round(100 * tf / BF16_PEAK_TFLOPS, 2),
                       "step_TFLOP/s": round(fl["flops"] / (t_step * 1e-3) / 1e12, 1),
                       "flops": fl["flops"], "sparsity": round(fl["sparsity"], 4)}
        log(f"[bench] {name}: prefill {t_att:.3f} ms -> {tf:.0f} TFLOP/s; step {t_step:.3f} ms; "
            f"sparsity {fl['sparsity']:.3f}")
        return fns, bufs, fl

    def backward_measure(name, w, inp, desc, fns, bufs, fl):
        """Gradients of the sparse prefill (loss sum(O * dO)) for the step's own lists and O."""
        import numpy as np
        # the training forward keeps each row's log-sum-exp for the backward
        lse = torch.empty(inp.Q.shape[:3], dtype=torch.float32, device=inp.Q.device)
        sas.sparse_prefill(inp.Q, inp.K, inp.V, inp.seq_lens, w.block, inp.q_start, bufs["idx"], bufs["nsel"],
                           bufs["gate"], sel_mode=w.sel, O=bufs["O"], lse=lse)
        dO = torch.zeros_like(inp.Q)
        for bi, b in enumerate(inp.seqs):
            dO[bi] = torch.from_numpy(np.ascontiguousarray(w.grad_out(b))).to(torch.bfloat16).to(dO.device)
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
                       "pct_mfma_peak": round(100 * tf / BF16_PEAK_TFLOPS, 2), "flops": bflops,
                       "workspace_bytes": need}
        log(f"[bench] {name}: backward {t_bwd:.3f} ms -> {tf:.0f} TFLOP/s")
        del grads, ws, dO

    def decode_measure(name, w, inp, desc, gist=False):
        fns, bufs = decode_step_setup(sas, w, inp, gist=gist)
        torch.cuda.synchronize()
        byw = decode_bytes(w, inp, bufs, gist=gist)
        t_step, _ = timer.time(fns["step"], K_, W_)
        t_att, _ = timer.time(fns["attend"], K_, W_)
        gbs = byw["total"] / (t_step * 1e-3) / 1e9
        extra[name] = {"workload": desc, "step_us": round(t_step * 1e3, 2), "attend_us": round(t_att * 1e3, 2),
                       "GB/s": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                       "attend_GB/s": round((byw["kv"] + byw["qo"]) / (t_att * 1e-3) / 1e9, 1),
                       "bytes_per_step": byw["total"]}
        log(f"[bench] {name}: step {t_step * 1e3:.1f} us -> {gbs:.0f} GB/s; attend {t_att * 1e3:.1f} us")

    if "prefill" in only:
        w3 = Workload(3)
        log("[bench] generating the 32K prefill workload")
        inp3 = upload(w3, [0])
        pf = prefill_measure("prefill_32k", w3, inp3, "prefill_b1_h28x4_d128_32768_blk128_top1/8+sink+current_gate")
        if "backward" in only:
            backward_measure("prefill_backward_32k", w3, inp3,
                             "backward of prefill_b1_h28x4_d128_32768_blk128_top1/8+sink+current_gate", *pf)
        del pf
        del inp3
        torch.cuda.empty_cache()
    if "gist" in only:
        w4 = Workload(4)
        log("[bench] generating the 128K gist decode workload")
        inp4 = upload(w4, list(range(w4.batch)), gist=True)
        decode_measure("gist_decode_128k", w4, inp4, "gist_decode_b4_h64x8_d128_ctx131073_chunk64_top104",
                       gist=True)
        del inp4
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
        log(f"[bench] hssa_decode_128k: step {t_step * 1e3:.1f} us -> {gbs:.0f} GB/s; attend {t_att * 1e3:.1f} us")
        del inp6, fns, bufs
        torch.cuda.empty_cache()
    if "mixed" in only:
        w5 = Workload(5)
        log("[bench] generating the mixed variable-length workload")
        inp5p = upload(w5, w5.prefill_seqs())
        desc5 = f"8 seqs, last 4096 rows, lens {inp5p.seq_lens}, 32/8 heads, per-head, 5% + current, gate"
        pf = prefill_measure("mixed_prefill_half", w5, inp5p, desc5)
        if "backward" in only:
            backward_measure("mixed_prefill_backward", w5, inp5p, "backward of " + desc5, *pf)
        del inp5p, pf
        torch.cuda.empty_cache()
        inp5d = upload(w5, w5.decode_seqs())
        decode_measure("mixed_decode_half", w5, inp5d,
                       f"8 seqs decode, lens {inp5d.seq_lens}, 32/8 heads, per-head, 5% + current, gate")
        del inp5d
        torch.cuda.empty_cache()
    if "copy" in only:
        # plain copy of known size: calibrates the profiler's HBM byte counters
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        b_ = torch.empty_like(a)
        for _ in range(3):
            b_.copy_(a)
        torch.cuda.synchronize()
        extra["copy_calibration_bytes"] = {"read": a.numel(), "write": a.numel()}

    if result is None:
        result = {"metric": "decode GB/s (%HBM peak) + prefill TFLOP/s (%MFMA peak) at sparsity 0.95",
                  "value": None, "unit": "GB/s", "n_gpus": 1, "steps": K_, "warmup": W_}
    result["extra"] = extra
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
