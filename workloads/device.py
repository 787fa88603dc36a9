"""Upload a workload's inputs into padded device tensors (torch), one sequence at a time.

Layouts: Q prefill [B, Hq, tq, d], Q decode [B, Hq, d], K/V [B, Hkv, Lmax, d],
gist K/V [B, Hkv, NCmax, d], meta-gist K/V [B, Hkv, NMmax, d]; rows past a sequence's length are zero.  Values are the
generator's (bf16-representable) numbers, converted exactly to the workload dtype.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

from .gen import Workload


@dataclass
class DeviceInputs:
    seqs: List[int]
    seq_lens: List[int]
    q_start: Optional[List[int]]     # None for decode
    Q: "object"
    K: "object"
    V: "object"
    gist_k: "object" = None
    gist_v: "object" = None
    host: Dict[int, dict] = field(default_factory=dict)   # kept numpy inputs of some sequences
    meta_k: "object" = None                                # [B, Hkv, NMmax, d] (two-level gist mode)
    meta_v: "object" = None


def upload(w: Workload, seqs: List[int], device="cuda", keep_host=(), lmax: Optional[int] = None,
           gist: bool = False, meta: bool = False) -> DeviceInputs:
    import torch
    dt = torch.bfloat16 if w.is_bf16() else torch.float32
    lens = [w.seq_lens[b] for b in seqs]
    kinds = {w.seq_kind[b] for b in seqs}
    assert len(kinds) == 1, "a call holds either prefill or decode sequences"
    decode = kinds == {"decode"}
    Lmax = lmax or max(lens)
    B = len(seqs)
    if decode:
        Q = torch.empty((B, w.hq, w.d), dtype=dt, device=device)
    else:
        Q = torch.empty((B, w.hq, w.tq, w.d), dtype=dt, device=device)
    K = torch.zeros((B, w.hkv, Lmax, w.d), dtype=dt, device=device)
    V = torch.zeros((B, w.hkv, Lmax, w.d), dtype=dt, device=device)
    gk = gv = None
    if gist:
        nc = max(L // w.block for L in lens)
        gk = torch.zeros((B, w.hkv, max(nc, 1), w.d), dtype=dt, device=device)
        gv = torch.zeros((B, w.hkv, max(nc, 1), w.d), dtype=dt, device=device)
    mk = mv = None
    if meta:
        nm = max(L // w.block for L in lens) // w.spec["group_chunks"]
        mk = torch.zeros((B, w.hkv, max(nm, 1), w.d), dtype=dt, device=device)
        mv = torch.zeros((B, w.hkv, max(nm, 1), w.d), dtype=dt, device=device)
    host = {}
    for i, b in enumerate(seqs):
        q = w.q(b)
        Kb, Vb = w.kv(b)
        L = w.seq_lens[b]
        if decode:
            Q[i].copy_(torch.from_numpy(q[:, 0, :]).to(dt))
        else:
            Q[i].copy_(torch.from_numpy(q).to(dt))
        K[i, :, :L].copy_(torch.from_numpy(Kb).to(dt))
        V[i, :, :L].copy_(torch.from_numpy(Vb).to(dt))
        entry = {}
        if gist:
            g_k, g_v = w.gist(b)
            nc = g_k.shape[1]
            if nc:
                gk[i, :, :nc].copy_(torch.from_numpy(g_k).to(dt))
                gv[i, :, :nc].copy_(torch.from_numpy(g_v).to(dt))
            entry.update(gist_k=g_k, gist_v=g_v)
        if meta:
            m_k, m_v = w.meta(b)
            if m_k.shape[1]:
                mk[i, :, :m_k.shape[1]].copy_(torch.from_numpy(m_k).to(dt))
                mv[i, :, :m_v.shape[1]].copy_(torch.from_numpy(m_v).to(dt))
            entry.update(meta_k=m_k, meta_v=m_v)
        if b in keep_host:
            entry.update(q=q, k=Kb, v=Vb)
            host[b] = entry
    torch.cuda.synchronize()
    q_start = None if decode else [w.q_start[b] for b in seqs]
    return DeviceInputs(seqs=list(seqs), seq_lens=lens, q_start=q_start, Q=Q, K=K, V=V, gist_k=gk, gist_v=gv,
                        host=host, meta_k=mk, meta_v=mv)
