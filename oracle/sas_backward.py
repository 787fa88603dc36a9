"""Backward of the gated block-sparse attention (test infrastructure only; CPU, float64).

Only the tests may import this module.  It differentiates the oracle's forward definition with
torch's autograd in float64 on the CPU: for each selection unit and each of its (row, head)
pairs, logits = scale * q K^T + M + g, with M = 0 for keys of the unit's selected blocks at or
before the row's position and -inf otherwise, and g the unit's log-gate of the key's block
([SAS] method, core modules 2-3: the selector score enters the logits through a log-softmax over
the kept set); O = softmax(logits) V.  For the loss sum(O * dO) it returns dQ, dK, dV, the
gradient of each unit's gate values (dgate, one per list entry) and the gradient of the
selector scores of the list entries through g = s - logsumexp over the list (dscore).

Pages cited by title: [SAS] "SAS: 通过端到端优化上下文排序的简单注意力稀疏化".
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Tuple

import numpy as np


def backward_sequence(Qb: np.ndarray, Kb: np.ndarray, Vb: np.ndarray, dOb: np.ndarray, L: int, q_start: int,
                      blk: int, units, gate: bool, scale: Optional[float] = None,
                      through_scores: bool = False) -> dict:
    """Qb, dOb: [hq, rows, d]; Kb, Vb: [hkv, >= L, d]; units: the oracle's selection units of this
    sequence (their .sel lists and .scores), as run_sequence leaves them.

    through_scores (with a gate, pooled representatives): the selector scores are not constants but
    the function of Q and K that the forward scored with, s_j = scale * qbar . r_j (qbar the mean of
    the unit's query vectors over its rows and heads, r_j the mean of block j's present keys), so dQ
    and dK also carry the gradient that reaches the scores through the gate; the lists stay fixed."""
    import torch
    hq, rows, d = Qb.shape
    hkv = Kb.shape[0]
    G = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    f64 = torch.float64
    Q = torch.tensor(np.asarray(Qb, np.float64), dtype=f64, requires_grad=True)
    K = torch.tensor(np.asarray(Kb[:, :L], np.float64), dtype=f64, requires_grad=True)
    V = torch.tensor(np.asarray(Vb[:, :L], np.float64), dtype=f64, requires_grad=True)
    dO = torch.tensor(np.asarray(dOb, np.float64), dtype=f64)
    keys = torch.arange(L)
    loss = torch.zeros((), dtype=f64)
    s_leaves: Dict[Tuple[int, int], torch.Tensor] = {}
    g_nodes: Dict[Tuple[int, int], torch.Tensor] = {}
    for u in units:
        if u.sel is None:
            continue
        sel = list(u.sel)
        key_u = (u.sel_head, u.c)
        if gate:
            if through_scores:
                kvh = u.heads[0] // G
                qbar = Q[list(u.heads), u.t_lo:u.t_hi].reshape(-1, d).mean(dim=0)
                reps = torch.stack([K[kvh, j * blk:min((j + 1) * blk, L)].mean(dim=0) for j in sel])
                s = scale * (reps @ qbar)
                s.retain_grad()
            else:
                s = torch.tensor([float(u.scores[j]) for j in sel], dtype=f64, requires_grad=True)
            g = s - torch.logsumexp(s, dim=0)
            g.retain_grad()
            s_leaves[key_u], g_nodes[key_u] = s, g
            gblk = torch.zeros(L // blk + 2, dtype=f64)
            gblk = gblk.index_put((torch.tensor(sel),), g)
            gkey = gblk[keys // blk]
        else:
            gkey = torch.zeros(L, dtype=f64)
        kv = u.heads[0] // G  # the unit's KV head
        in_sel = torch.zeros(L, dtype=torch.bool)
        for j in sel:
            in_sel[j * blk:min((j + 1) * blk, L)] = True
        for h in u.heads:
            pos = q_start + torch.arange(u.t_lo, u.t_hi)
            allow = in_sel[None, :] & (keys[None, :] <= pos[:, None])
            logits = (Q[h, u.t_lo:u.t_hi] @ K[kv].T) * scale + gkey[None, :]
            logits = logits.masked_fill(~allow, float("-inf"))
            P = torch.softmax(logits, dim=1)
            O = P @ V[kv]
            loss = loss + (O * dO[h, u.t_lo:u.t_hi]).sum()
    loss.backward()
    out = {"dQ": Q.grad.numpy(), "dK": K.grad.numpy(), "dV": V.grad.numpy(), "dgate": {}, "dscore": {}}
    for key_u, g in g_nodes.items():
        out["dgate"][key_u] = g.grad.numpy().copy()
        out["dscore"][key_u] = s_leaves[key_u].grad.numpy().copy()
    return out


def row_logsumexp(Qb: np.ndarray, Kb: np.ndarray, L: int, q_start: int, blk: int, units, gate: bool,
                  scale: Optional[float] = None) -> np.ndarray:
    """Natural-log log-sum-exp of each (head, row)'s logits scale * q.k + g over its unit's visible
    keys (the softmax normaliser of the forward above), float64 [hq, rows]; NaN for rows no unit
    covers."""
    hq, rows, d = Qb.shape
    G = hq // Kb.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.full((hq, rows), np.nan)
    for u in units:
        if u.sel is None:
            continue
        g = u.gate if gate else {}
        for h in u.heads:
            K = np.asarray(Kb[h // G], np.float64)
            for t in range(u.t_lo, u.t_hi):
                pos = q_start + t
                q = np.asarray(Qb[h, t], np.float64)
                logits = []
                for j in u.sel:
                    for s_ in range(j * blk, min((j + 1) * blk, L, pos + 1)):
                        logits.append(scale * float(q @ K[s_]) + (g.get(j, 0.0) if gate else 0.0))
                m = max(logits)
                out[h, t] = m + math.log(sum(math.exp(x - m) for x in logits))
    return out
