"""Content-selected block-sparse attention on MI355X (gfx950): thin Python binding.

Each function marshals torch tensors (device memory) and the current HIP stream into one
call of the C ABI in libsas.so (include/sas.h) and returns the outputs.  Every step of
the computation runs in the library's HIP kernels; when libsas.so is missing the import
of the first call raises.

Layouts (last dim contiguous):  Q, O [B, Hq, T, d] (decode: [B, Hq, d]);
K, V [B, Hkv, Lmax, d];  reps [B, Hkv, NBmax, d] fp32;  gist K/V [B, Hkv, NC, d];
scores [B*S*QB, NBmax] fp32;  idx / gate [B*S*QB, kcap];  nsel [B*S*QB].
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

from . import _lib
from ._lib import (SAS_BF16, SAS_F32, SAS_REPS_GIST, SAS_REPS_POOLED, SAS_SEL_GROUP, SAS_SEL_HEAD,
                   SasError, check, i32x, i64x, load)

__all__ = ["Budget", "block_reps", "block_scores", "topk_select", "select_decode", "sparse_prefill",
           "sparse_prefill_backward", "sparse_decode", "num_qblocks", "required_kcap", "SasError", "load", "sel_code"]


def _torch():
    import torch
    return torch


@dataclass
class Budget:
    """k = ceil(sqrt_num * sqrt(c + count_current) / sqrt_den) when sqrt_den > 0, else k_fixed, or
    ceil(frac_num * (c + count_current) / frac_den) when frac_den > 0; with coverage > 0, the smallest
    k whose top candidates hold that share of the softmax mass (capped by the rule when one is set)."""
    k_fixed: int = 0
    frac_num: int = 0
    frac_den: int = 0
    count_current: int = 0
    sink: bool = False
    gate: bool = False
    coverage: float = 0.0
    shared: bool = False
    sqrt_num: int = 0
    sqrt_den: int = 0

    def c_struct(self) -> _lib.Budget:
        return _lib.Budget(self.k_fixed, self.frac_num, self.frac_den, self.count_current,
                           int(bool(self.sink)), int(bool(self.gate)), float(self.coverage), int(bool(self.shared)),
                           int(self.sqrt_num), int(self.sqrt_den))


def sel_code(sel_mode) -> int:
    if sel_mode in (SAS_SEL_GROUP, "group"):
        return SAS_SEL_GROUP
    if sel_mode in (SAS_SEL_HEAD, "head"):
        return SAS_SEL_HEAD
    raise ValueError(f"sel_mode {sel_mode!r}")


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return SAS_BF16
    if t.dtype == torch.float32:
        return SAS_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


class _Prob:
    """sas_problem plus the host arrays it points to (kept alive for the call).  seq_lens: a sequence of
    ints (host lengths), or an int32 tensor on the GPU (lengths the kernels read from device memory)."""

    def __init__(self, batch, hq, hkv, d, block, dtype, max_len, seq_lens):
        if _is_device_lens(seq_lens):
            self.lens = seq_lens
            self.s = _lib.Problem(batch, hq, hkv, d, block, dtype, max_len,
                                  C.cast(C.c_void_p(seq_lens.data_ptr()), C.POINTER(C.c_int32)), 1)
        else:
            self.lens = i32x(seq_lens)
            self.s = _lib.Problem(batch, hq, hkv, d, block, dtype, max_len,
                                  C.cast(self.lens, C.POINTER(C.c_int32)), 0)

    @property
    def ref(self):
        return C.byref(self.s)


def _is_device_lens(seq_lens) -> bool:
    if hasattr(seq_lens, "is_cuda") and seq_lens.is_cuda:
        torch = _torch()
        if seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous():
            raise ValueError("device seq_lens must be a contiguous int32 tensor")
        return True
    return False


def _max_blocks(seq_lens, block, max_len) -> int:
    """Blocks of the longest sequence (device lengths: of the capacity max_len)."""
    if _is_device_lens(seq_lens):
        return -(-int(max_len) // block)
    return max(-(-int(L) // block) for L in seq_lens)


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else None


def _strides(t, n):
    return i64x(t.stride()[:n])


def _qstart(q_start):
    if q_start is None:
        return None
    return i32x(q_start)


def num_qblocks(tq: int, block: int) -> int:
    return int(load().sas_num_qblocks(tq, block))


def required_kcap(batch, hq, hkv, d, block, dtype, max_len, seq_lens, tq, q_start, budget: Budget) -> int:
    p = _Prob(batch, hq, hkv, d, block, dtype, max_len, seq_lens)
    qs = _qstart(q_start)
    bs = budget.c_struct()
    r = load().sas_required_kcap(p.ref, tq, qs, C.byref(bs))
    if r < 0:
        check(r, "sas_required_kcap")
    return int(r)


def block_reps(K, seq_lens: Sequence[int], block: int, hq: Optional[int] = None, reps=None, stream=None,
               first_block: Optional[Sequence[int]] = None, current_block: bool = False):
    """A1: fp32 mean of every block's keys; K [B, Hkv, Lmax, d] -> reps [B, Hkv, NBmax, d].

    first_block (one int per sequence): recompute only blocks first_block[b] .. NB_b - 1 of an
    existing ``reps`` (sas_block_reps_update), e.g. floor(L_old / block) after appending tokens.
    current_block (seq_lens a device tensor): recompute only the block holding each sequence's last
    position, found on the device (sas_block_reps_update with first_block NULL).
    """
    torch = _torch()
    B, hkv, lmax, d = K.shape
    nb = _max_blocks(seq_lens, block, lmax)
    if reps is None:
        if first_block is not None or current_block:
            raise ValueError("an incremental update needs the existing reps")
        reps = torch.empty((B, hkv, nb, d), dtype=torch.float32, device=K.device)
    p = _Prob(B, hq or hkv, hkv, d, block, _dtype_code(K), lmax, seq_lens)
    lib = load()
    if current_block:
        check(lib.sas_block_reps_update(p.ref, _ptr(K), _strides(K, 3), _ptr(reps), _strides(reps, 3), None,
                                        _stream(stream)), "sas_block_reps_update")
    elif first_block is None:
        check(lib.sas_block_reps(p.ref, _ptr(K), _strides(K, 3), _ptr(reps), _strides(reps, 3), _stream(stream)),
              "sas_block_reps")
    else:
        fb = i32x(first_block)
        check(lib.sas_block_reps_update(p.ref, _ptr(K), _strides(K, 3), _ptr(reps), _strides(reps, 3), fb,
                                        _stream(stream)), "sas_block_reps_update")
    return reps


def block_scores(Q, reps, seq_lens, block, hkv, max_len, q_start=None, sel_mode="group", gist=False,
                 scale=0.0, scores=None, workspace=None, stream=None):
    """A2: scores [B*S*QB, NBmax] fp32 (entries j <= c of each unit row are written).

    Q: [B, Hq, T, d] (prefill, q_start given) or [B, Hq, d] (decode).
    reps: fp32 pooled reps, or gist keys (gist=True) of Q's dtype.
    """
    torch = _torch()
    decode = q_start is None
    if decode:
        B, hq, d = Q.shape
        tq = 1
        qs = i64x([Q.stride(0), Q.stride(1), 0])
    else:
        B, hq, tq, d = Q.shape
        qs = _strides(Q, 3)
    sm = sel_code(sel_mode)
    S = hq if sm == SAS_SEL_HEAD else hkv
    nb = max(-(-int(L) // block) for L in seq_lens)
    QB = 1 if decode else num_qblocks(tq, block)
    if scores is None:
        scores = torch.full((B * S * QB, nb), float("-inf"), dtype=torch.float32, device=Q.device)
    p = _Prob(B, hq, hkv, d, block, _dtype_code(Q), max_len, seq_lens)
    lib = load()
    need = lib.sas_block_scores_workspace(p.ref, tq, sm) if not decode else 0
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=Q.device)
    check(lib.sas_block_scores(p.ref, _ptr(Q), qs, tq, _qstart(q_start), _ptr(reps),
                               SAS_REPS_GIST if gist else SAS_REPS_POOLED, _strides(reps, 3), sm, float(scale),
                               _ptr(scores), scores.stride(0), _ptr(workspace),
                               workspace.numel() if workspace is not None else 0, _stream(stream)),
          "sas_block_scores")
    return scores


def topk_select(scores, seq_lens, block, hq, hkv, d, dtype, max_len, budget: Budget, tq=1, q_start=None,
                sel_mode="group", kcap=None, idx=None, nsel=None, gate=None, stream=None):
    """A3: (idx [U, kcap] int32 ascending, -1 padded; nsel [U] int32; gate [U, kcap] fp32 or None)."""
    torch = _torch()
    sm = sel_code(sel_mode)
    B = len(seq_lens)
    p = _Prob(B, hq, hkv, d, block, dtype, max_len, seq_lens)
    bs = budget.c_struct()
    lib = load()
    if kcap is None:
        kcap = lib.sas_required_kcap(p.ref, tq, _qstart(q_start), C.byref(bs))
        if kcap < 0:
            check(kcap, "sas_required_kcap")
    U = scores.shape[0]
    if idx is None:
        idx = torch.empty((U, kcap), dtype=torch.int32, device=scores.device)
    if nsel is None:
        nsel = torch.empty((U,), dtype=torch.int32, device=scores.device)
    if budget.gate and gate is None:
        gate = torch.empty((U, kcap), dtype=torch.float32, device=scores.device)
    check(lib.sas_topk_select(p.ref, _ptr(scores), scores.stride(0), tq, _qstart(q_start), sm, C.byref(bs),
                              kcap, _ptr(idx), _ptr(nsel), _ptr(gate) if budget.gate else None, _stream(stream)),
          "sas_topk_select")
    return idx, nsel, (gate if budget.gate else None)


def select_decode(Q, reps, seq_lens, block, hkv, max_len, budget: Budget, sel_mode="group", gist=False,
                  scale=0.0, kcap=None, scores=None, idx=None, nsel=None, gate=None, workspace=None,
                  stream=None):
    """A2 + A3 fused for decode (one launch): (scores, idx, nsel, gate) as block_scores + topk_select.

    workspace: arrival counters, zero before first use (allocated zeroed when not given) and left
    zero by every call.
    """
    torch = _torch()
    B, hq, d = Q.shape
    sm = sel_code(sel_mode)
    S = hq if sm == SAS_SEL_HEAD else hkv
    nb = _max_blocks(seq_lens, block, max_len)
    p = _Prob(B, hq, hkv, d, block, _dtype_code(Q), max_len, seq_lens)
    bs = budget.c_struct()
    lib = load()
    if kcap is None:
        # device lengths: the capacity's kcap (a host problem at max_len)
        hp = _Prob(B, hq, hkv, d, block, _dtype_code(Q), max_len, [max_len] * B) if _is_device_lens(seq_lens) else p
        kcap = lib.sas_required_kcap(hp.ref, 1, None, C.byref(bs))
        if kcap < 0:
            check(kcap, "sas_required_kcap")
    if scores is None:
        scores = torch.full((B * S, nb), float("-inf"), dtype=torch.float32, device=Q.device)
    if idx is None:
        idx = torch.empty((B * S, kcap), dtype=torch.int32, device=Q.device)
    if nsel is None:
        nsel = torch.empty((B * S,), dtype=torch.int32, device=Q.device)
    if budget.gate and gate is None:
        gate = torch.empty((B * S, kcap), dtype=torch.float32, device=Q.device)
    if workspace is None:
        workspace = torch.zeros(lib.sas_select_decode_workspace(p.ref), dtype=torch.uint8, device=Q.device)
    check(lib.sas_select_decode(p.ref, _ptr(Q), _strides(Q, 2), _ptr(reps),
                                SAS_REPS_GIST if gist else SAS_REPS_POOLED, _strides(reps, 3), sm, float(scale),
                                C.byref(bs), kcap, _ptr(scores), scores.stride(0), _ptr(idx), _ptr(nsel),
                                _ptr(gate) if budget.gate else None, _ptr(workspace), workspace.numel(),
                                _stream(stream)),
          "sas_select_decode")
    return scores, idx, nsel, (gate if budget.gate else None)


def select_decode_workspace_bytes(B, hq, hkv, d, block, dtype, max_len, seq_lens) -> int:
    p = _Prob(B, hq, hkv, d, block, dtype, max_len, seq_lens)
    return int(load().sas_select_decode_workspace(p.ref))


def sparse_prefill(Q, K, V, seq_lens, block, q_start, idx, nsel, gate=None, sel_mode="group", scale=0.0,
                   O=None, stream=None, lse=None):
    """A4: O [B, Hq, T, d] = attention of each row over its unit's selected blocks (causal).
    lse: optional fp32 [B, Hq, T] tensor that receives each row's log-sum-exp (for the backward)."""
    torch = _torch()
    B, hq, tq, d = Q.shape
    _, hkv, lmax, _ = K.shape
    if K.stride() != V.stride():
        raise ValueError("K and V must share strides")
    if O is None:
        O = torch.empty_like(Q)
    if lse is not None and (not lse.is_contiguous() or tuple(lse.shape) != (B, hq, tq)):
        raise ValueError("lse must be a contiguous [B, Hq, T] tensor")
    p = _Prob(B, hq, hkv, d, block, _dtype_code(Q), lmax, seq_lens)
    check(load().sas_sparse_prefill_lse(p.ref, _ptr(Q), _strides(Q, 3), _ptr(K), _ptr(V), _strides(K, 3), tq,
                                        _qstart(q_start), sel_code(sel_mode), _ptr(idx), _ptr(nsel), _ptr(gate),
                                        idx.shape[1], float(scale), _ptr(O), _strides(O, 3), _ptr(lse),
                                        _stream(stream)),
          "sas_sparse_prefill")
    return O


def prefill_backward_workspace_bytes(B, hq, hkv, d, block, max_len, seq_lens, tq, sel_mode, kcap, gate) -> int:
    p = _Prob(B, hq, hkv, d, block, SAS_BF16, max_len, seq_lens)
    return int(load().sas_sparse_prefill_backward_workspace(p.ref, tq, sel_code(sel_mode), kcap, int(bool(gate))))


def sparse_prefill_backward(Q, K, V, O, dO, seq_lens, block, q_start, idx, nsel, gate=None, sel_mode="group",
                            scale=0.0, workspace=None, grads=None, stream=None, lse=None, reps=None):
    """Gradients of sparse_prefill for the loss sum(O * dO): (dQ, dK, dV, dgate, dscore), fp32
    (dgate and dscore are None without a gate).  grads: optional preallocated (dQ, dK, dV, dgate,
    dscore); dK/dV rows past a sequence's length are left as given (zeros when allocated here).
    lse: the forward's row log-sum-exp (sparse_prefill(..., lse=)), or None to recompute it.
    reps: the block representatives the selection scored (with a gate): the gradient then continues
    through the selector scores into dQ and dK."""
    torch = _torch()
    B, hq, tq, d = Q.shape
    _, hkv, lmax, _ = K.shape
    if K.stride() != V.stride() or O.stride() != dO.stride():
        raise ValueError("K and V (O and dO) must share strides")
    kcap = idx.shape[1]
    p = _Prob(B, hq, hkv, d, block, _dtype_code(Q), lmax, seq_lens)
    lib = load()
    if grads is None:
        f32 = dict(dtype=torch.float32, device=Q.device)
        dQ = torch.empty(B, hq, tq, d, **f32)
        dK = torch.zeros(B, hkv, lmax, d, **f32)
        dV = torch.zeros(B, hkv, lmax, d, **f32)
        dgate = torch.empty(idx.shape, **f32) if gate is not None else None
        dscore = torch.empty(idx.shape, **f32) if gate is not None else None
    else:
        dQ, dK, dV, dgate, dscore = grads
    if dK.stride() != dV.stride():
        raise ValueError("dK and dV must share strides")
    need = lib.sas_sparse_prefill_backward_workspace(p.ref, tq, sel_code(sel_mode), kcap, int(gate is not None))
    if workspace is None:
        workspace = torch.empty(max(1, need), dtype=torch.uint8, device=Q.device)
    check(lib.sas_sparse_prefill_backward(p.ref, _ptr(Q), _strides(Q, 3), _ptr(K), _ptr(V), _strides(K, 3), tq,
                                          _qstart(q_start), sel_code(sel_mode), _ptr(idx), _ptr(nsel), _ptr(gate),
                                          kcap, float(scale), _ptr(O), _ptr(dO), _strides(O, 3), _ptr(lse), _ptr(dQ),
                                          _strides(dQ, 3), _ptr(dK), _ptr(dV), _strides(dK, 3), _ptr(dgate),
                                          _ptr(dscore), _ptr(reps), _strides(reps, 3) if reps is not None else None,
                                          _ptr(workspace), workspace.numel(), _stream(stream)),
          "sas_sparse_prefill_backward")
    return dQ, dK, dV, dgate, dscore


def decode_workspace_bytes(B, hq, hkv, d, block, dtype, max_len, seq_lens, sel_mode, kcap, gist) -> int:
    p = _Prob(B, hq, hkv, d, block, dtype, max_len, seq_lens)
    return int(load().sas_sparse_decode_workspace(p.ref, sel_code(sel_mode), kcap, int(bool(gist))))


def sparse_decode(Q, K, V, seq_lens, block, idx, nsel, gate=None, sel_mode="group", scale=0.0, gist_k=None,
                  gist_v=None, O=None, workspace=None, stream=None):
    """A5/A6: O [B, Hq, d] for the row at position L_b - 1 (gist mode when gist_k/gist_v are given)."""
    torch = _torch()
    B, hq, d = Q.shape
    _, hkv, lmax, _ = K.shape
    if K.stride() != V.stride():
        raise ValueError("K and V must share strides")
    gist = gist_k is not None
    if gist and gist_k.stride() != gist_v.stride():
        raise ValueError("gist K and V must share strides")
    if O is None:
        O = torch.empty_like(Q)
    kcap = idx.shape[1]
    dt = _dtype_code(Q)
    p = _Prob(B, hq, hkv, d, block, dt, lmax, seq_lens)
    lib = load()
    need = lib.sas_sparse_decode_workspace(p.ref, sel_code(sel_mode), kcap, int(gist))
    if workspace is None and need:
        # arrival counters must start at zero (the library leaves them zero after each call)
        workspace = torch.zeros(need, dtype=torch.uint8, device=Q.device)
    check(lib.sas_sparse_decode(p.ref, _ptr(Q), _strides(Q, 2), _ptr(K), _ptr(V), _strides(K, 3),
                                _ptr(gist_k) if gist else None, _ptr(gist_v) if gist else None,
                                _strides(gist_k, 3) if gist else None, sel_code(sel_mode), _ptr(idx), _ptr(nsel),
                                _ptr(gate), kcap, float(scale), _ptr(O), _strides(O, 2), _ptr(workspace),
                                workspace.numel() if workspace is not None else 0, _stream(stream)),
          "sas_sparse_decode")
    return O


def sparse_decode_noalloc(Q, K, V, seq_lens, block, idx, nsel, gate=None, sel_mode="group", scale=0.0, gist_k=None,
                          gist_v=None, O=None, stream=None):
    """sparse_decode with the library's static scratch instead of a workspace
    (sas_sparse_decode_noalloc): the call allocates no device memory itself (O is allocated here
    when not given).  Calls that overlap in time on one GPU must not use it."""
    torch = _torch()
    B, hq, d = Q.shape
    _, hkv, lmax, _ = K.shape
    if K.stride() != V.stride():
        raise ValueError("K and V must share strides")
    gist = gist_k is not None
    if gist and gist_k.stride() != gist_v.stride():
        raise ValueError("gist K and V must share strides")
    if O is None:
        O = torch.empty_like(Q)
    p = _Prob(B, hq, hkv, d, block, _dtype_code(Q), lmax, seq_lens)
    check(load().sas_sparse_decode_noalloc(p.ref, _ptr(Q), _strides(Q, 2), _ptr(K), _ptr(V), _strides(K, 3),
                                           _ptr(gist_k) if gist else None, _ptr(gist_v) if gist else None,
                                           _strides(gist_k, 3) if gist else None, sel_code(sel_mode), _ptr(idx),
                                           _ptr(nsel), _ptr(gate), idx.shape[1], float(scale), _ptr(O), _strides(O, 2),
                                           _stream(stream)),
          "sas_sparse_decode_noalloc")
    return O


def hssa_select_decode(Q, gist_k, meta_k, seq_lens, block, hkv, max_len, group_chunks, k1, k2, sel_mode="group",
                       scale=0.0, kcap=None, gcap=None, idx=None, nsel=None, gidx=None, gsel=None, workspace=None,
                       stream=None):
    """Two-level gist selection for decode: (idx, nsel, gidx, gsel).

    idx [U, kcap]: expanded chunks ascending, then the current chunk; gidx [U, gcap]: opened groups
    ascending, then the trailing group (group_chunks chunks per group).
    """
    torch = _torch()
    B, hq, d = Q.shape
    sm = sel_code(sel_mode)
    S = hq if sm == SAS_SEL_HEAD else hkv
    nm_cap = ((int(max_len) - 1) // block) // group_chunks
    k1u = max(0, min(int(k1), nm_cap))
    if gcap is None:
        gcap = k1u + 1
    if kcap is None:
        kcap = min(int(k2), (k1u + 1) * group_chunks) + 1
    p = _Prob(B, hq, hkv, d, block, _dtype_code(Q), max_len, seq_lens)
    lib = load()
    dev = Q.device
    idx = idx if idx is not None else torch.empty((B * S, kcap), dtype=torch.int32, device=dev)
    nsel = nsel if nsel is not None else torch.empty((B * S,), dtype=torch.int32, device=dev)
    gidx = gidx if gidx is not None else torch.empty((B * S, gcap), dtype=torch.int32, device=dev)
    gsel = gsel if gsel is not None else torch.empty((B * S,), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(lib.sas_hssa_select_workspace(p.ref, sm, group_chunks, int(k1)), dtype=torch.uint8,
                                device=dev)
    check(lib.sas_hssa_select_decode(p.ref, _ptr(Q), _strides(Q, 2), _ptr(gist_k), _strides(gist_k, 3), _ptr(meta_k),
                                     _strides(meta_k, 3), group_chunks, sm, int(k1), int(k2), float(scale), kcap, gcap,
                                     _ptr(idx), _ptr(nsel), _ptr(gidx), _ptr(gsel), _ptr(workspace),
                                     workspace.numel(), _stream(stream)),
          "sas_hssa_select_decode")
    return idx, nsel, gidx, gsel


def hssa_decode(Q, K, V, seq_lens, block, gist_k, gist_v, meta_k, meta_v, group_chunks, idx, nsel, gidx,
                sel_mode="group", scale=0.0, O=None, workspace=None, stream=None):
    """Attention of the two-level gist selection: O [B, Hq, d] for the row at position L_b - 1."""
    torch = _torch()
    B, hq, d = Q.shape
    _, hkv, lmax, _ = K.shape
    for a, b_, what in ((K, V, "K and V"), (gist_k, gist_v, "gist K and V"), (meta_k, meta_v, "meta-gist K and V")):
        if a.stride() != b_.stride():
            raise ValueError(what + " must share strides")
    if O is None:
        O = torch.empty_like(Q)
    kcap, gcap = idx.shape[1], gidx.shape[1]
    p = _Prob(B, hq, hkv, d, block, _dtype_code(Q), lmax, seq_lens)
    lib = load()
    sm = sel_code(sel_mode)
    if workspace is None:
        # arrival counters must start at zero (the library leaves them zero after each call)
        workspace = torch.zeros(lib.sas_hssa_decode_workspace(p.ref, sm, kcap, gcap, group_chunks), dtype=torch.uint8,
                                device=Q.device)
    check(lib.sas_hssa_decode(p.ref, _ptr(Q), _strides(Q, 2), _ptr(K), _ptr(V), _strides(K, 3), _ptr(gist_k),
                              _ptr(gist_v), _strides(gist_k, 3), _ptr(meta_k), _ptr(meta_v), _strides(meta_k, 3),
                              group_chunks, sm, _ptr(idx), _ptr(nsel), kcap, _ptr(gidx), gcap, float(scale), _ptr(O),
                              _strides(O, 2), _ptr(workspace), workspace.numel(), _stream(stream)),
          "sas_hssa_decode")
    return O


def hssa_select_workspace_bytes(B, hq, hkv, d, block, max_len, seq_lens, sel_mode, group_chunks, k1) -> int:
    p = _Prob(B, hq, hkv, d, block, SAS_BF16, max_len, seq_lens)
    return int(load().sas_hssa_select_workspace(p.ref, sel_code(sel_mode), group_chunks, int(k1)))


def hssa_decode_workspace_bytes(B, hq, hkv, d, block, max_len, seq_lens, sel_mode, kcap, gcap, group_chunks) -> int:
    p = _Prob(B, hq, hkv, d, block, SAS_BF16, max_len, seq_lens)
    return int(load().sas_hssa_decode_workspace(p.ref, sel_code(sel_mode), kcap, gcap, group_chunks))


def block_reps_paged(K_pages, block_table, seq_lens, block: int, hkv: int, max_len: int, reps,
                     first_block: Optional[Sequence[int]] = None, hq: Optional[int] = None, stream=None):
    """A1 over a paged K: K_pages [num_pages, Hkv, block, d], block_table [B, ld] int32 (page of each
    block); reps [B, Hkv, NB, d] fp32 by logical block (first_block: only blocks from it on)."""
    B = block_table.shape[0]
    d = K_pages.shape[-1]
    p = _Prob(B, hq or hkv, hkv, d, block, _dtype_code(K_pages), max_len, seq_lens)
    fb = i32x(first_block) if first_block is not None else None
    check(load().sas_block_reps_paged(p.ref, _ptr(K_pages), _strides(K_pages, 3), _ptr(block_table),
                                      block_table.stride(0), _ptr(reps), _strides(reps, 3), fb, _stream(stream)),
          "sas_block_reps_paged")
    return reps


def sparse_decode_paged(Q, K_pages, V_pages, block_table, seq_lens, block, max_len, idx, nsel, gate=None,
                        sel_mode="group", scale=0.0, O=None, workspace=None, stream=None):
    """A5 over paged K/V (see block_reps_paged): O [B, Hq, d] for the row at position L_b - 1."""
    torch = _torch()
    B, hq, d = Q.shape
    hkv = K_pages.shape[1]
    if K_pages.stride() != V_pages.stride():
        raise ValueError("K and V pages must share strides")
    if O is None:
        O = torch.empty_like(Q)
    kcap = idx.shape[1]
    p = _Prob(B, hq, hkv, d, block, _dtype_code(Q), max_len, seq_lens)
    lib = load()
    if workspace is None:
        need = lib.sas_sparse_decode_workspace(p.ref, sel_code(sel_mode), kcap, 0)
        workspace = torch.zeros(max(need, 16), dtype=torch.uint8, device=Q.device)
    check(lib.sas_sparse_decode_paged(p.ref, _ptr(Q), _strides(Q, 2), _ptr(K_pages), _ptr(V_pages),
                                      _strides(K_pages, 3), _ptr(block_table), block_table.stride(0),
                                      sel_code(sel_mode), _ptr(idx), _ptr(nsel), _ptr(gate), kcap, float(scale),
                                      _ptr(O), _strides(O, 2), _ptr(workspace), workspace.numel(), _stream(stream)),
          "sas_sparse_decode_paged")
    return O


def sparse_prefill_paged(Q, K_pages, V_pages, block_table, seq_lens, block, max_len, q_start, idx, nsel, gate=None,
                         sel_mode="group", scale=0.0, O=None, stream=None):
    """A4 over paged K/V (see block_reps_paged): O like Q [B, Hq, tq, d]."""
    torch = _torch()
    B, hq, tq, d = Q.shape
    hkv = K_pages.shape[1]
    if K_pages.stride() != V_pages.stride():
        raise ValueError("K and V pages must share strides")
    if O is None:
        O = torch.empty_like(Q)
    p = _Prob(B, hq, hkv, d, block, _dtype_code(Q), max_len, seq_lens)
    check(load().sas_sparse_prefill_paged(p.ref, _ptr(Q), _strides(Q, 3), _ptr(K_pages), _ptr(V_pages),
                                          _strides(K_pages, 3), _ptr(block_table), block_table.stride(0), tq,
                                          _qstart(q_start), sel_code(sel_mode), _ptr(idx), _ptr(nsel), _ptr(gate),
                                          idx.shape[1], float(scale), _ptr(O), _strides(O, 3), _stream(stream)),
          "sas_sparse_prefill_paged")
    return O
