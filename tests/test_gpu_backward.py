"""GPU parity of the sparse-prefill backward against the float64 autograd oracle.

Both sides take the same inputs: the seeded Q/K/V/dO, the oracle's own block lists and gate values
(uploaded to the GPU as int32 / fp32) and the oracle's forward output O rounded to bf16.

Bar, per gradient tensor X (dQ, dK, dV, dgate, dscore):
  max |X_gpu - X_ref| <= 2e-2 * max |X_ref|   and   mean |X_gpu - X_ref| <= 2e-3 * max |X_ref|.
The GPU rounds P and dS to bf16 as matrix operands (relative error <= 2^-9 each, random in sign)
and D_row uses O in bf16; all sums are fp32.  A sum of n such terms is off by about 2^-9 times
the root-sum-square of its terms, a small fraction of max |X| for these inputs.
"""
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from workloads import Workload  # noqa: E402
from workloads.device import upload  # noqa: E402

from gpu_harness import say  # noqa: E402
import top_block_sparse_gist_amd as sas  # noqa: E402
from oracle import sas_oracle as orc  # noqa: E402
from oracle import sas_backward as orcb  # noqa: E402

MAX_REL = 2e-2
MEAN_REL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sas.load()
    yield


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def _check(name, got, ref, stats):
    err = np.abs(got - ref)
    top = float(np.abs(ref).max()) if ref.size else 0.0
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    stats[name] = (mx / max(top, 1e-30), mean / max(top, 1e-30), top)
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    assert mx <= MAX_REL * top + 1e-6, f"{name}: max-abs {mx:.3e} vs max|ref| {top:.3e}"
    assert mean <= MEAN_REL * top + 1e-7, f"{name}: mean-abs {mean:.3e} vs max|ref| {top:.3e}"


def run_backward_case(w: Workload, seqs=(0,), use_lse=False, through_scores=False):
    """use_lse: the GPU forward writes each row's log-sum-exp (checked against the oracle's to 1e-3
    absolute: fp32 sums of exact bf16 products) and the backward takes it instead of recomputing it."""
    seqs = list(seqs)
    say(f"[bwd] {w.name} seqs={seqs} sel={w.sel} d={w.d} blk={w.block} gate={w.gate} lse={use_lse}")
    inp = upload(w, seqs, keep_host=set(seqs))
    lens = inp.seq_lens
    B, blk, tq = len(seqs), w.block, w.tq
    S = w.hkv if w.sel == "group" else w.hq
    QB = sas.num_qblocks(tq, blk)
    scale = 1.0 / math.sqrt(w.d)
    # oracle forward: lists, gate values, O
    res = {}
    for b in seqs:
        h = inp.host[b]
        res[b] = orc.run_sequence(h["q"], h["k"], h["v"], w.seq_lens[b], w.q_start[b], blk, w.sel,
                                  k_fixed=w.k_fixed, frac_num=w.frac_num, frac_den=w.frac_den,
                                  count_current=w.count_current, sink=w.sink, gate=w.gate, scale=scale,
                                  coverage=w.spec.get("coverage", 0.0), shared=w.spec.get("shared", False))
    kcap = max(len(u.sel) for r in res.values() for u in r.units if u.sel is not None)
    units = B * S * QB
    idx = np.full((units, kcap), -1, np.int32)
    nsel = np.zeros(units, np.int32)
    gate = np.zeros((units, kcap), np.float32)
    O = torch.zeros_like(inp.Q)
    dO = torch.zeros_like(inp.Q)
    for bi, b in enumerate(seqs):
        r = res[b]
        q0 = w.q_start[b]
        for u in r.units:
            x = (bi * S + u.sel_head) * QB + (u.c - q0 // blk)
            nsel[x] = len(u.sel)
            idx[x, :len(u.sel)] = u.sel
            if w.gate:
                gate[x, :len(u.sel)] = [u.gate[j] for j in u.sel]
        O[bi, :, :w.rows[b]] = _bf16(r.O).to(O.device)
        dO[bi, :, :w.rows[b]] = _bf16(w.grad_out(b)).to(O.device)
    dev = inp.Q.device
    t_idx = torch.from_numpy(idx).to(dev)
    t_nsel = torch.from_numpy(nsel).to(dev)
    t_gate = torch.from_numpy(gate).to(dev) if w.gate else None
    lse = None
    if use_lse:
        lse = torch.full(inp.Q.shape[:3], float("nan"), dtype=torch.float32, device=dev)
        sas.sparse_prefill(inp.Q, inp.K, inp.V, lens, blk, inp.q_start, t_idx, t_nsel, t_gate, sel_mode=w.sel,
                           lse=lse)
        torch.cuda.synchronize()
        lse_h = lse.cpu().numpy()
        for bi, b in enumerate(seqs):
            h = inp.host[b]
            ref = orcb.row_logsumexp(h["q"], h["k"], w.seq_lens[b], w.q_start[b], blk, res[b].units, w.gate, scale)
            err = float(np.abs(lse_h[bi, :, :w.rows[b]] - ref).max())
            say(f"[bwd] lse[{b}] max-abs {err:.2e}")
            assert err <= 1e-3, f"row log-sum-exp differs by {err:.3e}"
    reps = sas.block_reps(inp.K, lens, blk) if through_scores else None
    dQ, dK, dV, dgate, dscore = sas.sparse_prefill_backward(inp.Q, inp.K, inp.V, O, dO, lens, blk, inp.q_start,
                                                            t_idx, t_nsel, t_gate, sel_mode=w.sel, lse=lse, reps=reps)
    plain = None
    if through_scores:
        # the same call without the representatives isolates the selector path's contribution
        plain = sas.sparse_prefill_backward(inp.Q, inp.K, inp.V, O, dO, lens, blk, inp.q_start, t_idx, t_nsel,
                                            t_gate, sel_mode=w.sel, lse=lse)
        plain = (plain[0].cpu().numpy(), plain[1].cpu().numpy())
    torch.cuda.synchronize()
    say("[bwd] gpu done")
    dQ, dK, dV = dQ.cpu().numpy(), dK.cpu().numpy(), dV.cpu().numpy()
    if w.gate:
        dgate, dscore = dgate.cpu().numpy(), dscore.cpu().numpy()
    stats = {}
    for bi, b in enumerate(seqs):
        h = inp.host[b]
        L, q0, rows = w.seq_lens[b], w.q_start[b], w.rows[b]
        ref = orcb.backward_sequence(h["q"], h["k"], h["v"], w.grad_out(b), L, q0, blk, res[b].units, w.gate,
                                     scale, through_scores=through_scores)
        _check(f"dQ[{b}]", dQ[bi, :, :rows], ref["dQ"], stats)
        _check(f"dK[{b}]", dK[bi, :, :L], ref["dK"], stats)
        if through_scores:
            refp = orcb.backward_sequence(h["q"], h["k"], h["v"], w.grad_out(b), L, q0, blk, res[b].units, w.gate,
                                          scale)
            _check(f"selector path dQ[{b}]", dQ[bi, :, :rows] - plain[0][bi, :, :rows], ref["dQ"] - refp["dQ"], stats)
            _check(f"selector path dK[{b}]", dK[bi, :, :L] - plain[1][bi, :, :L], ref["dK"] - refp["dK"], stats)
        _check(f"dV[{b}]", dV[bi, :, :L], ref["dV"], stats)
        if w.gate:
            g_got, g_ref, s_got, s_ref = [], [], [], []
            for u in res[b].units:
                x = (bi * S + u.sel_head) * QB + (u.c - q0 // blk)
                n = len(u.sel)
                g_got.append(dgate[x, :n]); g_ref.append(ref["dgate"][(u.sel_head, u.c)])
                s_got.append(dscore[x, :n]); s_ref.append(ref["dscore"][(u.sel_head, u.c)])
                assert not dgate[x, n:].any() and not dscore[x, n:].any(), "padding entries must be 0"
            _check(f"dgate[{b}]", np.concatenate(g_got), np.concatenate(g_ref), stats)
            _check(f"dscore[{b}]", np.concatenate(s_got), np.concatenate(s_ref), stats)
    for k, (a, m, top) in stats.items():
        say(f"[bwd] {k}: max-abs/max|ref| {a:.2e}  mean-abs/max|ref| {m:.2e}  (max|ref| {top:.3g})")
    return stats


def test_backward_group_unaligned_sink_gate():
    """Per-group units (G = 2), q_start off a block boundary, a partial last block, d = 128."""
    w = Workload(3, overrides=dict(tag="bwd_unaligned", seq_len=1000, tq=300, block=64, hq=4, hkv=2,
                                   frac_num=1, frac_den=4, sink=True, gate=True))
    run_backward_case(w)
    run_backward_case(w, use_lse=True)


def test_backward_per_head_d64_block128():
    """Per-head units (64-row and partial), d = 64, 128-key blocks (two tiles per block)."""
    w = Workload(3, overrides=dict(tag="bwd_head64", seq_len=1500, tq=600, block=128, d=64, hq=8, hkv=2,
                                   sel="head", frac_num=1, frac_den=4, sink=True, gate=True))
    run_backward_case(w)


def test_backward_per_head_sink_forward_lse():
    """Per-head units with a sink (block 0 kept by all 64 units of the KV head), the forward's row
    log-sum-exp handed to the backward."""
    w = Workload(3, overrides=dict(tag="bwd_headsink", seq_len=1024, tq=1024, block=64, hq=4, hkv=1, sel="head",
                                   frac_num=0, frac_den=0, k_fixed=2, sink=True, gate=True))
    run_backward_case(w, use_lse=True)


def test_backward_block_list_split_into_segments():
    """16 heads per KV head share each unit (2048 flattened rows), so a work item holds 16 units; the
    sink block is kept by all 18 units and its list is cut into two items whose dK/dV partial sums
    meet in atomic adds."""
    w = Workload(3, overrides=dict(tag="bwd_split", seq_len=2304, tq=2304, block=128, hq=16, hkv=1,
                                   frac_num=0, frac_den=0, k_fixed=2, sink=True, gate=True))
    run_backward_case(w)


@pytest.mark.parametrize("sel", ["group", "head"])
def test_backward_through_the_selector_scores(sel):
    """The gradient carried on from dscore through the pooled query and the block means into dQ and
    dK (the block representatives passed to the backward), against the oracle's through-scores mode."""
    w = Workload(3, overrides=dict(tag="bwd_chain" + sel, seq_len=1000, tq=300, block=64 if sel == "group" else 128,
                                   d=128 if sel == "group" else 64, hq=4, hkv=2, sel=sel, frac_num=1, frac_den=4,
                                   sink=True, gate=True))
    run_backward_case(w, through_scores=True)


def test_backward_shared_budget_lists_of_varying_length():
    """Per-head lists under a budget shared by the 4 heads of a KV group (lengths differ per head)."""
    w = Workload(3, overrides=dict(tag="bwd_shared", seq_len=1200, tq=700, block=64, hq=8, hkv=2, sel="head",
                                   frac_num=0, frac_den=0, k_fixed=3, sink=True, gate=True, shared=True))
    run_backward_case(w)


def test_backward_coverage_budget_d64():
    """Per-group lists from a coverage budget (the smallest top set holding 80 % of the selector's
    softmax mass), d = 64."""
    w = Workload(3, overrides=dict(tag="bwd_cov", seq_len=1100, tq=500, block=64, d=64, hq=4, hkv=1,
                                   frac_num=0, frac_den=0, k_fixed=0, sink=False, gate=True, coverage=0.8))
    run_backward_case(w)


def test_backward_group_no_gate_block128_seven_heads():
    """No gate (dgate/dscore not written), G = 7 (896 rows per unit: 7 row tiles), 128-key blocks."""
    w = Workload(3, overrides=dict(tag="bwd_nogate", seq_len=1536, tq=1536, block=128, hq=14, hkv=2,
                                   frac_num=1, frac_den=8, sink=True, gate=False))
    run_backward_case(w)


def test_backward_two_sequences_ragged():
    """Two sequences of different lengths in one call (the shorter one's rows past its length unused)."""
    w = Workload(3, overrides=dict(tag="bwd_two", seq_lens=[1300, 700], batch=2, tq=256, block=64, hq=4, hkv=2,
                                   frac_num=1, frac_den=4, sink=False, gate=True))
    run_backward_case(w, seqs=[0, 1], use_lse=True)


def test_backward_full_32k_prefill_properties():
    """The 32K prefill at full size, in the launch configuration bench.py times (its own lists, the
    forward's log-sum-exp).  Identities that hold at any size, since each row's P sums to 1 over its
    keys and so its dS sums to 0:
      sum over keys of dV[b, g] = sum of dO over the rows of the heads of group g;
      sum over keys of dK[b, g] = 0;  sum over a unit's list of dgate = 0 up to the bf16 rounding of O
      (and dscore = dgate then);
    and a second call gives the same bits for dQ, dgate and dscore, and for dK/dV outside the blocks
    whose unit lists were cut into several work items."""
    w = Workload(3)
    say(f"[bwd-full] {w.name}")
    inp = upload(w, [0])
    lens, blk, tq = inp.seq_lens, w.block, w.tq
    Lmax = inp.K.shape[2]
    budget = sas.Budget(k_fixed=w.k_fixed, frac_num=w.frac_num, frac_den=w.frac_den,
                        count_current=w.count_current, sink=w.sink, gate=w.gate)
    reps = sas.block_reps(inp.K, lens, blk)
    scores = sas.block_scores(inp.Q, reps, lens, blk, w.hkv, Lmax, q_start=inp.q_start, sel_mode=w.sel)
    idx, nsel, gate = sas.topk_select(scores, lens, blk, w.hq, w.hkv, w.d, sas.SAS_BF16, Lmax, budget, tq=tq,
                                      q_start=inp.q_start, sel_mode=w.sel)
    lse = torch.empty(inp.Q.shape[:3], dtype=torch.float32, device=inp.Q.device)
    O = sas.sparse_prefill(inp.Q, inp.K, inp.V, lens, blk, inp.q_start, idx, nsel, gate, sel_mode=w.sel, lse=lse)
    g = torch.Generator(device="cpu").manual_seed(w.seed)
    dO = torch.randn(inp.Q.shape, generator=g, dtype=torch.float32).to(torch.bfloat16).to(inp.Q.device)
    r1 = sas.sparse_prefill_backward(inp.Q, inp.K, inp.V, O, dO, lens, blk, inp.q_start, idx, nsel, gate,
                                     sel_mode=w.sel, lse=lse)
    r2 = sas.sparse_prefill_backward(inp.Q, inp.K, inp.V, O, dO, lens, blk, inp.q_start, idx, nsel, gate,
                                     sel_mode=w.sel, lse=lse)
    torch.cuda.synchronize()
    say("[bwd-full] gpu done")
    dQ, dK, dV, dgate, dscore = r1
    for x in (dQ, dK, dV, dgate, dscore):
        assert torch.isfinite(x).all()
    G = w.hq // w.hkv
    L = lens[0]
    dOf = dO.float()[0]
    for gi in range(w.hkv):
        want = dOf[gi * G:(gi + 1) * G].sum(dim=(0, 1))
        got = dV[0, gi, :L].sum(dim=0)
        err = float((got - want).abs().max())
        scale_v = float(dV[0, gi, :L].abs().sum(dim=0).max())
        say(f"[bwd-full] group {gi}: |sum dV - sum dO| {err:.3e} (sum |dV| {scale_v:.3e})")
        assert err <= 1e-3 * scale_v
        ksum = float(dK[0, gi, :L].sum(dim=0).abs().max())
        scale_k = float(dK[0, gi, :L].abs().sum(dim=0).max())
        say(f"[bwd-full] group {gi}: |sum dK| {ksum:.3e} (sum |dK| {scale_k:.3e})")
        assert ksum <= 1e-3 * scale_k
    # Each row's dS sums to dO . (O - O_bf16) rather than 0, since D_row takes the forward's bf16 O:
    # at most 2^-8 sum_d |dO_d O_d| per row (round-to-nearest: |O - O_bf16| <= 2^-9 |O|, doubled for
    # margin).  So |sum of a unit's dgate| <= the sum of that over the unit's rows and heads, plus fp32
    # noise.
    QB = sas.num_qblocks(tq, blk)
    e_row = (dO.float()[0].abs() * O.float()[0].abs()).sum(-1) * 2.0 ** -8          # [hq, tq]
    nb = tq // blk
    bound = e_row.view(w.hkv, G, nb, blk).sum(dim=(1, 3))                            # [hkv, nb]
    gs = dgate.sum(dim=1).abs().view(w.hkv, QB)[:, :nb]
    noise = 1e-4 * float(dgate.abs().sum(dim=1).max())
    excess = float((gs - bound - noise).max())
    say(f"[bwd-full] |sum dgate| per unit: max {float(gs.max()):.3e}, its rounding bound up to "
        f"{float(bound.max()):.3e}; worst excess {excess:.3e}")
    assert excess <= 0
    # dscore - dgate = -exp(g) sum(dgate) with exp(g) <= 1
    diff = (dscore - dgate).abs().max(dim=1).values
    assert bool((diff <= dgate.sum(dim=1).abs() * 1.0001 + 1e-5 * float(dgate.abs().max())).all())
    assert torch.equal(r2[0], dQ) and torch.equal(r2[3], dgate) and torch.equal(r2[4], dscore)
    # dK/dV: bitwise equal outside blocks kept by more units than one work item holds
    same = (r2[1][0] == dK[0]).all(dim=-1) & (r2[2][0] == dV[0]).all(dim=-1)   # [hkv, Lmax]
    frac = float(same[:, :L].float().mean())
    say(f"[bwd-full] dK/dV rows bitwise equal across two calls: {frac:.4f}")
    assert frac >= 0.9


def _unit_alone(h, dO_b, un, G, sel, blk, q0):
    """The unit's own slice of the inputs: its heads' query/dO rows and its KV head, re-indexed so
    that the oracle's backward builds a graph of this unit only (head 0.., KV head 0, rows 0..)."""
    g = un.heads[0] // G
    heads = list(un.heads)
    q = h["q"][heads, un.t_lo:un.t_hi]
    do = dO_b[heads, un.t_lo:un.t_hi]
    u2 = orc.Unit(sel_head=0, c=un.c, t_lo=0, t_hi=un.t_hi - un.t_lo, heads=tuple(range(len(heads))),
                  scores=un.scores, sel=un.sel, k=un.k, gate=un.gate)
    return q, h["k"][g:g + 1], h["v"][g:g + 1], do, q0 + un.t_lo, u2


def run_backward_full_sampled(w, seqs, keep, unit_sample, n_blocks, max_units_per_block, seed):
    """Full size, in the launch configuration bench.py times: the GPU's own lists, gates, O and
    log-sum-exp.  Each unit's dQ rows, dgate and dscore depend only on that unit, and each block's
    dK/dV rows only on the units that keep it, so sampled units and sampled blocks (with every unit
    keeping them) are compared with the float64 oracle, at the bars above."""
    say(f"[bwd-sampled] {w.name} seqs={seqs} keep={keep} units={unit_sample} blocks={n_blocks}")
    inp = upload(w, seqs, keep_host=set(keep))
    lens, blk, tq = inp.seq_lens, w.block, w.tq
    Lmax = inp.K.shape[2]
    S = w.hkv if w.sel == "group" else w.hq
    G = w.hq // w.hkv
    QB = sas.num_qblocks(tq, blk)
    scale = 1.0 / math.sqrt(w.d)
    budget = sas.Budget(k_fixed=w.k_fixed, frac_num=w.frac_num, frac_den=w.frac_den,
                        count_current=w.count_current, sink=w.sink, gate=w.gate)
    reps = sas.block_reps(inp.K, lens, blk)
    scores = sas.block_scores(inp.Q, reps, lens, blk, w.hkv, Lmax, q_start=inp.q_start, sel_mode=w.sel)
    idx, nsel, gate = sas.topk_select(scores, lens, blk, w.hq, w.hkv, w.d, sas.SAS_BF16, Lmax, budget, tq=tq,
                                      q_start=inp.q_start, sel_mode=w.sel)
    lse = torch.empty(inp.Q.shape[:3], dtype=torch.float32, device=inp.Q.device)
    O = sas.sparse_prefill(inp.Q, inp.K, inp.V, lens, blk, inp.q_start, idx, nsel, gate, sel_mode=w.sel, lse=lse)
    dO = torch.zeros_like(inp.Q)
    for bi, b in enumerate(seqs):
        dO[bi] = _bf16(w.grad_out(b)).to(dO.device)
    dQ, dK, dV, dgate, dscore = sas.sparse_prefill_backward(inp.Q, inp.K, inp.V, O, dO, lens, blk, inp.q_start, idx,
                                                            nsel, gate, sel_mode=w.sel, lse=lse)
    torch.cuda.synchronize()
    say("[bwd-sampled] gpu done")
    idx_h, nsel_h = idx.cpu().numpy(), nsel.cpu().numpy()
    dgate_h, dscore_h = dgate.cpu().numpy(), dscore.cpu().numpy()
    rng = np.random.default_rng(seed)
    acc = {k: ([], []) for k in ("dQ", "dgate", "dscore", "dK", "dV")}
    n_units = n_blk = 0
    for b in keep:
        bi = seqs.index(b)
        h = inp.host[b]
        L, q0 = w.seq_lens[b], w.q_start[b]
        dO_b = w.grad_out(b)
        reps_o = np.stack([orc.block_reps(h["k"][g], L, blk) for g in range(w.hkv)])
        units = orc.make_units(q0, w.rows[b], blk, w.hq, w.hkv, w.sel)
        slot = {}
        for un in units:
            x = (bi * S + un.sel_head) * QB + (un.c - q0 // blk)
            slot[(un.sel_head, un.c)] = x
            un.sel = [int(j) for j in idx_h[x, :nsel_h[x]]]
            g = orc.kv_head_of(un, G, w.sel)
            un.scores = orc.unit_scores(orc.unit_query_vectors(h["q"], un), reps_o[g], un.c + 1, scale)
        dQ_b = dQ[bi].cpu().numpy()
        for x in rng.choice(len(units), size=min(unit_sample, len(units)), replace=False):
            un = units[int(x)]
            q, k, v, do, qs, u2 = _unit_alone(h, dO_b, un, G, w.sel, blk, q0)
            ref = orcb.backward_sequence(q, k, v, do, L, qs, blk, [u2], w.gate, scale)
            acc["dQ"][0].append(dQ_b[list(un.heads), un.t_lo:un.t_hi].ravel())
            acc["dQ"][1].append(ref["dQ"].ravel())
            if w.gate:
                n = len(un.sel)
                xs = slot[(un.sel_head, un.c)]
                acc["dgate"][0].append(dgate_h[xs, :n]); acc["dgate"][1].append(ref["dgate"][(0, un.c)])
                acc["dscore"][0].append(dscore_h[xs, :n]); acc["dscore"][1].append(ref["dscore"][(0, un.c)])
            n_units += 1
        # blocks: every unit of the KV head that keeps the block contributes to its dK/dV rows
        keepers = {}
        for un in units:
            for j in un.sel:
                keepers.setdefault((orc.kv_head_of(un, G, w.sel), j), []).append(un)
        cands = [(g, j, us) for (g, j), us in sorted(keepers.items()) if len(us) <= max_units_per_block]
        for x in rng.choice(len(cands), size=min(n_blocks, len(cands)), replace=False):
            g, j, us = cands[int(x)]
            lo, hi = j * blk, min((j + 1) * blk, L)
            rk = np.zeros((hi - lo, w.d))
            rv = np.zeros((hi - lo, w.d))
            for un in us:
                q, k, v, do, qs, u2 = _unit_alone(h, dO_b, un, G, w.sel, blk, q0)
                ref = orcb.backward_sequence(q, k, v, do, L, qs, blk, [u2], w.gate, scale)
                rk += ref["dK"][0, lo:hi]
                rv += ref["dV"][0, lo:hi]
            acc["dK"][0].append(dK[bi, g, lo:hi].cpu().numpy().ravel()); acc["dK"][1].append(rk.ravel())
            acc["dV"][0].append(dV[bi, g, lo:hi].cpu().numpy().ravel()); acc["dV"][1].append(rv.ravel())
            n_blk += 1
            say(f"[bwd-sampled] sequence {b}, KV head {g}, block {j}: {len(us)} units")
    stats = {}
    for name, (got, ref) in acc.items():
        if got:
            _check(name, np.concatenate(got), np.concatenate(ref), stats)
    for k_, (a, m, top) in stats.items():
        say(f"[bwd-sampled] {k_}: max-abs/max|ref| {a:.2e}  mean-abs/max|ref| {m:.2e}  (max|ref| {top:.3g})")
    say(f"[bwd-sampled] {n_units} units, {n_blk} blocks checked")
    assert n_units >= unit_sample and n_blk >= 1
    return stats


@pytest.mark.timeout(900)
def test_backward_full_32k_sampled_against_the_oracle():
    """The 32K prefill (28/4 heads, 128-key blocks, top c/8 + sink + current, gate): 48 units (896
    query vectors each) and 4 blocks with all the units that keep them."""
    w = Workload(3)
    run_backward_full_sampled(w, [0], [0], unit_sample=48, n_blocks=4, max_units_per_block=24, seed=13)


@pytest.mark.timeout(900)
def test_backward_full_mixed_prefill_sampled_against_the_oracle():
    """The mixed batch's prefill half (8 sequences of 4096 rows, per-head lists at sparsity 0.95,
    gate), as bench.py times it: 64 units and 6 blocks in each of 2 sequences."""
    w = Workload(5)
    seqs = w.prefill_seqs()
    run_backward_full_sampled(w, seqs, [seqs[1], seqs[6]], unit_sample=64, n_blocks=6, max_units_per_block=40,
                              seed=17)


def test_backward_few_rows_per_unit():
    """tq = 5 rows across a block boundary, per-head units of 2-3 rows: every 32-row step is mostly
    padding (rows past the unit masked, staged rows clamped to the unit's last)."""
    w = Workload(3, overrides=dict(tag="bwd_few", seq_len=646, tq=5, block=64, hq=6, hkv=2, sel="head",
                                   frac_num=0, frac_den=0, k_fixed=3, sink=True, gate=True))
    run_backward_case(w, use_lse=True, through_scores=True)
