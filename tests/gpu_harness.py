"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI binding, run the
CPU oracle on the same seeded inputs, and compare them to the stated bars.

Bars:
  * block lists: bit-exact, except where the oracle's k-th and (k+1)-th candidate scores
    differ by less than 1e-5 relative; there the lists may differ only by blocks whose
    oracle scores lie within that band of the k-th score, and the attention output is then
    checked against the oracle run on the GPU's list;
  * outputs: fp32 max-abs <= 1e-4; bf16 max-abs <= 2e-2 and mean-abs <= 2e-3.
"""
from __future__ import annotations

import math
import sys
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

import top_block_sparse_gist_amd as sas
from oracle import sas_oracle as orc
from workloads import Workload
from workloads.device import upload

TIE_REL = 1e-5
F32_MAX_ABS = 1e-4
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


@dataclass
class Report:
    units: int = 0
    tie_band_units: int = 0
    max_abs: float = 0.0
    mean_abs_num: float = 0.0
    mean_abs_den: int = 0
    score_max_rel: float = 0.0
    gate_max_abs: float = 0.0
    reps_max_abs: float = 0.0

    @property
    def mean_abs(self):
        return self.mean_abs_num / max(1, self.mean_abs_den)


def list_matches(oracle_sel: List[int], gpu_sel: List[int], scores: np.ndarray, c: int, k: int, sink: bool
                 ) -> Tuple[bool, bool, str]:
    """(ok, in_tie_band, why).  Applies the tie rule to one unit."""
    if list(oracle_sel) == list(gpu_sel):
        return True, False, ""
    forced = {c} | ({0} if (sink and c > 0) else set())
    if not forced <= set(gpu_sel) or len(gpu_sel) != len(oracle_sel) or sorted(set(gpu_sel)) != list(gpu_sel):
        return False, False, f"malformed list {gpu_sel} vs {oracle_sel}"
    cand = [j for j in range(c) if j not in forced]
    ranked = sorted(cand, key=lambda j: (-scores[j], j))
    if k == 0 or k >= len(ranked):
        return False, False, f"lists differ with no choice to make: {gpu_sel} vs {oracle_sel}"
    sk, sk1 = scores[ranked[k - 1]], scores[ranked[k]]
    band = TIE_REL * max(abs(sk), abs(sk1))
    if abs(sk - sk1) >= band:
        return False, False, f"k-th/k+1-th gap {abs(sk - sk1):.3e} >= band {band:.3e}: {gpu_sel} vs {oracle_sel}"
    allowed = {j for j in cand if abs(scores[j] - sk) <= band}
    diff = set(gpu_sel) ^ set(oracle_sel)
    if not diff <= allowed:
        return False, True, f"difference {sorted(diff)} outside the tie band {sorted(allowed)}"
    return True, True, ""


COVERAGE_REL = 1e-5


def coverage_length_ok(scores: np.ndarray, c: int, sink: bool, tau: float, k: int) -> bool:
    """A coverage budget summed in fp32 may stop one candidate early or late where the exact share
    of that candidate lies within COVERAGE_REL of tau: k is accepted when the exact share of the
    top k reaches tau (within the band) and that of the top k - 1 does not (within the band)."""
    forced = {c} | ({0} if (sink and c > 0) else set())
    cand = [j for j in range(c) if j not in forced]
    ranked = sorted(cand, key=lambda j: (-float(scores[j]), j))
    sv = np.array([float(scores[j]) for j in ranked])
    e = np.exp(sv - sv.max())
    cum = np.cumsum(e) / e.sum()
    if k < 1 or k > len(cum):
        return False
    reach = cum[k - 1] >= tau * (1 - COVERAGE_REL)
    short = k == 1 or cum[k - 2] < tau * (1 + COVERAGE_REL)
    return bool(reach and short)


def selection_matches(un, gsel: List[int], scores: np.ndarray, budget) -> Tuple[bool, bool, str]:
    """list_matches, plus (coverage budgets) a list one entry longer or shorter than the oracle's
    when the coverage band allows that length; such a list counts as inside the tie band."""
    if budget.coverage <= 0:
        return list_matches(un.sel, gsel, scores, un.c, un.k, budget.sink)
    nforced = 1 + (1 if (budget.sink and un.c > 0) else 0)
    k_gpu = len(gsel) - nforced
    if k_gpu == un.k:
        return list_matches(un.sel, gsel, scores, un.c, un.k, budget.sink)
    capped = budget.k_fixed > 0 or budget.frac_den > 0 or budget.sqrt_den > 0
    if capped and k_gpu > un.k:
        return False, False, f"{k_gpu} kept above the cap's {un.k}"
    if not coverage_length_ok(scores, un.c, budget.sink, budget.coverage, k_gpu):
        return False, False, f"coverage keeps {k_gpu} blocks, the oracle {un.k}, outside the band"
    exp = orc.topk_blocks(scores, un.c, k_gpu, budget.sink)
    ok, _, why = list_matches(exp, gsel, scores, un.c, k_gpu, budget.sink)
    return ok, True, why


def joint_matches(units, gpu_lists: Dict[int, List[int]], sink: bool) -> Tuple[bool, bool, str]:
    """Shared budget: the GPU's kept (head, block) pairs over the group's heads must be the
    oracle's, or differ only by pairs whose scores lie within TIE_REL of the K-th kept score
    (then the lists count as inside the tie band)."""
    c = units[0].c
    forced = {c} | ({0} if (sink and c > 0) else set())
    rows = {un.sel_head: un.scores for un in units}
    ora = {(un.sel_head, j) for un in units for j in un.sel if j not in forced}
    gpu = set()
    for h, lst in gpu_lists.items():
        if not forced <= set(lst) or sorted(set(lst)) != lst:
            return False, False, f"head {h}: malformed list {lst}"
        gpu |= {(h, j) for j in lst if j not in forced}
    if gpu == ora:
        return True, False, ""
    if len(gpu) != len(ora):
        return False, False, f"{len(gpu)} pairs kept, the oracle keeps {len(ora)}"
    cand = [(h, j) for h in rows for j in range(c) if j not in forced]
    ranked = sorted(cand, key=lambda hj: (-float(rows[hj[0]][hj[1]]), hj[0], hj[1]))
    K = len(ora)
    if K == 0 or K >= len(ranked):
        return False, False, "pairs differ with no choice to make"
    sk, sk1 = float(rows[ranked[K - 1][0]][ranked[K - 1][1]]), float(rows[ranked[K][0]][ranked[K][1]])
    band = TIE_REL * max(abs(sk), abs(sk1))
    if abs(sk - sk1) >= band:
        return False, False, f"K-th/K+1-th gap {abs(sk - sk1):.3e} >= band {band:.3e}"
    allowed = {hj for hj in cand if abs(float(rows[hj[0]][hj[1]]) - sk) <= band}
    if not (gpu ^ ora) <= allowed:
        return False, True, "pairs differ outside the tie band"
    return True, True, ""


def out_check(rep: Report, gpu: np.ndarray, ref: np.ndarray, bf16: bool) -> None:
    d = np.abs(gpu.astype(np.float64) - ref)
    assert np.isfinite(gpu).all(), "non-finite GPU output"
    rep.max_abs = max(rep.max_abs, float(d.max()))
    rep.mean_abs_num += float(d.sum())
    rep.mean_abs_den += d.size


def assert_report(rep: Report, bf16: bool) -> None:
    if bf16:
        assert rep.max_abs <= BF16_MAX_ABS, f"max-abs {rep.max_abs:.3e} > {BF16_MAX_ABS}"
        assert rep.mean_abs <= BF16_MEAN_ABS, f"mean-abs {rep.mean_abs:.3e} > {BF16_MEAN_ABS}"
    else:
        assert rep.max_abs <= F32_MAX_ABS, f"max-abs {rep.max_abs:.3e} > {F32_MAX_ABS}"


def sel_count(w: Workload) -> int:
    return w.hkv if w.sel == "group" else w.hq


def budget_of(w: Workload) -> sas.Budget:
    return sas.Budget(k_fixed=w.k_fixed, frac_num=w.frac_num, frac_den=w.frac_den,
                      count_current=w.count_current, sink=w.sink, gate=w.gate,
                      coverage=float(w.spec.get("coverage", 0.0)), shared=bool(w.spec.get("shared", False)),
                      sqrt_num=w.sqrt_num, sqrt_den=w.sqrt_den)


def run_case(w: Workload, seqs: List[int], unit_sample: Optional[int] = None, seed: int = 0,
             budget_override: Optional[sas.Budget] = None, check_scores: bool = True, keep_n: int = 2,
             unit_keys=()) -> Report:
    """Run the whole path for the given sequences (all prefill or all decode) and compare.

    unit_sample: compare a seeded sample of that many units per kept sequence (keep_n sequences kept
    on the host) instead of every unit; unit_keys: (selector head, current block) pairs compared in
    every kept sequence besides the sample."""
    import torch
    bf16 = w.is_bf16()
    gist = w.kind == "gist_decode"
    decode = w.seq_kind[seqs[0]] == "decode"
    rng = np.random.default_rng(seed)
    budget = budget_override or budget_of(w)
    S = sel_count(w)
    say(f"[case] {w.name} seqs={seqs} decode={decode} gist={gist} sample={unit_sample}")
    # which sequences get oracle attention (sampled runs keep at most 2 sequences on the host)
    keep = list(seqs) if unit_sample is None else list(rng.choice(seqs, size=min(keep_n, len(seqs)), replace=False))
    inp = upload(w, seqs, keep_host=set(int(x) for x in keep), gist=gist)
    lens = inp.seq_lens
    B = len(seqs)
    Lmax = inp.K.shape[2]
    dtype_code = sas.SAS_BF16 if bf16 else sas.SAS_F32
    tq = 1 if decode else w.tq
    # ---- GPU path
    if gist:
        reps = inp.gist_k
    else:
        reps = sas.block_reps(inp.K, lens, w.block, hq=w.hq)
    scores = sas.block_scores(inp.Q, reps, lens, w.block, w.hkv, Lmax, q_start=inp.q_start, sel_mode=w.sel,
                              gist=gist)
    idx, nsel, gate = sas.topk_select(scores, lens, w.block, w.hq, w.hkv, w.d, dtype_code, Lmax, budget, tq=tq,
                                      q_start=inp.q_start, sel_mode=w.sel)
    fused = None
    if decode and max((L - 1) // w.block for L in lens) <= 2048 and budget.coverage > 0:
        # coverage budgets sum fp32 shares in each path's own order: both lists are checked against
        # the oracle below (a length may differ by one inside the coverage band)
        _, i2, n2, _ = sas.select_decode(inp.Q, reps, lens, w.block, w.hkv, Lmax, budget, sel_mode=w.sel,
                                         gist=gist, kcap=idx.shape[1])
        torch.cuda.synchronize()
        fused = (i2.cpu().numpy(), n2.cpu().numpy())
    elif decode and max((L - 1) // w.block for L in lens) <= 2048 and not (budget.shared and w.group > 4):
        # the fused decode selection must give the same scores, lists and gates as the two calls
        s2, i2, n2, g2 = sas.select_decode(inp.Q, reps, lens, w.block, w.hkv, Lmax, budget, sel_mode=w.sel,
                                           gist=gist, kcap=idx.shape[1])
        torch.cuda.synchronize()
        assert torch.equal(n2, nsel), "fused selection: nsel differs from the two-call path"
        assert torch.equal(i2, idx), "fused selection: lists differ from the two-call path"
        if g2 is not None:
            assert torch.allclose(g2, gate, rtol=0, atol=1e-6), "fused selection: gates differ"
        scores, idx, nsel, gate = s2, i2, n2, g2
        say("[case] fused decode selection == two-call selection")
    if decode:
        O = sas.sparse_decode(inp.Q, inp.K, inp.V, lens, w.block, idx, nsel, gate, sel_mode=w.sel,
                              gist_k=inp.gist_k if gist else None, gist_v=inp.gist_v if gist else None)
    else:
        O = sas.sparse_prefill(inp.Q, inp.K, inp.V, lens, w.block, inp.q_start, idx, nsel, gate, sel_mode=w.sel)
    torch.cuda.synchronize()
    say("[case] gpu path done")
    reps_h = reps.float().cpu().numpy() if not gist else None
    scores_h = scores.cpu().numpy()
    idx_h = idx.cpu().numpy()
    nsel_h = nsel.cpu().numpy()
    gate_h = gate.cpu().numpy() if gate is not None else None
    O_h = O.float().cpu().numpy()
    QB = 1 if decode else sas.num_qblocks(w.tq, w.block)
    rep = Report()
    for bi, b in enumerate(seqs):
        if int(b) not in inp.host:
            continue
        hst = inp.host[int(b)]
        L = w.seq_lens[b]
        q0 = w.q_start[b]
        Qb = hst["q"]
        units = orc.make_units(q0, w.rows[b], w.block, w.hq, w.hkv, w.sel)
        chosen = set(range(len(units)))
        if unit_sample is not None:
            chosen = set(int(x) for x in rng.choice(len(units), size=min(unit_sample, len(units)), replace=False))
            chosen |= {x for x, un in enumerate(units) if (un.sel_head, un.c) in set(unit_keys)}
        keyset = {(units[x].sel_head, units[x].c) for x in chosen}
        filt = lambda u: (u.sel_head, u.c) in keyset  # noqa: E731
        # oracle: reps/scores/selection for chosen units, no attention yet
        gk = hst.get("gist_k") if gist else None
        gv = hst.get("gist_v") if gist else None
        r = orc.run_sequence(Qb, hst["k"], hst["v"], L, q0, w.block, w.sel, k_fixed=budget.k_fixed,
                             frac_num=budget.frac_num, frac_den=budget.frac_den,
                             count_current=budget.count_current, sink=budget.sink, gate=budget.gate,
                             gist_k=gk, gist_v=gv, unit_filter=filt, attend=False, coverage=budget.coverage,
                             shared=budget.shared, sqrt_num=budget.sqrt_num, sqrt_den=budget.sqrt_den)
        if not gist:
            nb = orc.num_blocks(L, w.block)
            dr = np.abs(reps_h[bi, :, :nb] - r.reps)
            rep.reps_max_abs = max(rep.reps_max_abs, float(dr.max()))
            assert dr.max() <= 1e-5 * (1.0 + np.abs(r.reps).max()), f"reps differ by {dr.max():.3e}"
        explicit = {}
        band_units = set()
        if budget.shared:
            # a shared budget is checked per group: the kept (head, block) pairs of the G heads
            groups = {}
            for un in r.units:
                if un.scores is not None:
                    groups.setdefault((un.sel_head // w.group, un.c), []).append(un)
            for (g, c), us in groups.items():
                gl = {}
                for un in us:
                    u = (bi * S + un.sel_head) * QB + (un.c - q0 // w.block)
                    gl[un.sel_head] = [int(x) for x in idx_h[u, :int(nsel_h[u])]]
                ok, band, why = joint_matches(us, gl, budget.sink)
                assert ok, f"sequence {b}, KV head {g}, block {c}: {why}"
                if band:
                    band_units |= {(un.sel_head, un.c) for un in us}
        for un in r.units:
            if un.scores is None:
                continue
            u = (bi * S + un.sel_head) * QB + (un.c - q0 // w.block)
            s_or = un.scores
            s_gpu = scores_h[u, : un.c + 1].astype(np.float64)
            if check_scores:
                fin = np.isfinite(s_or)
                assert (np.isfinite(s_gpu) == fin).all(), f"unit {u}: -inf pattern differs"
                if fin.any():
                    err = np.abs(s_gpu[fin] - s_or[fin])
                    tol = 1e-5 * (1.0 + np.abs(s_or[fin]).max())
                    assert err.max() <= tol, f"unit {u}: scores differ by {err.max():.3e} (tol {tol:.1e})"
                    rep.score_max_rel = max(rep.score_max_rel, float(err.max() / (1.0 + np.abs(s_or[fin]).max())))
            n = int(nsel_h[u])
            gsel = [int(x) for x in idx_h[u, :n]]
            assert all(int(x) == -1 for x in idx_h[u, n:]), f"unit {u}: padding is not -1"
            if budget.shared:
                ok, tie, why = True, (un.sel_head, un.c) in band_units, ""
                if not tie:
                    assert gsel == list(un.sel), f"unit {u}: {gsel} != {un.sel}"
            else:
                ok, tie, why = selection_matches(un, gsel, s_or, budget)
            assert ok, f"unit {u} (head {un.sel_head}, block {un.c}): {why}"
            if fused is not None:
                fs = [int(x) for x in fused[0][u, :fused[1][u]]]
                ok2, _, why2 = selection_matches(un, fs, s_or, budget)
                assert ok2, f"unit {u} (head {un.sel_head}, block {un.c}), fused selection: {why2}"
            rep.units += 1
            if tie:
                rep.tie_band_units += 1
                gv_ = orc.gate_values(s_or, gsel) if budget.gate else None
                explicit[(un.sel_head, un.c)] = (gsel, gv_)
            elif budget.gate:
                ref_g = np.array([un.gate[j] for j in un.sel])
                dg = np.abs(gate_h[u, :n] - ref_g).max()
                rep.gate_max_abs = max(rep.gate_max_abs, float(dg))
                assert dg <= 1e-4, f"unit {u}: gate differs by {dg:.3e}"
        # oracle attention for the chosen units (with the GPU list inside the tie band)
        r2 = orc.run_sequence(Qb, hst["k"], hst["v"], L, q0, w.block, w.sel, k_fixed=budget.k_fixed,
                              frac_num=budget.frac_num, frac_den=budget.frac_den,
                              count_current=budget.count_current, sink=budget.sink, gate=budget.gate,
                              gist_k=gk, gist_v=gv, unit_filter=filt, reps=r.reps, explicit=explicit,
                              coverage=budget.coverage, shared=budget.shared, sqrt_num=budget.sqrt_num,
                              sqrt_den=budget.sqrt_den)
        mask = ~np.isnan(r2.O[:, :, 0])
        gpu_rows = O_h[bi] if not decode else O_h[bi][:, None, :]
        out_check(rep, gpu_rows[mask], r2.O[mask], bf16)
    assert rep.units > 0
    assert_report(rep, bf16)
    say(f"[case] ok units={rep.units} tie_band={rep.tie_band_units} max_abs={rep.max_abs:.3e} "
        f"mean_abs={rep.mean_abs:.3e} reps_err={rep.reps_max_abs:.2e} score_rel={rep.score_max_rel:.2e} "
        f"gate_err={rep.gate_max_abs:.2e}")
    return rep
