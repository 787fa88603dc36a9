"""CPU oracle for content-selected block-sparse attention (test infrastructure only).

Only the tests, the package's smoke check and the CPU-baseline leg of the benchmark
may import this module; the product path (the HIP library and its Python binding)
never does.  Everything is plain numpy in float64 after an exact upcast of the
(float32 or bf16-valued) inputs.  The module shares no code, table or helper with
the GPU path.

Pages cited below (by title; section in brackets):
  [SAS]  "SAS: 通过端到端优化上下文排序的简单注意力稀疏化"  (ai-feeds.com, paper 2609.13141)
  [BLOG] "稀疏注意力"  (blog.vegetog.com, ai-infra/sparse-attention)
  [GSA]  "开源大模型注意力机制演进:从全注意力到门控稀疏注意力的工程实践"  (ruibaoantu.com)
  [SSA]  "通过Gist Token的简化稀疏注意力"  (ai-feeds.com, paper 2604.20920)
  [SF]   "稀疏注意力的Trade-offs：Transformer大语言模型实证研究"  (review of The Sparse Frontier)

What is computed (plain definitions, no blocking or fusion beyond them):
  1. block representative of block j = mean of the present keys of that block
     ([SF] 2.1, representation heuristics: block-pooled token representations;
     [GSA] section 4, pseudo-code step 1 aggregates keys per block).
     Gist mode: the representative is the given gist key ([SSA] method, relevance scoring).
  2. selection unit = the (query row, query head) pairs that share one block list:
     decode -> one row; prefill -> the rows of one query block ([SF] 2.1 key constraint:
     prefill selects block to block).  Per KV group (rows x the group's heads pooled) or
     per query head ([SSA] method item 2, grouped expansion for GQA).
  3. score of block j for unit u = mean over (row, head) in u of scale * q . r_j.
  4. top-k by (score descending, block index ascending) among the blocks before the
     current one, plus the current block always and block 0 when the sink is on
     ([SAS] core modules 3 and 4; [BLOG] 4.6; [SF] 2.2.3 Star Attention).
  5. optional gate: g(j) = s_j - log sum_{j' in Sel} exp(s_j'), added inside the
     softmax ([SAS] core insight and core modules 2-3: the selector's score enters the
     logits in log form, normalised by a softmax over the kept set that includes the
     current block).
  6. attention = softmax(q K^T * scale + M + g) V with M = 0 for allowed keys and
     -inf otherwise ([BLOG] sections 1 and 2).  Allowed: keys of selected blocks at
     positions <= the row's position.  Gist mode adds the gist tokens of the complete,
     non-selected chunks before the current one ([SSA] method items 2 and 3).

Readings taken where the pages leave a step open are listed in the repository's design
notes; each is restated at the function that applies it.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

NEG_INF = float("-inf")


# ---------------------------------------------------------------------------------------------
# 1. block representatives
# ---------------------------------------------------------------------------------------------
def num_blocks(L: int, blk: int) -> int:
    return (L + blk - 1) // blk


def block_reps(K: np.ndarray, L: int, blk: int) -> np.ndarray:
    """Mean-pooled key of every block of one (sequence, KV head) slab.

    K: [>= L, d].  Returns [ceil(L/blk), d] float64; block j covers positions
    [j*blk, min((j+1)*blk, L)) and its representative is the sum of those keys divided
    by their count (the last block may be partial).  [SF] 2.1; [GSA] section 4 step 1.
    """
    K = np.asarray(K, dtype=np.float64)
    nb = num_blocks(L, blk)
    out = np.empty((nb, K.shape[1]), dtype=np.float64)
    for j in range(nb):
        lo, hi = j * blk, min((j + 1) * blk, L)
        out[j] = K[lo:hi].sum(axis=0) / float(hi - lo)
    return out


# ---------------------------------------------------------------------------------------------
# 2. selection units
# ---------------------------------------------------------------------------------------------
@dataclass
class Unit:
    """One selection unit of one sequence.

    sel_head: KV head g (per-group selection) or query head h (per-head selection).
    c: block index of the unit's query rows (the current block).
    t_lo, t_hi: local query-row range [t_lo, t_hi) (positions q_start + t).
    heads: query heads whose rows belong to the unit.
    """
    sel_head: int
    c: int
    t_lo: int
    t_hi: int
    heads: Tuple[int, ...]
    scores: Optional[np.ndarray] = None       # [c+1] (index j <= c), float64
    sel: Optional[List[int]] = None           # ascending block ids (forced ones included)
    k: int = 0                                # budget actually used for the top-k part
    gate: Optional[Dict[int, float]] = None   # block id -> log-gate value (None if gate off)


def query_blocks(q_start: int, rows: int, blk: int) -> List[Tuple[int, int, int]]:
    """(c, t_lo, t_hi) for every block c touched by positions q_start .. q_start+rows-1."""
    out = []
    t = 0
    while t < rows:
        p = q_start + t
        c = p // blk
        t_hi = min(rows, (c + 1) * blk - q_start)
        out.append((c, t, t_hi))
        t = t_hi
    return out


def make_units(q_start: int, rows: int, blk: int, hq: int, hkv: int, sel_mode: str) -> List[Unit]:
    """Enumerate units in (selector head, query block) order.  sel_mode: 'group' | 'head'."""
    G = hq // hkv
    units = []
    nsel = hkv if sel_mode == "group" else hq
    for s in range(nsel):
        heads = tuple(range(s * G, (s + 1) * G)) if sel_mode == "group" else (s,)
        for (c, t_lo, t_hi) in query_blocks(q_start, rows, blk):
            units.append(Unit(sel_head=s, c=c, t_lo=t_lo, t_hi=t_hi, heads=heads))
    return units


def kv_head_of(unit: Unit, G: int, sel_mode: str) -> int:
    return unit.sel_head if sel_mode == "group" else unit.sel_head // G


# ---------------------------------------------------------------------------------------------
# 3. scores
# ---------------------------------------------------------------------------------------------
def unit_query_vectors(Qb: np.ndarray, unit: Unit) -> np.ndarray:
    """All query vectors of the unit, [rows * heads, d] float64.  Qb: [hq, rows, d]."""
    q = np.asarray(Qb[list(unit.heads), unit.t_lo:unit.t_hi, :], dtype=np.float64)
    return q.reshape(-1, q.shape[-1])


def unit_scores(qvecs: np.ndarray, reps: np.ndarray, upto: int, scale: float) -> np.ndarray:
    """s_j for j in [0, upto): the mean over the unit's query vectors of scale * q . r_j.

    Written as the definition (mean of the per-vector dot products), not as a dot with a
    pooled query; the two agree by linearity.  [GSA] section 4 step 1; [SSA] method item 1
    (query against every historical gist); reading: a unit's score averages its rows and
    heads, as for the grouped decode workload whose scores average a group's query heads.
    """
    if upto <= 0:
        return np.zeros(0, dtype=np.float64)
    dots = qvecs @ np.asarray(reps[:upto], dtype=np.float64).T      # [n, upto]
    return dots.sum(axis=0) / float(qvecs.shape[0]) * scale


# ---------------------------------------------------------------------------------------------
# 4. budget and top-k
# ---------------------------------------------------------------------------------------------
def sqrt_budget(n: int, num: int, den: int) -> int:
    """Length-adaptive (sub-linear) budget: ceil(num * sqrt(n) / den), n = c + count_current blocks.

    [SF] 4.3.2 (iso-error curve): the budget that holds one error level falls from 1/10 of a 16K
    context to 1/20 of a 64K one, so the kept tokens double while the length quadruples, which is
    growth as the square root of the length; [SF] 4.4.1-4.4.2: fixed-ratio budgets are suboptimal,
    grow the budget sub-linearly with length.  Reading: k grows as sqrt(n) with a coefficient
    num/den.  Evaluated exactly: num * sqrt(n) = sqrt(num^2 n), and k * den is an integer, so the
    smallest k with k * den >= sqrt(num^2 n) is the ceiling of ceil(sqrt(num^2 n)) / den.
    """
    if n <= 0 or num <= 0:
        return 0
    x = num * num * n
    r = math.isqrt(x)
    if r * r < x:
        r += 1
    return -(-r // den)


def budget_k(c: int, n_cand: int, k_fixed: int, frac_num: int, frac_den: int, count_current: int,
             sqrt_num: int = 0, sqrt_den: int = 0) -> int:
    """Number of blocks the top-k part keeps for a unit whose current block is c.

    Fixed budget: k_fixed.  Fractional budget: ceil(frac_num * (c + count_current) / frac_den)
    in integers (the pages state budgets as a kept fraction, [GSA] section 4 pseudo-code
    keep_ratio, [SF] 1.2: 0.95 sparsity keeps 1/20).  Square-root budget (sqrt_den > 0, which takes
    precedence): sqrt_budget(c + count_current, sqrt_num, sqrt_den).  Never more than the candidates.
    """
    if sqrt_den > 0:
        k = sqrt_budget(c + count_current, sqrt_num, sqrt_den)
    elif frac_den == 0:
        k = k_fixed
    else:
        num = frac_num * (c + count_current)
        k = (num + frac_den - 1) // frac_den
    return max(0, min(n_cand, k))


def coverage_k(scores: Sequence[float], c: int, sink: bool, tau: float) -> int:
    """Coverage budget ([SF] 2.3, threshold-based allocation: keep units until a share of the
    attention mass is covered).  Reading: the candidates' mass is the softmax of their selector
    scores; the budget is the smallest k such that the first k candidates in (score descending,
    index ascending) order hold a share >= tau of it (forced blocks are not candidates and do not
    count).  0 when there is no candidate.
    """
    forced = {c}
    if sink:
        forced.add(0)
    cand = [j for j in range(c) if j not in forced]
    if not cand:
        return 0
    ranked = sorted(cand, key=lambda j: (-float(scores[j]), j))
    s = np.array([float(scores[j]) for j in ranked], dtype=np.float64)
    e = np.exp(s - s.max())
    cum = np.cumsum(e)
    return int(np.searchsorted(cum, tau * cum[-1], side="left")) + 1


def topk_blocks(scores: Sequence[float], c: int, k: int, sink: bool) -> List[int]:
    """Selected block set of a unit, ascending.

    Candidates are the blocks strictly before the current block c, minus the forced ones.
    The k best by (score descending, index ascending) are kept; the current block is always
    added ([SAS] core insight: the always-kept current block), and block 0 when the sink is
    on ([SF] 2.2.3: local block plus the first prefix block).  Ties go to the lower index
    (the pages are silent; the lower index is the stated rule for this library).
    """
    forced = {c}
    if sink:
        forced.add(0)
    cand = [j for j in range(c) if j not in forced]
    ranked = sorted(cand, key=lambda j: (-float(scores[j]), j))
    return sorted(set(ranked[:k]) | forced)


def gate_values(scores: Sequence[float], sel: Sequence[int]) -> Dict[int, float]:
    """log of the softmax over the selected set of the selector scores ([SAS] core modules 2-3).

    g(j) = s_j - log(sum_{j' in Sel} exp(s_j')), computed with the maximum subtracted.
    Temperature 1 (the scores already carry the 1/sqrt(d) scale).
    """
    v = np.array([float(scores[j]) for j in sel], dtype=np.float64)
    m = v.max()
    lse = m + math.log(float(np.exp(v - m).sum()))
    return {int(j): float(scores[j]) - lse for j in sel}


# ---------------------------------------------------------------------------------------------
# 5./6. attention
# ---------------------------------------------------------------------------------------------
def _softmax_rows(logits: np.ndarray) -> np.ndarray:
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    return e / e.sum(axis=1, keepdims=True)


def attend_unit(qrows: np.ndarray, pos: np.ndarray, K: np.ndarray, V: np.ndarray, L: int, blk: int,
                sel: Sequence[int], gate: Optional[Dict[int, float]], scale: float,
                mode: str = "skip", gist_k: Optional[np.ndarray] = None,
                gist_v: Optional[np.ndarray] = None, gist_ids: Sequence[int] = ()) -> np.ndarray:
    """softmax(q K^T * scale + M + g) V for the rows of one unit.

    qrows: [n, d]; pos: [n] absolute positions of the rows; K, V: [>= L, d] of the unit's KV
    head.  Key sigma is allowed iff its block is in ``sel`` and sigma <= the row's position
    (and sigma < L).  ``g`` is the unit's log-gate per block (0 when None).
    mode 'literal': every key's logit is formed and the mask M (0 / -inf) is added, as in
    [BLOG] section 2; mode 'skip': only allowed keys are visited.  The two give identical
    float64 results because exp(-inf) is exactly 0 and the kept terms are summed in the
    same key order.
    Gist mode ([SSA] method items 2-3): ``gist_ids`` lists the chunks whose gist token joins
    the key set (complete, non-selected chunks before the current one); gist j contributes
    key gist_k[j] and value gist_v[j], with no gate.  Gist tokens follow the raw keys in
    the key order.
    """
    q = np.asarray(qrows, dtype=np.float64)
    n = q.shape[0]
    pos = np.asarray(pos, dtype=np.int64)
    gate = gate or {}
    sel_set = set(int(j) for j in sel)
    if mode == "literal":
        keys = np.arange(L)
        Kd = np.asarray(K[:L], dtype=np.float64)
        Vd = np.asarray(V[:L], dtype=np.float64)
        logits = (q @ Kd.T) * scale                                     # [n, L]
        blocks = keys // blk
        allowed_blk = np.array([int(b) in sel_set for b in blocks], dtype=bool)
        g = np.array([gate.get(int(b), 0.0) for b in blocks], dtype=np.float64)
        M = np.where(allowed_blk[None, :] & (keys[None, :] <= pos[:, None]), 0.0, NEG_INF)
        logits = logits + M + g[None, :]
        vals = Vd
    elif mode == "skip":
        keys = np.concatenate([np.arange(j * blk, min((j + 1) * blk, L)) for j in sorted(sel_set)]) \
            if sel_set else np.zeros(0, dtype=np.int64)
        Kd = np.asarray(K[keys], dtype=np.float64)
        vals = np.asarray(V[keys], dtype=np.float64)
        g = np.array([gate.get(int(k) // blk, 0.0) for k in keys], dtype=np.float64)
        logits = (q @ Kd.T) * scale + g[None, :]
        logits = np.where(keys[None, :] <= pos[:, None], logits, NEG_INF)
    else:
        raise ValueError(mode)
    if len(gist_ids):
        gk = np.asarray(gist_k[list(gist_ids)], dtype=np.float64)
        gv = np.asarray(gist_v[list(gist_ids)], dtype=np.float64)
        logits = np.concatenate([logits, (q @ gk.T) * scale], axis=1)
        vals = np.concatenate([vals, gv], axis=0)
    p = _softmax_rows(logits)
    return p @ vals


# ---------------------------------------------------------------------------------------------
# whole-sequence drivers
# ---------------------------------------------------------------------------------------------
@dataclass
class SeqResult:
    reps: np.ndarray                   # [hkv, NB, d] (gist mode: the gist keys)
    units: List[Unit]
    O: np.ndarray                      # [hq, rows, dv]; NaN where not computed
    pairs: int = 0                     # visible raw (row, key) pairs over computed rows
    gist_pairs: int = 0                # visible gist (row, gist) pairs over computed rows


def joint_topk(rows: Dict[int, np.ndarray], c: int, k_total: int, sink: bool) -> Dict[int, List[int]]:
    """Budget shared by the heads of a group ([SF] 2.3, Ada-KV: the top k x h entries over all h
    heads, so that heads with sharper scores keep more).  Reading: the candidates of every head
    (blocks before c, minus the forced ones) compete as (head, block) pairs ranked by (score
    descending, head ascending, block ascending); the first k_total pairs are kept and each head's
    list is its kept blocks plus its forced blocks, ascending."""
    forced = {c} | ({0} if (sink and c > 0) else set())
    pairs = [(h, j) for h in sorted(rows) for j in range(c) if j not in forced]
    ranked = sorted(pairs, key=lambda hj: (-float(rows[hj[0]][hj[1]]), hj[0], hj[1]))
    kept = ranked[:max(0, min(k_total, len(ranked)))]
    return {h: sorted({j for (hh, j) in kept if hh == h} | forced) for h in rows}


def run_sequence(Qb: np.ndarray, Kb: np.ndarray, Vb: np.ndarray, L: int, q_start: int, blk: int,
                 sel_mode: str, k_fixed: int = 0, frac_num: int = 0, frac_den: int = 0,
                 count_current: int = 0, sink: bool = False, gate: bool = False,
                 scale: Optional[float] = None, gist_k: Optional[np.ndarray] = None,
                 coverage: float = 0.0, shared: bool = False, sqrt_num: int = 0, sqrt_den: int = 0,
                 gist_v: Optional[np.ndarray] = None, mode: str = "skip",
                 unit_filter=None, attend: bool = True, reps: Optional[np.ndarray] = None,
                 explicit: Optional[Dict[Tuple[int, int], Tuple[List[int], Optional[Dict[int, float]]]]] = None
                 ) -> SeqResult:
    """Oracle for one sequence: reps -> scores -> top-k (+forced, +gate) -> attention.

    Qb: [hq, rows, d] rows at positions q_start..q_start+rows-1 (decode: rows == 1 at L-1).
    Kb, Vb: [hkv, >= L, d].  gist_k/gist_v: [hkv, >= c, d] switch on gist mode (decode).
    shared (per-head selection only): the G heads of a KV group at one query block share a budget
    of G times the per-head k (joint_topk).
    unit_filter(unit) -> bool restricts which units are attended (and, unless the budget is
    shared, scored; a shared budget scores every head of a filtered unit's group).
    explicit[(sel_head, c)] = (sel, gate) replaces the unit's own selection (used to check the
    attention step on a list produced elsewhere when selections differ inside the tie band).
    """
    hq, rows, d = Qb.shape
    hkv = Kb.shape[0]
    G = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    gist_mode = gist_k is not None
    if gist_mode and gate:
        raise ValueError("the log-gate is not defined for gist tokens")
    if shared and sel_mode != "head":
        raise ValueError("a shared budget needs per-head selection")
    if reps is None:
        if gist_mode:
            reps = np.asarray(gist_k, dtype=np.float64)
        else:
            reps = np.stack([block_reps(Kb[g], L, blk) for g in range(hkv)])
    units = make_units(q_start, rows, blk, hq, hkv, sel_mode)
    O = np.full((hq, rows, Vb.shape[-1]), np.nan)
    pairs = 0
    gpairs = 0
    chosen = [u for u in units if unit_filter is None or unit_filter(u)]
    if shared:
        groups = {(kv_head_of(u, G, sel_mode), u.c) for u in chosen}
        scored = [u for u in units if (kv_head_of(u, G, sel_mode), u.c) in groups]
    else:
        scored = chosen
    # ---- scores and budgets
    for u in scored:
        g = kv_head_of(u, G, sel_mode)
        qv = unit_query_vectors(Qb, u)
        if gist_mode:
            # gists exist for the complete chunks before the current one only
            s = np.full(u.c + 1, NEG_INF)
            s[:u.c] = unit_scores(qv, reps[g], u.c, scale)
        else:
            s = unit_scores(qv, reps[g], u.c + 1, scale)
        u.scores = s
        n_cand = u.c - (1 if (sink and u.c > 0) else 0)
        rule_k = budget_k(u.c, n_cand, k_fixed, frac_num, frac_den, count_current, sqrt_num, sqrt_den)
        if coverage > 0.0:
            # coverage budget, capped by the fixed, fractional or square-root rule when one is given
            kc = coverage_k(s, u.c, sink and u.c > 0, coverage)
            capped = k_fixed > 0 or frac_den > 0 or sqrt_den > 0
            u.k = min(kc, rule_k) if capped else kc
        else:
            u.k = rule_k
    # ---- selection
    if shared:
        by_group: Dict[Tuple[int, int], List[Unit]] = {}
        for u in scored:
            by_group.setdefault((kv_head_of(u, G, sel_mode), u.c), []).append(u)
        for (g, c), us in by_group.items():
            lists = joint_topk({u.sel_head: u.scores for u in us}, c, sum(u.k for u in us), sink)
            for u in us:
                u.sel = lists[u.sel_head]
                u.gate = gate_values(u.scores, u.sel) if gate else None
    else:
        for u in scored:
            u.sel = topk_blocks(u.scores, u.c, u.k, sink)
            u.gate = gate_values(u.scores, u.sel) if gate else None
    # ---- attention
    for u in chosen:
        g = kv_head_of(u, G, sel_mode)
        sel, gv = u.sel, u.gate
        if explicit is not None and (u.sel_head, u.c) in explicit:
            sel, gv = explicit[(u.sel_head, u.c)]
        if not attend:
            continue
        gist_ids = [j for j in range(u.c) if j not in set(sel)] if gist_mode else []
        for h in u.heads:
            qrows = Qb[h, u.t_lo:u.t_hi, :]
            pos = q_start + np.arange(u.t_lo, u.t_hi)
            O[h, u.t_lo:u.t_hi, :] = attend_unit(qrows, pos, Kb[g], Vb[g], L, blk, sel, gv, scale, mode,
                                                 gist_k[g] if gist_mode else None,
                                                 gist_v[g] if gist_mode else None, gist_ids)
            pairs += visible_raw_pairs(pos, sel, blk, L)
            gpairs += len(gist_ids) * len(pos)
    return SeqResult(reps=reps, units=units, O=O, pairs=pairs, gist_pairs=gpairs)


def visible_raw_pairs(pos: np.ndarray, sel: Sequence[int], blk: int, L: int) -> int:
    """Number of (row, raw key) pairs a row set may attend: keys of selected blocks at <= the row."""
    pos = np.asarray(pos, dtype=np.int64)
    total = 0
    for j in sel:
        hi = np.minimum(np.minimum((j + 1) * blk, L), pos + 1)
        total += int(np.clip(hi - j * blk, 0, None).sum())
    return total


def dense_causal_pairs(q_start: int, rows: int) -> int:
    """(row, key) pairs of full causal attention for the rows: sum over rows of (p + 1)."""
    return sum(q_start + t + 1 for t in range(rows))


def sparsity(computed_pairs: int, full_pairs: int) -> float:
    """1 - computed / full ([SF] 1.2)."""
    return 1.0 - computed_pairs / float(full_pairs)


# ---------------------------------------------------------------------------------------------
# 7. two-level gist selection (H-SSA), decode
# ---------------------------------------------------------------------------------------------
# [SSA] method, hierarchical extension: meta-gist tokens ("gists of gists") make a second level;
# a coarse choice among them comes first, then the ordinary gists of the chosen part are scored
# and the best chunks expanded.  The pages give no more detail; the readings taken here:
#   H1  a group is M consecutive chunks; group i (chunks iM .. iM+M-1) has a meta-gist only when
#       it is complete and lies wholly before the current chunk c: i < floor(c / M);
#   H2  level 1 keeps the top-k1 complete groups by meta-gist score (ties to the lower index);
#       the trailing group (chunks floor(c/M)*M .. c-1, no meta-gist yet) is always open, as the
#       current block always is;
#   H3  level 2 keeps the top-k2 chunks of the open groups by gist score (ties to the lower
#       index); the current chunk is always attended raw;
#   H4  the key set is the raw tokens of the expanded chunks and of the current chunk (up to the
#       row), the gists of the open groups' chunks that were not expanded, and the meta-gists of
#       the complete groups that were not opened; no gate (as in gist mode);
#   H5  scores are those of step 3 (mean over the unit's heads of scale * q . x).

@dataclass
class HssaUnit:
    sel_head: int
    c: int
    heads: Tuple[int, ...]
    meta_scores: np.ndarray            # [floor(c/M)]
    groups: List[int]                  # opened groups, ascending; the last is the trailing group
    cand: List[int]                    # chunks of the opened groups (< c), ascending
    gist_scores: np.ndarray            # [c]: -inf outside cand
    sel: List[int]                     # expanded chunks + the current chunk, ascending
    k1: int = 0
    k2: int = 0


def topk_among(scores: Sequence[float], cand: Sequence[int], k: int) -> List[int]:
    """The k best of ``cand`` by (score descending, index ascending), ascending."""
    ranked = sorted(cand, key=lambda j: (-float(scores[j]), j))
    return sorted(ranked[:k])


def hssa_select(qv: np.ndarray, gist_k: np.ndarray, meta_k: np.ndarray, c: int, M: int, k1: int, k2: int,
                scale: float) -> Tuple[np.ndarray, List[int], List[int], np.ndarray, List[int], int, int]:
    """Readings H1-H3 for one unit with query vectors ``qv``: (meta scores, opened groups,
    candidate chunks, gist scores, expanded chunks + c, k1 used, k2 used)."""
    nm = c // M
    s1 = unit_scores(qv, meta_k, nm, scale)
    k1u = max(0, min(k1, nm))
    groups = topk_among(s1, range(nm), k1u) + [nm]
    cand = [j for j in range(c) if j // M in set(groups)]
    s2 = np.full(c, NEG_INF)
    if cand:
        full = unit_scores(qv, gist_k, c, scale)
        s2[cand] = full[cand]
    k2u = max(0, min(k2, len(cand)))
    sel = topk_among(s2, cand, k2u) + [c]
    return s1, groups, cand, s2, sel, k1u, k2u


def hssa_decode_sequence(Qb: np.ndarray, Kb: np.ndarray, Vb: np.ndarray, L: int, blk: int, sel_mode: str,
                         M: int, k1: int, k2: int, gist_k: np.ndarray, gist_v: np.ndarray,
                         meta_k: np.ndarray, meta_v: np.ndarray, scale: Optional[float] = None,
                         attend: bool = True, mode: str = "skip",
                         explicit: Optional[Dict[int, Tuple[List[int], List[int]]]] = None
                         ) -> Tuple[List[HssaUnit], np.ndarray]:
    """H-SSA decode of one sequence at position L - 1 (readings H1-H5).

    Qb: [hq, 1, d]; Kb, Vb: [hkv, >= L, d]; gist_k/gist_v: [hkv, >= c, d]; meta_k/meta_v:
    [hkv, >= floor(c/M), d].  explicit[sel_head] = (groups, sel) replaces a unit's own choice
    (attention checked on lists produced elsewhere when they differ inside the tie band).
    Returns the units and O [hq, 1, d].
    """
    hq, rows, d = Qb.shape
    assert rows == 1
    hkv = Kb.shape[0]
    G = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    c = (L - 1) // blk
    nm = c // M
    units = make_units(L - 1, 1, blk, hq, hkv, sel_mode)
    out_units: List[HssaUnit] = []
    O = np.full((hq, 1, Vb.shape[-1]), np.nan)
    for u in units:
        g = kv_head_of(u, G, sel_mode)
        qv = unit_query_vectors(Qb, u)
        s1, groups, cand, s2, sel, k1u, k2u = hssa_select(qv, gist_k[g], meta_k[g], c, M, k1, k2, scale)
        out_units.append(HssaUnit(u.sel_head, c, u.heads, s1, groups, cand, s2, sel, k1u, k2u))
        if not attend:
            continue
        if explicit is not None and u.sel_head in explicit:
            groups, sel = explicit[u.sel_head]
            cand = [j for j in range(c) if j // M in set(groups)]
        sel_set = set(sel)
        gist_ids = [j for j in cand if j not in sel_set]
        meta_ids = [i for i in range(nm) if i not in set(groups)]
        # gists, then meta-gists, follow the raw keys (both enter without a gate)
        extra_k = np.concatenate([np.asarray(gist_k[g][gist_ids], dtype=np.float64).reshape(-1, d),
                                  np.asarray(meta_k[g][meta_ids], dtype=np.float64).reshape(-1, d)])
        extra_v = np.concatenate([np.asarray(gist_v[g][gist_ids], dtype=np.float64).reshape(-1, Vb.shape[-1]),
                                  np.asarray(meta_v[g][meta_ids], dtype=np.float64).reshape(-1, Vb.shape[-1])])
        ids = list(range(len(gist_ids) + len(meta_ids)))
        for h in u.heads:
            O[h, 0, :] = attend_unit(Qb[h, 0:1, :], np.array([L - 1]), Kb[g], Vb[g], L, blk, sel, None, scale,
                                     mode, extra_k, extra_v, ids)[0]
    return out_units, O
