"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each test checks the oracle against something it does not compute itself: a pattern
printed on the pages (tests/golden), a hand-worked example, a library routine
(torch's scaled_dot_product_attention in float64 on the CPU, numpy reductions), a
brute-force enumeration, or a closed form.  Together they are chosen so that a dropped
term, a wrong sign or index, or a transposed operand in any oracle step fails one of them.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

from oracle import sas_oracle as o
from workloads import Workload, round_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_matrix(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(x) for x in line.split()])
    return np.array(rows)


def _sdpa(q, k, v, additive):
    """torch SDPA in float64 on the CPU with an additive float mask [n, L]."""
    qt = torch.from_numpy(np.asarray(q, np.float64))[None, None]
    kt = torch.from_numpy(np.asarray(k, np.float64))[None, None]
    vt = torch.from_numpy(np.asarray(v, np.float64))[None, None]
    mt = torch.from_numpy(np.asarray(additive, np.float64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt)[0, 0].numpy()


# ------------------------------------------------------------------------------------ P1
def test_window_pattern_from_topk_recency():
    """Token-level blocks with recency scores and k = w - 1 = 2 reproduce the printed w=3 window."""
    L, d = 6, 2
    q = np.zeros((1, L, d)); q[0, :, 0] = math.sqrt(2.0)          # score of key j == j
    K = np.zeros((1, L, d)); K[0, :, 0] = np.arange(L)
    V = np.eye(L)[None]                                            # output row == attention weights
    r = o.run_sequence(q, K, V, L, 0, 1, "group", k_fixed=2)
    mask = (r.O[0] > 0).astype(int)
    np.testing.assert_array_equal(mask, _load_matrix("window_w3_pattern.txt"))


# ------------------------------------------------------------------------------------ P2
def test_block_pattern_from_explicit_lists():
    """The printed 4x4 block-sparse pattern is what the mask expansion of its block lists gives."""
    blk, L, d = 3, 12, 4
    rng = np.random.default_rng(0)
    q = rng.standard_normal((1, L, d)); K = rng.standard_normal((1, L, d))
    V = np.eye(L)[None]
    lists = {0: [0], 1: [0, 1], 2: [1, 2], 3: [0, 2, 3]}           # Q1:{1} Q2:{1,2} Q3:{2,3} Q4:{1,3,4}
    explicit = {(0, c): (sel, None) for c, sel in lists.items()}
    r = o.run_sequence(q, K, V, L, 0, blk, "group", k_fixed=0, explicit=explicit)
    tok = r.O[0] > 0                                                # [query token, key token]
    blocks = tok.reshape(4, blk, 4, blk).any(axis=(1, 3)).astype(int)
    np.testing.assert_array_equal(blocks, _load_matrix("block_sparse_4x4_pattern.txt"))


# ------------------------------------------------------------------------------------ hand example
def test_hand_worked_three_keys():
    g = {}
    with open(os.path.join(GOLDEN, "hand_three_keys.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, a, b = line.split()
                g[name] = (float(a), float(b))
    q = np.array([[[math.sqrt(2.0), 0.0]]])
    K = np.array([[[0.0, 0.0], [math.log(3.0), 0.0], [0.0, 0.0]]])
    V = np.array([[[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]]])
    for name, kw in (("dense", dict(k_fixed=5)), ("top1", dict(k_fixed=1)),
                     ("top1_gate", dict(k_fixed=1, gate=True))):
        r = o.run_sequence(q, K, V, 3, 2, 1, "group", **kw)
        np.testing.assert_allclose(r.O[0, 0], g[name], rtol=0, atol=1e-14)


# ------------------------------------------------------------------------------------ P3
@pytest.mark.parametrize("q_start,rows", [(0, 37), (20, 17)])
@pytest.mark.parametrize("sel_mode", ["group", "head"])
def test_all_blocks_is_dense_causal_sdpa(q_start, rows, sel_mode):
    """Budget >= #blocks with the gate off is dense causal attention (torch SDPA, float64)."""
    rng = np.random.default_rng(1)
    hq, hkv, d, L, blk = 4, 2, 8, 37, 4
    Q = rng.standard_normal((hq, rows, d)); K = rng.standard_normal((hkv, L, d)); V = rng.standard_normal((hkv, L, d))
    r = o.run_sequence(Q, K, V, L, q_start, blk, sel_mode, k_fixed=100)
    pos = q_start + np.arange(rows)
    add = np.where(np.arange(L)[None, :] <= pos[:, None], 0.0, -np.inf)
    for h in range(hq):
        ref = _sdpa(Q[h], K[h // 2], V[h // 2], add)
        np.testing.assert_allclose(r.O[h], ref, rtol=0, atol=1e-12)


# ------------------------------------------------------------------------------------ P4
@pytest.mark.parametrize("gate", [False, True])
@pytest.mark.parametrize("sink", [False, True])
def test_selected_equals_sdpa_with_minus_inf_mask(gate, sink):
    """Sparse output == dense attention with unselected blocks at -inf (+ the gate), via SDPA."""
    rng = np.random.default_rng(2)
    hq, hkv, d, L, blk = 6, 2, 16, 53, 5
    q_start, rows = 11, 42
    Q = rng.standard_normal((hq, rows, d)); K = rng.standard_normal((hkv, L, d)); V = rng.standard_normal((hkv, L, d))
    r = o.run_sequence(Q, K, V, L, q_start, blk, "group", k_fixed=3, sink=sink, gate=gate)
    lit = o.run_sequence(Q, K, V, L, q_start, blk, "group", k_fixed=3, sink=sink, gate=gate, mode="literal")
    np.testing.assert_allclose(r.O, lit.O, rtol=0, atol=1e-13)
    G = hq // hkv
    for u in r.units:
        for h in u.heads:
            pos = q_start + np.arange(u.t_lo, u.t_hi)
            keys = np.arange(L)
            ok = np.isin(keys // blk, u.sel)[None, :] & (keys[None, :] <= pos[:, None])
            add = np.where(ok, 0.0, -np.inf)
            if gate:
                add = add + np.array([u.gate.get(int(j), 0.0) for j in keys // blk])[None, :]
            ref = _sdpa(Q[h, u.t_lo:u.t_hi], K[h // G], V[h // G], add)
            np.testing.assert_allclose(r.O[h, u.t_lo:u.t_hi], ref, rtol=0, atol=1e-12)


# ------------------------------------------------------------------------------------ P5
def _brute_topk(scores, c, k, sink):
    forced = {c} | ({0} if sink else set())
    cand = [j for j in range(c) if j not in forced]
    best = None
    for sub in itertools.combinations(cand, min(k, len(cand))):
        key = (sorted((scores[j] for j in sub), reverse=True), [-x for x in sorted(sub)])
        # best = lexicographically largest sorted score vector; among equal, smallest indices
        if best is None or key[0] > best[0][0] or (key[0] == best[0][0] and sorted(sub) < best[1]):
            best = (key, sorted(sub))
    return sorted(set(best[1]) | forced)


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(3)
    for trial in range(300):
        c = int(rng.integers(0, 11))
        scores = [float(x) for x in rng.integers(0, 4, size=c + 1)]   # many exact ties
        sink = bool(rng.integers(0, 2))
        k = int(rng.integers(0, c + 2))
        assert o.topk_blocks(scores, c, k, sink) == _brute_topk(scores, c, k, sink), (scores, c, k, sink)


def test_topk_prefers_lower_index_on_ties_and_keeps_forced():
    assert o.topk_blocks([1.0, 5.0, 5.0, 5.0, 0.0], 4, 2, False) == [1, 2, 4]
    assert o.topk_blocks([9.0, 5.0, 5.0, 7.0, 0.0], 4, 1, True) == [0, 3, 4]
    assert o.topk_blocks([0.0], 0, 3, True) == [0]


# ------------------------------------------------------------------------------------ budgets
def test_budget_rules():
    # fixed budget, capped by the candidate count
    assert o.budget_k(c=511, n_cand=511, k_fixed=16, frac_num=0, frac_den=0, count_current=0) == 16
    assert o.budget_k(c=3, n_cand=3, k_fixed=16, frac_num=0, frac_den=0, count_current=0) == 3
    # top 1/8 of the prior blocks: ceil(c/8)
    assert [o.budget_k(c, c, 0, 1, 8, 0) for c in (0, 1, 8, 9, 255)] == [0, 1, 1, 2, 32]
    # 5% of the visible blocks (c+1), rounded up
    assert [o.budget_k(c, c, 0, 1, 20, 1) for c in (0, 19, 20, 2047)] == [0, 1, 2, 103]


# ------------------------------------------------------------------------------------ P6
def test_gate_constant_shift_invariance():
    rng = np.random.default_rng(4)
    d, L, blk = 8, 24, 4
    q = rng.standard_normal((5, d)); K = rng.standard_normal((L, d)); V = rng.standard_normal((L, d))
    pos = np.arange(19, 24)
    sel = [0, 2, 5]
    g = o.gate_values([0.3] * 6, sel)
    assert all(abs(v + math.log(3.0)) < 1e-15 for v in g.values())
    a = o.attend_unit(q, pos, K, V, L, blk, sel, g, 0.5)
    b = o.attend_unit(q, pos, K, V, L, blk, sel, None, 0.5)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)
    assert o.gate_values([2.5], [0]) == {0: 0.0}


# ------------------------------------------------------------------------------------ P7
def test_gate_block_decomposition_closed_form():
    """With the gate, out = sum_j pi_j Z_j o_j / sum_j pi_j Z_j (pi = softmax over Sel of s)."""
    rng = np.random.default_rng(5)
    hq, hkv, d, L, blk = 2, 1, 8, 40, 8
    Q = rng.standard_normal((hq, 1, d)); K = rng.standard_normal((hkv, L, d)); V = rng.standard_normal((hkv, L, d))
    r = o.run_sequence(Q, K, V, L, L - 1, blk, "head", k_fixed=2, gate=True)
    sc = 1.0 / math.sqrt(d)
    for u in r.units:
        h = u.sel_head
        s = u.scores
        pi = np.exp(np.array([s[j] for j in u.sel]) - max(s[j] for j in u.sel))
        pi /= pi.sum()
        num = np.zeros(d); den = 0.0
        for w, j in zip(pi, u.sel):
            lo, hi = j * blk, min((j + 1) * blk, L)
            logit = K[0, lo:hi] @ Q[h, 0] * sc
            e = np.exp(logit)
            Z = e.sum()
            oj = (e[:, None] * V[0, lo:hi]).sum(axis=0) / Z
            num += w * Z * oj; den += w * Z
        np.testing.assert_allclose(r.O[h, 0], num / den, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------------------------ P8 / scores
def test_scores_closed_form():
    """Constant-key blocks: rep = that key, score = scale * mean(q) . key (hand values)."""
    d, blk, L = 4, 2, 6
    K = np.zeros((1, L, d))
    K[0, 0:2] = [1, 0, 0, 0]; K[0, 2:4] = [0, 2, 0, 0]; K[0, 4:6] = [1, 1, 1, 1]
    Q = np.zeros((2, 2, d))                                   # 2 heads of one group, rows at 4, 5
    Q[0, 0] = [2, 0, 0, 0]; Q[0, 1] = [0, 0, 0, 2]; Q[1, 0] = [0, 4, 0, 0]; Q[1, 1] = [2, 2, 2, 2]
    V = np.zeros((1, L, d))
    r = o.run_sequence(Q, K, V, L, 4, blk, "group", k_fixed=0, scale=0.5)
    (u,) = r.units
    # mean q = (1, 1.5, 0.5, 1); scores = 0.5 * (1, 3, 4)
    np.testing.assert_allclose(u.scores, [0.5, 1.5, 2.0], rtol=0, atol=1e-15)
    # per-head selection: head 0 mean q = (1,0,0,1) -> 0.5*(1, 0, 2); head 1 = (1,3,1,1) -> 0.5*(1, 6, 6)
    r2 = o.run_sequence(Q, K, V, L, 4, blk, "head", k_fixed=0, scale=0.5)
    np.testing.assert_allclose(r2.units[0].scores, [0.5, 0.0, 1.0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(r2.units[1].scores, [0.5, 3.0, 3.0], rtol=0, atol=1e-15)


def test_score_linearity_pooled_query():
    rng = np.random.default_rng(6)
    qv = rng.standard_normal((50, 16)); reps = rng.standard_normal((9, 16))
    s = o.unit_scores(qv, reps, 9, 0.25)
    np.testing.assert_allclose(s, 0.25 * (qv.mean(axis=0) @ reps.T), rtol=1e-13, atol=1e-14)


# ------------------------------------------------------------------------------------ P9
def test_decode_equals_last_prefill_row():
    rng = np.random.default_rng(7)
    hq, hkv, d, blk = 4, 2, 16, 8
    L = blk * 9 + 1                                           # last block holds only position L-1
    Q = rng.standard_normal((hq, L, d)); K = rng.standard_normal((hkv, L, d)); V = rng.standard_normal((hkv, L, d))
    kw = dict(k_fixed=3, gate=True, sink=True)
    pre = o.run_sequence(Q, K, V, L, 0, blk, "head", **kw)
    dec = o.run_sequence(Q[:, L - 1:], K, V, L, L - 1, blk, "head", **kw)
    np.testing.assert_allclose(dec.O[:, 0], pre.O[:, L - 1], rtol=0, atol=1e-13)


# ------------------------------------------------------------------------------------ P11 gist limits
def test_gist_limits():
    rng = np.random.default_rng(8)
    hq, hkv, d, blk = 2, 1, 8, 4
    L = blk * 7 + 3                                           # 7 complete chunks, query in chunk 7
    Q = rng.standard_normal((hq, 1, d)); K = rng.standard_normal((hkv, L, d)); V = rng.standard_normal((hkv, L, d))
    gk = rng.standard_normal((hkv, 7, d)); gv = rng.standard_normal((hkv, 7, d))
    p = L - 1
    # every chunk expanded: plain causal attention over the raw tokens
    r = o.run_sequence(Q, K, V, L, p, blk, "group", k_fixed=100, gist_k=gk, gist_v=gv)
    add = np.zeros((1, L))
    for h in range(hq):
        np.testing.assert_allclose(r.O[h], _sdpa(Q[h], K[0], V[0], add), rtol=0, atol=1e-12)
    assert r.gist_pairs == 0
    # nothing expanded: the 7 gists plus the raw tokens of the current chunk
    r0 = o.run_sequence(Q, K, V, L, p, blk, "group", k_fixed=0, gist_k=gk, gist_v=gv)
    kk = np.concatenate([gk[0], K[0, 7 * blk:L]]); vv = np.concatenate([gv[0], V[0, 7 * blk:L]])
    for h in range(hq):
        np.testing.assert_allclose(r0.O[h], _sdpa(Q[h], kk, vv, np.zeros((1, kk.shape[0]))), rtol=0, atol=1e-12)
    assert r0.gist_pairs == 7 * hq and r0.pairs == 3 * hq


# ------------------------------------------------------------------------------------ P12 reps
def test_reps_closed_forms_and_library_mean():
    rng = np.random.default_rng(9)
    d, blk = 8, 4
    K = rng.standard_normal((4 * blk + 1, d))
    K[blk:2 * blk] = K[blk]                                   # constant block
    reps = o.block_reps(K, 4 * blk + 1, blk)
    assert reps.shape == (5, d)
    np.testing.assert_array_equal(reps[1], K[blk])
    np.testing.assert_array_equal(reps[4], K[4 * blk])        # 1-token partial block
    np.testing.assert_allclose(reps[:4], K[:4 * blk].reshape(4, blk, d).mean(axis=1), rtol=1e-14, atol=1e-15)
    reps2 = o.block_reps(K, 4 * blk - 2, blk)                 # partial block of 2 tokens
    np.testing.assert_allclose(reps2[3], K[3 * blk:4 * blk - 2].mean(axis=0), rtol=1e-14)


# ------------------------------------------------------------------------------------ P13 sparsity
def test_sparsity_accounting_tiny_prefill_closed_form():
    """Config 1: sum over query blocks of (min(c,4)*64*64 + 64*65/2) = 254,464 visible pairs."""
    w = Workload(1)
    Q = w.q(0); K, V = w.kv(0)
    r = o.run_sequence(Q, K, V, w.seq_lens[0], 0, w.block, "group", k_fixed=4)
    closed = sum(min(c, 4) * 64 * 64 + 64 * 65 // 2 for c in range(16))
    assert r.pairs == closed == 254464
    assert abs(o.sparsity(r.pairs, o.dense_causal_pairs(0, 1024)) - (1 - 254464 / 524800)) < 1e-15


def test_sparsity_accounting_block_rules():
    # decode, 32K context, 64-token blocks, 16 + current: 17 blocks of 64 keys per row
    assert 1 - 17 * 64 / 32768 == pytest.approx(0.96680, abs=1e-5)
    # causal prefill, 256 blocks of 128, ceil(c/8) + sink + current
    per_head = 0
    for c in range(256):
        n = len(o.topk_blocks(list(range(c + 1)), c, o.budget_k(c, max(c - 1, 0), 0, 1, 8, 0), True))
        per_head += (n - 1) * 128 * 128 + 128 * 129 // 2
    assert per_head == 74956800
    # gist decode: 104 expanded chunks, 1 raw token of the current chunk, 1944 gists
    assert 104 * 64 + 1 + (2048 - 104) == 8601


def test_workload_inputs_are_bf16_and_seeded():
    w = Workload(2, mini=True)
    K, V = w.kv(3)
    np.testing.assert_array_equal(K, round_bf16(K))
    K2, _ = Workload(2, mini=True).kv(3)
    np.testing.assert_array_equal(K, K2)
    assert K.shape == (8, 4096, 128)


# ------------------------------------------------------------------------------------ H-SSA
def _hssa_data(seed, hq, hkv, d, blk, L):
    rng = np.random.default_rng(seed)
    c = (L - 1) // blk
    Q = rng.standard_normal((hq, 1, d)); K = rng.standard_normal((hkv, L, d)); V = rng.standard_normal((hkv, L, d))
    gk = rng.standard_normal((hkv, c, d)); gv = rng.standard_normal((hkv, c, d))
    mk = rng.standard_normal((hkv, c, d)); mv = rng.standard_normal((hkv, c, d))
    return Q, K, V, gk, gv, mk, mv


@pytest.mark.parametrize("sel_mode", ["group", "head"])
def test_hssa_with_every_group_open_is_gist_selection(sel_mode):
    """k1 >= the complete groups: every chunk is a candidate and no meta-gist is visible, so the
    two-level choice is the one-level gist selection with k = k2, bit for bit."""
    hq, hkv, d, blk, M = 4, 2, 8, 4, 3
    L = blk * 17 + 2                                               # c = 17: 5 complete groups + 2 trailing chunks
    Q, K, V, gk, gv, mk, mv = _hssa_data(31, hq, hkv, d, blk, L)
    units, O = o.hssa_decode_sequence(Q, K, V, L, blk, sel_mode, M, 5, 6, gk, gv, mk, mv)
    r = o.run_sequence(Q, K, V, L, L - 1, blk, sel_mode, k_fixed=6, gist_k=gk, gist_v=gv)
    for hu, su in zip(units, r.units):
        assert hu.groups == [0, 1, 2, 3, 4, 5] and hu.cand == list(range(17))
        assert hu.sel == list(su.sel)
    assert np.array_equal(O, r.O)


def test_hssa_with_every_chunk_expanded_is_dense_causal():
    hq, hkv, d, blk, M = 2, 1, 8, 4, 2
    L = blk * 9 + 1
    Q, K, V, gk, gv, mk, mv = _hssa_data(32, hq, hkv, d, blk, L)
    _, O = o.hssa_decode_sequence(Q, K, V, L, blk, "group", M, 100, 100, gk, gv, mk, mv)
    for h in range(hq):
        np.testing.assert_allclose(O[h], _sdpa(Q[h], K[0], V[0], np.zeros((1, L))), rtol=0, atol=1e-12)


def test_hssa_nothing_opened_attends_meta_gists_and_the_current_chunk():
    """k1 = k2 = 0 with c a multiple of M (no trailing chunk): the key set is every meta-gist
    plus the raw tokens of the current chunk, checked with the library routine over that set."""
    hq, hkv, d, blk, M = 2, 1, 8, 4, 4
    L = blk * 12 + 3                                               # c = 12 = 3 complete groups of 4
    Q, K, V, gk, gv, mk, mv = _hssa_data(33, hq, hkv, d, blk, L)
    units, O = o.hssa_decode_sequence(Q, K, V, L, blk, "group", M, 0, 0, gk, gv, mk, mv)
    assert units[0].groups == [3] and units[0].cand == [] and units[0].sel == [12]
    kk = np.concatenate([K[0, 12 * blk:L], mk[0, :3]]); vv = np.concatenate([V[0, 12 * blk:L], mv[0, :3]])
    for h in range(hq):
        np.testing.assert_allclose(O[h], _sdpa(Q[h], kk, vv, np.zeros((1, kk.shape[0]))), rtol=0, atol=1e-12)


def test_hssa_selection_invariants_and_key_set():
    """Level 1 and level 2 each keep a top set (no kept score below a dropped one, ties to the
    lower index), the trailing group is always open, and the attended key set follows the
    visibility rules: checked against the library routine with a mask built key by key."""
    hq, hkv, d, blk, M = 2, 1, 8, 2, 3
    for seed, L, k1, k2 in [(34, 2 * 23 + 1, 2, 3), (35, 2 * 24 + 2, 1, 5), (36, 2 * 7 + 1, 5, 2)]:
        Q, K, V, gk, gv, mk, mv = _hssa_data(seed, hq, hkv, d, blk, L)
        # plant exact ties: repeat some meta-gists and gists
        mk[0, 1] = mk[0, 0]; gk[0, 4] = gk[0, 3]
        units, O = o.hssa_decode_sequence(Q, K, V, L, blk, "group", M, k1, k2, gk, gv, mk, mv)
        u = units[0]
        c, nm = u.c, u.c // M
        qbar = Q[:, 0, :].mean(axis=0)
        s1 = np.array([qbar @ mk[0, i] for i in range(nm)]) / math.sqrt(d)
        s2 = np.array([qbar @ gk[0, j] for j in range(c)]) / math.sqrt(d)
        opened = [i for i in u.groups if i < nm]
        assert u.groups[-1] == nm and len(opened) == min(k1, nm)
        closed = [i for i in range(nm) if i not in opened]
        for a in opened:
            for b in closed:
                assert s1[a] > s1[b] + 1e-12 or (abs(s1[a] - s1[b]) <= 1e-12 and a < b)
        cand = [j for j in range(c) if j // M in set(u.groups)]
        assert u.cand == cand and len(cand) <= (min(k1, nm) + 1) * M
        exp = [j for j in u.sel if j != c]
        assert u.sel[-1] == c and len(exp) == min(k2, len(cand))
        for a in exp:
            for b in set(cand) - set(exp):
                assert s2[a] > s2[b] + 1e-12 or (abs(s2[a] - s2[b]) <= 1e-12 and a < b)
        # the key set, key by key: raw tokens, gists, meta-gists
        keys, vals, add = [], [], []
        for t in range(L):
            keys.append(K[0, t]); vals.append(V[0, t]); add.append(0.0 if t // blk in u.sel else -np.inf)
        for j in range(c):
            keys.append(gk[0, j]); vals.append(gv[0, j])
            add.append(0.0 if (j // M in set(u.groups) and j not in u.sel) else -np.inf)
        for i in range(nm):
            keys.append(mk[0, i]); vals.append(mv[0, i]); add.append(0.0 if i not in u.groups else -np.inf)
        kk, vv, mask = np.array(keys), np.array(vals), np.array(add)[None, :]
        for h in range(hq):
            np.testing.assert_allclose(O[h], _sdpa(Q[h], kk, vv, mask), rtol=0, atol=1e-12)


# ------------------------------------------------------------------------------------ coverage budget
def test_coverage_budget_closed_form():
    """Scores log p with p = (1/2, 1/4, 1/8, 1/16, 1/16): the top-k shares are 1/2, 3/4, 7/8, 15/16, 1."""
    p = np.array([0.0625, 0.5, 0.125, 0.25, 0.0625])           # blocks 0..4, current block 5
    s = list(np.log(p)) + [0.0]
    for tau, k in [(0.3, 1), (0.5 - 1e-9, 1), (0.74, 2), (0.76, 3), (0.9, 4), (0.95, 5), (1.0 - 1e-12, 5)]:
        assert o.coverage_k(s, 5, False, tau) == k, tau
    # with the sink, block 0 is forced and leaves the candidates: shares over blocks 1..4
    assert o.coverage_k(s, 5, True, 0.5) == 1          # 0.5 / 0.9375 = 0.53
    assert o.coverage_k(s, 5, True, 0.93) == 3         # (0.5 + 0.25 + 0.125) / 0.9375 = 0.933
    assert o.coverage_k(s, 0, False, 0.5) == 0          # no candidate


def test_coverage_budget_brute_force_with_ties():
    """The coverage budget is the smallest size of any candidate subset holding a share >= tau
    (enumerated), and the list is the top set of that size under the lower-index tie rule."""
    rng = np.random.default_rng(41)
    for trial in range(60):
        c = int(rng.integers(1, 9))
        s = list(rng.integers(-3, 3, size=c).astype(float) * 0.5) + [0.0]
        tau = float(rng.uniform(0.05, 1.0))
        e = np.exp(np.array(s[:c]) - max(s[:c]))
        best = min(len(sub) for r in range(1, c + 1) for sub in itertools.combinations(range(c), r)
                   if e[list(sub)].sum() >= tau * e.sum() * (1 - 1e-12))
        k = o.coverage_k(s, c, False, tau)
        assert k == best, (s, tau, k, best)
        assert o.topk_blocks(s, c, k, False)[:-1] == sorted(sorted(range(c), key=lambda j: (-s[j], j))[:k])


def test_coverage_budget_in_a_sequence():
    """run_sequence with a coverage budget: each unit keeps the covering top set, capped by the
    fixed budget when one is given; tau -> 1 keeps every candidate."""
    rng = np.random.default_rng(42)
    hq, hkv, d, blk, L = 4, 2, 8, 4, 4 * 13 + 1
    Q = rng.standard_normal((hq, 1, d)); K = rng.standard_normal((hkv, L, d)); V = rng.standard_normal((hkv, L, d))
    r = o.run_sequence(Q, K, V, L, L - 1, blk, "group", coverage=0.6, sink=True, attend=False)
    for un in r.units:
        assert un.k == o.coverage_k(un.scores, un.c, True, 0.6) and len(un.sel) == un.k + 2
    r = o.run_sequence(Q, K, V, L, L - 1, blk, "group", coverage=0.6, k_fixed=2, sink=True, attend=False)
    assert all(un.k == min(2, o.coverage_k(un.scores, un.c, True, 0.6)) for un in r.units)
    r = o.run_sequence(Q, K, V, L, L - 1, blk, "group", coverage=1.0, attend=False)
    assert all(un.k == un.c for un in r.units)


# ------------------------------------------------------------------------------------ shared budget
def test_joint_topk_closed_forms():
    rng = np.random.default_rng(51)
    c = 12
    row = rng.standard_normal(c + 1)
    # identical rows: every head keeps the per-head top-k
    lists = o.joint_topk({0: row, 1: row, 2: row}, c, 3 * 4, False)
    assert all(lists[h] == o.topk_blocks(row, c, 4, False) for h in range(3))
    # one head, or a budget of one head's k: the per-head selection
    assert o.joint_topk({5: row}, c, 4, True)[5] == o.topk_blocks(row, c, 4, True)
    # a head whose scores all exceed the other's takes the budget first
    hi = row + 100.0
    lists = o.joint_topk({0: row, 1: hi}, c, 2 * 7, False)
    assert lists[1] == list(range(c + 1)) and lists[0] == o.topk_blocks(row, c, 2 * 7 - c, False)
    # the budget caps at the candidate count
    lists = o.joint_topk({0: row, 1: row}, 3, 50, True)
    assert lists[0] == lists[1] == [0, 1, 2, 3]


def test_joint_topk_is_a_top_set_with_planted_ties():
    """Every kept (head, block) pair ranks above every dropped one: higher score, or an equal score
    and a lower (head, block); forced blocks are in every list."""
    rng = np.random.default_rng(52)
    for trial in range(40):
        G, c = int(rng.integers(1, 5)), int(rng.integers(1, 15))
        rows = {h: rng.integers(-2, 3, size=c + 1).astype(float) for h in range(G)}
        sink = bool(rng.integers(0, 2))
        K = int(rng.integers(0, G * c + 2))
        lists = o.joint_topk(rows, c, K, sink)
        forced = {c} | ({0} if (sink and c > 0) else set())
        kept = {(h, j) for h in range(G) for j in lists[h] if j not in forced}
        cand = {(h, j) for h in range(G) for j in range(c) if j not in forced}
        assert len(kept) == min(K, len(cand)) and all(forced <= set(lists[h]) for h in range(G))
        for (h, j) in kept:
            for (h2, j2) in cand - kept:
                assert rows[h][j] > rows[h2][j2] or (rows[h][j] == rows[h2][j2] and (h, j) < (h2, j2))


def test_shared_budget_in_a_sequence():
    """Per-head prefill units of one query block share G * k; the lists do not depend on which
    units are attended, and the attended output is the masked softmax of each head's list."""
    rng = np.random.default_rng(53)
    hq, hkv, d, blk, L, tq = 4, 2, 8, 4, 4 * 11 + 2, 9
    Q = rng.standard_normal((hq, tq, d)); K = rng.standard_normal((hkv, L, d)); V = rng.standard_normal((hkv, L, d))
    r = o.run_sequence(Q, K, V, L, L - tq, blk, "head", k_fixed=2, sink=True, gate=True, shared=True)
    byg = {}
    for u in r.units:
        byg.setdefault((u.sel_head // 2, u.c), []).append(u)
    for (g, c), us in byg.items():
        lists = o.joint_topk({u.sel_head: u.scores for u in us}, c, 2 * len(us), True)
        assert all(u.sel == lists[u.sel_head] for u in us)
        assert sum(len(u.sel) - len({c} | ({0} if c > 0 else set())) for u in us) == min(4, 2 * max(c - 1, 0))
    keep = {(r.units[0].sel_head, r.units[0].c)}
    r2 = o.run_sequence(Q, K, V, L, L - tq, blk, "head", k_fixed=2, sink=True, gate=True, shared=True,
                        unit_filter=lambda u: (u.sel_head, u.c) in keep)
    assert r2.units[0].sel == r.units[0].sel
    u = r.units[0]
    h = u.heads[0]
    pos = (L - tq) + np.arange(u.t_lo, u.t_hi)
    keys = np.arange(L)
    g = np.array([u.gate.get(int(k) // blk, 0.0) for k in keys])
    allow = np.isin(keys // blk, u.sel)[None, :] & (keys[None, :] <= pos[:, None])
    add = np.where(allow, 0.0, -np.inf) + g[None, :]
    ref = _sdpa(Q[h, u.t_lo:u.t_hi], K[h // 2], V[h // 2], add)
    np.testing.assert_allclose(r.O[h, u.t_lo:u.t_hi], ref, rtol=0, atol=1e-12)


# ------------------------------------------------------------------------------------ backward
def _loss_numpy(Q, K, V, dO, L, q0, blk, sel_mode, explicit, gate):
    r = o.run_sequence(Q, K, V, L, q0, blk, sel_mode, k_fixed=2, sink=True, gate=gate, explicit=explicit)
    return float((r.O * dO).sum())


@pytest.mark.parametrize("sel_mode", ["group", "head"])
def test_backward_matches_finite_differences_of_the_forward_oracle(sel_mode):
    """The autograd backward against central differences of the numpy forward oracle, with each
    unit's list held fixed: entries of Q, K, V, one gate value, and one selector score (through
    the gate's log-softmax)."""
    from oracle import sas_backward as ob
    rng = np.random.default_rng(61)
    hq, hkv, d, blk, L, tq = 4, 2, 8, 4, 4 * 9 + 3, 10
    q0 = L - tq
    Q = rng.standard_normal((hq, tq, d)); K = rng.standard_normal((hkv, L, d)); V = rng.standard_normal((hkv, L, d))
    dO = rng.standard_normal((hq, tq, d))
    r = o.run_sequence(Q, K, V, L, q0, blk, sel_mode, k_fixed=2, sink=True, gate=True, attend=False)
    fixed = {(u.sel_head, u.c): (list(u.sel), dict(u.gate)) for u in r.units}
    grads = ob.backward_sequence(Q, K, V, dO, L, q0, blk, r.units, gate=True)
    eps = 1e-6

    def fd(mutate):
        plus, minus = mutate(+eps), mutate(-eps)
        return (_loss_numpy(*plus) - _loss_numpy(*minus)) / (2 * eps)

    def with_arr(arr_name, index):
        def mutate(e):
            arrs = {"Q": Q.copy(), "K": K.copy(), "V": V.copy()}
            arrs[arr_name][index] += e
            return (arrs["Q"], arrs["K"], arrs["V"], dO, L, q0, blk, sel_mode, fixed, True)
        return mutate
    for name, index in [("Q", (1, 3, 2)), ("Q", (3, 9, 7)), ("K", (0, 30, 1)), ("K", (1, 5, 4)),
                        ("V", (1, 33, 0)), ("V", (0, 2, 6))]:
        got = grads["d" + name][index]
        assert abs(got - fd(with_arr(name, index))) <= 1e-6 * (1 + abs(got)), (name, index)
    u = r.units[-1]
    key_u = (u.sel_head, u.c)
    j0 = u.sel[0]

    def with_gate(e):
        sel, g = fixed[key_u]
        g2 = dict(g); g2[j0] += e
        ex = dict(fixed); ex[key_u] = (sel, g2)
        return (Q, K, V, dO, L, q0, blk, sel_mode, ex, True)

    assert abs(grads["dgate"][key_u][0] - fd(with_gate)) <= 1e-6

    def with_score(e):
        s2 = np.array(u.scores, dtype=np.float64); s2[j0] += e
        ex = dict(fixed); ex[key_u] = (fixed[key_u][0], o.gate_values(s2, fixed[key_u][0]))
        return (Q, K, V, dO, L, q0, blk, sel_mode, ex, True)

    assert abs(grads["dscore"][key_u][0] - fd(with_score)) <= 1e-6
    # the log-softmax Jacobian: dscore = dgate - exp(g) * sum(dgate)
    g = np.array([u.gate[j] for j in u.sel])
    dg = grads["dgate"][key_u]
    np.testing.assert_allclose(grads["dscore"][key_u], dg - np.exp(g) * dg.sum(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("sel_mode", ["group", "head"])
def test_backward_through_scores_matches_finite_differences(sel_mode):
    """With the selector scores taken as the function of Q and K the forward scored with (pooled
    query . block mean), the autograd dQ and dK against central differences of the numpy forward
    oracle in which every unit's gate is recomputed from the perturbed Q and K (lists fixed); and
    the gradient differs from the constant-score one (the selector path is not empty)."""
    from oracle import sas_backward as ob
    rng = np.random.default_rng(67)
    hq, hkv, d, blk, L, tq = 4, 2, 8, 4, 4 * 9 + 3, 10
    q0 = L - tq
    scale = 1.0 / np.sqrt(d)
    Q = rng.standard_normal((hq, tq, d)); K = rng.standard_normal((hkv, L, d)); V = rng.standard_normal((hkv, L, d))
    dO = rng.standard_normal((hq, tq, d))
    r = o.run_sequence(Q, K, V, L, q0, blk, sel_mode, k_fixed=2, sink=True, gate=True, attend=False)
    grads = ob.backward_sequence(Q, K, V, dO, L, q0, blk, r.units, gate=True, through_scores=True)
    plain = ob.backward_sequence(Q, K, V, dO, L, q0, blk, r.units, gate=True)
    G = hq // hkv

    def loss(Qx, Kx):
        reps = np.stack([o.block_reps(Kx[g], L, blk) for g in range(hkv)])
        ex = {}
        for u in r.units:
            g = u.heads[0] // G
            sc = o.unit_scores(o.unit_query_vectors(Qx, u), reps[g], u.c + 1, scale)
            ex[(u.sel_head, u.c)] = (list(u.sel), o.gate_values(sc, u.sel))
        return _loss_numpy(Qx, Kx, V, dO, L, q0, blk, sel_mode, ex, True)
    eps = 1e-6
    for name, index in [("Q", (1, 3, 2)), ("Q", (3, 9, 7)), ("K", (0, 30, 1)), ("K", (1, 5, 4)), ("K", (0, 1, 3))]:
        def at(e):
            Qx, Kx = Q.copy(), K.copy()
            (Qx if name == "Q" else Kx)[index] += e
            return loss(Qx, Kx)
        want = (at(eps) - at(-eps)) / (2 * eps)
        got = grads["d" + name][index]
        assert abs(got - want) <= 1e-6 * (1 + abs(got)), (name, index, got, want)
    assert np.abs(grads["dK"] - plain["dK"]).max() > 1e-6
    np.testing.assert_allclose(grads["dV"], plain["dV"], rtol=0, atol=1e-12)


def test_backward_all_blocks_gate_off_is_sdpa_backward():
    """Every block selected and no gate: the gradients of dense causal attention, from torch's
    scaled_dot_product_attention in float64."""
    from oracle import sas_backward as ob
    rng = np.random.default_rng(62)
    hq, hkv, d, blk, L = 2, 1, 8, 4, 4 * 6 + 1
    Q = rng.standard_normal((hq, L, d)); K = rng.standard_normal((hkv, L, d)); V = rng.standard_normal((hkv, L, d))
    dO = rng.standard_normal((hq, L, d))
    r = o.run_sequence(Q, K, V, L, 0, blk, "group", k_fixed=100, attend=False)
    grads = ob.backward_sequence(Q, K, V, dO, L, 0, blk, r.units, gate=False)
    qt = torch.tensor(Q, dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(np.repeat(K, hq, axis=0), dtype=torch.float64, requires_grad=True)
    vt = torch.tensor(np.repeat(V, hq, axis=0), dtype=torch.float64, requires_grad=True)
    out = torch.nn.functional.scaled_dot_product_attention(qt[None], kt[None], vt[None], is_causal=True)[0]
    (out * torch.tensor(dO)).sum().backward()
    np.testing.assert_allclose(grads["dQ"], qt.grad.numpy(), rtol=0, atol=1e-10)
    np.testing.assert_allclose(grads["dK"], kt.grad.numpy().sum(axis=0, keepdims=True), rtol=0, atol=1e-10)
    np.testing.assert_allclose(grads["dV"], vt.grad.numpy().sum(axis=0, keepdims=True), rtol=0, atol=1e-10)


def test_row_logsumexp_closed_forms():
    """Row log-sum-exp of the backward oracle: with K = 0 and no gate every visible logit is 0, so it
    equals log(number of visible keys) = log(pos + 1) under a dense causal selection; the row at
    position 0 sees key 0 only, so it equals that one logit, scale q.k0 + g(0)."""
    import math
    from oracle import sas_oracle as o
    from oracle import sas_backward as ob
    rng = np.random.default_rng(7)
    hq, hkv, d, blk, L = 2, 1, 8, 4, 19
    Q = rng.standard_normal((hq, L, d))
    K0 = np.zeros((hkv, L, d))
    r = o.run_sequence(Q, K0, K0, L, 0, blk, "group", k_fixed=100, attend=False)
    lse = ob.row_logsumexp(Q, K0, L, 0, blk, r.units, gate=False)
    np.testing.assert_allclose(lse, np.log(np.arange(1, L + 1))[None, :].repeat(hq, 0), rtol=0, atol=1e-12)
    K = rng.standard_normal((hkv, L, d))
    r = o.run_sequence(Q, K, K, L, 0, blk, "group", k_fixed=2, sink=True, gate=True, attend=False)
    lse = ob.row_logsumexp(Q, K, L, 0, blk, r.units, gate=True, scale=0.5)
    u0 = [u for u in r.units if u.c == 0][0]
    for h in range(hq):
        assert abs(lse[h, 0] - (0.5 * float(Q[h, 0] @ K[0, 0]) + u0.gate[0])) <= 1e-12
    # a row past the first block sees more keys than one, so its value differs from its first logit
    assert np.isfinite(lse).all()
