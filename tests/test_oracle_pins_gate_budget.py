"""More pins of the CPU oracle (CPU only): the gated row log-sum-exp, what the unit-level gate does to
causality, and the square-root (length-adaptive) budget.

Each test checks the oracle against something it does not compute itself: a closed form over keys
that are constant within each block, exact equality of two oracle runs that differ only in inputs the
checked row must not see, a brute-force search over integers, or the iso-error table printed on the
page "稀疏注意力的Trade-offs：Transformer大语言模型实证研究" (section 4.3.2).
"""
import math

import numpy as np
import pytest

from oracle import sas_oracle as o
from oracle import sas_backward as ob


# ------------------------------------------------------------------------------------ gated lse
def test_row_logsumexp_with_gate_closed_form():
    """Keys constant within each block: a row at position p sees n_j(p) copies of key k_j in each
    selected block j, so its log-sum-exp is log sum_j n_j(p) exp(scale q.k_j + g_j) in closed form.
    The budget keeps one block besides the current one, so every unit past the first block has two
    blocks with different selector scores and non-zero gate values; a dropped gate term, the gate of
    the wrong block or a wrong visible-key count changes the value."""
    rng = np.random.default_rng(31)
    hq, hkv, d, blk, L = 2, 1, 8, 4, 22
    nb = o.num_blocks(L, blk)
    kblock = rng.standard_normal((nb, d))
    K = np.repeat(kblock, blk, axis=0)[None, :L]
    Q = rng.standard_normal((hq, L, d))
    scale = 0.4
    r = o.run_sequence(Q, K, K, L, 0, blk, "group", k_fixed=1, gate=True, scale=scale, attend=False)
    lse = ob.row_logsumexp(Q, K, L, 0, blk, r.units, gate=True, scale=scale)
    big_gate = 0
    for u in r.units:
        if u.c > 0:
            assert len(u.sel) == 2
            big_gate += int(min(abs(u.gate[j]) for j in u.sel) > 0.05)
        for h in u.heads:
            for t in range(u.t_lo, u.t_hi):
                p = t
                terms = []
                for j in u.sel:
                    n = min(blk, L - j * blk, p - j * blk + 1)
                    if n > 0:
                        terms.append(n * math.exp(scale * float(Q[h, t] @ kblock[j]) + u.gate[j]))
                want = math.log(sum(terms))
                assert abs(lse[h, t] - want) <= 1e-12 * max(1.0, abs(want)), (u.c, h, t, lse[h, t], want)
    assert big_gate >= 3, "the pin needs units whose gate values are far from zero"


# ------------------------------------------------------------------------------------ O6: the gate is per unit
def _causality_setup():
    rng = np.random.default_rng(5)
    hq, hkv, d, blk, L = 2, 1, 8, 8, 40
    Q = rng.standard_normal((hq, L, d))
    K = rng.standard_normal((hkv, L, d))
    V = rng.standard_normal((hkv, L, d))
    K2 = K.copy()
    K2[0, 37] += 3.0 * rng.standard_normal(d)        # a key after row 33, in row 33's own block (4)
    return Q, K, V, K2, blk, L


def test_mask_is_causal_and_the_gate_is_a_unit_value():
    """Row 33 sits in block 4 with rows 32..39.  Perturbing key 37 (after the row, same block):
    gate off -> row 33's output is unchanged, bit for bit; gate on with the lists and gate values
    held fixed -> unchanged; gate on with the scores recomputed -> the lists stay the same (only the
    current block's score moves), the gate values move, and row 33 equals the unperturbed keys run
    with the perturbed run's gate values: the later key reaches the row only through its unit's gate
    values, never through the attention weights."""
    Q, K, V, K2, blk, L = _causality_setup()
    kw = dict(k_fixed=2, sink=True)
    t = 33
    a = o.run_sequence(Q, K, V, L, 0, blk, "group", **kw)
    b = o.run_sequence(Q, K2, V, L, 0, blk, "group", **kw)
    np.testing.assert_array_equal(a.O[:, t], b.O[:, t])
    assert not np.array_equal(a.O[:, 37], b.O[:, 37])               # the perturbation is real
    g1 = o.run_sequence(Q, K, V, L, 0, blk, "group", gate=True, **kw)
    u1 = [u for u in g1.units if u.c == 4][0]
    fixed = {(u1.sel_head, 4): (u1.sel, u1.gate)}
    g2 = o.run_sequence(Q, K2, V, L, 0, blk, "group", gate=True, explicit=fixed, **kw)
    np.testing.assert_array_equal(g1.O[:, t], g2.O[:, t])
    g3 = o.run_sequence(Q, K2, V, L, 0, blk, "group", gate=True, **kw)
    u3 = [u for u in g3.units if u.c == 4][0]
    assert u3.sel == u1.sel
    assert max(abs(u3.gate[j] - u1.gate[j]) for j in u1.sel) > 1e-3
    g4 = o.run_sequence(Q, K, V, L, 0, blk, "group", gate=True, explicit={(u3.sel_head, 4): (u3.sel, u3.gate)}, **kw)
    np.testing.assert_array_equal(g3.O[:, t], g4.O[:, t])
    assert np.abs(g3.O[:, t] - g1.O[:, t]).max() > 1e-6             # the unit-level gate did move the row


# ------------------------------------------------------------------------------------ square-root budget
def _smallest_k_by_search(n, num, den):
    """Linear search with exact integer compares: the smallest k >= 0 with k den >= num sqrt(n)."""
    k = 0
    while (k * den) ** 2 < num * num * n:
        k += 1
    return k


def test_sqrt_budget_brute_force():
    for num, den in ((8, 5), (1, 1), (3, 7), (16, 1), (5, 2)):
        for n in range(0, 2200):
            assert o.sqrt_budget(n, num, den) == _smallest_k_by_search(n, num, den), (n, num, den)


def test_sqrt_budget_perfect_squares_and_float_agreement():
    for m in range(0, 60):
        assert o.sqrt_budget(m * m, 8, 5) == -(-8 * m // 5)
        assert o.sqrt_budget(m * m, 1, 1) == m
    # away from exact boundaries the value is the real-valued ceiling
    rng = np.random.default_rng(3)
    for n in rng.integers(1, 1 << 20, size=400):
        x = 8 * math.sqrt(int(n)) / 5
        if abs(x - round(x)) > 1e-6:
            assert o.sqrt_budget(int(n), 8, 5) == math.ceil(x)


def test_sqrt_budget_reproduces_the_iso_error_table():
    """[SF] 4.3.2 prints the budget that holds a relative error of about 0.2: 1/10 at 16K, 1/15 at
    32K and 1/20 at 64K.  A square-root rule fitted to the 16K entry (64-token blocks: 256 blocks,
    k = 1.6 sqrt(n) = 25.6 blocks, the rule ceil(8 sqrt(n) / 5)) must give 1/20 at 64K (the two
    endpoints pin the exponent to 1/2: the kept tokens double while the length quadruples) and a
    fraction between 1/10 and 1/20 at 32K, as the table does; a fixed-ratio rule cannot meet both ends."""
    blk = 64
    frac = {}
    for L in (16384, 32768, 65536):
        n = L // blk
        k = o.sqrt_budget(n, 8, 5)
        frac[L] = k * blk / L
    assert abs(frac[16384] - 1 / 10) <= 0.002
    assert abs(frac[65536] - 1 / 20) <= 0.002
    assert 1 / 20 < frac[32768] < 1 / 10
    # sub-linear: four times the length keeps twice the blocks (perfect squares), never more
    for m in (4, 9, 16, 25):
        assert o.sqrt_budget(4 * m * m, 8, 5) <= 2 * o.sqrt_budget(m * m, 8, 5)
    ks = [o.sqrt_budget(n, 8, 5) for n in range(1, 4097)]
    assert all(b >= a for a, b in zip(ks, ks[1:]))                           # non-decreasing
    assert ks[4095] / 4096 < ks[255] / 256 < ks[15] / 16                     # kept fraction falls


def test_sqrt_budget_in_a_prefill_sequence():
    """Each unit keeps min(candidates, ceil(num sqrt(c + count_current) / den)) blocks plus its forced
    ones; with the sink forced, a capped coverage budget keeps no more than the rule."""
    rng = np.random.default_rng(17)
    hq, hkv, d, blk, L = 2, 1, 8, 4, 160
    Q = rng.standard_normal((hq, L, d))
    K = rng.standard_normal((hkv, L, d))
    r = o.run_sequence(Q, K, K, L, 0, blk, "group", sqrt_num=3, sqrt_den=2, count_current=1, sink=True, attend=False)
    for u in r.units:
        ncand = u.c - (1 if u.c > 0 else 0)
        want = min(ncand, _smallest_k_by_search(u.c + 1, 3, 2))
        assert u.k == want
        assert len(u.sel) == want + (2 if u.c > 0 else 1)
    rc = o.run_sequence(Q, K, K, L, 0, blk, "group", sqrt_num=3, sqrt_den=2, count_current=1, sink=True,
                        coverage=0.99, attend=False)
    for u, v in zip(r.units, rc.units):
        assert v.k <= u.k
