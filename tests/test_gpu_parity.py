"""GPU parity of the HIP path (through the C ABI binding) against the CPU oracle.

Every case runs reps -> scores -> top-k -> attention on the GPU and compares block
representatives, scores, block lists (tie rule), gates and outputs with the oracle on
the same seeded inputs.  Small cases compare every unit; the full-size configurations
(the shapes the benchmark times) compare a seeded sample of units.
"""
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from workloads import Workload  # noqa: E402

from gpu_harness import run_case, say  # noqa: E402
import top_block_sparse_gist_amd as sas  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sas.load()
    yield


# ------------------------------------------------------------------------------ the five workloads, small
def test_c1_tiny_prefill_f32():
    w = Workload(1)
    run_case(w, [0])


def test_c2_decode_mini():
    w = Workload(2, mini=True)
    run_case(w, list(range(w.batch)))


def test_c3_prefill_mini():
    w = Workload(3, mini=True)
    run_case(w, [0])


def test_c4_gist_decode_mini():
    w = Workload(4, mini=True)
    run_case(w, list(range(w.batch)))


def test_c5_mixed_mini_prefill_half():
    w = Workload(5, mini=True)
    run_case(w, w.prefill_seqs())


def test_c5_mixed_mini_decode_half():
    w = Workload(5, mini=True)
    run_case(w, w.decode_seqs())


# ------------------------------------------------------------------------------ edge cases
def test_decode_ragged_lengths_sink_gate():
    """L = 1 (only the current block), partial blocks, k larger than the candidates."""
    w = Workload(2, overrides=dict(tag="ragged", seq_lens=[1, 63, 64, 65, 200, 4097, 777, 3000], k_fixed=3,
                                   sink=True, gate=True, seq_len=None))
    run_case(w, list(range(8)))


def test_decode_per_head_block128_d64():
    w = Workload(2, overrides=dict(tag="h128d64", seq_lens=[129, 1000, 4096, 2500], batch=4, block=128, d=64,
                                   sel="head", k_fixed=2, gate=True, hq=8, hkv=2))
    run_case(w, list(range(4)))


def test_prefill_unaligned_rows_and_partial_blocks():
    """q_start not on a block boundary, tq not a multiple of the block, per-group G=2."""
    w = Workload(3, overrides=dict(tag="unaligned", seq_len=1000, tq=300, block=64, hq=4, hkv=2,
                                   frac_num=1, frac_den=4, sink=True, gate=True))
    run_case(w, [0])


def test_prefill_short_rows_per_head():
    w = Workload(3, overrides=dict(tag="short", seq_len=520, tq=17, block=64, hq=6, hkv=2, sel="head",
                                   frac_num=0, frac_den=0, k_fixed=2, sink=False, gate=True))
    run_case(w, [0])


@pytest.mark.parametrize("sel", ["group", "head"])
def test_prefill_head_dim_64(sel):
    """d = 64: per-group units (4 heads x 128-block rows: 128-row workgroups, swizzled 16-byte copies,
    a partial last block) and per-head units (64-row workgroups, padded one-row copies)."""
    w = Workload(3, overrides=dict(tag="d64" + sel, seq_len=1500, tq=600, block=128 if sel == "group" else 64,
                                   d=64, hq=8, hkv=2, sel=sel, frac_num=1, frac_den=4, sink=True, gate=True))
    run_case(w, [0])


def test_prefill_zero_budget_only_current_and_sink():
    w = Workload(3, overrides=dict(tag="k0", seq_len=2048, tq=2048, block=128, hq=4, hkv=1,
                                   frac_num=0, frac_den=0, k_fixed=0, sink=True, gate=True))
    run_case(w, [0])


def test_decode_group_and_gist_d64():
    """d = 64 on the bf16 decode path: per-group lists with sink and gate, and gist mode."""
    w = Workload(2, overrides=dict(tag="g64", seq_lens=[300, 2000, 4096, 1000], batch=4, d=64, k_fixed=4,
                                   sink=True, gate=True, hq=8, hkv=2, seq_len=None))
    run_case(w, list(range(4)))
    wg = Workload(4, overrides=dict(tag="gist64", d=64, seq_len=5000, batch=2, k_fixed=6, hq=8, hkv=2))
    run_case(wg, [0, 1])


def test_decode_per_head_sixteen_heads_per_kv_head():
    """Per-head selection with G = 16: each wave of the fused selection's last workgroup takes
    four units in turn; 5 % budget over ~80-700 candidates."""
    w = Workload(2, overrides=dict(tag="h16", seq_lens=[45000, 5000], batch=2, sel="head", hq=32, hkv=2,
                                   k_fixed=0, frac_num=1, frac_den=20, gate=True, seq_len=None))
    run_case(w, [0, 1])


def test_decode_group_block128_sink_gate():
    w = Workload(2, overrides=dict(tag="g128", seq_lens=[5000, 300, 129, 8000], batch=4, block=128, k_fixed=3,
                                   sink=True, gate=True, hq=8, hkv=2, seq_len=None))
    run_case(w, list(range(4)))


def test_decode_beyond_fused_selection_limit():
    """Current block 2187 > 2048: selection by the two calls, then a 10-entry list in decode."""
    w = Workload(2, overrides=dict(tag="long", seq_lens=[140000], batch=1, hq=8, hkv=2, k_fixed=8, sink=True,
                                   gate=True, seq_len=None))
    run_case(w, [0])


def test_decode_group_long_lists_sink_gate():
    """Per-group selection over 468-1562 candidates: the last selection workgroup's 4 waves share
    each unit's candidates (counts, tie ranks, gate sums and output offsets combined across
    waves), with sink and gate."""
    w = Workload(2, overrides=dict(tag="glong", seq_lens=[30000, 45000, 70000, 100000], batch=4, k_fixed=40,
                                   sink=True, gate=True, hq=8, hkv=2, seq_len=None))
    run_case(w, list(range(4)))


def test_decode_three_tiles_per_wave():
    """74-entry lists over 64 units: at two tiles per wave the grid would need two rounds of
    resident workgroups on a 256-CU device, so each wave takes three tiles; ragged lengths leave
    some units short of the capacity (workgroups past their list exit), with sink and gate."""
    w = Workload(2, overrides=dict(tag="tpw3", seq_lens=[16000, 9000, 12000, 16384, 4000, 15000, 7000, 16300],
                                   batch=8, k_fixed=72, sink=True, gate=True, seq_len=None))
    run_case(w, list(range(8)))


def test_prefill_group_few_rows():
    """20 query rows x 2 heads per unit: 64-row workgroups on per-group lists."""
    w = Workload(3, overrides=dict(tag="few", seq_len=700, tq=20, block=64, hq=4, hkv=2, frac_num=1, frac_den=4,
                                   sink=True, gate=True))
    run_case(w, [0])


def test_decode_f32_and_gist_f32():
    w = Workload(2, overrides=dict(tag="f32", dtype="f32", seq_lens=[100, 1500, 4096, 64], batch=4, k_fixed=3,
                                   gate=True, hq=8, hkv=2))
    run_case(w, list(range(4)))
    wg = Workload(4, overrides=dict(tag="f32", dtype="f32", seq_len=4097, batch=2, k_fixed=5, hq=8, hkv=2))
    run_case(wg, [0, 1])


def test_gist_decode_when_current_chunk_is_complete():
    """L a multiple of the chunk: the current chunk has a gist, which must not be used."""
    w = Workload(4, overrides=dict(tag="aligned", seq_len=8192, batch=2, k_fixed=7))
    run_case(w, [0, 1])


def test_decode_equals_last_prefill_row_on_gpu():
    """Decode at L-1 == the last row of a full prefill when that row is alone in its block."""
    L = 64 * 9 + 1
    w = Workload(3, overrides=dict(tag="p9", seq_len=L, tq=L, block=64, hq=4, hkv=2, sel="head", frac_num=0,
                                   frac_den=0, k_fixed=3, sink=True, gate=True, batch=1))
    from workloads.device import upload
    inp = upload(w, [0])
    dt = sas.SAS_BF16
    b = sas.Budget(k_fixed=3, sink=True, gate=True)
    reps = sas.block_reps(inp.K, inp.seq_lens, w.block)
    # prefill over all rows
    sc = sas.block_scores(inp.Q, reps, inp.seq_lens, w.block, w.hkv, L, q_start=[0], sel_mode="head")
    idx, nsel, gate = sas.topk_select(sc, inp.seq_lens, w.block, w.hq, w.hkv, w.d, dt, L, b, tq=L, q_start=[0],
                                      sel_mode="head")
    Op = sas.sparse_prefill(inp.Q, inp.K, inp.V, inp.seq_lens, w.block, [0], idx, nsel, gate, sel_mode="head")
    # decode of the last row
    Qd = inp.Q[:, :, L - 1, :].contiguous()
    sd = sas.block_scores(Qd, reps, inp.seq_lens, w.block, w.hkv, L, sel_mode="head")
    idd, nsd, gd = sas.topk_select(sd, inp.seq_lens, w.block, w.hq, w.hkv, w.d, dt, L, b, sel_mode="head")
    Od = sas.sparse_decode(Qd, inp.K, inp.V, inp.seq_lens, w.block, idd, nsd, gd, sel_mode="head")
    torch.cuda.synchronize()
    a = Op[0, :, L - 1].float().cpu().numpy()
    d_ = np.abs(a - Od[0].float().cpu().numpy()).max()
    say(f"[p9] decode vs last prefill row max-abs {d_:.3e}")
    assert d_ <= 2e-2


def test_explicit_block_pattern_prefill_on_gpu():
    """The printed 4x4 block pattern, given as explicit lists, reaches exactly those key blocks."""
    B, hq, hkv, d, blk, L = 1, 1, 1, 128, 64, 256
    g = torch.Generator().manual_seed(0)
    Q = torch.zeros((B, hq, L, d), dtype=torch.bfloat16)
    K = torch.zeros((B, hkv, L, d), dtype=torch.bfloat16)
    # V = one-hot of the key's block in dims 0..3: the output shows the weight on each key block
    V = torch.zeros((B, hkv, L, d), dtype=torch.bfloat16)
    for j in range(4):
        V[0, 0, j * blk:(j + 1) * blk, j] = 1.0
    lists = {0: [0], 1: [0, 1], 2: [1, 2], 3: [0, 2, 3]}
    qb = sas.num_qblocks(L, blk)           # unit slots per (sequence, head); the last one is empty
    idx = torch.full((qb, 4), -1, dtype=torch.int32)
    nsel = torch.zeros(qb, dtype=torch.int32)
    for c, sel in lists.items():
        idx[c, :len(sel)] = torch.tensor(sel, dtype=torch.int32)
        nsel[c] = len(sel)
    O = sas.sparse_prefill(Q.cuda(), K.cuda(), V.cuda(), [L], blk, [0], idx.cuda(), nsel.cuda(), None)
    w = O[0, 0, :, :4].float().cpu().numpy().reshape(4, blk, 4)
    pattern = (w > 0).any(axis=1).astype(int)
    golden = np.loadtxt(os.path.join(os.path.dirname(__file__), "golden", "block_sparse_4x4_pattern.txt"),
                        dtype=int)
    np.testing.assert_array_equal(pattern, golden)


# ------------------------------------------------------------------------------ full sizes, sampled units
@pytest.mark.timeout(600)
def test_c2_decode_full_sampled():
    w = Workload(2)
    run_case(w, list(range(w.batch)), unit_sample=16, seed=2)


@pytest.mark.timeout(600)
def test_c3_prefill_full_sampled():
    """32 random units plus all 4 KV heads of the last 8 query blocks (the longest lists: 33-34
    blocks of 128 keys over 896 rows each)."""
    w = Workload(3)
    last = [(g, c) for g in range(w.hkv) for c in range(248, 256)]
    rep = run_case(w, [0], unit_sample=32, seed=3, unit_keys=last)
    assert rep.units >= 64


@pytest.mark.timeout(600)
def test_c4_gist_decode_full_sampled():
    w = Workload(4)
    run_case(w, list(range(w.batch)), unit_sample=8, seed=4)


@pytest.mark.timeout(600)
def test_c5_prefill_half_full_sampled():
    """64 per-head units in each of 4 of the 8 prefill sequences, plus the last query block of every
    head in them (the longest lists)."""
    w = Workload(5)
    last = [(h, (w.seq_lens[b] - 1) // w.block) for b in w.prefill_seqs() for h in range(w.hq)]
    rep = run_case(w, w.prefill_seqs(), unit_sample=64, seed=5, keep_n=4, unit_keys=last)
    assert rep.units >= 256


@pytest.mark.timeout(600)
def test_c5_decode_half_full_sampled():
    w = Workload(5)
    run_case(w, w.decode_seqs(), unit_sample=32, seed=6)


# ------------------------------------------------------------------------------ exact ties
@pytest.mark.parametrize("lens", [[64 * 40 + 5, 64 * 34], [64 * 700 + 9, 64 * 40 + 1]], ids=["c_le_512", "c_gt_512"])
def test_exact_ties_go_to_the_lower_block(lens):
    """Blocks repeat with period 4, so their representatives, and hence their scores, are equal
    bit for bit: the lists (both selection paths) must be the oracle's, lowest indices first."""
    from oracle import sas_oracle as orc
    from workloads.gen import round_bf16
    B, hq, hkv, d, blk, k = len(lens), 8, 2, 128, 64, 6
    rng = np.random.default_rng(11)
    Lmax = max(lens)
    base = round_bf16(rng.standard_normal((hkv, 4, blk, d), dtype=np.float32))
    K = np.zeros((B, hkv, Lmax, d), dtype=np.float32)
    for b, L in enumerate(lens):
        for j in range(-(-L // blk)):
            n = min(blk, L - j * blk)
            K[b, :, j * blk:j * blk + n] = base[:, j % 4, :n]
    V = round_bf16(rng.standard_normal((B, hkv, Lmax, d), dtype=np.float32))
    Q = round_bf16(rng.standard_normal((B, hq, d), dtype=np.float32))
    Kd = torch.from_numpy(K).to(torch.bfloat16).cuda()
    Qd = torch.from_numpy(Q).to(torch.bfloat16).cuda()
    bud = sas.Budget(k_fixed=k)
    reps = sas.block_reps(Kd, lens, blk)
    sc = sas.block_scores(Qd, reps, lens, blk, hkv, Lmax)
    idx, nsel, _ = sas.topk_select(sc, lens, blk, hq, hkv, d, sas.SAS_BF16, Lmax, bud)
    _, idx2, nsel2, _ = sas.select_decode(Qd, reps, lens, blk, hkv, Lmax, bud, kcap=idx.shape[1])
    torch.cuda.synchronize()
    idx_h, nsel_h = idx.cpu().numpy(), nsel.cpu().numpy()
    assert torch.equal(idx, idx2) and torch.equal(nsel, nsel2), "fused selection differs from the two-call path"
    ties = 0
    for b, L in enumerate(lens):
        r = orc.run_sequence(Q[b][:, None, :], K[b], V[b], L, L - 1, blk, "group", k_fixed=k, attend=False)
        for un in r.units:
            u = b * hkv + un.sel_head
            got = [int(x) for x in idx_h[u, :nsel_h[u]]]
            assert got == list(un.sel), f"sequence {b}, KV head {un.sel_head}: {got} != {list(un.sel)}"
            s = np.sort(un.scores[:un.c])[::-1]
            ties += int(s[k - 1] == s[k])
    say(f"[ties] {ties} of {B * hkv} units have the k-th and (k+1)-th scores exactly equal")
    assert ties == B * hkv


# ------------------------------------------------------------------------------ decode loop
def test_decode_loop_incremental_reps():
    """A decode loop that appends one token per sequence per step: sas_block_reps_update pools
    only the block the token lands in, and the reps then equal a full sas_block_reps bit for bit;
    each step's selection and output match the oracle at the new length (lengths cross block
    boundaries: a block fills up, a new one opens with a single token)."""
    from oracle import sas_oracle as orc
    from workloads.gen import round_bf16
    from gpu_harness import list_matches, BF16_MAX_ABS, BF16_MEAN_ABS
    lens = [1000, 2047, 4096, 63]
    steps, B, hq, hkv, d, blk, k = 3, 4, 8, 2, 128, 64, 4
    Lmax = max(lens) + steps
    rng = np.random.default_rng(29)
    K = round_bf16(rng.standard_normal((B, hkv, Lmax, d), dtype=np.float32))
    V = round_bf16(rng.standard_normal((B, hkv, Lmax, d), dtype=np.float32))
    Q = round_bf16(rng.standard_normal((B, hq, d), dtype=np.float32))
    Kd = torch.from_numpy(K).to(torch.bfloat16).cuda()
    Vd = torch.from_numpy(V).to(torch.bfloat16).cuda()
    Qd = torch.from_numpy(Q).to(torch.bfloat16).cuda()
    bud = sas.Budget(k_fixed=k, sink=True, gate=True)
    nbmax = -(-Lmax // blk)
    reps = torch.zeros((B, hkv, nbmax, d), dtype=torch.float32, device="cuda")
    sas.block_reps(Kd, lens, blk, reps=reps)
    for step in range(steps):
        old, lens = lens, [L + 1 for L in lens]
        sas.block_reps(Kd, lens, blk, reps=reps, first_block=[L // blk for L in old])
        full = sas.block_reps(Kd, lens, blk, reps=torch.full_like(reps, float("nan")))
        scores, idx, nsel, gate = sas.select_decode(Qd, reps, lens, blk, hkv, Lmax, bud)
        O = sas.sparse_decode(Qd, Kd, Vd, lens, blk, idx, nsel, gate)
        torch.cuda.synchronize()
        for b, L in enumerate(lens):
            nb = -(-L // blk)
            assert torch.equal(reps[b, :, :nb], full[b, :, :nb]), f"step {step}: reps of sequence {b} differ"
        idx_h, nsel_h, O_h = idx.cpu().numpy(), nsel.cpu().numpy(), O.float().cpu().numpy()
        err_sum, err_n = 0.0, 0
        for b, L in enumerate(lens):
            r = orc.run_sequence(Q[b][:, None, :], K[b], V[b], L, L - 1, blk, "group", k_fixed=k, sink=True,
                                 gate=True)
            explicit = {}
            for un in r.units:
                u = b * hkv + un.sel_head
                got = [int(x) for x in idx_h[u, :nsel_h[u]]]
                ok, band, why = list_matches(un.sel, got, un.scores, un.c, un.k, True)
                assert ok, f"step {step}, sequence {b}, KV head {un.sel_head}: {why}"
                if band:
                    explicit[(un.sel_head, un.c)] = (got, orc.gate_values(un.scores, got))
            if explicit:
                r = orc.run_sequence(Q[b][:, None, :], K[b], V[b], L, L - 1, blk, "group", k_fixed=k, sink=True,
                                     gate=True, explicit=explicit)
            diff = np.abs(O_h[b] - r.O[:, 0, :])
            assert diff.max() <= BF16_MAX_ABS, f"step {step}, sequence {b}: max-abs {diff.max():.3e}"
            err_sum += float(diff.sum())
            err_n += diff.size
        assert err_sum / err_n <= BF16_MEAN_ABS
        say(f"[loop] step {step}: lengths {lens}, reps equal a full pass, lists and outputs match")


# ------------------------------------------------------------------------------ coverage budgets
def test_coverage_budget_decode_group():
    """Uncapped coverage on per-group decode units (fused and two-call selection, one wave and the
    four-wave top-k), then capped with sink and gate."""
    w = Workload(2, overrides=dict(tag="cov", seq_lens=[3000, 5000, 8000, 1500, 40000, 33000], batch=6, hq=8,
                                   hkv=2, k_fixed=0, coverage=0.5, seq_len=None))
    run_case(w, list(range(6)))
    w2 = Workload(2, overrides=dict(tag="covcap", seq_lens=[3000, 9000, 700], batch=3, hq=8, hkv=2, k_fixed=6,
                                    coverage=0.3, sink=True, gate=True, seq_len=None))
    run_case(w2, list(range(3)))


def test_coverage_budget_decode_per_head_and_gist():
    w = Workload(2, overrides=dict(tag="covh", seq_lens=[20000, 6000], batch=2, sel="head", hq=8, hkv=2,
                                   k_fixed=0, coverage=0.25, gate=True, seq_len=None))
    run_case(w, [0, 1])
    wg = Workload(4, overrides=dict(tag="covg", seq_len=9000, batch=2, hq=8, hkv=2, k_fixed=0, coverage=0.4))
    run_case(wg, [0, 1])


def test_coverage_budget_prefill():
    """Per-group and per-head prefill units through the two-call top-k."""
    w = Workload(3, overrides=dict(tag="cov", seq_len=3000, tq=1000, hq=8, hkv=2, frac_num=0, frac_den=0,
                                   k_fixed=0, coverage=0.35, sink=True, gate=True))
    run_case(w, [0])
    wh = Workload(3, overrides=dict(tag="covh", seq_len=2500, tq=600, hq=4, hkv=2, block=64, sel="head",
                                    frac_num=0, frac_den=0, k_fixed=5, coverage=0.6, gate=True))
    run_case(wh, [0])


# ------------------------------------------------------------------------------ paged KV cache
def _paged_copy(K, V, lens, blk, seed):
    """Scatter the blocks of contiguous K/V [B, Hkv, Lmax, d] into shuffled pages of one block
    each, [num_pages, Hkv, blk, d] (plus unused pages), and return (K_pages, V_pages, table)."""
    B, hkv, _, d = K.shape
    nbs = [-(-L // blk) for L in lens]
    npages = sum(nbs) + 5
    perm = np.random.default_rng(seed).permutation(npages)
    Kp = torch.zeros((npages, hkv, blk, d), dtype=K.dtype, device=K.device)
    Vp = torch.zeros_like(Kp)
    table = torch.full((B, max(nbs) + 3), -1, dtype=torch.int32)
    n = 0
    for b, L in enumerate(lens):
        for j in range(nbs[b]):
            pg = int(perm[n]); n += 1
            rows = min(blk, L - j * blk)
            Kp[pg, :, :rows] = K[b, :, j * blk:j * blk + rows]
            Vp[pg, :, :rows] = V[b, :, j * blk:j * blk + rows]
            table[b, j] = pg
    return Kp, Vp, table.cuda()


@pytest.mark.parametrize("sel,blk", [("group", 64), ("head", 128)])
def test_paged_decode_equals_contiguous(sel, blk):
    """The same cache, paged in shuffled pages with a block table: reps (full and incremental) and
    decode outputs equal the contiguous path's bit for bit; that path is checked against the
    oracle, on the same workload, first."""
    from workloads.device import upload
    w = Workload(2, overrides=dict(tag=f"paged{blk}", seq_lens=[5000, 777, 12345, 64 * 30], batch=4, hq=8, hkv=2,
                                   block=blk, sel=sel, k_fixed=5, sink=True, gate=True, seq_len=None))
    run_case(w, list(range(4)))
    inp = upload(w, list(range(4)))
    lens, Lmax = inp.seq_lens, inp.K.shape[2]
    Kp, Vp, table = _paged_copy(inp.K, inp.V, lens, blk, seed=7)
    reps = sas.block_reps(inp.K, lens, blk)
    reps_p = torch.full_like(reps, float("nan"))
    sas.block_reps_paged(Kp, table, lens, blk, w.hkv, Lmax, reps_p, hq=w.hq)
    # incremental form over pages: pool the last block of every sequence again
    sas.block_reps_paged(Kp, table, lens, blk, w.hkv, Lmax, reps_p, first_block=[(L - 1) // blk for L in lens],
                         hq=w.hq)
    budget = sas.Budget(k_fixed=5, sink=True, gate=True)
    _, idx, nsel, gate = sas.select_decode(inp.Q, reps, lens, blk, w.hkv, Lmax, budget, sel_mode=sel)
    O = sas.sparse_decode(inp.Q, inp.K, inp.V, lens, blk, idx, nsel, gate, sel_mode=sel)
    Op = sas.sparse_decode_paged(inp.Q, Kp, Vp, table, lens, blk, Lmax, idx, nsel, gate, sel_mode=sel)
    torch.cuda.synchronize()
    for b, L in enumerate(lens):
        nb = -(-L // blk)
        assert torch.equal(reps[b, :, :nb], reps_p[b, :, :nb]), f"sequence {b}: paged reps differ"
    assert torch.equal(O, Op), "paged decode differs from the contiguous decode"
    say(f"[paged] blk {blk} {sel}: reps and outputs equal the contiguous path bit for bit")


@pytest.mark.parametrize("sel,blk,d", [("group", 128, 128), ("head", 64, 128), ("head", 64, 64)])
def test_paged_prefill_equals_contiguous(sel, blk, d):
    """Prefill over a paged cache (shuffled one-block pages) equals the contiguous prefill bit for
    bit: 128-row workgroups with swizzled copies, 64-row ones with padded rows (d 128) and with
    swizzled rows (d 64), partial last blocks included; the contiguous path is checked against the
    oracle on the same workload first."""
    from workloads.device import upload
    w = Workload(3, overrides=dict(tag=f"paged{sel}{blk}{d}", seq_lens=[3000, 1777], seq_len=None, batch=2, tq=900,
                                   hq=8, hkv=2, d=d, block=blk, sel=sel, frac_num=1, frac_den=4, sink=True, gate=True))
    run_case(w, [0, 1])
    inp = upload(w, [0, 1])
    lens, Lmax = inp.seq_lens, inp.K.shape[2]
    budget = sas.Budget(frac_num=1, frac_den=4, sink=True, gate=True)
    reps = sas.block_reps(inp.K, lens, blk, hq=w.hq)
    scores = sas.block_scores(inp.Q, reps, lens, blk, w.hkv, Lmax, q_start=inp.q_start, sel_mode=sel)
    idx, nsel, gate = sas.topk_select(scores, lens, blk, w.hq, w.hkv, d, sas.SAS_BF16, Lmax, budget, tq=w.tq,
                                      q_start=inp.q_start, sel_mode=sel)
    O = sas.sparse_prefill(inp.Q, inp.K, inp.V, lens, blk, inp.q_start, idx, nsel, gate, sel_mode=sel)
    Kp, Vp, table = _paged_copy(inp.K, inp.V, lens, blk, seed=9)
    Op = sas.sparse_prefill_paged(inp.Q, Kp, Vp, table, lens, blk, Lmax, inp.q_start, idx, nsel, gate, sel_mode=sel)
    torch.cuda.synchronize()
    assert torch.equal(O, Op), "paged prefill differs from the contiguous prefill"
    say(f"[paged] prefill {sel} blk {blk} d {d}: equal to the contiguous path bit for bit")


def test_decode_and_prefill_at_the_batch_limit():
    """64 sequences (the largest batch a call takes), ragged lengths from 1 token up, per-group and
    per-head decode with sink and gate; then a 64-sequence prefill."""
    rng = np.random.default_rng(77)
    lens = [int(x) for x in rng.integers(1, 3000, size=64)]
    w = Workload(2, overrides=dict(tag="b64", seq_lens=lens, batch=64, hq=4, hkv=2, k_fixed=3, sink=True, gate=True,
                                   seq_len=None))
    run_case(w, list(range(64)), unit_sample=24)
    wh = Workload(2, overrides=dict(tag="b64h", seq_lens=lens, batch=64, hq=4, hkv=2, sel="head", k_fixed=2,
                                    gate=True, seq_len=None))
    run_case(wh, list(range(64)), unit_sample=24)
    lp = [int(x) for x in rng.integers(200, 1500, size=64)]
    wp = Workload(3, overrides=dict(tag="b64", seq_lens=lp, seq_len=None, batch=64, tq=150, hq=4, hkv=2, block=64,
                                    frac_num=1, frac_den=4, sink=True, gate=True))
    run_case(wp, list(range(64)), unit_sample=40)


# ------------------------------------------------------------------------------ shared budgets
def test_shared_budget_decode():
    """Per-head decode units whose 4 heads share 4 k: fused selection (one head per wave, one and
    four registers of candidates) and the two-call selection must agree with the oracle; then 8
    heads per KV head through the two-call path only."""
    w = Workload(2, overrides=dict(tag="sh4", seq_lens=[5000, 300, 40000, 12000], batch=4, sel="head", hq=8, hkv=2,
                                   k_fixed=6, sink=True, gate=True, shared=True, seq_len=None))
    run_case(w, list(range(4)))
    w8 = Workload(2, overrides=dict(tag="sh8", seq_lens=[7000, 2000], batch=2, sel="head", hq=16, hkv=2, k_fixed=3,
                                    gate=True, shared=True, seq_len=None))
    run_case(w8, [0, 1])


def test_shared_budget_prefill():
    w = Workload(3, overrides=dict(tag="sh", seq_len=3000, tq=800, hq=8, hkv=2, block=64, sel="head", frac_num=1,
                                   frac_den=8, sink=True, gate=True, shared=True))
    run_case(w, [0])


# ------------------------------------------------------------------------------ near ties
def test_near_tie_output_checked_on_the_gpu_list():
    """Two planted needle blocks whose exact scores differ by ~1e-11 relative (inside the 1e-5 tie
    band, not equal): the oracle keeps the later one, fp32 scoring sees a tie and keeps the earlier
    one.  The lists must differ only inside the band, and the output is then compared with the
    oracle run on the GPU's own list (the explicit-list branch), with and without the gate."""
    w = Workload(2, overrides=dict(tag="ntie", seq_lens=[3000, 5000, 2000, 7000], batch=4, hq=8, hkv=2, k_fixed=1,
                                   needles=0, near_tie=True, seq_len=None))
    rep = run_case(w, list(range(4)))
    assert rep.tie_band_units > 0, "no unit took the tie-band branch"
    wg = Workload(2, overrides=dict(tag="ntieg", seq_lens=[3000, 5000, 2000, 7000], batch=4, hq=8, hkv=2, k_fixed=1,
                                    needles=0, near_tie=True, gate=True, sink=True, seq_len=None))
    repg = run_case(wg, list(range(4)))
    assert repg.tie_band_units > 0, "no unit took the tie-band branch"


# ------------------------------------------------------------------------------ square-root budgets
def test_sqrt_budget_decode():
    """k = ceil(8 sqrt(c + 1) / 5) (a 16K context keeps 1/10, a 64K one 1/20): per-group units
    through the fused selection (one wave and the four-wave top-k) and the two calls, then per-head
    units with the gate as in the mixed batch."""
    w = Workload(2, overrides=dict(tag="sqrtg", seq_lens=[3000, 16384, 65536, 40000], batch=4, hq=8, hkv=2,
                                   k_fixed=0, sqrt_num=8, sqrt_den=5, count_current=1, seq_len=None))
    run_case(w, list(range(4)))
    wh = Workload(2, overrides=dict(tag="sqrth", seq_lens=[20000, 6000], batch=2, sel="head", hq=8, hkv=2, k_fixed=0,
                                    sqrt_num=8, sqrt_den=5, count_current=1, gate=True, seq_len=None))
    run_case(wh, [0, 1])


def test_sqrt_budget_prefill():
    """Per-group (sink, gate) and per-head prefill units through the two-call top-k."""
    w = Workload(3, overrides=dict(tag="sqrt", seq_len=4000, tq=1200, hq=8, hkv=2, block=64, frac_num=0, frac_den=0,
                                   k_fixed=0, sqrt_num=3, sqrt_den=2, sink=True, gate=True))
    run_case(w, [0])
    wh = Workload(3, overrides=dict(tag="sqrth", seq_len=2600, tq=700, hq=4, hkv=2, block=64, sel="head",
                                    frac_num=0, frac_den=0, k_fixed=0, sqrt_num=1, sqrt_den=1, count_current=1,
                                    gate=True))
    run_case(wh, [0])


# ------------------------------------------------------------------------------ paged decode loop
def test_paged_decode_loop_against_the_oracle():
    """A decode loop over a paged cache: each step appends one token per sequence into its page (a
    fresh page from a shuffled free list when the token opens a block), updates the block table,
    pools again only the blocks from floor(L_old / blk) on through the table, selects, and attends
    through the table; every step's reps, lists and outputs are compared with the oracle on the
    contiguous cache at the new length (lengths cross block boundaries)."""
    from oracle import sas_oracle as orc
    from workloads.gen import round_bf16
    from gpu_harness import list_matches, BF16_MAX_ABS, BF16_MEAN_ABS
    lens = [1000, 127, 4096, 63]
    steps, B, hq, hkv, d, blk, k = 3, 4, 8, 2, 128, 64, 4
    Lmax = max(lens) + steps
    nbmax = -(-Lmax // blk)
    rng = np.random.default_rng(41)
    K = round_bf16(rng.standard_normal((B, hkv, Lmax, d), dtype=np.float32))
    V = round_bf16(rng.standard_normal((B, hkv, Lmax, d), dtype=np.float32))
    Q = round_bf16(rng.standard_normal((B, hq, d), dtype=np.float32))
    Qd = torch.from_numpy(Q).to(torch.bfloat16).cuda()
    npages = B * nbmax + 7
    free = [int(x) for x in rng.permutation(npages)]
    Kp = torch.zeros((npages, hkv, blk, d), dtype=torch.bfloat16, device="cuda")
    Vp = torch.zeros_like(Kp)
    table_h = torch.full((B, nbmax), -1, dtype=torch.int32)

    def write_tokens(b, lo, hi):
        for j in range(lo // blk, -(-hi // blk)):
            if int(table_h[b, j]) < 0:
                table_h[b, j] = free.pop()
            a, e = max(lo, j * blk), min(hi, (j + 1) * blk)
            pg = int(table_h[b, j])
            Kp[pg, :, a - j * blk:e - j * blk] = torch.from_numpy(K[b, :, a:e]).to(torch.bfloat16).cuda()
            Vp[pg, :, a - j * blk:e - j * blk] = torch.from_numpy(V[b, :, a:e]).to(torch.bfloat16).cuda()

    for b, L in enumerate(lens):
        write_tokens(b, 0, L)
    table = table_h.cuda()
    bud = sas.Budget(k_fixed=k, sink=True, gate=True)
    reps = torch.zeros((B, hkv, nbmax, d), dtype=torch.float32, device="cuda")
    sas.block_reps_paged(Kp, table, lens, blk, hkv, Lmax, reps, hq=hq)
    for step in range(steps):
        old, lens = lens, [L + 1 for L in lens]
        for b in range(B):
            write_tokens(b, old[b], lens[b])
        table.copy_(table_h)
        sas.block_reps_paged(Kp, table, lens, blk, hkv, Lmax, reps, first_block=[L // blk for L in old], hq=hq)
        _, idx, nsel, gate = sas.select_decode(Qd, reps, lens, blk, hkv, Lmax, bud)
        O = sas.sparse_decode_paged(Qd, Kp, Vp, table, lens, blk, Lmax, idx, nsel, gate)
        torch.cuda.synchronize()
        reps_h, idx_h, nsel_h, O_h = reps.cpu().numpy(), idx.cpu().numpy(), nsel.cpu().numpy(), O.float().cpu().numpy()
        err_sum, err_n = 0.0, 0
        for b, L in enumerate(lens):
            r = orc.run_sequence(Q[b][:, None, :], K[b], V[b], L, L - 1, blk, "group", k_fixed=k, sink=True,
                                 gate=True)
            nb = -(-L // blk)
            dr = np.abs(reps_h[b, :, :nb] - r.reps).max()
            assert dr <= 1e-5 * (1.0 + np.abs(r.reps).max()), f"step {step}, sequence {b}: reps differ by {dr:.3e}"
            explicit = {}
            for un in r.units:
                u = b * hkv + un.sel_head
                got = [int(x) for x in idx_h[u, :nsel_h[u]]]
                ok, band, why = list_matches(un.sel, got, un.scores, un.c, un.k, True)
                assert ok, f"step {step}, sequence {b}, KV head {un.sel_head}: {why}"
                if band:
                    explicit[(un.sel_head, un.c)] = (got, orc.gate_values(un.scores, got))
            if explicit:
                r = orc.run_sequence(Q[b][:, None, :], K[b], V[b], L, L - 1, blk, "group", k_fixed=k, sink=True,
                                     gate=True, explicit=explicit)
            diff = np.abs(O_h[b] - r.O[:, 0, :])
            assert diff.max() <= BF16_MAX_ABS, f"step {step}, sequence {b}: max-abs {diff.max():.3e}"
            err_sum += float(diff.sum())
            err_n += diff.size
        assert err_sum / err_n <= BF16_MEAN_ABS
        say(f"[paged-loop] step {step}: lengths {lens}, pages in use {B * nbmax + 7 - len(free)}, "
            f"reps, lists and outputs match the oracle")


@pytest.mark.parametrize("sel,d", [("group", 128), ("head", 64)])
def test_prefill_scores_against_gist_keys(sel, d):
    """Prefill block scores with gist keys as representatives (bf16 keys into the fp32 score
    product): every unit's row against the oracle's definition (mean over the unit's query vectors
    of scale * q . g_j) for the complete chunks before its current one, -inf for the rest up to c."""
    from oracle import sas_oracle as orc
    rng = np.random.default_rng(7)
    B, hq, hkv, blk = 2, 8, 2, 64
    lens, tq = [2000, 1500], 600
    q_start = [L - tq for L in lens]
    Lmax = max(lens)
    NC = Lmax // blk
    Q = torch.from_numpy(rng.standard_normal((B, hq, tq, d)).astype(np.float32)).to(torch.bfloat16)
    gk = torch.from_numpy(rng.standard_normal((B, hkv, NC, d)).astype(np.float32)).to(torch.bfloat16)
    scores = sas.block_scores(Q.cuda(), gk.cuda(), lens, blk, hkv, Lmax, q_start=q_start, sel_mode=sel, gist=True)
    torch.cuda.synchronize()
    sc = scores.cpu().numpy().astype(np.float64)
    S = hkv if sel == "group" else hq
    QB = sas.num_qblocks(tq, blk)
    scale = 1.0 / np.sqrt(d)
    worst = 0.0
    for b in range(B):
        Qb = Q[b].float().numpy()
        units = orc.make_units(q_start[b], tq, blk, hq, hkv, sel)
        for un in units:
            u = (b * S + un.sel_head) * QB + (un.c - q_start[b] // blk)
            g = orc.kv_head_of(un, hq // hkv, sel)
            have = min(lens[b] // blk, un.c)
            ref = orc.unit_scores(orc.unit_query_vectors(Qb, un), gk[b, g].float().numpy(), have, scale)
            got = sc[u, :un.c + 1]
            assert np.isneginf(got[have:]).all(), f"unit {u}: entries past the complete chunks are not -inf"
            err = np.abs(got[:have] - ref).max() if have else 0.0
            tol = 1e-5 * (1.0 + np.abs(ref).max()) if have else 0.0
            assert err <= tol, f"unit {u}: scores differ by {err:.3e} (tol {tol:.1e})"
            worst = max(worst, err / (1.0 + (np.abs(ref).max() if have else 0.0)))
    say(f"[case] gist-key prefill scores {sel} d{d}: max rel err {worst:.2e}")
