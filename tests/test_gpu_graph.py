"""The benchmark replays the decode and prefill steps from HIP graphs: every replay must give
the eager result (the library records no memset nodes; this checks it stays that way)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

import top_block_sparse_gist_amd as sas  # noqa: E402
from workloads import Workload  # noqa: E402
from workloads.device import upload  # noqa: E402


def _capture(fn):
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sas.load()


@pytest.mark.parametrize("cfg", [2, 5])
def test_decode_step_graph_replays_match_eager(cfg):
    w = Workload(cfg, mini=True)
    seqs = w.decode_seqs()
    inp = upload(w, seqs)
    lens = inp.seq_lens
    Lmax = inp.K.shape[2]
    bud = sas.Budget(k_fixed=w.k_fixed, frac_num=w.frac_num, frac_den=w.frac_den, count_current=w.count_current,
                     sink=w.sink, gate=w.gate)
    reps = sas.block_reps(inp.K, lens, w.block)
    scores = sas.block_scores(inp.Q, reps, lens, w.block, w.hkv, Lmax, sel_mode=w.sel)
    idx, nsel, gate = sas.topk_select(scores, lens, w.block, w.hq, w.hkv, w.d, sas.SAS_BF16, Lmax, bud,
                                      sel_mode=w.sel)
    O = torch.empty_like(inp.Q)
    ws = torch.zeros(sas.decode_workspace_bytes(len(lens), w.hq, w.hkv, w.d, w.block, sas.SAS_BF16, Lmax, lens,
                                                w.sel, idx.shape[1], False), dtype=torch.uint8, device="cuda")

    sel_ws = torch.zeros(sas.select_decode_workspace_bytes(len(lens), w.hq, w.hkv, w.d, w.block, sas.SAS_BF16,
                                                           Lmax, lens), dtype=torch.uint8, device="cuda")

    def step():
        # the two-launch step the benchmark replays: fused selection, then attention
        sas.select_decode(inp.Q, reps, lens, w.block, w.hkv, Lmax, bud, sel_mode=w.sel, kcap=idx.shape[1],
                          scores=scores, idx=idx, nsel=nsel, gate=gate, workspace=sel_ws)
        sas.sparse_decode(inp.Q, inp.K, inp.V, lens, w.block, idx, nsel, gate, sel_mode=w.sel, O=O, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref_O, ref_idx = O.clone(), idx.clone()
    g = _capture(step)
    for r in range(4):
        O.zero_()
        idx.fill_(7)
        scores.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx), f"replay {r}: lists differ"
        assert torch.equal(O, ref_O), f"replay {r}: outputs differ"


def test_prefill_step_graph_replays_match_eager():
    w = Workload(3, mini=True)
    inp = upload(w, [0])
    lens = inp.seq_lens
    L = lens[0]
    bud = sas.Budget(frac_num=1, frac_den=8, sink=True, gate=True)
    reps = sas.block_reps(inp.K, lens, w.block)
    ws = torch.empty(w.hkv * sas.num_qblocks(w.tq, w.block) * w.d * 4, dtype=torch.uint8, device="cuda")
    scores = sas.block_scores(inp.Q, reps, lens, w.block, w.hkv, L, q_start=[0], workspace=ws)
    idx, nsel, gate = sas.topk_select(scores, lens, w.block, w.hq, w.hkv, w.d, sas.SAS_BF16, L, bud, tq=w.tq,
                                      q_start=[0])
    O = torch.empty_like(inp.Q)

    def step():
        sas.block_reps(inp.K, lens, w.block, reps=reps)
        sas.block_scores(inp.Q, reps, lens, w.block, w.hkv, L, q_start=[0], scores=scores, workspace=ws)
        sas.topk_select(scores, lens, w.block, w.hq, w.hkv, w.d, sas.SAS_BF16, L, bud, tq=w.tq, q_start=[0],
                        idx=idx, nsel=nsel, gate=gate)
        sas.sparse_prefill(inp.Q, inp.K, inp.V, lens, w.block, [0], idx, nsel, gate, O=O)

    step()
    torch.cuda.synchronize()
    ref = O.clone()
    g = _capture(step)
    for r in range(3):
        O.zero_()
        reps.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(O, ref), f"replay {r}: outputs differ"


def test_training_step_graph_replays_match_eager():
    """Forward with the row log-sum-exp, then the backward (its workspace is cleared by a fill
    kernel inside the call, not a memset node), replayed from a graph with the workspace and the
    gradients scribbled over between replays."""
    w = Workload(3, overrides=dict(tag="graph_bwd", seq_len=2048, tq=2048, block=128, hq=8, hkv=2,
                                   frac_num=1, frac_den=4, sink=True, gate=True))
    inp = upload(w, [0])
    lens = inp.seq_lens
    L = lens[0]
    bud = sas.Budget(frac_num=1, frac_den=4, sink=True, gate=True)
    reps = sas.block_reps(inp.K, lens, w.block)
    scores = sas.block_scores(inp.Q, reps, lens, w.block, w.hkv, L, q_start=[0])
    idx, nsel, gate = sas.topk_select(scores, lens, w.block, w.hq, w.hkv, w.d, sas.SAS_BF16, L, bud, tq=w.tq,
                                      q_start=[0])
    O = torch.empty_like(inp.Q)
    lse = torch.empty(inp.Q.shape[:3], dtype=torch.float32, device="cuda")
    gen = torch.Generator(device="cpu").manual_seed(5)
    dO = torch.randn(inp.Q.shape, generator=gen).to(torch.bfloat16).cuda()
    f32 = dict(dtype=torch.float32, device="cuda")
    grads = (torch.empty(inp.Q.shape, **f32), torch.zeros(inp.K.shape, **f32), torch.zeros(inp.K.shape, **f32),
             torch.empty(idx.shape, **f32), torch.empty(idx.shape, **f32))
    need = sas.prefill_backward_workspace_bytes(1, w.hq, w.hkv, w.d, w.block, L, lens, w.tq, w.sel, idx.shape[1],
                                                True)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def step():
        sas.sparse_prefill(inp.Q, inp.K, inp.V, lens, w.block, [0], idx, nsel, gate, O=O, lse=lse)
        sas.sparse_prefill_backward(inp.Q, inp.K, inp.V, O, dO, lens, w.block, [0], idx, nsel, gate,
                                    workspace=ws, grads=grads, lse=lse)

    step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in grads]
    g = _capture(step)
    for r in range(3):
        for x in grads:
            x.fill_(float("nan"))
        grads[1].zero_()
        grads[2].zero_()
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, x, y in zip(("dQ", "dK", "dV", "dgate", "dscore"), grads, ref):
            assert torch.equal(x, y), f"replay {r}: {name} differs"


@pytest.mark.parametrize("sel", ["group", "head"])
def test_decode_loop_with_device_lengths_from_one_graph(sel):
    """A decode loop whose step -- pool the current block again, fused scores + top-k, attention -- is
    captured ONCE with the lengths in device memory and replayed while every sequence grows by one
    token per step (lengths cross block boundaries: a block fills up, a new one opens with one token).
    Between replays, outside the graph, the new token's K/V and the step's queries are written and the
    device lengths incremented.  Each replay must match the oracle at the new lengths (reps, lists under
    the tie rule, outputs to the bf16 bars) and the same step run eagerly with host lengths, bit for bit."""
    from oracle import sas_oracle as orc
    from workloads.gen import round_bf16
    from gpu_harness import list_matches, BF16_MAX_ABS, BF16_MEAN_ABS, say
    lens = [1000, 127, 4095, 63]
    steps, B, hq, hkv, d, blk = 4, 4, 8, 2, 128, 64
    Lmax = 4200
    rng = np.random.default_rng(53 if sel == "group" else 59)
    K = round_bf16(rng.standard_normal((B, hkv, Lmax, d), dtype=np.float32))
    V = round_bf16(rng.standard_normal((B, hkv, Lmax, d), dtype=np.float32))
    Qs = round_bf16(rng.standard_normal((steps, B, hq, d), dtype=np.float32))
    Kd = torch.zeros((B, hkv, Lmax, d), dtype=torch.bfloat16, device="cuda")
    Vd = torch.zeros_like(Kd)
    for b, L in enumerate(lens):
        Kd[b, :, :L] = torch.from_numpy(K[b, :, :L]).to(torch.bfloat16).cuda()
        Vd[b, :, :L] = torch.from_numpy(V[b, :, :L]).to(torch.bfloat16).cuda()
    Qd = torch.zeros((B, hq, d), dtype=torch.bfloat16, device="cuda")
    lens_dev = torch.tensor(lens, dtype=torch.int32, device="cuda")
    bud = sas.Budget(k_fixed=0, frac_num=1, frac_den=20, count_current=1, sink=True, gate=True) if sel == "head" \
        else sas.Budget(k_fixed=4, sink=True, gate=True)
    kcap = sas.required_kcap(B, hq, hkv, d, blk, sas.SAS_BF16, Lmax, [Lmax] * B, 1, None, bud)
    S = hq if sel == "head" else hkv
    nbm = -(-Lmax // blk)
    reps = torch.zeros((B, hkv, nbm, d), dtype=torch.float32, device="cuda")
    sas.block_reps(Kd, lens, blk, reps=reps)
    scores = torch.full((B * S, nbm), float("-inf"), dtype=torch.float32, device="cuda")
    idx = torch.empty((B * S, kcap), dtype=torch.int32, device="cuda")
    nsel = torch.empty((B * S,), dtype=torch.int32, device="cuda")
    gate = torch.empty((B * S, kcap), dtype=torch.float32, device="cuda")
    O = torch.empty_like(Qd)
    sel_ws = torch.zeros(sas.select_decode_workspace_bytes(B, hq, hkv, d, blk, sas.SAS_BF16, Lmax, [Lmax] * B),
                         dtype=torch.uint8, device="cuda")
    dec_ws = torch.zeros(sas.decode_workspace_bytes(B, hq, hkv, d, blk, sas.SAS_BF16, Lmax, [Lmax] * B, sel, kcap,
                                                    False), dtype=torch.uint8, device="cuda")

    def step():
        sas.block_reps(Kd, lens_dev, blk, reps=reps, current_block=True)
        sas.select_decode(Qd, reps, lens_dev, blk, hkv, Lmax, bud, sel_mode=sel, kcap=kcap, scores=scores, idx=idx,
                          nsel=nsel, gate=gate, workspace=sel_ws)
        sas.sparse_decode(Qd, Kd, Vd, lens_dev, blk, idx, nsel, gate, sel_mode=sel, O=O, workspace=dec_ws)

    # capture at the starting lengths (the capture's warm-up call pools the current blocks again,
    # which leaves reps unchanged)
    Qd.copy_(torch.from_numpy(Qs[0]).to(torch.bfloat16))
    g = _capture(step)
    for s in range(steps):
        for b in range(B):
            L = lens[b]
            Kd[b, :, L] = torch.from_numpy(K[b, :, L]).to(torch.bfloat16).cuda()
            Vd[b, :, L] = torch.from_numpy(V[b, :, L]).to(torch.bfloat16).cuda()
        lens = [L + 1 for L in lens]
        lens_dev.copy_(torch.tensor(lens, dtype=torch.int32))
        Qd.copy_(torch.from_numpy(Qs[s]).to(torch.bfloat16))
        g.replay()
        torch.cuda.synchronize()
        r_idx, r_nsel, r_O, r_reps = idx.clone(), nsel.clone(), O.clone(), reps.clone()
        # the same step eagerly, with host lengths
        full = sas.block_reps(Kd, lens, blk, reps=torch.full_like(reps, float("nan")))
        _, e_idx, e_nsel, e_gate = sas.select_decode(Qd, full, lens, blk, hkv, Lmax, bud, sel_mode=sel, kcap=kcap)
        e_O = sas.sparse_decode(Qd, Kd, Vd, lens, blk, e_idx, e_nsel, e_gate, sel_mode=sel)
        torch.cuda.synchronize()
        for b, L in enumerate(lens):
            nb = -(-L // blk)
            assert torch.equal(r_reps[b, :, :nb], full[b, :, :nb]), f"step {s}: reps of sequence {b} differ"
        assert torch.equal(r_nsel, e_nsel) and torch.equal(r_idx, e_idx), f"step {s}: lists differ from eager"
        assert torch.equal(r_O, e_O), f"step {s}: outputs differ from the eager host-length step"
        idx_h, nsel_h, O_h = r_idx.cpu().numpy(), r_nsel.cpu().numpy(), r_O.float().cpu().numpy()
        err_sum, err_n = 0.0, 0
        for b, L in enumerate(lens):
            kw = dict(frac_num=1, frac_den=20, count_current=1) if sel == "head" else dict(k_fixed=4)
            r = orc.run_sequence(Qs[s][b][:, None, :], K[b], V[b], L, L - 1, blk, sel, sink=True, gate=True, **kw)
            explicit = {}
            for un in r.units:
                u = b * S + un.sel_head
                got = [int(x) for x in idx_h[u, :nsel_h[u]]]
                ok, band, why = list_matches(un.sel, got, un.scores, un.c, un.k, True)
                assert ok, f"step {s}, sequence {b}, unit {un.sel_head}: {why}"
                if band:
                    explicit[(un.sel_head, un.c)] = (got, orc.gate_values(un.scores, got))
            if explicit:
                r = orc.run_sequence(Qs[s][b][:, None, :], K[b], V[b], L, L - 1, blk, sel, sink=True, gate=True,
                                     explicit=explicit, **kw)
            diff = np.abs(O_h[b] - r.O[:, 0, :])
            assert diff.max() <= BF16_MAX_ABS, f"step {s}, sequence {b}: max-abs {diff.max():.3e}"
            err_sum += float(diff.sum())
            err_n += diff.size
        assert err_sum / err_n <= BF16_MEAN_ABS
        say(f"[graph-loop {sel}] replay {s}: lengths {lens} match the oracle and the eager host-length step")
