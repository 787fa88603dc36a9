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
