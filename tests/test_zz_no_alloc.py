"""sas_sparse_decode_noalloc (decode with the library's static scratch array) against sas_sparse_decode
(decode with a caller workspace), through the C ABI.

Both run the same kernels on the same lists, so the outputs must agree bit for bit (stricter than the
bf16 output bar).  Calls in a row share the array: a large call, then a smaller one (fewer sequences
and units, shorter contexts), then per-head units with a gate, then gist mode; each is compared with
the workspace entry point on the same inputs.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from workloads import Workload  # noqa: E402
from workloads.device import upload  # noqa: E402

from gpu_harness import budget_of, say  # noqa: E402
import top_block_sparse_gist_amd as sas  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sas.load()
    yield


def _compare(w, seqs, gist=False):
    inp = upload(w, seqs, gist=gist)
    lens, Lmax = inp.seq_lens, inp.K.shape[2]
    budget = budget_of(w)
    reps = inp.gist_k if gist else sas.block_reps(inp.K, lens, w.block)
    _, idx, nsel, gate = sas.select_decode(inp.Q, reps, lens, w.block, w.hkv, Lmax, budget, sel_mode=w.sel, gist=gist)
    gk, gv = (inp.gist_k, inp.gist_v) if gist else (None, None)
    ref = sas.sparse_decode(inp.Q, inp.K, inp.V, lens, w.block, idx, nsel, gate, sel_mode=w.sel, gist_k=gk, gist_v=gv)
    got = torch.full_like(ref, float("nan"))
    sas.sparse_decode_noalloc(inp.Q, inp.K, inp.V, lens, w.block, idx, nsel, gate, sel_mode=w.sel, gist_k=gk,
                              gist_v=gv, O=got)
    torch.cuda.synchronize()
    need = sas.decode_workspace_bytes(len(lens), w.hq, w.hkv, w.d, w.block, sas.SAS_BF16, Lmax, lens, w.sel,
                                      idx.shape[1], gist)
    say(f"[noalloc] {w.name}: {len(lens)} sequences, scratch {need} bytes, equal: {torch.equal(got, ref)}")
    assert torch.equal(got, ref), "the no-alloc decode differs from the workspace decode"
    return need


def test_noalloc_decode_equals_the_workspace_decode():
    big = Workload(2, mini=True)                                      # 8 x 4096 tokens, 32/8 heads
    n1 = _compare(big, list(range(big.batch)))
    small = Workload(2, overrides=dict(tag="na_small", seq_lens=[1000, 300], batch=2, hq=8, hkv=2, k_fixed=3,
                                       sink=True, gate=True, seq_len=None))
    n2 = _compare(small, [0, 1])
    assert n2 < n1
    head = Workload(2, overrides=dict(tag="na_head", seq_lens=[5000, 64, 2500], batch=3, hq=8, hkv=2, sel="head",
                                      k_fixed=0, frac_num=1, frac_den=20, count_current=1, gate=True, seq_len=None))
    _compare(head, [0, 1, 2])
    gist = Workload(4, overrides=dict(tag="na_gist", seq_len=9000, batch=2, hq=8, hkv=2, k_fixed=6))
    _compare(gist, [0, 1], gist=True)
    # the large call again after the smaller ones: the counters left by them are cleared
    _compare(big, list(range(big.batch)))


def test_noalloc_decode_refuses_calls_beyond_the_array():
    """A call whose scratch would exceed SAS_DECODE_NOALLOC_SCRATCH_BYTES is refused with
    SAS_ERR_WORKSPACE on the host, before anything is launched."""
    B, hq, hkv, d, blk, kcap = 64, 32, 8, 128, 64, 300
    lens = [64 * 20] * B
    need = sas.decode_workspace_bytes(B, hq, hkv, d, blk, sas.SAS_BF16, max(lens), lens, "head", kcap, False)
    assert need > sas._lib.SAS_DECODE_NOALLOC_SCRATCH_BYTES
    Q = torch.zeros((B, hq, d), dtype=torch.bfloat16, device="cuda")
    K = torch.empty((B, hkv, max(lens), d), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((B * hq, kcap), dtype=torch.int32, device="cuda")
    nsel = torch.zeros((B * hq,), dtype=torch.int32, device="cuda")
    with pytest.raises(sas.SasError) as ei:
        sas.sparse_decode_noalloc(Q, K, K, lens, blk, idx, nsel, None, sel_mode="head")
    assert ei.value.status == sas._lib.SAS_ERR_WORKSPACE
    assert "static array" in str(ei.value)
