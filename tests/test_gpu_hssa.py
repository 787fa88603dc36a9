"""GPU parity of the two-level gist selection (meta-gists) and its attention against the oracle.

Lists: the opened groups must equal the oracle's; the expanded chunks follow the tie rule of
the one-level selection.  Outputs: the bf16 tolerances.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from workloads import Workload  # noqa: E402
from workloads.device import upload  # noqa: E402

from gpu_harness import list_matches, say, BF16_MAX_ABS, BF16_MEAN_ABS  # noqa: E402
import top_block_sparse_gist_amd as sas  # noqa: E402
from oracle import sas_oracle as orc  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sas.load()
    yield


def run_hssa_case(w: Workload, seqs, unit_sample=None, seed=0):
    M, k1, k2 = w.spec["group_chunks"], w.spec["k_groups"], w.k_fixed
    inp = upload(w, seqs, gist=True, meta=True)
    lens = inp.seq_lens
    Lmax = inp.K.shape[2]
    say(f"[hssa] {w.name} seqs={seqs} lens={lens} M={M} k1={k1} k2={k2} sel={w.sel}")
    idx, nsel, gidx, gsel = sas.hssa_select_decode(inp.Q, inp.gist_k, inp.meta_k, lens, w.block, w.hkv, Lmax, M,
                                                   k1, k2, sel_mode=w.sel)
    O = sas.hssa_decode(inp.Q, inp.K, inp.V, lens, w.block, inp.gist_k, inp.gist_v, inp.meta_k, inp.meta_v, M,
                        idx, nsel, gidx, sel_mode=w.sel)
    torch.cuda.synchronize()
    idx_h, nsel_h = idx.cpu().numpy(), nsel.cpu().numpy()
    gidx_h, gsel_h = gidx.cpu().numpy(), gsel.cpu().numpy()
    O_h = O.float().cpu().numpy()
    S = w.hq if w.sel == "head" else w.hkv
    rng = np.random.default_rng(seed)
    err_max, err_sum, err_n, band_hits = 0.0, 0.0, 0, 0
    for i, bseq in enumerate(seqs):
        L = lens[i]
        q = w.q(bseq)
        K, V = w.kv(bseq)
        gk, gv = w.gist(bseq)
        mk, mv = w.meta(bseq)
        units, _ = orc.hssa_decode_sequence(q, K, V, L, w.block, w.sel, M, k1, k2, gk, gv, mk, mv, attend=False)
        keep = range(len(units)) if unit_sample is None else sorted(rng.choice(len(units), unit_sample, replace=False))
        explicit = {}
        for ui in keep:
            un = units[ui]
            u = i * S + un.sel_head
            groups = [int(x) for x in gidx_h[u, :gsel_h[u]]]
            assert groups == un.groups, f"sequence {bseq}, unit {un.sel_head}: groups {groups} != {un.groups}"
            assert (gidx_h[u, gsel_h[u]:] == -1).all()
            got = [int(x) for x in idx_h[u, :nsel_h[u]]]
            ok, band, why = list_matches(un.sel, got, un.gist_scores, un.c, un.k2, False)
            assert ok, f"sequence {bseq}, unit {un.sel_head}: {why}"
            assert (idx_h[u, nsel_h[u]:] == -1).all()
            if band:
                band_hits += 1
                explicit[un.sel_head] = (groups, got)
        kept = {units[ui].sel_head for ui in keep}
        _, Oref = orc.hssa_decode_sequence(q, K, V, L, w.block, w.sel, M, k1, k2, gk, gv, mk, mv,
                                           explicit=explicit)
        for un in units:
            if un.sel_head not in kept:
                continue
            for h in un.heads:
                d = np.abs(O_h[i, h] - Oref[h, 0])
                assert np.isfinite(O_h[i, h]).all()
                err_max = max(err_max, float(d.max()))
                err_sum += float(d.sum())
                err_n += d.size
    mean = err_sum / max(1, err_n)
    say(f"[hssa] ok max_abs={err_max:.3e} mean_abs={mean:.3e} tie_band={band_hits}")
    assert err_max <= BF16_MAX_ABS, f"max-abs {err_max:.3e}"
    assert mean <= BF16_MEAN_ABS, f"mean-abs {mean:.3e}"


def test_hssa_mini():
    w = Workload(6, mini=True)
    run_hssa_case(w, list(range(w.batch)))


def test_hssa_full_sampled():
    """The benchmark's shape: 128K tokens, 64 groups of 32 chunks, 8 opened, 104 chunks expanded.
    Every unit (KV head) of two of the four sequences: the oracle forms all of a sequence's units
    anyway."""
    w = Workload(6)
    run_hssa_case(w, [0, 1])


def test_hssa_per_head_ragged():
    """Per-head units, ragged lengths: no complete group (c < M), c a multiple of M (empty trailing
    group), L a multiple of the chunk, k1 above the group count."""
    w = Workload(6, overrides=dict(tag="ragged", seq_lens=[300, 64 * 40 + 1, 64 * 141, 4100], seq_len=None, batch=4,
                                   sel="head", hq=8, hkv=2, group_chunks=8, k_groups=3, k_fixed=9))
    run_hssa_case(w, list(range(4)))


def test_hssa_all_groups_opened_and_d64():
    w = Workload(6, overrides=dict(tag="d64", seq_len=6000, batch=2, hq=8, hkv=2, d=64, group_chunks=16,
                                   k_groups=10, k_fixed=20))
    run_hssa_case(w, [0, 1])


def test_hssa_many_candidates_four_wave_topk():
    """(k1 + 1) * M > 512 candidate chunks: the level-2 top-k runs on the four waves together."""
    w = Workload(6, overrides=dict(tag="wide", seq_len=70000, batch=2, hq=8, hkv=2, group_chunks=64, k_groups=12,
                                   k_fixed=40))
    run_hssa_case(w, [0, 1])
