"""The C ABI library loads, exports every declared symbol, and rejects invalid calls on the host.

These tests make no compute call: every call below fails host-side validation, which makes
no HIP call, so they run on a machine without a GPU.
"""
import ctypes as C
import os
import re

import pytest

from top_block_sparse_gist_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sas.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libsas.so not built")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sas_[a-z_0-9]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    lib = _lib.load()
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.EXPORTED)


def _problem(batch=2, hq=8, hkv=2, d=128, block=64, dtype=_lib.SAS_BF16, max_len=1000, lens=(1000, 700)):
    arr = _lib.i32x(lens)
    p = _lib.Problem(batch, hq, hkv, d, block, dtype, max_len, C.cast(arr, C.POINTER(C.c_int32)))
    return p, arr


FAKE = C.c_void_p(0x10000)   # 16-byte aligned non-NULL; never dereferenced (validation fails first)


def _reps(lib, p, **kw):
    ks = _lib.i64x([8 * 1000 * 128, 1000 * 128, 128])
    rs = _lib.i64x([2 * 16 * 128, 16 * 128, 128])
    return lib.sas_block_reps(C.byref(p), kw.get("K", FAKE), ks, kw.get("reps", FAKE), rs, None)


def test_reps_validation_codes():
    lib = _lib.load()
    p, a = _problem()
    assert lib.sas_block_reps(None, FAKE, _lib.i64x([1, 1, 1]), FAKE, _lib.i64x([1, 1, 1]), None) == _lib.SAS_ERR_NULL
    assert _reps(lib, p, K=None) == _lib.SAS_ERR_NULL
    p2, a2 = _problem(d=96)
    assert _reps(lib, p2) == _lib.SAS_ERR_UNSUPPORTED
    p3, a3 = _problem(block=32)
    assert _reps(lib, p3) == _lib.SAS_ERR_UNSUPPORTED
    p4, a4 = _problem(hq=6, hkv=4)
    assert _reps(lib, p4) == _lib.SAS_ERR_SHAPE
    p5, a5 = _problem(lens=(1001, 5))
    assert _reps(lib, p5) == _lib.SAS_ERR_SHAPE
    assert b"seq_lens[0]" in lib.sas_last_error()
    p6, a6 = _problem(batch=65, lens=[10] * 65)
    assert _reps(lib, p6) == _lib.SAS_ERR_UNSUPPORTED
    p7, a7 = _problem(dtype=7)
    assert _reps(lib, p7) == _lib.SAS_ERR_UNSUPPORTED
    # misaligned pointer
    assert _reps(lib, p, K=C.c_void_p(0x10002)) == _lib.SAS_ERR_SHAPE


def test_reps_update_validation_codes():
    """The incremental form validates like the full one, plus its per-sequence first block."""
    lib = _lib.load()
    p, a = _problem()  # lengths 1000 and 700: 16 and 11 blocks
    ks = _lib.i64x([8 * 1000 * 128, 1000 * 128, 128])
    rs = _lib.i64x([2 * 16 * 128, 16 * 128, 128])

    def upd(first, K=FAKE):
        fb = None if first is None else _lib.i32x(first)
        return lib.sas_block_reps_update(C.byref(p), K, ks, FAKE, rs, fb, None)

    assert upd(None) == _lib.SAS_ERR_NULL
    assert upd([15, 10], K=None) == _lib.SAS_ERR_NULL
    assert upd([-1, 0]) == _lib.SAS_ERR_SHAPE
    assert upd([16, 12]) == _lib.SAS_ERR_SHAPE
    assert b"first_block[1] = 12" in lib.sas_last_error()
    assert upd([15, 10], K=C.c_void_p(0x10002)) == _lib.SAS_ERR_SHAPE
    p2, a2 = _problem(d=96)
    assert lib.sas_block_reps_update(C.byref(p2), FAKE, ks, FAKE, rs, _lib.i32x([0, 0]), None) == \
        _lib.SAS_ERR_UNSUPPORTED


def test_num_qblocks_and_required_kcap():
    lib = _lib.load()
    assert lib.sas_num_qblocks(1, 64) == 1
    assert lib.sas_num_qblocks(64, 64) == 2
    assert lib.sas_num_qblocks(4096, 64) == 65
    assert lib.sas_num_qblocks(0, 64) < 0
    p, a = _problem(lens=(32768, 32768), max_len=32768)
    b16 = _lib.Budget(16, 0, 0, 0, 0, 0)
    assert lib.sas_required_kcap(C.byref(p), 1, None, C.byref(b16)) == 17
    # ceil(c/8) + sink + current over the full prefill of 256 blocks of 128 (c = 255 -> 32 + 2)
    p1, a1 = _problem(batch=1, hq=28, hkv=4, block=128, lens=(32768,), max_len=32768)
    b8 = _lib.Budget(0, 1, 8, 0, 1, 1)
    qs = _lib.i32x([0])
    assert lib.sas_required_kcap(C.byref(p1), 32768, qs, C.byref(b8)) == 34
    # 5% of (c+1) + current at c = 2047 -> 103 + 1
    p2, a2 = _problem(batch=1, lens=(131072,), max_len=131072)
    b20 = _lib.Budget(0, 1, 20, 1, 0, 1)
    assert lib.sas_required_kcap(C.byref(p2), 1, None, C.byref(b20)) == 104
    bad = _lib.Budget(-1, 0, 0, 0, 0, 0)
    assert lib.sas_required_kcap(C.byref(p2), 1, None, C.byref(bad)) == _lib.SAS_ERR_SHAPE


def test_scores_topk_validation_codes():
    lib = _lib.load()
    p, a = _problem()
    qs3 = _lib.i64x([8 * 100 * 128, 100 * 128, 128])
    rs = _lib.i64x([2 * 16 * 128, 16 * 128, 128])
    # decode needs tq == 1
    assert lib.sas_block_scores(C.byref(p), FAKE, qs3, 5, None, FAKE, 0, rs, 0, 0.0, FAKE, 16, None, 0,
                                None) == _lib.SAS_ERR_SHAPE
    # rows beyond the sequence
    qst = _lib.i32x([950, 0])
    assert lib.sas_block_scores(C.byref(p), FAKE, qs3, 100, qst, FAKE, 0, rs, 0, 0.0, FAKE, 16, FAKE, 1 << 20,
                                None) == _lib.SAS_ERR_SHAPE
    # scores_ld too small (needs 16 blocks)
    assert lib.sas_block_scores(C.byref(p), FAKE, qs3, 1, None, FAKE, 0, rs, 0, 0.0, FAKE, 15, None, 0,
                                None) == _lib.SAS_ERR_SHAPE
    # prefill workspace too small
    qs0 = _lib.i32x([0, 0])
    assert lib.sas_block_scores(C.byref(p), FAKE, qs3, 100, qs0, FAKE, 0, rs, 0, 0.0, FAKE, 16, FAKE, 16,
                                None) == _lib.SAS_ERR_WORKSPACE
    # bad selection mode / negative scale
    assert lib.sas_block_scores(C.byref(p), FAKE, qs3, 1, None, FAKE, 0, rs, 7, 0.0, FAKE, 16, None, 0,
                                None) == _lib.SAS_ERR_SHAPE
    assert lib.sas_block_scores(C.byref(p), FAKE, qs3, 1, None, FAKE, 0, rs, 0, -1.0, FAKE, 16, None, 0,
                                None) == _lib.SAS_ERR_SHAPE
    b = _lib.Budget(4, 0, 0, 0, 0, 1)
    # kcap below the required 5, gate requested without a gate buffer
    assert lib.sas_topk_select(C.byref(p), FAKE, 16, 1, None, 0, C.byref(b), 4, FAKE, FAKE, FAKE,
                               None) == _lib.SAS_ERR_SHAPE
    assert lib.sas_topk_select(C.byref(p), FAKE, 16, 1, None, 0, C.byref(b), 5, FAKE, FAKE, None,
                               None) == _lib.SAS_ERR_NULL
    assert lib.sas_topk_select(C.byref(p), FAKE, 16, 1, None, 0, None, 5, FAKE, FAKE, FAKE,
                               None) == _lib.SAS_ERR_NULL


def test_attention_validation_codes():
    lib = _lib.load()
    p, a = _problem()
    qs3 = _lib.i64x([8 * 100 * 128, 100 * 128, 128])
    kvs = _lib.i64x([2 * 1000 * 128, 1000 * 128, 128])
    qs2 = _lib.i64x([8 * 128, 128])
    # prefill without q_start
    assert lib.sas_sparse_prefill(C.byref(p), FAKE, qs3, FAKE, FAKE, kvs, 100, None, 0, FAKE, FAKE, None, 8, 0.0,
                                  FAKE, qs3, None) == _lib.SAS_ERR_NULL
    # odd row stride for bf16 (not a multiple of 8 elements)
    bad = _lib.i64x([8 * 100 * 128, 100 * 128, 130])
    qs0 = _lib.i32x([0, 0])
    assert lib.sas_sparse_prefill(C.byref(p), FAKE, bad, FAKE, FAKE, kvs, 100, qs0, 0, FAKE, FAKE, None, 8, 0.0,
                                  FAKE, qs3, None) == _lib.SAS_ERR_SHAPE
    # bf16 K/V slab of one (sequence, KV head) beyond 32-bit byte offsets: 1000 rows at a 2^22-element stride
    huge = _lib.i64x([1 << 40, 1 << 32, 1 << 22])
    assert lib.sas_sparse_prefill(C.byref(p), FAKE, qs3, FAKE, FAKE, huge, 100, qs0, 0, FAKE, FAKE, None, 8, 0.0,
                                  FAKE, qs3, None) == _lib.SAS_ERR_UNSUPPORTED
    # decode: gist with a gate is not defined; half a gist pair is an error; workspace too small
    gs = _lib.i64x([2 * 15 * 128, 15 * 128, 128])
    assert lib.sas_sparse_decode(C.byref(p), FAKE, qs2, FAKE, FAKE, kvs, FAKE, FAKE, gs, 0, FAKE, FAKE, FAKE, 8, 0.0,
                                 FAKE, qs2, FAKE, 1 << 30, None) == _lib.SAS_ERR_UNSUPPORTED
    assert lib.sas_sparse_decode(C.byref(p), FAKE, qs2, FAKE, FAKE, kvs, FAKE, None, gs, 0, FAKE, FAKE, None, 8, 0.0,
                                 FAKE, qs2, FAKE, 1 << 30, None) == _lib.SAS_ERR_NULL
    need = lib.sas_sparse_decode_workspace(C.byref(p), 0, 8, 0)
    assert need > 0
    assert lib.sas_sparse_decode(C.byref(p), FAKE, qs2, FAKE, FAKE, kvs, None, None, None, 0, FAKE, FAKE, None, 8,
                                 0.0, FAKE, qs2, FAKE, need - 1, None) == _lib.SAS_ERR_WORKSPACE
    # a list capacity whose split-K records per unit exceed what the merge can stage in LDS:
    # 16 heads per KV head at d 128 hold 383 records; kcap 4000 at two tiles per wave needs 500
    p16, a16 = _problem(hq=32, hkv=2)
    need16 = lib.sas_sparse_decode_workspace(C.byref(p16), 0, 4000, 0)
    assert lib.sas_sparse_decode(C.byref(p16), FAKE, qs2, FAKE, FAKE, kvs, None, None, None, 0, FAKE, FAKE, None,
                                 4000, 0.0, FAKE, qs2, FAKE, need16, None) == _lib.SAS_ERR_UNSUPPORTED
    assert b"merge holds 383" in lib.sas_last_error()
    need_ok = lib.sas_sparse_decode_workspace(C.byref(p16), 0, 3000, 0)
    assert need_ok > 0  # 3000 entries: 375 records, within the merge
    # units of one head (per-head lists) run one tile per wave and stage V in half tiles: the merge
    # holds 2729 records of 4 tiles, so 10,916 entries of 64 keys fit and 10,917 do not
    ph, aph = _problem()
    need_ph = lib.sas_sparse_decode_workspace(C.byref(ph), _lib.SAS_SEL_HEAD, 10917, 0)
    assert lib.sas_sparse_decode(C.byref(ph), FAKE, qs2, FAKE, FAKE, kvs, None, None, None, _lib.SAS_SEL_HEAD, FAKE,
                                 FAKE, None, 10917, 0.0, FAKE, qs2, FAKE, need_ph, None) == _lib.SAS_ERR_UNSUPPORTED
    assert b"needs 2730 split-K records per unit; the merge holds 2729" in lib.sas_last_error()
    # more than 16 query heads per KV head in per-group decode
    p9, a9 = _problem(hq=34, hkv=2)
    need9 = lib.sas_sparse_decode_workspace(C.byref(p9), 0, 8, 0)
    assert lib.sas_sparse_decode(C.byref(p9), FAKE, qs2, FAKE, FAKE, kvs, None, None, None, 0, FAKE, FAKE, None, 8,
                                 0.0, FAKE, qs2, FAKE, need9, None) == _lib.SAS_ERR_UNSUPPORTED


def test_hssa_validation_codes():
    """Two-level gist selection and attention: host validation (no HIP call)."""
    lib = _lib.load()
    p, a = _problem(lens=(1000, 700))
    q2 = _lib.i64x([8 * 128, 128])
    s3 = _lib.i64x([2 * 16 * 128, 16 * 128, 128])
    ws = C.c_size_t(1 << 20)

    # max_len 1000, blk 64: current chunk <= 15, so 3 complete groups of 4 chunks
    def sel(M=4, k1=2, k2=3, kcap=8, gcap=4, ptr=FAKE, prob=p, sm=_lib.SAS_SEL_GROUP):
        return lib.sas_hssa_select_decode(C.byref(prob), ptr, q2, FAKE, s3, FAKE, s3, M, sm, k1, k2, 0.0, kcap, gcap,
                                          FAKE, FAKE, FAKE, FAKE, FAKE, ws, None)

    assert sel(ptr=None) == _lib.SAS_ERR_NULL
    assert sel(M=3) == _lib.SAS_ERR_UNSUPPORTED
    assert sel(M=65) == _lib.SAS_ERR_UNSUPPORTED
    assert sel(k1=-1) == _lib.SAS_ERR_SHAPE
    assert sel(gcap=2) == _lib.SAS_ERR_SHAPE          # 2 opened + the trailing group
    assert b"gcap 2 < 3" in lib.sas_last_error()
    assert sel(k1=9, gcap=3) == _lib.SAS_ERR_SHAPE    # k1 capped at the 3 groups: 4 entries
    assert sel(kcap=3) == _lib.SAS_ERR_SHAPE          # 3 expanded + the current chunk
    assert sel(sm=7) == _lib.SAS_ERR_SHAPE
    pf, af = _problem(dtype=_lib.SAS_F32)
    assert sel(prob=pf) == _lib.SAS_ERR_UNSUPPORTED
    assert lib.sas_hssa_select_workspace(C.byref(p), _lib.SAS_SEL_GROUP, 8, 2) > 0
    assert lib.sas_hssa_select_workspace(C.byref(p), _lib.SAS_SEL_GROUP, 2, 2) == 0

    def dec(M=8, kcap=8, gcap=4, ptr=FAKE, wbytes=1 << 30):
        return lib.sas_hssa_decode(C.byref(p), FAKE, q2, FAKE, FAKE, s3, FAKE, FAKE, s3, ptr, FAKE, s3, M,
                                   _lib.SAS_SEL_GROUP, FAKE, FAKE, kcap, FAKE, gcap, 0.0, FAKE, q2, FAKE,
                                   C.c_size_t(wbytes), None)

    assert dec(ptr=None) == _lib.SAS_ERR_NULL
    assert dec(M=2) == _lib.SAS_ERR_UNSUPPORTED
    assert dec(gcap=0) == _lib.SAS_ERR_SHAPE
    assert dec(wbytes=16) == _lib.SAS_ERR_WORKSPACE
    need = lib.sas_hssa_decode_workspace(C.byref(p), _lib.SAS_SEL_GROUP, 8, 4, 8)
    assert need > 0 and dec(wbytes=need - 1) == _lib.SAS_ERR_WORKSPACE


def test_paged_validation_codes():
    lib = _lib.load()
    p, a = _problem(lens=(1000, 700))           # 16 and 11 blocks of 64
    ps = _lib.i64x([2 * 64 * 128, 64 * 128, 128])
    rs = _lib.i64x([2 * 16 * 128, 16 * 128, 128])

    def reps(table=FAKE, ld=16, pstride=ps):
        return lib.sas_block_reps_paged(C.byref(p), FAKE, pstride, table, ld, FAKE, rs, None, None)

    assert reps(table=None) == _lib.SAS_ERR_NULL
    assert reps(ld=15) == _lib.SAS_ERR_SHAPE
    assert b"table_ld 15 < 16" in lib.sas_last_error()
    assert reps(pstride=_lib.i64x([64 * 128, 64 * 128, 128])) == _lib.SAS_ERR_SHAPE   # two heads cannot fit
    q2 = _lib.i64x([8 * 128, 128])

    def dec(table=FAKE, ld=16, wbytes=1 << 30, prob=p):
        return lib.sas_sparse_decode_paged(C.byref(prob), FAKE, q2, FAKE, FAKE, ps, table, ld, _lib.SAS_SEL_GROUP,
                                           FAKE, FAKE, None, 8, 0.0, FAKE, q2, FAKE, C.c_size_t(wbytes), None)

    assert dec(table=None) == _lib.SAS_ERR_NULL
    assert dec(ld=3) == _lib.SAS_ERR_SHAPE
    assert dec(wbytes=8) == _lib.SAS_ERR_WORKSPACE
    pf, af = _problem(dtype=_lib.SAS_F32, lens=(1000, 700))
    assert dec(prob=pf) == _lib.SAS_ERR_UNSUPPORTED


def test_paged_prefill_validation_codes():
    lib = _lib.load()
    p, a = _problem(lens=(1000, 700))
    ps = _lib.i64x([2 * 64 * 128, 64 * 128, 128])
    q3 = _lib.i64x([8 * 1000 * 128, 1000 * 128, 128])
    qs = _lib.i32x([900, 600])

    def pf(table=FAKE, ld=16, tq=100, q_start=qs):
        return lib.sas_sparse_prefill_paged(C.byref(p), FAKE, q3, FAKE, FAKE, ps, table, ld, tq, q_start,
                                            _lib.SAS_SEL_GROUP, FAKE, FAKE, None, 8, 0.0, FAKE, q3, None)

    assert pf(table=None) == _lib.SAS_ERR_NULL
    assert pf(q_start=None) == _lib.SAS_ERR_NULL
    assert pf(ld=10) == _lib.SAS_ERR_SHAPE
    assert pf(tq=200) == _lib.SAS_ERR_SHAPE            # q_start + tq > L for the second sequence


def test_shared_budget_validation():
    lib = _lib.load()
    p, a = _problem(hq=16, hkv=2, lens=(5000, 700), max_len=5000)
    bad = _lib.Budget(4, 0, 0, 0, 0, 0, 0.0, 2)
    assert lib.sas_required_kcap(C.byref(p), 1, None, C.byref(bad)) == _lib.SAS_ERR_SHAPE
    both = _lib.Budget(4, 0, 0, 0, 0, 0, 0.5, 1)
    assert lib.sas_required_kcap(C.byref(p), 1, None, C.byref(both)) == _lib.SAS_ERR_UNSUPPORTED
    sh = _lib.Budget(4, 0, 0, 0, 1, 0, 0.0, 1)
    # 8 heads per KV head share 8 x 4: a list may hold min(32, candidates) + current + sink
    assert lib.sas_required_kcap(C.byref(p), 1, None, C.byref(sh)) == 32 + 2
    p2, a2 = _problem(hq=16, hkv=2, lens=(1000, 700))
    assert lib.sas_required_kcap(C.byref(p2), 1, None, C.byref(sh)) == 14 + 2   # capped: 14 candidates
    q2 = _lib.i64x([16 * 128, 128])
    r3 = _lib.i64x([2 * 16 * 128, 16 * 128, 128])
    ws = C.c_size_t(1 << 20)
    # the fused selection takes at most 4 heads per KV head when they share a budget
    assert lib.sas_select_decode(C.byref(p), FAKE, q2, FAKE, _lib.SAS_REPS_POOLED, r3, _lib.SAS_SEL_HEAD, 0.0,
                                 C.byref(sh), 40, FAKE, 16, FAKE, FAKE, None, FAKE, ws, None) == \
        _lib.SAS_ERR_UNSUPPORTED
    # per-group selection cannot share a budget
    assert lib.sas_select_decode(C.byref(p), FAKE, q2, FAKE, _lib.SAS_REPS_POOLED, r3, _lib.SAS_SEL_GROUP, 0.0,
                                 C.byref(sh), 40, FAKE, 16, FAKE, FAKE, None, FAKE, ws, None) == _lib.SAS_ERR_SHAPE


def test_prefill_backward_validation_codes():
    lib = _lib.load()
    p, a = _problem(lens=(1000, 700))
    kv = _lib.i64x([2 * 1000 * 128, 1000 * 128, 128])
    q3 = _lib.i64x([8 * 128 * 128, 128 * 128, 128])
    qs = _lib.i32x([872, 572])
    need = lib.sas_sparse_prefill_backward_workspace(C.byref(p), 128, _lib.SAS_SEL_GROUP, 8, 1)
    assert need > 0
    assert lib.sas_sparse_prefill_backward_workspace(C.byref(p), 128, _lib.SAS_SEL_GROUP, 40000, 1) == 0
    # the gate adds the partial sums and the entry positions
    assert lib.sas_sparse_prefill_backward_workspace(C.byref(p), 128, _lib.SAS_SEL_GROUP, 8, 0) < need

    def bw(gate=None, dgate=FAKE, ws=FAKE, wsb=None, q_start=qs, kcap=8, dQ=FAKE, prob=p, reps=None):
        return lib.sas_sparse_prefill_backward(C.byref(prob), FAKE, q3, FAKE, FAKE, kv, 128, q_start,
                                               _lib.SAS_SEL_GROUP, FAKE, FAKE, gate, kcap, 0.0, FAKE, FAKE, q3, None,
                                               dQ, q3, FAKE, FAKE, kv, dgate, FAKE, reps, kv, ws,
                                               need if wsb is None else wsb, None)

    assert bw(q_start=None) == _lib.SAS_ERR_NULL
    assert bw(dQ=None) == _lib.SAS_ERR_NULL
    assert bw(ws=None) == _lib.SAS_ERR_NULL
    assert bw(gate=FAKE, dgate=None) == _lib.SAS_ERR_NULL          # a gate needs dgate and dscore
    assert bw(reps=FAKE) == _lib.SAS_ERR_SHAPE                      # the selector's gradient needs a gate
    assert bw(kcap=0) == _lib.SAS_ERR_SHAPE
    assert bw(kcap=40000) == _lib.SAS_ERR_SHAPE
    assert bw(gate=FAKE, wsb=need - 1) == _lib.SAS_ERR_WORKSPACE
    pf, af = _problem(lens=(1000, 700), dtype=_lib.SAS_F32)
    assert bw(prob=pf) == _lib.SAS_ERR_UNSUPPORTED                  # bf16 only
    # the forward's log-sum-exp output exists on the bf16 path only
    assert lib.sas_sparse_prefill_lse(C.byref(pf), FAKE, q3, FAKE, FAKE, kv, 128, qs, _lib.SAS_SEL_GROUP, FAKE,
                                      FAKE, None, 8, 0.0, FAKE, q3, FAKE, None) == _lib.SAS_ERR_UNSUPPORTED
