"""Host-side arithmetic of the library that the GPU path depends on (CPU only, no compute call).

  * the dK/dV kernel of the backward splits a unit's flattened (head, row) index f into
    (f / rows, f % rows) with a 20-bit reciprocal multiply on 32-bit integers; it must be exact for
    every shape the host accepts (rows <= 128, at most 64 query heads per per-group unit);
  * the square-root budget (sas_budget.sqrt_num / sqrt_den) through sas_required_kcap, and the
    host's rejections of out-of-range budgets and of per-group backward units it cannot map.
"""
import ctypes as C
import math
import os

import numpy as np
import pytest

from top_block_sparse_gist_amd import _lib

needs_lib = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libsas.so not built")

FAKE = C.c_void_p(0x10000)   # 16-byte aligned non-NULL; never dereferenced (validation fails first)


def test_backward_row_split_is_exact_for_every_accepted_shape():
    """inv = ceil(2^20 / rows); ((f * inv) mod 2^32) >> 20 must equal f // rows for every flattened
    index f < rows * G, rows 1..128 and G 1..64 (the largest G the host accepts for per-group units;
    per-head units have f < rows)."""
    for rows in range(1, 129):
        inv = ((1 << 20) + rows - 1) // rows
        f = np.arange(rows * 64, dtype=np.uint64)
        got = ((f * np.uint64(inv)) & np.uint64(0xFFFFFFFF)) >> np.uint64(20)
        np.testing.assert_array_equal(got, f // np.uint64(rows), err_msg=f"rows {rows}")
    # one head more per unit and the split goes wrong for some row count: the host bound is tight enough
    bad = 0
    for rows in range(1, 129):
        inv = ((1 << 20) + rows - 1) // rows
        f = np.arange(rows * 80, dtype=np.uint64)
        got = ((f * np.uint64(inv)) & np.uint64(0xFFFFFFFF)) >> np.uint64(20)
        bad += int((got != f // np.uint64(rows)).any())
    assert bad > 0


def _problem(batch=1, hq=8, hkv=2, d=128, block=64, max_len=131072, lens=(131072,)):
    arr = _lib.i32x(lens)
    return _lib.Problem(batch, hq, hkv, d, block, _lib.SAS_BF16, max_len, C.cast(arr, C.POINTER(C.c_int32))), arr


@needs_lib
def test_required_kcap_with_the_square_root_budget():
    lib = _lib.load()
    p, a = _problem()
    # decode at c = 2047, n = c + 1 = 2048: ceil(8 sqrt(2048) / 5) = 73 blocks + the current one
    b = _lib.Budget(0, 0, 0, 1, 0, 1, 0.0, 0, 8, 5)
    assert lib.sas_required_kcap(C.byref(p), 1, None, C.byref(b)) == math.ceil(8 * math.sqrt(2048) / 5) + 1 == 74
    # the rule takes precedence over a fractional one given beside it
    b2 = _lib.Budget(0, 1, 20, 1, 0, 1, 0.0, 0, 8, 5)
    assert lib.sas_required_kcap(C.byref(p), 1, None, C.byref(b2)) == 74
    # a prefill of 4096 rows ending at the last block: the largest unit is the last one
    qs = _lib.i32x([131072 - 4096])
    b3 = _lib.Budget(0, 0, 0, 0, 1, 1, 0.0, 0, 1, 1)
    assert lib.sas_required_kcap(C.byref(p), 4096, qs, C.byref(b3)) == math.ceil(math.sqrt(2047)) + 2
    for bad in (_lib.Budget(0, 0, 0, 0, 0, 0, 0.0, 0, -1, 5), _lib.Budget(0, 0, 0, 0, 0, 0, 0.0, 0, 8, -5),
                _lib.Budget(0, 0, 0, 0, 0, 0, 0.0, 0, 70000, 5)):
        assert lib.sas_required_kcap(C.byref(p), 1, None, C.byref(bad)) == _lib.SAS_ERR_SHAPE


@needs_lib
def test_backward_rejects_per_group_units_beyond_the_row_split():
    lib = _lib.load()
    p, a = _problem(hq=130, hkv=2, lens=(1000,), max_len=1000)   # 65 query heads per KV head
    s3 = _lib.i64x([130 * 1000 * 128, 1000 * 128, 128])
    k3 = _lib.i64x([2 * 1000 * 128, 1000 * 128, 128])
    qs = _lib.i32x([0])
    r = lib.sas_sparse_prefill_backward(C.byref(p), FAKE, s3, FAKE, FAKE, k3, 1000, qs, _lib.SAS_SEL_GROUP, FAKE,
                                        FAKE, None, 4, 0.0, FAKE, FAKE, s3, None, FAKE, s3, FAKE, FAKE, k3, None,
                                        None, None, None, FAKE, 1 << 30, None)
    assert r == _lib.SAS_ERR_UNSUPPORTED
    assert b"per KV head" in lib.sas_last_error()


@needs_lib
def test_device_lengths_are_refused_where_the_host_needs_them():
    """seq_lens in device memory (seq_lens_device = 1) serve the decode loop's entry points only; the
    others refuse them before anything is launched, and a bad flag is a shape error."""
    lib = _lib.load()
    lens = _lib.i32x([4096, 4096])
    dev = _lib.Problem(2, 8, 2, 128, 64, _lib.SAS_BF16, 4096, C.cast(lens, C.POINTER(C.c_int32)), 1)
    bad = _lib.Problem(2, 8, 2, 128, 64, _lib.SAS_BF16, 4096, C.cast(lens, C.POINTER(C.c_int32)), 2)
    b = _lib.Budget(4, 0, 0, 0, 0, 0)
    assert lib.sas_required_kcap(C.byref(dev), 1, None, C.byref(b)) == _lib.SAS_ERR_UNSUPPORTED
    assert lib.sas_required_kcap(C.byref(bad), 1, None, C.byref(b)) == _lib.SAS_ERR_SHAPE
    qs3 = _lib.i64x([8 * 4096 * 128, 4096 * 128, 128])
    rs = _lib.i64x([2 * 64 * 128, 64 * 128, 128])
    r = lib.sas_block_scores(C.byref(dev), FAKE, qs3, 1, None, FAKE, _lib.SAS_REPS_POOLED, rs, _lib.SAS_SEL_GROUP,
                             0.0, FAKE, 64, None, 0, None)
    assert r == _lib.SAS_ERR_UNSUPPORTED
    assert b"host memory" in lib.sas_last_error()
    r = lib.sas_topk_select(C.byref(dev), FAKE, 64, 1, None, _lib.SAS_SEL_GROUP, C.byref(b), 8, FAKE, FAKE, None, None)
    assert r == _lib.SAS_ERR_UNSUPPORTED
    # the incremental reps of a decode loop: the block to pool is found on the device, so no first_block
    ks = _lib.i64x([2 * 4096 * 128, 4096 * 128, 128])
    first = _lib.i32x([63, 63])
    r = lib.sas_block_reps_update(C.byref(dev), FAKE, ks, FAKE, rs, first, None)
    assert r == _lib.SAS_ERR_SHAPE
    assert b"first_block must be NULL" in lib.sas_last_error()
