"""The library's C++ block manager (host code, no GPU) against the oracle's,
and pa_copy_blocks' host validation."""
import ctypes

import numpy as np
import pytest

import oracle
import paged_kv_cache_443_amd as pa
from paged_kv_cache_443_amd import _lib
from paged_kv_cache_443_amd._lib import (PA_BF16, PA_ERR_BAD_SHAPE, PA_ERR_INVALID_BLOCK, PA_ERR_MISALIGNED,
                                         PA_ERR_NULL_PTR, PA_ERR_OUT_OF_BLOCKS, PA_OK, PaKvCache)


def test_pages_examples():
    bm = pa.BlockManager(64, 16)
    tables = []
    for L in (100, 50, 200):
        t = []
        for pos in range(L):
            slot, copies = bm.append_slot(t, pos)
            assert copies == [] and slot == t[pos // 16] * 16 + pos % 16
        tables.append(t)
    assert [len(t) for t in tables] == [7, 4, 13] and bm.num_free() == 64 - 24
    # beams of the block-pool figure
    bm = pa.BlockManager(16, 16)
    beam1 = []
    for pos in range(40):
        bm.append_slot(beam1, pos)
    beam2 = bm.fork(beam1)
    slot, copies = bm.append_slot(beam2, 40)
    assert beam2[:2] == beam1[:2] and copies == [(beam1[2], beam2[2])] and slot == beam2[2] * 16 + 8
    assert [bm.refcount(b) for b in beam1] == [2, 2, 1]


def test_matches_the_oracle_on_random_operations():
    """Same operations on both managers give the same slots, copies, tables
    and reference counts (allocation is lowest-id-first in both)."""
    rng = np.random.default_rng(42)
    N = 200
    ours, ref = pa.BlockManager(N, 16), oracle.BlockManager(N, 16)
    t_ours, t_ref, lens = [], [], []
    for step in range(4000):
        op = int(rng.integers(0, 12))
        if op == 0 and t_ours:
            i = int(rng.integers(len(t_ours)))
            t_ours.append(ours.fork(t_ours[i]))
            t_ref.append(ref.fork(t_ref[i]))
            lens.append(lens[i])
        elif op == 1 and t_ours:
            i = int(rng.integers(len(t_ours)))
            ours.free(t_ours.pop(i))
            ref.free(t_ref.pop(i))
            lens.pop(i)
        elif op == 2 or not t_ours:
            t_ours.append([])
            t_ref.append([])
            lens.append(0)
        else:
            i = int(rng.integers(len(t_ours)))
            try:
                want = ref.append_slot(t_ref[i], lens[i])
            except oracle.OutOfBlocks:
                with pytest.raises(pa.OutOfBlocks):
                    ours.append_slot(t_ours[i], lens[i])
                continue
            got = ours.append_slot(t_ours[i], lens[i])
            assert got == want, step
            lens[i] += 1
        assert t_ours == t_ref, step
        assert ours.num_free() == ref.num_free(), step
    assert [ours.refcount(b) for b in range(N)] == [int(r) for r in ref.refcount]


def test_rejected_calls_change_nothing():
    bm = pa.BlockManager(4, 16)
    a = bm.allocate(3)
    assert a == [0, 1, 2]
    with pytest.raises(pa.OutOfBlocks):
        bm.allocate(2)
    assert bm.num_free() == 1
    with pytest.raises(pa.PAError):
        bm.free([0, 0])  # block 0 holds one reference, not two
    assert bm.refcount(0) == 1
    with pytest.raises(pa.PAError):
        bm.fork([0, 3])  # block 3 is free
    assert [bm.refcount(b) for b in range(4)] == [1, 1, 1, 0]
    with pytest.raises(pa.PAError):
        bm.append_slot([0], 17)  # position 17 needs block 1 of a one-block table
    assert bm.refcount(7) == -1 and bm.refcount(-1) == -1


def test_c_abi_argument_checks():
    L = _lib.lib()
    h = ctypes.c_void_p()
    assert L.pa_bm_create(0, 16, ctypes.byref(h)) == PA_ERR_BAD_SHAPE
    # slots are int32: a pool whose slot range overflows it is refused
    assert L.pa_bm_create(2 ** 27, 16, ctypes.byref(h)) == PA_ERR_BAD_SHAPE
    assert L.pa_bm_create(2 ** 26, 32, ctypes.byref(h)) == PA_ERR_BAD_SHAPE
    assert L.pa_bm_create(4, 16, None) == PA_ERR_NULL_PTR
    assert L.pa_bm_create(4, 16, ctypes.byref(h)) == PA_OK
    try:
        I = ctypes.c_int32
        assert L.pa_bm_allocate(h, -1, None) == PA_ERR_BAD_SHAPE
        assert L.pa_bm_allocate(h, 1, None) == PA_ERR_NULL_PTR
        ids = (I * 8)()
        assert L.pa_bm_allocate(h, 5, ids) == PA_ERR_OUT_OF_BLOCKS
        assert L.pa_bm_num_free(h) == 4
        assert L.pa_bm_free(h, ids, 0) == PA_OK
        bad = (I * 1)(9)
        assert L.pa_bm_free(h, bad, 1) == PA_ERR_INVALID_BLOCK
        tl, slot, pair = I(0), I(0), (I * 2)()
        table = (I * 1)()
        assert L.pa_bm_append_slot(h, table, ctypes.byref(tl), 1, 3, ctypes.byref(slot), pair) == PA_ERR_BAD_SHAPE
        assert L.pa_bm_append_slot(h, table, ctypes.byref(tl), 0, 0, ctypes.byref(slot), pair) == PA_ERR_BAD_SHAPE
        assert L.pa_bm_append_slot(h, table, ctypes.byref(tl), 1, 0, ctypes.byref(slot), pair) == PA_OK
        assert tl.value == 1 and table[0] == 0 and slot.value == 0 and list(pair) == [-1, -1]
    finally:
        L.pa_bm_destroy(h)


def test_copy_blocks_host_validation():
    L = _lib.lib()
    A = 0x7F0000000000
    c = PaKvCache(A + 0x1000, A + 0x2000, None, None, 8, 2, 16, 128, PA_BF16)
    assert L.pa_copy_blocks(ctypes.byref(c), None, 0, None) == PA_OK  # no-op
    assert L.pa_copy_blocks(ctypes.byref(c), None, 2, None) == PA_ERR_NULL_PTR
    assert L.pa_copy_blocks(ctypes.byref(c), A + 0x3002, 2, None) == PA_ERR_MISALIGNED
    assert L.pa_copy_blocks(ctypes.byref(c), A + 0x3000, -1, None) == PA_ERR_BAD_SHAPE
    c_bad = PaKvCache(A + 0x1000, A + 0x2000, A, A, 8, 2, 16, 128, PA_BF16)  # scales on a bf16 cache
    assert L.pa_copy_blocks(ctypes.byref(c_bad), A + 0x3000, 1, None) == PA_ERR_NULL_PTR
