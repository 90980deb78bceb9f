"""Pins of the oracle's block copy and block manager (no GPU)."""
import numpy as np
import pytest

import oracle
import pinlib


def test_allocation_example_from_pages():
    """Sequences of 100, 50 and 200 tokens grown one token at a time with
    16-token blocks hold 7, 4 and 13 blocks, 24 in all, and never copy
    (page "LLM推理优化", section 3.2 allocation example)."""
    g = pinlib.golden("block_counts.json")
    bm = oracle.BlockManager(64, g["block_size"])
    tables = []
    for L in g["total"]["lengths"]:
        t = []
        for pos in range(L):
            slot, copies = bm.append_slot(t, pos)
            assert copies == []
            assert slot == t[pos // 16] * 16 + pos % 16
        tables.append(t)
    assert [len(t) for t in tables] == [7, 4, 13]
    assert 64 - bm.num_free() == g["total"]["blocks"]
    ids = [b for t in tables for b in t]
    assert len(set(ids)) == len(ids)  # no block shared without a fork


def check_beams(Manager):
    """Two beams of a 40-token request share the first blocks and the second
    beam writes into a private copy of the last one (page "字节跳动 AI Infra
    (2)", PagedAttention block-pool figure: beam 1 [B1, B3, B6], beam 2
    [B1, B3, B6'])."""
    bm = Manager(16, 16)
    beam1 = []
    for pos in range(40):
        bm.append_slot(beam1, pos)
    assert len(beam1) == 3  # request A: 40 tokens -> 3 blocks
    beam2 = bm.fork(beam1)
    assert list(bm.refcount[beam1]) == [2, 2, 2]
    slot, copies = bm.append_slot(beam2, 40)
    assert beam2[:2] == beam1[:2] and beam2[2] != beam1[2]
    assert copies == [(beam1[2], beam2[2])]
    assert slot == beam2[2] * 16 + 8
    assert bm.refcount[beam1[2]] == 1 and bm.refcount[beam2[2]] == 1
    assert list(bm.refcount[beam1[:2]]) == [2, 2]
    # the first beam now owns its last block alone: no copy
    slot1, copies1 = bm.append_slot(beam1, 40)
    assert copies1 == [] and slot1 == beam1[2] * 16 + 8
    # a new block starts at position 48 for both, without copies
    for t in (beam1, beam2):
        for pos in range(41, 49):
            _, c = bm.append_slot(t, pos)
            assert c == []
    assert beam1[3] != beam2[3]


def test_beam_fork_and_copy_on_write_as_in_the_figure():
    check_beams(oracle.BlockManager)


def check_invariants(Manager):
    """References equal table entries; releasing every table frees the pool."""
    rng = np.random.default_rng(0)
    bm = Manager(256, 16)
    tables, lens = [], []
    for step in range(3000):
        op = rng.integers(0, 10)
        if op == 0 and tables:
            i = int(rng.integers(len(tables)))
            tables.append(bm.fork(tables[i]))
            lens.append(lens[i])
        elif op == 1 and tables:
            i = int(rng.integers(len(tables)))
            bm.free(tables.pop(i))
            lens.pop(i)
        elif op == 2 or not tables:
            tables.append([])
            lens.append(0)
        else:
            i = int(rng.integers(len(tables)))
            try:
                slot, copies = bm.append_slot(tables[i], lens[i])
            except oracle.OutOfBlocks:
                continue
            lens[i] += 1
            for s, d in copies:
                assert bm.refcount[d] == 1 and bm.refcount[s] >= 1
        counts = np.zeros(256, np.int64)
        for t in tables:
            for b in t:
                counts[b] += 1
        assert np.array_equal(counts, bm.refcount), step
    for t in tables:
        bm.free(t)
    assert bm.num_free() == 256


def test_manager_invariants_random_ops():
    check_invariants(oracle.BlockManager)


class _KeepsSourceReference(oracle.BlockManager):
    """Mutant: copy-on-write that forgets to drop the source's reference."""

    def append_slot(self, table, length):
        slot, copies = super().append_slot(table, length)
        for s, _ in copies:
            self.refcount[s] += 1
        return slot, copies


class _NeverCopies(oracle.BlockManager):
    """Mutant: writes into shared blocks without copying them."""

    def append_slot(self, table, length):
        bs = self.block_size
        j, off = divmod(int(length), bs)
        if j == len(table):
            table.append(self.allocate(1)[0])
        return table[j] * bs + off, []


@pytest.mark.parametrize("mutant", [_KeepsSourceReference, _NeverCopies])
def test_manager_mutants_are_caught(mutant):
    caught = 0
    for check in (check_beams, check_invariants):
        try:
            check(mutant)
        except AssertionError:
            caught += 1
    assert caught >= 1


def test_out_of_blocks_and_misuse():
    bm = oracle.BlockManager(2, 16)
    bm.allocate(2)
    with pytest.raises(oracle.OutOfBlocks):
        bm.allocate(1)
    bm.free([0])
    with pytest.raises(ValueError):
        bm.free([0])
    with pytest.raises(ValueError):
        bm.fork([0])
    with pytest.raises(ValueError):
        bm.append_slot([1], 17)  # position 17 needs a block 1 that the table lacks


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16", "i8"])
def test_copy_blocks_moves_exactly_the_blocks(kv_dtype):
    rng = np.random.default_rng(1)
    nb, H, bs, D = 6, 2, 16, 32
    c = oracle.PagedCache.empty(kv_dtype, nb, H, bs, D, poison=False)
    # distinct contents in every (block, slot): write tokens through append
    K = pinlib.dyadic(rng, (nb * bs, H, D))
    V = pinlib.dyadic(rng, (nb * bs, H, D))
    oracle.append(c, K, V, np.arange(nb * bs))
    before = oracle.PagedCache(c.kv_dtype, nb, H, bs, D, c.k.copy(), c.v.copy(),
                               None if c.k_scale is None else c.k_scale.copy(),
                               None if c.v_scale is None else c.v_scale.copy())
    oracle.copy_blocks(c, [(1, 4), (3, 0)])
    offs = np.arange(bs)
    for h in range(H):
        for dst, src in ((4, 1), (0, 3), (1, 1), (2, 2), (3, 3), (5, 5)):
            got_k = c.k_rows(np.full(bs, dst), h, offs)
            got_v = c.v_rows(np.full(bs, dst), h, offs)
            assert np.array_equal(got_k, before.k_rows(np.full(bs, src), h, offs))
            assert np.array_equal(got_v, before.v_rows(np.full(bs, src), h, offs))


def test_copy_blocks_reads_the_pool_before_the_call_and_checks_pairs():
    c = oracle.PagedCache.empty("f32", 4, 1, 16, 16, poison=False)
    c.k[:] = np.arange(4, dtype=np.float32)[:, None, None, None]
    with pytest.raises(ValueError):
        oracle.copy_blocks(c, [(0, 1), (1, 2)])  # 1 is both a destination and a source
    with pytest.raises(ValueError):
        oracle.copy_blocks(c, [(0, 2), (1, 2)])  # destination twice
    with pytest.raises(IndexError):
        oracle.copy_blocks(c, [(0, 4)])
    oracle.copy_blocks(c, [(3, 0), (2, 1)])
    assert [float(c.k[b].flat[0]) for b in range(4)] == [3.0, 2.0, 2.0, 3.0]


# ---- swap between a GPU pool and a host pool --------------------------------


def _swap_round_trip(kv_dtype, swap):
    """Swap one sequence's blocks out to a host pool, let another sequence
    reuse (overwrite) its GPU blocks, swap it back in under other ids and
    rewrite its table: its decode is exactly what it was.  Returns True when
    that holds."""
    rng = np.random.default_rng(21)
    Hq, Hkv, D, bs = 4, 2, 32, 16
    lens = [37, 50, 16]
    Ks = [pinlib.dyadic(rng, (L, Hkv, D)) for L in lens]
    Vs = [pinlib.dyadic(rng, (L, Hkv, D)) for L in lens]
    cache, tb, cl = pinlib.paged_from_dense(Ks, Vs, bs, kv_dtype, rng, spare=8)
    q = pinlib.dyadic(rng, (len(lens), Hq, D))
    before = oracle.decode(q, cache, tb, cl, 0.3)
    victim = 1
    nblk = -(-lens[victim] // bs)
    gpu_ids = [int(b) for b in tb[victim, :nblk]]
    host = oracle.PagedCache.empty(kv_dtype, 9, Hkv, bs, D)
    host_ids = [8 - i for i in range(nblk)]
    swap(cache, host, list(zip(gpu_ids, host_ids)))
    # the freed GPU blocks are reused by someone else
    cache.k[gpu_ids] = cache.k[0]
    cache.v[gpu_ids] = -cache.v[0]
    if cache.k_scale is not None:
        cache.k_scale[gpu_ids] = 0
        cache.v_scale[gpu_ids] = 0
    used = {int(b) for b in tb[tb >= 0].ravel()}
    free = [b for b in range(cache.num_blocks) if b not in used]
    new_ids = free[:nblk]
    swap(host, cache, list(zip(host_ids, new_ids)))
    tb2 = tb.copy()
    tb2[victim, :nblk] = new_ids
    after = oracle.decode(q, cache, tb2, cl, 0.3)
    return np.array_equal(after, before)


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16", "i8"])
def test_swap_out_and_in_decodes_exactly_as_before(kv_dtype):
    """A preempted sequence's KV moved to host memory and back under new
    block ids decodes bit for bit as before (page "vLLM框架是怎么做推理加速的",
    section 2: swapped requests resume; page "字节跳动 AI Infra (2)",
    PagedAttention question: KV swapped to CPU when memory runs short)."""
    assert _swap_round_trip(kv_dtype, oracle.swap_blocks)


def _swap_k_only(src, dst, pairs):
    for s, d in pairs:
        dst.k[d] = src.k[s]


def _swap_without_scales(src, dst, pairs):
    for s, d in pairs:
        dst.k[d] = src.k[s]
        dst.v[d] = src.v[s]


def _swap_first_head_only(src, dst, pairs):
    for s, d in pairs:
        dst.k[d, 0] = src.k[s, 0]
        dst.v[d, 0] = src.v[s, 0]
        if src.k_scale is not None:
            dst.k_scale[d] = src.k_scale[s]
            dst.v_scale[d] = src.v_scale[s]


@pytest.mark.parametrize("mutant,kv_dtype", [(_swap_k_only, "bf16"), (_swap_without_scales, "i8"),
                                             (_swap_first_head_only, "f32")])
def test_swap_mutants_are_caught(mutant, kv_dtype):
    assert not _swap_round_trip(kv_dtype, mutant)


def test_swap_moves_exactly_the_blocks_and_checks_its_arguments():
    rng = np.random.default_rng(3)
    g = oracle.PagedCache.empty("i8", 5, 2, 16, 32, poison=False)
    K = pinlib.dyadic(rng, (5 * 16, 2, 32))
    oracle.append(g, K, -K, np.arange(5 * 16))
    h = oracle.PagedCache.empty("i8", 3, 2, 16, 32)
    g_before = (g.k.copy(), g.v.copy(), g.k_scale.copy(), g.v_scale.copy())
    h_before = (h.k.copy(), h.v.copy(), h.k_scale.copy(), h.v_scale.copy())
    oracle.swap_blocks(g, h, [(4, 0), (1, 2)])
    for a, b in zip((g.k, g.v, g.k_scale, g.v_scale), g_before):
        assert np.array_equal(a, b)  # the source pool is only read
    for got, src_arr, untouched in zip((h.k, h.v, h.k_scale, h.v_scale), g_before, h_before):
        assert np.array_equal(got[0], src_arr[4]) and np.array_equal(got[2], src_arr[1])
        assert np.array_equal(got[1], untouched[1], equal_nan=True)
    with pytest.raises(ValueError):
        oracle.swap_blocks(g, g, [(0, 1)])  # one pool: that is copy_blocks
    with pytest.raises(ValueError):
        oracle.swap_blocks(g, oracle.PagedCache.empty("i8", 3, 2, 32, 32), [(0, 0)])  # layouts differ
    with pytest.raises(IndexError):
        oracle.swap_blocks(g, h, [(5, 0)])
    with pytest.raises(IndexError):
        oracle.swap_blocks(g, h, [(0, 3)])
    with pytest.raises(ValueError):
        oracle.swap_blocks(g, h, [(0, 1), (2, 1)])
