"""Physical-block bookkeeping and block copies, written from their definitions.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

* ``copy_blocks``: copying physical block ``src`` to ``dst`` makes every K/V
  element (and int8 scale) of ``dst``, for every kv head and every in-block
  slot, equal to that of ``src``.  All copies of one call read the pool as it
  was before the call.  This is the copy half of copy-on-write (page
  "字节跳动 AI Infra (2)", PagedAttention question, block-pool figure: two
  beams share blocks B1 and B3, and the second beam's last block B6' is a
  copy of B6; page "LLM推理优化", section 3.2: shared blocks are copied when
  one sharer writes).
* ``BlockManager``: a pool of ``num_blocks`` physical blocks with reference
  counts.  Blocks are handed out on demand (page "LLM推理优化", section 3.2:
  blocks are allocated as a sequence grows; 100, 50 and 200 tokens take 7, 4
  and 13 blocks of 16) and shared between sequences by counting references
  (a fork shares every block of the parent's table).  Before a sequence writes
  a token into a block that another sequence also references, the block is
  copied into a fresh one that only the writer references (copy-on-write).

* ``swap_blocks``: the same whole-block copy between two pools of one
  layout, a GPU pool and a host pool.  When GPU memory runs short, or a
  request is preempted, its KV cache is moved to CPU memory and brought back
  before it runs again (page "字节跳动 AI Infra (2)", PagedAttention question,
  scheduling list, and the preemption/swap row of the third question's
  layer-4 table; page "vLLM框架是怎么做推理加速的", section 2 (swapped queue,
  long requests swapped out to CPU) and its second follow-up (a swap costs
  10-20 ms)).  A block's contents are the same wherever it lives, so a
  sequence swapped out and back in under new block ids decodes exactly as
  before.

Readings where the pages are silent: free blocks are handed out lowest id
first; a fork shares the parent's blocks (no copy happens until a write); a
write into a shared block copies that block only; a swap copies whole blocks
(every kv head, and the scales of an int8 cache) between pools of the same
layout, and its block ids are independent in the two pools.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

from .layout import PagedCache


def copy_blocks(cache: PagedCache, pairs: Sequence[Tuple[int, int]]) -> None:
    """Copy physical blocks ``src -> dst`` for every (src, dst) in ``pairs``.

    Preconditions (checked): ids in range, destinations distinct, no
    destination is also a source.
    """
    pairs = [(int(s), int(d)) for s, d in pairs]
    srcs = [s for s, _ in pairs]
    dsts = [d for _, d in pairs]
    for b in srcs + dsts:
        if not 0 <= b < cache.num_blocks:
            raise IndexError(f"block {b} outside the pool")
    if len(set(dsts)) != len(dsts):
        raise ValueError("a destination block appears twice")
    if set(dsts) & set(srcs):
        raise ValueError("a destination block is also a source")
    before_k = cache.k.copy()
    before_v = cache.v.copy()
    before_ks = None if cache.k_scale is None else cache.k_scale.copy()
    before_vs = None if cache.v_scale is None else cache.v_scale.copy()
    for s, d in pairs:
        cache.k[d] = before_k[s]
        cache.v[d] = before_v[s]
        if before_ks is not None:
            cache.k_scale[d] = before_ks[s]
            cache.v_scale[d] = before_vs[s]


def swap_blocks(src: PagedCache, dst: PagedCache, pairs: Sequence[Tuple[int, int]]) -> None:
    """Copy block ``s`` of pool ``src`` to block ``d`` of pool ``dst`` for every
    (s, d) in ``pairs`` (swap out: GPU pool -> host pool; swap in: the reverse).

    Preconditions (checked): two distinct pools of one layout (kv dtype, kv
    heads, block size, head dim), ids in range of their own pool,
    destinations distinct.
    """
    if src is dst:
        raise ValueError("swap_blocks moves blocks between two pools; use copy_blocks within one")
    if (src.kv_dtype, src.Hkv, src.bs, src.D) != (dst.kv_dtype, dst.Hkv, dst.bs, dst.D):
        raise ValueError("the two pools differ in layout")
    pairs = [(int(s), int(d)) for s, d in pairs]
    for s, d in pairs:
        if not 0 <= s < src.num_blocks:
            raise IndexError(f"source block {s} outside its pool")
        if not 0 <= d < dst.num_blocks:
            raise IndexError(f"destination block {d} outside its pool")
    dsts = [d for _, d in pairs]
    if len(set(dsts)) != len(dsts):
        raise ValueError("a destination block appears twice")
    for s, d in pairs:
        dst.k[d] = src.k[s]
        dst.v[d] = src.v[s]
        if src.k_scale is not None:
            dst.k_scale[d] = src.k_scale[s]
            dst.v_scale[d] = src.v_scale[s]


class OutOfBlocks(RuntimeError):
    pass


class BlockManager:
    """Reference counts of a pool of physical blocks (host bookkeeping)."""

    def __init__(self, num_blocks: int, block_size: int):
        if num_blocks < 1 or block_size < 1:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.refcount = np.zeros(self.num_blocks, dtype=np.int64)

    # ---- pool -------------------------------------------------------------
    def num_free(self) -> int:
        return int(np.sum(self.refcount == 0))

    def allocate(self, n: int) -> List[int]:
        """``n`` free blocks, lowest ids first, each with one reference."""
        free = np.flatnonzero(self.refcount == 0)
        if len(free) < n:
            raise OutOfBlocks(f"{n} blocks requested, {len(free)} free")
        ids = [int(b) for b in free[:n]]
        self.refcount[ids] += 1
        return ids

    def free(self, ids: Sequence[int]) -> None:
        """Drop one reference to each block (a block is free at zero)."""
        for b in ids:
            if self.refcount[b] <= 0:
                raise ValueError(f"block {b} is not in use")
            self.refcount[b] -= 1

    def fork(self, table: Sequence[int]) -> List[int]:
        """A child's table sharing every block of ``table`` (one more reference each)."""
        for b in table:
            if self.refcount[b] <= 0:
                raise ValueError(f"block {b} is not in use")
            self.refcount[b] += 1
        return list(table)

    # ---- a sequence grows by one token --------------------------------------
    def append_slot(self, table: List[int], length: int) -> Tuple[int, List[Tuple[int, int]]]:
        """Make room for the token at position ``length`` of the sequence whose
        block table is ``table`` (modified in place).

        Returns (slot, copies): the slot (physical block * block_size + offset)
        the token is written to, and the (src, dst) block copies that must be
        carried out before the write.  A new block is taken when the position
        starts a block; a block still referenced by another sequence is
        replaced by a private copy first.
        """
        bs = self.block_size
        j, off = divmod(int(length), bs)
        if j > len(table) or (j == len(table) and off != 0):
            raise ValueError("length does not follow the blocks of the table")
        copies: List[Tuple[int, int]] = []
        if j == len(table):
            table.append(self.allocate(1)[0])
        elif self.refcount[table[j]] > 1:
            src = table[j]
            dst = self.allocate(1)[0]
            self.refcount[src] -= 1
            table[j] = dst
            copies.append((src, dst))
        return table[j] * bs + off, copies
