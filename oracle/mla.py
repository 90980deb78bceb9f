"""MLA (multi-head latent attention) decode over a paged latent cache, float64.

TEST INFRASTRUCTURE (see ``oracle/__init__``).  Plain definitions: the heads'
keys and values are recovered from the cached latent rows explicitly, then
attended as in ``oracle.decode``.

Source: page "字节跳动 AI Infra (2)", question on KV-cache principles, the MLA
paragraph and the MLA row of its optimisation table.  Each token's K and V
are compressed jointly into one latent vector c (512 wide in the page's
example); the cache stores only c, and at inference the keys are recovered
as K = c W_up_K, mapping d_compress to num_heads x head_dim, so attention is
computed as over the full-width K/V.  Readings where the page is silent:

* V is recovered the same way with its own matrix, V = c W_up_V (the page
  says K and V are compressed jointly and writes out only the K projection);
* the column of W_up (a d_compress x (num_heads * head_dim) matrix) for head
  h, channel d is h * head_dim + d (heads are consecutive column blocks);
* the cache is paged like the K/V cache: latent row of logical position t in
  physical block block_table[t // bs] at offset t % bs, stored row-major
  ``[num_blocks][bs][d_c]``;
* scores are scaled by the caller's ``scale`` (1/sqrt(head_dim) in the
  workloads, the page's divide by sqrt(d)).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class LatentCache:
    """Host latent cache: values (float64, exact copies of the stored bf16) ``[num_blocks, bs, d_c]``."""

    c: np.ndarray

    @property
    def num_blocks(self) -> int:
        return self.c.shape[0]

    @property
    def bs(self) -> int:
        return self.c.shape[1]

    @property
    def d_c(self) -> int:
        return self.c.shape[2]

    @classmethod
    def empty(cls, num_blocks: int, bs: int, d_c: int, poison: bool = True) -> "LatentCache":
        return cls(np.full((num_blocks, bs, d_c), np.nan if poison else 0.0, dtype=np.float64))


def mla_append(cache: LatentCache, rows: np.ndarray, slots: np.ndarray) -> None:
    """Write latent rows ``[T, d_c]`` into slots (block = s // bs, offset = s % bs); s < 0 skips."""
    rows = np.asarray(rows, np.float64)
    for i, s in enumerate(np.asarray(slots, np.int64)):
        if s < 0:
            continue
        pb, off = divmod(int(s), cache.bs)
        if pb >= cache.num_blocks:
            continue
        cache.c[pb, off, :] = rows[i]


def mla_gather(cache: LatentCache, table_row: np.ndarray, length: int) -> np.ndarray:
    """Latent rows (float64 ``[L, d_c]``) of logical positions 0 .. L-1 of one sequence."""
    t = np.arange(int(length), dtype=np.int64)
    pbs = table_row[t // cache.bs].astype(np.int64)
    if np.any(pbs < 0) or np.any(pbs >= cache.num_blocks):
        raise IndexError("block table entry out of range for a used position")
    return cache.c[pbs, t % cache.bs, :]


def mla_expand(c_rows: np.ndarray, w_up: np.ndarray, H: int, d_h: int) -> np.ndarray:
    """Per-head vectors recovered from latent rows: ``[L, H, d_h]`` = (c W_up) with column
    h * d_h + d giving head h, channel d."""
    full = np.asarray(c_rows, np.float64) @ np.asarray(w_up, np.float64)  # [L, H * d_h]
    return full.reshape(full.shape[0], H, d_h)


def mla_decode(q: np.ndarray, cache: LatentCache, w_uk: np.ndarray, w_uv: np.ndarray,
               block_tables: np.ndarray, context_lens: np.ndarray, scale: float) -> np.ndarray:
    """MLA decode output ``[B, H, d_h]`` (float64).

    For sequence b with L cached tokens and query head h:
        K_t = c_t W_uk (head h's columns),  V_t = c_t W_uv (head h's columns),
        s_t = scale * q[b, h] . K_t,
        out[b, h] = sum_t exp(s_t - m) V_t / sum_t exp(s_t - m),  m = max_t s_t.
    L = 0 gives a zero row.
    """
    q = np.asarray(q, np.float64)
    B, H, d_h = q.shape
    out = np.zeros((B, H, d_h), np.float64)
    for b in range(B):
        L = int(context_lens[b])
        if L == 0:
            continue
        C = mla_gather(cache, block_tables[b], L)
        K = mla_expand(C, w_uk, H, d_h)
        V = mla_expand(C, w_uv, H, d_h)
        for h in range(H):
            s = float(scale) * (K[:, h, :] @ q[b, h])
            w = np.exp(s - s.max())
            out[b, h] = (w @ V[:, h, :]) / w.sum()
    return out


def mla_build_cache(workload, poison: bool = True) -> LatentCache:
    """Host latent cache holding every cached token of an ``MlaWorkload``."""
    s = workload.spec
    cache = LatentCache.empty(workload.num_blocks, s.bs, s.d_c, poison=poison)
    for b in range(s.B):
        L = int(workload.context_lens[b])
        if L:
            mla_append(cache, workload.latent(b), workload.slots(b))
    return cache
