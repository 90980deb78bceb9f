"""Algorithmic byte counts for the paged-decode path (roofline denominators).

These are the bytes the method has to move, not what a kernel happens to
fetch: K and V of every valid cached token (shared prefix blocks once),
int8 scales, the queries read and outputs written, the used block-table
entries and context lengths.  KV-split scratch (partials) is overhead and
not counted.
"""
from __future__ import annotations

from typing import Iterable, Optional

import numpy as np

ELEM_BYTES = {"f32": 4, "bf16": 2, "i8": 1, "i4": 0.5}
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak, vendor figure (no sparsity)


def kv_cache_bytes_per_sequence(layers: int, heads: int, seq_len: int, head_dim: int, dtype_bytes: int) -> int:
    """KV bytes of one sequence: K and V, every layer and head, every token.

    The memory formula on page "LLM推理优化", section 1.2 (two tensors times
    layers, heads, sequence length, head_dim and element size).  ``heads``
    is the number of K/V heads actually stored (fewer than the query heads
    under GQA).
    """
    return 2 * int(layers) * int(heads) * int(seq_len) * int(head_dim) * int(dtype_bytes)


def decode_bytes(context_lens: Iterable[int], *, Hq: int, Hkv: int, D: int, bs: int, kv_dtype: str,
                 q_dtype: str, out_dtype: str, shared_tokens: int = 0) -> int:
    """Bytes one decode launch over the batch must move.

    ``shared_tokens``: positions whose (block, kv head) tiles another
    sequence of the batch already reads (prefix-shared blocks); counted once.
    """
    L = np.asarray(list(context_lens), dtype=np.int64)
    B = len(L)
    toks = int(L.sum()) - int(shared_tokens)
    e = ELEM_BYTES[kv_dtype]
    kv = toks * Hkv * D * 2 * e
    if kv_dtype in ("i8", "i4"):
        kv += toks * Hkv * 2 * 2  # fp16 K and V scale per (token, kv head)
    qo = B * Hq * D * (ELEM_BYTES[q_dtype] + ELEM_BYTES[out_dtype])
    tables = int(np.sum((L + bs - 1) // bs)) * 4 + B * 4
    return int(kv + qo + tables)


def multi_bytes(context_lens: Iterable[int], query_counts: Iterable[int], *, Hq: int, Hkv: int, D: int, bs: int,
                kv_dtype: str, q_dtype: str, out_dtype: str) -> int:
    """Bytes one causal multi-query launch must move: every cached K/V row
    once, the query and output rows of every new token, the tables and the
    row offsets."""
    L = np.asarray(list(context_lens), dtype=np.int64)
    n = np.asarray(list(query_counts), dtype=np.int64)
    rows = int(n.sum())
    e = ELEM_BYTES[kv_dtype]
    toks = int(L.sum())
    kv = toks * Hkv * D * 2 * e
    if kv_dtype in ("i8", "i4"):
        kv += toks * Hkv * 2 * 2
    qo = rows * Hq * D * (ELEM_BYTES[q_dtype] + ELEM_BYTES[out_dtype])
    tables = int(np.sum((L + bs - 1) // bs)) * 4 + len(L) * 4 + (len(L) + 1) * 4
    return int(kv + qo + tables)


def multi_flops(context_lens: Iterable[int], query_counts: Iterable[int], *, Hq: int, D: int) -> int:
    """Flops of causal multi-query attention: 2·D for q·k plus 2·D for p·v
    per (query row, head, visible position); query token i of a sequence
    with n new tokens and L cached ones sees L - n + i + 1 positions."""
    total = 0
    for L, n in zip(context_lens, query_counts):
        L, n = int(L), int(n)
        total += n * (L - n) + n * (n + 1) // 2  # sum of L - n + i + 1 over i < n
    return int(4 * D * Hq * total)


def append_bytes(num_tokens: int, *, Hkv: int, D: int, kv_dtype: str, src_dtype: str) -> int:
    """Bytes one cache append moves: source rows read, cache rows (+ scales) written, slots read."""
    T = int(num_tokens)
    rd = T * Hkv * D * 2 * ELEM_BYTES[src_dtype] + T * 4
    wr = T * Hkv * D * 2 * ELEM_BYTES[kv_dtype]
    if kv_dtype in ("i8", "i4"):
        wr += T * Hkv * 2 * 2
    return int(rd + wr)


def split_scratch_bytes(B: int, Hq: int, D: int, num_partitions_used: int) -> int:
    """Partial outputs and LSEs written by the split pass and read by the merge (overhead)."""
    return int(2 * num_partitions_used * (D + 1) * 4 * Hq) if B else 0


def mla_bytes(context_lens: Iterable[int], *, H: int, d_h: int, d_c: int, bs: int) -> int:
    """Bytes one MLA decode over a latent cache must move: the latent row (bf16)
    of every cached token once, the two bf16 up-projections, q read and out
    written (bf16), the used block-table entries and the context lengths.
    The workspace (absorbed queries, partials) is overhead and not counted."""
    L = np.asarray(list(context_lens), dtype=np.int64)
    B = len(L)
    latent = int(L.sum()) * d_c * 2
    weights = 2 * d_c * H * d_h * 2
    qo = B * H * d_h * 2 * 2
    tables = int(np.sum((L + bs - 1) // bs)) * 4 + B * 4
    return int(latent + weights + qo + tables)


def mla_flops(context_lens: Iterable[int], *, H: int, d_h: int, d_c: int) -> int:
    """Algorithmic flops of MLA decode in the absorbed form: per cached token and
    head a d_c-wide score and a d_c-wide weighted sum (4 d_c), plus the query
    absorption and the output projection (2 d_c d_h each) per (sequence, head)."""
    L = np.asarray(list(context_lens), dtype=np.int64)
    return int(int(L.sum()) * H * 4 * d_c + len(L) * H * 4 * d_c * d_h)
