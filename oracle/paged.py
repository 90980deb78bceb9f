"""Paged decode attention, KV-split partials and cache append, in float64.

TEST INFRASTRUCTURE (see ``oracle/__init__``).  Plain definitions; no
tiling, no online softmax, no fusion.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .layout import PagedCache, f32_to_bf16_bits_exact
from .quant import quantize_int4, quantize_int8


def blocks_for(length: int, block_size: int) -> int:
    """Number of cache blocks a sequence of ``length`` tokens occupies.

    Blocks hold ``block_size`` tokens each and the last one may be partly
    filled (page "LLM推理优化", section 3.2 allocation example: 100, 50 and
    200 tokens at 16 per block take 7, 4 and 13 blocks).
    """
    return (int(length) + int(block_size) - 1) // int(block_size)


def gather_sequence(cache: PagedCache, table_row: np.ndarray, length: int, kv_head: int,
                    start: int = 0, stop: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """K and V (float64 ``[n, D]``) of logical positions [start, stop) of one sequence.

    Logical position t lives in physical block ``table_row[t // bs]`` at
    offset ``t % bs`` (the block-table walk of the kernel sketch on page
    "字节跳动 AI Infra (2)", PagedAttention question).
    """
    stop = length if stop is None else stop
    t = np.arange(start, stop, dtype=np.int64)
    pbs = table_row[t // cache.bs].astype(np.int64)
    if np.any(pbs < 0) or np.any(pbs >= cache.num_blocks):
        raise IndexError("block table entry out of range for a used position")
    offs = t % cache.bs
    return cache.k_rows(pbs, kv_head, offs), cache.v_rows(pbs, kv_head, offs)


def kv_head_for(h: int, Hq: int, Hkv: int) -> int:
    """K/V head read by query head h: consecutive groups of Hq/Hkv query heads
    share one K/V head (GQA; MQA when Hkv = 1; MHA when Hkv = Hq).  Page
    "LLM推理优化", section 1.3, says several query heads share a K/V head but
    not which ones; grouping consecutive heads is the plain reading."""
    return h // (Hq // Hkv)


def _scores(q_row: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    # s_t = scale * sum_d q[d] * k_t[d]
    return float(scale) * (K @ q_row)


def _softmax_apply(s: np.ndarray, V: np.ndarray) -> Tuple[np.ndarray, float]:
    """(sum_t softmax(s)_t v_t, log sum_t exp(s_t)) for a non-empty range."""
    m = s.max()
    w = np.exp(s - m)
    total = w.sum()
    return (w @ V) / total, float(m + np.log(total))


def decode(q: np.ndarray, cache: PagedCache, block_tables: np.ndarray, context_lens: np.ndarray,
           scale: float) -> np.ndarray:
    """Decode attention output ``[B, Hq, D]`` (float64).

    For sequence b with L = context_lens[b] cached tokens (the newest token
    included, since its K/V row was appended before attending) and query
    head h, kv head = h // (Hq / Hkv) (consecutive query heads share one K/V
    head: GQA, page "LLM推理优化" section 1.3):

        s_t = scale * q[b, h] . k_t,        t = 0 .. L-1
        out[b, h] = sum_t exp(s_t - m) v_t / sum_t exp(s_t - m),   m = max_t s_t

    (softmax is unchanged by subtracting m).  L = 0 gives a zero row.
    Source: page "字节跳动 AI Infra (2)", KV-cache question, step-t equations.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    assert Hq % cache.Hkv == 0 and D == cache.D
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        if L == 0:
            continue
        for h in range(Hq):
            K, V = gather_sequence(cache, block_tables[b], L, kv_head_for(h, Hq, cache.Hkv))
            out[b, h] = _softmax_apply(_scores(q[b, h], K, scale), V)[0]
    return out


def decode_multi(q: np.ndarray, q_start: np.ndarray, cache: PagedCache, block_tables: np.ndarray,
                 context_lens: np.ndarray, scale: float) -> np.ndarray:
    """Causal attention of several new query tokens per sequence, ``[total, Hq, D]`` (float64).

    Sequence b holds n_b = q_start[b + 1] - q_start[b] new tokens: the last
    n_b of its L = context_lens[b] cached tokens (their K/V rows already
    appended).  Query token i of b (row q_start[b] + i) sits at position
    p = L - n_b + i and attends to the cached tokens t <= p only:

        out[row, h] = sum_{t <= p} exp(s_t - m) v_t / sum_{t <= p} exp(s_t - m),
        s_t = scale * q[row, h] . k_t.

    This is the step-t attention of page "字节跳动 AI Infra (2)" (KV-cache
    question) applied to each new token in turn, the shape of a chunked
    prefill (page "vLLM框架是怎么做推理加速的", section 3) and of verifying
    draft tokens; n_b = 1 is ``decode``.
    """
    q = np.asarray(q, dtype=np.float64)
    total, Hq, D = q.shape
    assert Hq % cache.Hkv == 0 and D == cache.D
    B = len(context_lens)
    assert len(q_start) == B + 1 and int(q_start[B]) == total
    out = np.zeros((total, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        r0, r1 = int(q_start[b]), int(q_start[b + 1])
        n = r1 - r0
        if n == 0:
            continue
        if n > L:
            raise ValueError("more new tokens than cached tokens")
        for i in range(n):
            p = L - n + i
            for h in range(Hq):
                K, V = gather_sequence(cache, block_tables[b], p + 1, kv_head_for(h, Hq, cache.Hkv))
                out[r0 + i, h] = _softmax_apply(_scores(q[r0 + i, h], K, scale), V)[0]
    return out


def decode_partials(q: np.ndarray, cache: PagedCache, block_tables: np.ndarray, context_lens: np.ndarray,
                    scale: float, partition_size: int, max_partitions: int) -> Tuple[np.ndarray, np.ndarray]:
    """KV-split partials: ``part_out [B, Hq, Pmax, D]`` and ``part_lse [B, Hq, Pmax]``.

    Partition p of a sequence covers positions T_p = [p*P, min((p+1)*P, L)).
    For a non-empty T_p: lse_p = log sum_{t in T_p} exp(s_t) (natural log) and
    o_p = softmax over T_p applied to the v_t.  An empty T_p gives o_p = 0,
    lse_p = -inf.  (Splitting along the KV length: FlashDecoding, page
    "字节跳动 AI Infra (2)", third question, layer-2 table.)
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    assert Hq % cache.Hkv == 0 and D == cache.D
    P = int(partition_size)
    part_out = np.zeros((B, Hq, max_partitions, D), dtype=np.float64)
    part_lse = np.full((B, Hq, max_partitions), -np.inf, dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        if L == 0:
            continue
        n_parts = (L + P - 1) // P
        if n_parts > max_partitions:
            raise ValueError("max_partitions too small for this sequence")
        for h in range(Hq):
            kv = kv_head_for(h, Hq, cache.Hkv)
            for p in range(n_parts):
                K, V = gather_sequence(cache, block_tables[b], L, kv, p * P, min((p + 1) * P, L))
                part_out[b, h, p], part_lse[b, h, p] = _softmax_apply(_scores(q[b, h], K, scale), V)
    return part_out, part_lse


def merge_partials(part_out: np.ndarray, part_lse: np.ndarray, context_lens: np.ndarray,
                   partition_size: int) -> np.ndarray:
    """Combine KV-split partials into the decode output (float64 ``[B, Hq, D]``).

    With M = max_p lse_p over the sequence's partitions and
    w_p = exp(lse_p - M):  out = sum_p w_p o_p / sum_p w_p.  This reproduces
    softmax over the union of the ranges because exp(lse_p) is the
    unnormalised weight mass of range p (online-softmax statistics, page
    "LLM推理优化", section 2.2).  A sequence with no tokens gives 0.
    """
    B, Hq, Pmax, D = part_out.shape
    out = np.zeros((B, Hq, D), dtype=np.float64)
    P = int(partition_size)
    for b in range(B):
        L = int(context_lens[b])
        n_parts = (L + P - 1) // P
        if n_parts == 0:
            continue
        lse = np.asarray(part_lse[b, :, :n_parts], dtype=np.float64)  # [Hq, n]
        M = lse.max(axis=1, keepdims=True)
        w = np.exp(lse - M)
        out[b] = np.einsum("hp,hpd->hd", w, np.asarray(part_out[b, :, :n_parts], np.float64)) / w.sum(axis=1)[:, None]
    return out


def append(cache: PagedCache, key: np.ndarray, value: np.ndarray, slot_mapping: np.ndarray) -> None:
    """Write tokens' K/V rows (``[T, Hkv, D]`` values) into their cache slots.

    Slot s >= 0 names physical block s // bs, offset s % bs; s < 0 is skipped.
    fp32 / bf16 caches store the source values unchanged; an int8 (int4)
    cache stores ``quantize_int8`` (``quantize_int4``) codes and fp16 scales
    per (token, kv head).
    Appending the new token's K and V to the cache is the concatenation step
    of the step-t equations (page "字节跳动 AI Infra (2)", KV-cache question).
    """
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    if not np.any(keep):
        return
    slots = slots[keep]
    key = np.asarray(key)[keep]
    value = np.asarray(value)[keep]
    if len(np.unique(slots)) != len(slots):
        raise ValueError("duplicate slots")
    pbs = slots // cache.bs
    offs = slots % cache.bs
    if np.any(pbs >= cache.num_blocks):
        raise IndexError("slot beyond the pool")
    if cache.kv_dtype == "f32":
        cache.store(pbs, offs, np.asarray(key, np.float32), np.asarray(value, np.float32))
    elif cache.kv_dtype == "bf16":
        cache.store(pbs, offs, f32_to_bf16_bits_exact(key), f32_to_bf16_bits_exact(value))
    else:
        # the quantised caches' source tensors are bf16
        f32_to_bf16_bits_exact(key), f32_to_bf16_bits_exact(value)
        quantize = quantize_int8 if cache.kv_dtype == "i8" else quantize_int4
        kq, ks = quantize(key)
        vq, vs = quantize(value)
        cache.store(pbs, offs, kq, vq, ks, vs)


def build_cache(workload, include_last: bool = True, seqs=None, poison: bool = True) -> PagedCache:
    """Host cache holding the workload's tokens, written through ``append``.

    ``include_last=False`` leaves out each sequence's newest token (the one
    a decode step appends).  ``seqs`` restricts the sequences written.
    """
    s = workload.spec
    cache = PagedCache.empty(s.kv_dtype, workload.num_blocks, s.Hkv, s.bs, s.D, poison=poison)
    seqs = range(s.B) if seqs is None else seqs
    for b in seqs:
        L = int(workload.context_lens[b])
        n = L if include_last else max(L - 1, 0)
        if n == 0:
            continue
        K, V = workload.tokens(b)
        if b in workload.pair_of:
            # the shared prefix blocks already hold these values (written by the
            # first beam); write only this beam's private positions
            start = workload.shared_blocks[b] * s.bs
        else:
            start = 0
        if start >= n:
            continue
        append(cache, K[start:n], V[start:n], workload.slots(b, start, n))
    return cache
