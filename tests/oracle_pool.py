"""Oracle outputs for whole full-size batches, computed in worker processes.

The oracle is plain fp64 numpy, one sequence (or one query row) at a time;
a full-size batch is minutes of one core, so the GPU tests hand chunks of
sequences to a pool of spawned processes.  Each worker rebuilds the seeded
workload itself (inputs come only from ``workloads``), writes the host cache
of its chunk through the oracle's append and returns the oracle's decode.
Workers import numpy, ``workloads`` and ``oracle`` only: no torch, no GPU.
"""
from __future__ import annotations

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor
from typing import Dict, List, Sequence, Tuple

import numpy as np


def workers() -> int:
    return max(1, min(8, os.cpu_count() or 1))


def _with_partners(w, seqs: Sequence[int]) -> List[int]:
    """The chunk plus the beams whose prefix blocks it shares (they write them)."""
    return sorted(set(seqs) | {w.pair_of[b] for b in seqs if b in w.pair_of})


def _one_thread():
    """Each worker keeps its BLAS to one thread (the pool is the parallelism)."""
    from threadpoolctl import threadpool_limits

    return threadpool_limits(limits=1)


def _decode_job(args) -> Tuple[List[int], np.ndarray]:
    cfg, overrides, seqs = args
    import oracle
    from workloads import make_workload

    with _one_thread():
        w = make_workload(cfg, **overrides)
        oc = oracle.build_cache(w, seqs=_with_partners(w, seqs))
        want = oracle.decode(w.q[seqs], oc, w.block_tables[seqs], w.context_lens[seqs], w.spec.scale)
    return list(seqs), want


def _rows_job(args) -> Tuple[List[Tuple[int, int]], np.ndarray]:
    """Query rows of a multi-query step on a custom workload: row (b, i) is
    new token i of sequence b's n, attending to the context cut at its own
    position."""
    custom, n, rows = args
    import oracle
    from workloads import make_custom

    with _one_thread():
        w = make_custom(**custom)
        counts = np.full(w.B, n, np.int32)
        q_start, q = w.multi_queries(counts)
        oc = oracle.build_cache(w, seqs=sorted({b for b, _ in rows}))
        out = np.empty((len(rows), w.spec.Hq, w.spec.D), np.float64)
        for j, (b, i) in enumerate(rows):
            r = int(q_start[b]) + i
            cut = np.array([int(w.context_lens[b]) - n + i + 1], np.int32)
            out[j] = oracle.decode(q[r:r + 1], oc, w.block_tables[b:b + 1], cut, w.spec.scale)[0]
    return rows, out


def _deal(items: Sequence, weights: Sequence[float], parts: int) -> List[list]:
    """Items dealt into ``parts`` chunks of similar total weight (heaviest first)."""
    order = np.argsort(-np.asarray(weights, np.float64), kind="stable")
    chunks: List[list] = [[] for _ in range(parts)]
    load = np.zeros(parts)
    for k in order:
        j = int(np.argmin(load))
        chunks[j].append(items[k])
        load[j] += weights[k]
    return [sorted(c) for c in chunks if c]


def _pool():
    return ProcessPoolExecutor(max_workers=workers(), mp_context=mp.get_context("spawn"))


def whole_batch_decode(cfg: int, overrides: Dict, context_lens: np.ndarray) -> np.ndarray:
    """The oracle's decode of every sequence of workload ``cfg`` (float64 [B, Hq, D])."""
    B = len(context_lens)
    chunks = _deal(list(range(B)), [float(L) + 64.0 for L in context_lens], 2 * workers())
    parts = {}
    with _pool() as ex:
        for seqs, want in ex.map(_decode_job, [(cfg, overrides, c) for c in chunks]):
            for j, b in enumerate(seqs):
                parts[b] = want[j]
    return np.stack([parts[b] for b in range(B)])


def rows_decode(custom: Dict, n: int, rows: Sequence[Tuple[int, int]], context_lens: np.ndarray) -> np.ndarray:
    """The oracle's output for the given (sequence, new token) rows, in order."""
    chunks = _deal(list(rows), [float(context_lens[b]) for b, _ in rows], 2 * workers())
    got = {}
    with _pool() as ex:
        for rs, out in ex.map(_rows_job, [(custom, n, c) for c in chunks]):
            for j, r in enumerate(rs):
                got[tuple(r)] = out[j]
    return np.stack([got[tuple(r)] for r in rows])
