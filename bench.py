#!/usr/bin/env python3
"""Paged-attention decode benchmark on one MI355X.

One step is one decode iteration of the whole path over a batch that is
already resident in HBM: every sequence appends its newest K/V token to
the paged cache, then attends over its cache -- issued as a serving loop
issues it, one ``pa_append_decode`` call (one fused kernel), or
``pa_append_decode_split`` + ``pa_reduce`` for the long-context workload.
Before each timed step a sequential read of a 1 GiB scratch buffer with the
library's read probe (``pa_probe_read``, ordinary loads) evicts the L2s and
the 256 MB Infinity Cache with clean lines, so the K/V reads come from HBM
and no write-back of earlier data lands inside the timed kernels.  Kernel
times come from HIP events recorded on the stream the kernels run on
(torch's current stream, which the binding launches on).

Printed: ONE JSON line.  The headline workload is the largest one, the
INT8 KV-cache GQA decode plus cache append (256 sequences of 1024-8192
tokens).  ``value`` is its effective HBM rate: algorithmic bytes (K/V of
every cached token -- prefix-shared blocks once -- int8 scales, q, out,
used block-table entries, context lengths, and the appended rows) divided
by the median step time.  ``roofline`` reports the step's dominant kernel
against the 8 TB/s HBM peak and against the probe's rate for the same tile
pattern; every other workload carries the same block.

  python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--config 5]
                  [--others 2,3,4] [--no-cpu-baseline]

The ``cpu_baseline`` leg times the fp64 CPU oracle (the parity reference,
not a tuned CPU implementation) on one host core over a bounded sample of
the headline workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged-decode attention µs/step + effective KV-read GB/s (% of HBM peak)"
HEADLINE = 5


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=HEADLINE, choices=[1, 2, 3, 4, 5],
                    help="workload timed for the headline value")
    ap.add_argument("--others", default="2,3,4",
                    help="comma-separated workloads also timed and summarised ('' for none); the int8 "
                         "workload's shapes with an int4 cache are added whenever workload 5 runs")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--flush-mib", type=int, default=1024)
    ap.add_argument("--probe-mib", type=int, default=2048, help="buffer of the read-bandwidth probe ('0': skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="upper bound on the oracle's timed CPU work")
    ap.add_argument("--no-multi-shapes", action="store_true",
                    help="skip the extra multi-query shapes (verification and chunked-prefill sizes)")
    ap.add_argument("--no-mla", action="store_true", help="skip the MLA latent-cache decode")
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="seconds each timed call runs untimed first, so the GPU clocks settle (0 for profiler runs)")
    ap.add_argument("--json-out", default=None, help="also write the JSON line to this file")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device copy of this size first (calibrates rocprofv3 byte counters)")
    return ap.parse_args(argv)


# --------------------------------------------------------------------------
# one workload on the GPU
# --------------------------------------------------------------------------


class Case:
    """A workload resident on the GPU, with its step and its byte counts."""

    def __init__(self, cfg: int, seed, torch, pa, perfmodel, **overrides):
        from workloads import make_workload
        from workloads.device import append_tokens, meta, new_token_batch, poisoned_cache

        self.torch = torch
        self.pa = pa
        t0 = time.time()
        self.w = w = make_workload(cfg, seed, **overrides)
        s = self.s = w.spec
        log(f"cfg{cfg} {s.name}: B={w.B} tokens={w.total_tokens()} pool={w.num_blocks} blocks; filling cache")
        self.cache = poisoned_cache(w)
        append_tokens(w, self.cache, include_last=False)
        self.kn, self.vn, self.slots = new_token_batch(w)
        self.q, self.tables, self.lens = meta(w)
        self.out_dtype = torch.bfloat16 if s.q_dtype == "bf16" else torch.float32
        self.out = torch.empty(self.q.shape, dtype=self.out_dtype, device=self.q.device)
        self.split = s.partition_size is not None
        if self.split:
            self.pmax = pa.max_partitions(self.tables.shape[1], s.bs, s.partition_size)
            B, Hq, D = self.q.shape
            self.part_out = torch.empty((B, Hq, self.pmax, D), dtype=torch.float32, device=self.q.device)
            self.part_lse = torch.empty((B, Hq, self.pmax), dtype=torch.float32, device=self.q.device)
        torch.cuda.synchronize()
        log(f"cfg{cfg}: cache filled in {time.time() - t0:.1f}s")

        shared = sum(S * s.bs for S in w.shared_blocks.values())
        kw = dict(Hq=s.Hq, Hkv=s.Hkv, D=s.D, bs=s.bs, kv_dtype=s.kv_dtype, q_dtype=s.q_dtype,
                  out_dtype="bf16" if self.out_dtype == torch.bfloat16 else "f32")
        self.decode_bytes = perfmodel.decode_bytes(w.context_lens, shared_tokens=shared, **kw)
        self.decode_bytes_logical = perfmodel.decode_bytes(w.context_lens, **kw)
        # the split pass reads everything the decode reads but writes partials, not out
        self.split_kernel_bytes = self.decode_bytes - w.B * s.Hq * s.D * (2 if kw["out_dtype"] == "bf16" else 4)
        n_new = int((self.slots.cpu() >= 0).sum())
        self.append_bytes = perfmodel.append_bytes(n_new, Hkv=s.Hkv, D=s.D, kv_dtype=s.kv_dtype,
                                                   src_dtype="f32" if s.kv_dtype == "f32" else "bf16")
        self.step_bytes = self.decode_bytes + self.append_bytes
        if self.split:
            used = int(sum(-(-int(L) // s.partition_size) for L in w.context_lens))
            self.scratch_bytes = perfmodel.split_scratch_bytes(w.B, s.Hq, s.D, used)
        else:
            self.scratch_bytes = 0

    def step(self):
        """One decode step as a serving loop issues it: one call (pa_append_decode),
        or append + split pass in one call (pa_append_decode_split) and the merge
        for the KV-split workload."""
        pa, s = self.pa, self.s
        if self.split:
            pa.append_decode_split(self.kn, self.vn, self.slots, self.q, self.cache, self.tables, self.lens, s.scale,
                                   s.partition_size, self.part_out, self.part_lse)
            pa.reduce(self.part_out, self.part_lse, self.lens, s.partition_size, self.out)
        else:
            pa.append_decode(self.kn, self.vn, self.slots, self.q, self.cache, self.tables, self.lens, s.scale,
                             self.out)

    def kernels(self):
        """The step's kernels, and the unfused calls, by name (each is timed alone)."""
        pa, s = self.pa, self.s
        ks = {}
        if self.split:
            ks["append_decode_split"] = lambda: pa.append_decode_split(
                self.kn, self.vn, self.slots, self.q, self.cache, self.tables, self.lens, s.scale, s.partition_size,
                self.part_out, self.part_lse)
            ks["reduce"] = lambda: pa.reduce(self.part_out, self.part_lse, self.lens, s.partition_size, self.out)
            ks["decode_split"] = lambda: pa.decode_split(self.q, self.cache, self.tables, self.lens, s.scale,
                                                         s.partition_size, self.part_out, self.part_lse)
        else:
            ks["decode"] = lambda: pa.decode(self.q, self.cache, self.tables, self.lens, s.scale, self.out)
        ks["append"] = lambda: pa.reshape_and_cache(self.kn, self.vn, self.slots, self.cache)
        return ks

    def decode_f32(self):
        """The same decode into an fp32 output (parity check of the timed path)."""
        torch, pa, s = self.torch, self.pa, self.s
        out = torch.empty(self.q.shape, dtype=torch.float32, device=self.q.device)
        if self.split:
            pa.decode_split(self.q, self.cache, self.tables, self.lens, s.scale, s.partition_size,
                            self.part_out, self.part_lse)
            pa.reduce(self.part_out, self.part_lse, self.lens, s.partition_size, out)
        else:
            pa.decode(self.q, self.cache, self.tables, self.lens, s.scale, out)
        torch.cuda.synchronize()
        return out

    def free(self):
        for name in ("cache", "q", "tables", "lens", "out", "part_out", "part_lse", "kn", "vn", "slots"):
            if hasattr(self, name):
                delattr(self, name)


class Flush:
    """Evicts the L2s and the Infinity Cache: one sequential pass of the
    library's read probe (ordinary loads) over a 1 GiB buffer, which leaves
    the caches holding clean lines only."""

    def __init__(self, torch, pa, mib: int, device):
        self.pa = pa
        self.buf = torch.ones(mib * (1 << 20) // 4, dtype=torch.int32, device=device)
        self.sink = torch.zeros(1, dtype=torch.int32, device=device)

    def __call__(self):
        self.pa.probe_read(self.buf, "seq", self.sink)


def stats_us(v) -> dict:
    """mean, median, p10, p90 of durations in ms, as microseconds."""
    v = sorted(v)
    return {"mean_us": 1e3 * sum(v) / len(v), "median_us": 1e3 * v[len(v) // 2],
            "p10_us": 1e3 * v[len(v) // 10], "p90_us": 1e3 * v[(9 * len(v)) // 10]}


SETTLE_S = 1.0  # set from --settle-s


def _timed(torch, fn, steps: int, warmup: int, flush, settle_s=None) -> list:
    """Durations (ms) of ``fn`` over ``steps`` calls, one event pair around each
    call, the caches flushed before each.  First the calls run untimed for at
    least ``settle_s`` seconds and ``warmup`` calls: after seconds of host
    work (filling a cache) the GPU's clocks have dropped, and the first calls
    measured up to 20 % slower than a serving loop's steady state."""
    t_end = time.perf_counter() + (SETTLE_S if settle_s is None else settle_s)
    while True:
        for _ in range(8):
            flush()
            fn()
        torch.cuda.synchronize()
        if time.perf_counter() >= t_end:
            break
    for _ in range(warmup):
        flush()
        fn()
    torch.cuda.synchronize()
    se = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in se:
        flush()  # evict L2 and Infinity Cache: the K/V reads come from HBM
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in se]


def time_case(case: Case, steps: int, warmup: int, flush) -> dict:
    """The step timed by one event pair around it; then each of its kernels
    timed alone in a loop of its own (events between back-to-back launches
    would add their own gaps to the kernels' times)."""
    torch = case.torch
    t0 = time.perf_counter()
    step = _timed(torch, case.step, steps, warmup, flush)
    wall = time.perf_counter() - t0
    r = {"step": stats_us(step), "wall_ms_per_step_incl_flush": 1e3 * wall / steps}
    ks = case.kernels()
    for name, fn in ks.items():
        r[name] = stats_us(_timed(torch, fn, steps, warmup, flush))
    if "decode" in ks and case.s.kv_dtype == "bf16" and case.s.D == 128 and case.s.G <= 16:
        # arithmetic A/B: the same pa_decode on the vector ALUs (PA_DECODE_VALU=1)
        os.environ["PA_DECODE_VALU"] = "1"
        try:
            r["decode_valu"] = stats_us(_timed(torch, ks["decode"], steps, warmup, flush))
        finally:
            del os.environ["PA_DECODE_VALU"]
    return r


# --------------------------------------------------------------------------
# read-bandwidth probe (the achievable HBM read rate for each access pattern)
# --------------------------------------------------------------------------


def probe_pattern(s) -> tuple:
    """The probe pattern of a workload's K/V gather: one (block, kv head) tile
    of K, read as the decode kernel reads it (non-temporal for bf16 tiles,
    ordinary loads for quantised ones)."""
    elem = {"f32": 4, "bf16": 2, "i8": 1, "i4": 0.5}[s.kv_dtype]
    tile = int(s.bs * s.D * elem)
    return ("tiles_nt" if s.kv_dtype in ("bf16", "f32") else "tiles", tile)


def run_probe(torch, pa, mib: int, steps: int, flush, patterns) -> dict:
    """Median read rate of pa_probe_read over a ``mib`` MiB buffer: one
    sequential pass (ordinary and non-temporal loads) and each (mode, tile
    bytes) pattern, the caches flushed before each pass."""
    dev = torch.device("cuda:0")
    buf = torch.ones(mib * (1 << 20) // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    res = {"buffer_mib": mib}
    todo = [("seq", 0), ("seq_nt", 0)] + sorted(set(patterns))
    for mode, tile in todo:
        nbytes = {}

        def run():
            nbytes["n"] = pa.probe_read(buf, mode, sink, tile_bytes=tile or 4096)

        t = stats_us(_timed(torch, run, steps, 3, flush))
        key = mode if not tile else f"{mode}_{tile}"
        res[key] = {"GBps": round(nbytes["n"] / t["median_us"] / 1e3, 1), "bytes": nbytes["n"],
                    "median_us": round(t["median_us"], 2)}
        log(f"probe {key}: {res[key]}")
    del buf, sink
    torch.cuda.empty_cache()
    return res


def time_copy_blocks(case: Case, steps: int, warmup: int, flush, max_pairs: int = 1024) -> dict:
    """pa_copy_blocks on the workload's pool: used blocks copied into unused ones
    (the copy of copy-on-write, at a batch size that fills the GPU)."""
    torch, pa = case.torch, case.pa
    import numpy as np

    used = case.w.used_blocks()
    free = np.setdiff1d(np.arange(case.w.num_blocks), used)
    n = int(min(max_pairs, len(used), len(free)))
    if n == 0:
        return {}
    rng = np.random.default_rng(5)
    pairs = np.stack([rng.choice(used, n, replace=False), rng.choice(free, n, replace=False)], axis=1)
    dev_pairs = torch.from_numpy(pairs.astype(np.int32)).to(case.q.device)
    us = stats_us(_timed(torch, lambda: pa.copy_blocks(case.cache, dev_pairs), steps, warmup, flush))["median_us"]
    s = case.s
    elem = {"f32": 4, "bf16": 2, "i8": 1, "i4": 0.5}[s.kv_dtype]
    per_block = int(s.Hkv * s.bs * s.D * elem * 2) + (s.Hkv * s.bs * 2 * 2 if s.kv_dtype in ("i8", "i4") else 0)
    moved = n * per_block * 2 + n * 8  # read and written, plus the pairs
    return {"pairs": n, "bytes": moved, "us": round(us, 2), "GBps": round(moved / us / 1e3, 1)}


def time_multi(case: Case, steps: int, warmup: int, flush, perfmodel, q_len: int = 4) -> dict:
    """pa_decode_multi on the workload's cache: q_len new tokens per sequence
    (a small chunked-prefill chunk, or q_len draft tokens to verify), each
    attending causally to the cached positions up to its own."""
    torch, pa, w, s = case.torch, case.pa, case.w, case.s
    import numpy as np
    from workloads.device import to_dev_values

    counts = np.minimum(w.context_lens, q_len).astype(np.int32)
    q_start, q = w.multi_queries(counts)
    dev = case.q.device
    qd = to_dev_values(q, s.q_dtype, dev)
    qs = torch.from_numpy(q_start).to(dev)
    out = torch.empty(qd.shape, dtype=case.out_dtype, device=dev)

    def run():
        pa.decode_multi(qd, qs, q_len, case.cache, case.tables, case.lens, s.scale, out)

    us = stats_us(_timed(torch, run, steps, warmup, flush))["median_us"]
    nbytes = perfmodel.multi_bytes(w.context_lens, counts, Hq=s.Hq, Hkv=s.Hkv, D=s.D, bs=s.bs,
                                   kv_dtype=s.kv_dtype, q_dtype=s.q_dtype,
                                   out_dtype="bf16" if case.out_dtype == torch.bfloat16 else "f32")
    return {"q_len": q_len, "query_rows": int(counts.sum()), "bytes": nbytes, "us": round(us, 2),
            "GBps": round(nbytes / us / 1e3, 1), "frac_of_peak": round(nbytes / us / 1e3 / perfmodel.HBM_PEAK_GBPS, 4)}


def time_swap(case: Case, steps: int, warmup: int, max_pairs: int = 1024) -> dict:
    """pa_swap_blocks: used blocks of the workload's pool out to a pinned host
    pool and back into unused GPU blocks (the preemption copy), timed per
    direction with HIP events."""
    torch, pa = case.torch, case.pa
    import numpy as np

    used = case.w.used_blocks()
    free = np.setdiff1d(np.arange(case.w.num_blocks), used)
    n = int(min(max_pairs, len(used), len(free)))
    if n == 0:
        return {}
    s = case.s
    host = pa.KVCache.allocate(n, s.Hkv, s.bs, s.D, s.kv_dtype, device="cpu")
    rng = np.random.default_rng(6)
    src = rng.choice(used, n, replace=False)
    dst = rng.choice(free, n, replace=False)
    dev = case.q.device
    out_pairs = torch.from_numpy(np.stack([src, np.arange(n)], 1).astype(np.int32)).to(dev)
    in_pairs = torch.from_numpy(np.stack([np.arange(n), dst], 1).astype(np.int32)).to(dev)
    res = {}
    for name, a, b, pairs in (("out", case.cache, host, out_pairs), ("in", host, case.cache, in_pairs)):
        for _ in range(warmup):
            pa.swap_blocks(a, b, pairs)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for e0, e1 in ev:
            e0.record()
            pa.swap_blocks(a, b, pairs)
            e1.record()
        torch.cuda.synchronize()
        us = stats_us([e0.elapsed_time(e1) for e0, e1 in ev])["median_us"]
        elem = {"f32": 4, "bf16": 2, "i8": 1, "i4": 0.5}[s.kv_dtype]
        per_block = int(s.Hkv * s.bs * s.D * elem * 2) + (s.Hkv * s.bs * 2 * 2 if s.kv_dtype in ("i8", "i4") else 0)
        res[name] = {"us": round(us, 2), "GBps": round(n * per_block / us / 1e3, 1)}
    res.update({"pairs": n, "bytes_each_way": n * per_block})
    del host
    return res


# multi-query shapes beyond the headline workload's 4-token step: (name, heads,
# kv heads, cached tokens per sequence, new tokens per sequence, sequences)
MULTI_SHAPES = [
    ("gqa70b-verify8", 64, 8, 2048, 8, 32),      # 8 draft tokens to verify, 70B-shaped heads
    ("mha13b-chunk512", 40, 40, 2048, 512, 8),   # 512-token chunked-prefill chunks, 13B-shaped heads
    ("gqa70b-chunk512", 64, 8, 2048, 512, 8),
]


def time_multi_shape(torch, pa, perfmodel, shape, steps: int, warmup: int, flush) -> dict:
    """pa_decode_multi on a synthetic cache of its own (bf16, D 128, bs 16)."""
    import numpy as np
    from workloads import make_custom
    from workloads.device import append_tokens, meta, to_dev_values

    name, Hq, Hkv, L, n, B = shape
    w = make_custom(B=B, Hq=Hq, Hkv=Hkv, D=128, bs=16, kv_dtype="bf16", lengths=[L] * B, seed=11)
    dev = torch.device("cuda:0")
    cache = pa.KVCache.allocate(w.num_blocks, Hkv, 16, 128, "bf16", dev)
    append_tokens(w, cache)
    counts = np.full(B, n, np.int32)
    q_start, q = w.multi_queries(counts)
    _, tables, lens = meta(w)
    qd = to_dev_values(q, "bf16")
    qs = torch.from_numpy(q_start).to(dev)
    out = torch.empty(qd.shape, dtype=torch.bfloat16, device=dev)

    def run():
        pa.decode_multi(qd, qs, n, cache, tables, lens, w.spec.scale, out)

    us = stats_us(_timed(torch, run, steps, warmup, flush))["median_us"]
    nbytes = perfmodel.multi_bytes(w.context_lens, counts, Hq=Hq, Hkv=Hkv, D=128, bs=16, kv_dtype="bf16",
                                   q_dtype="bf16", out_dtype="bf16")
    flops = perfmodel.multi_flops(w.context_lens, counts, Hq=Hq, D=128)
    del cache, qd, out
    torch.cuda.empty_cache()
    return {"q_len": n, "batch": B, "cached_tokens": L, "q_heads": Hq, "kv_heads": Hkv, "us": round(us, 2),
            "GBps": round(nbytes / us / 1e3, 1), "frac_of_hbm_peak": round(nbytes / us / 1e3 / perfmodel.HBM_PEAK_GBPS, 4),
            "TFLOPs": round(flops / us / 1e6, 1),
            "frac_of_mfma_peak": round(flops / us / 1e6 / perfmodel.MFMA_BF16_PEAK_TFLOPS, 4)}


# single-token decode with a whole MQA group on one kv head: (name, heads,
# kv heads, cached tokens per sequence, sequences, kv dtype)
MQA_SHAPES = [
    ("mqa64-bf16", 64, 1, 4096, 128, "bf16"),
    ("mqa64-int8", 64, 1, 4096, 128, "i8"),
    ("mqa32-bf16", 32, 1, 4096, 128, "bf16"),
]


def time_decode_shape(torch, pa, perfmodel, shape, steps: int, warmup: int, flush) -> dict:
    """pa_decode on a synthetic cache of its own (D 128, bs 16)."""
    from workloads import make_custom
    from workloads.device import append_tokens, meta

    name, Hq, Hkv, L, B, kv = shape
    w = make_custom(B=B, Hq=Hq, Hkv=Hkv, D=128, bs=16, kv_dtype=kv, lengths=[L] * B, seed=12)
    dev = torch.device("cuda:0")
    cache = pa.KVCache.allocate(w.num_blocks, Hkv, 16, 128, kv, dev)
    append_tokens(w, cache)
    q, tables, lens = meta(w)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)

    P = 512  # KV split: more work-groups than the 128-256 units of a single pass
    pmax = pa.max_partitions(tables.shape[1], 16, P)
    po = torch.empty((B, Hq, pmax, 128), dtype=torch.float32, device=dev)
    pl = torch.empty((B, Hq, pmax), dtype=torch.float32, device=dev)

    def single():
        pa.decode(q, cache, tables, lens, w.spec.scale, out)

    def split():
        pa.decode_split(q, cache, tables, lens, w.spec.scale, P, po, pl)
        pa.reduce(po, pl, lens, P, out)

    def timed(run):
        return stats_us(_timed(torch, run, steps, warmup, flush))["median_us"]

    us, us_split = timed(single), timed(split)
    nbytes = perfmodel.decode_bytes(w.context_lens, Hq=Hq, Hkv=Hkv, D=128, bs=16, kv_dtype=kv, q_dtype="bf16",
                                    out_dtype="bf16")
    del cache, out, po, pl
    torch.cuda.empty_cache()
    frac = lambda t: round(nbytes / t / 1e3 / perfmodel.HBM_PEAK_GBPS, 4)  # noqa: E731
    return {"batch": B, "cached_tokens": L, "q_heads": Hq, "kv_heads": Hkv, "kv_dtype": kv, "us": round(us, 2),
            "GBps": round(nbytes / us / 1e3, 1), "frac_of_hbm_peak": frac(us),
            "split_512_plus_merge_us": round(us_split, 2), "split_frac_of_hbm_peak": frac(us_split)}


def time_mla(torch, pa, perfmodel, steps: int, warmup: int, flush) -> dict:
    """pa_mla_decode on the MLA latent-cache batch (128 sequences of 1024-8192
    tokens, 16 heads of 128 over a 512-wide latent, bf16): one call = query
    absorption, the attention pass over the latent cache, merge and output
    projection.  Algorithmic bytes: every cached latent row once, the two
    up-projections, q, out and the tables."""
    from workloads import make_mla
    from workloads.device import mla_fill, mla_to_dev

    w = make_mla()
    s = w.spec
    dev = torch.device("cuda:0")
    t0 = time.time()
    cache = mla_fill(w, dev)
    torch.cuda.synchronize()
    log(f"mla: {s.name} B={w.B} tokens={w.total_tokens()} latent cache filled in {time.time() - t0:.1f}s")
    q, wk, wv = mla_to_dev(w.q, dev), mla_to_dev(w.w_uk, dev), mla_to_dev(w.w_uv, dev)
    tables = torch.from_numpy(w.block_tables).to(dev)
    lens = torch.from_numpy(w.context_lens).to(dev)
    P = s.partition_size
    ws = torch.empty(pa.mla_workspace_bytes(w.B, s.H, cache, tables.shape[1], P), dtype=torch.uint8, device=dev)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    t = stats_us(_timed(torch, lambda: pa.mla_decode(q, wk, wv, cache, tables, lens, s.scale, P, ws, out), steps,
                        warmup, flush))
    nbytes = perfmodel.mla_bytes(w.context_lens, H=s.H, d_h=s.d_h, d_c=s.d_c, bs=s.bs)
    flops = perfmodel.mla_flops(w.context_lens, H=s.H, d_h=s.d_h, d_c=s.d_c)
    us = t["median_us"]
    del cache, ws, out, q, wk, wv
    torch.cuda.empty_cache()
    return {"workload": s.name, "batch": w.B, "q_heads": s.H, "head_dim": s.d_h, "latent_dim": s.d_c,
            "block_size": s.bs, "partition_size": P, "cached_tokens": w.total_tokens(),
            "us": round(us, 2), "us_stats": {k: round(v, 2) for k, v in t.items()}, "bytes": nbytes,
            "GBps": round(nbytes / us / 1e3, 1), "frac_of_hbm_peak": round(nbytes / us / 1e3 / perfmodel.HBM_PEAK_GBPS, 4),
            "TFLOPs": round(flops / us / 1e6, 1),
            "frac_of_mfma_peak": round(flops / us / 1e6 / perfmodel.MFMA_BF16_PEAK_TFLOPS, 4)}


def summarise(case: Case, t: dict, peak: float, probe: dict) -> dict:
    """A workload's line: the step (median and spread), every kernel timed
    alone, and the roofline block of the step's dominant kernel."""
    s = case.s
    step = t["step"]
    med = step["median_us"]
    if case.split:
        # append + split pass in one kernel, then the merge
        dom_name, dom = "pa_append_decode_split", t["append_decode_split"]
        dom_bytes = case.split_kernel_bytes + case.append_bytes
    else:
        # the step is one pa_append_decode call: one fused kernel for these workloads
        dom_name, dom = "pa_append_decode", step
        dom_bytes = case.step_bytes
    achieved = dom_bytes / dom["mean_us"] / 1e3
    mode, tile = probe_pattern(s)
    pkey = f"{mode}_{tile}"
    probe_gbps = probe.get(pkey, {}).get("GBps") if probe else None
    traffic = measured_traffic(s.name)
    roofline = {
        "bound": "hbm",
        "kernel": dom_name,
        "achieved": round(achieved, 1),
        "peak": peak,
        "unit": "GB/s",
        "frac": round(achieved / peak, 4),
        "traffic": traffic["bytes"] if traffic else None,
        "algorithmic_bytes_per_launch": dom_bytes,
        "avg_launch_us": round(dom["mean_us"], 2),
        "median_launch_us": round(dom["median_us"], 2),
        "probe_pattern": pkey,
        "probe_GBps": probe_gbps,
        "frac_of_probe": round(achieved / probe_gbps, 4) if probe_gbps else None,
    }
    if traffic:
        roofline["traffic_source"] = traffic["source"]
        roofline["traffic_over_algorithmic"] = round(traffic["bytes"] / dom_bytes, 4)
    return {
        "workload": s.name,
        "us_per_step": round(med, 2),
        "step_GBps": round(case.step_bytes / med / 1e3, 1),
        "step_frac_of_peak": round(case.step_bytes / med / 1e3 / peak, 4),
        "step_us_stats": {k: round(v, 2) for k, v in step.items()},  # mean, median, p10, p90
        "kernel_mean_us": {k: round(v["mean_us"], 2) for k, v in t.items() if isinstance(v, dict)},
        "kernel_median_us": {k: round(v["median_us"], 2) for k, v in t.items() if isinstance(v, dict)},
        "roofline": roofline,
        "bytes": {"step": case.step_bytes, "decode": case.decode_bytes,
                  "decode_logical": case.decode_bytes_logical, "append": case.append_bytes,
                  "split_scratch_overhead": case.scratch_bytes},
    }


# --------------------------------------------------------------------------
# HBM traffic of the dominant kernel (from rocprofv3 counter passes)
# --------------------------------------------------------------------------

KERNEL_SOURCES = ("pa_decode_mfma.hip", "pa_device.h", "pa_append_row.h")


def kernel_source_hash() -> str:
    """sha256 over what the decode kernels are built from: their source file,
    the device helpers, the append row code the fused kernels share and the
    parameter struct they take."""
    import hashlib
    import re

    csrc = os.path.join(ROOT, "paged_kv_cache_443_amd", "csrc")
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    with open(os.path.join(csrc, "pa_internal.h"), encoding="utf-8") as f:
        m = re.search(r"struct DecodeParams \{.*?\};", f.read(), re.S)
    h.update(m.group(0).encode() if m else b"")
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch recorded in profiles/ for this workload's dominant
    kernel, or None when there is no record or the kernel sources changed since
    the counters were taken.  Record lines: ``key: value``."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path, encoding="utf-8") as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return {"bytes": int(float(rec["traffic_bytes_per_launch"])), "source": os.path.relpath(path, ROOT)}
    except (KeyError, ValueError):
        return None


# --------------------------------------------------------------------------
# CPU baseline: the oracle, one core, bounded sample
# --------------------------------------------------------------------------


def cpu_baseline(case: Case, budget_s: float, perfmodel, gpu_out_f32, min_s: float = 10.0,
                 max_seqs: int = 40) -> dict:
    """The oracle on one host core over a bounded sample of the timed
    workload: its first ``max_seqs`` sequences (the oracle's cache is built
    for those only, untimed), decoded in order until ``budget_s`` of work, and
    passed over again until ``min_s`` when one pass is shorter (the rate
    counts every sequence decoded; parity is checked on the first pass)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle

    w, s = case.w, case.s
    n = min(w.B, max_seqs)
    host_cores = os.cpu_count()
    allowed = sorted(os.sched_getaffinity(0))
    log(f"cpu baseline: building the oracle's cache for {n} sequences (not timed)")
    oc = oracle.build_cache(w, seqs=range(n))
    os.sched_setaffinity(0, {allowed[0]})
    done, work, secs, toks, errs, passes = [], [], 0.0, 0, [], 0
    try:
        with threadpool_limits(limits=1):
            while secs < min_s and secs < budget_s:
                passes += 1
                for b in range(n):
                    sl = [b]
                    t0 = time.perf_counter()
                    want = oracle.decode(w.q[sl], oc, w.block_tables[sl], w.context_lens[sl], s.scale)
                    secs += time.perf_counter() - t0
                    work.append(b)
                    if passes == 1:
                        done.append(b)
                        toks += int(w.context_lens[b])
                        errs.append(float(np.max(np.abs(gpu_out_f32[b].astype(np.float64) - want[0]))))
                    if secs >= budget_s:
                        break
    finally:
        os.sched_setaffinity(0, set(allowed))
    kw = dict(Hq=s.Hq, Hkv=s.Hkv, D=s.D, bs=s.bs, kv_dtype=s.kv_dtype, q_dtype=s.q_dtype,
              out_dtype="bf16" if s.q_dtype == "bf16" else "f32")
    work_bytes = perfmodel.decode_bytes(w.context_lens[work], **kw)  # every sequence decoded, repeats included
    work_tokens = int(w.context_lens[work].sum())
    return {
        "value": round(work_bytes / secs / 1e9, 3),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"oracle.decode (numpy fp64) over sequences 0..{done[-1]} of {w.B} ({toks} cached tokens) of "
                   f"the timed workload, {passes} pass(es), one host core of {host_cores}"),
        "seconds": round(secs, 2),
        "us_per_step_equiv": round(secs * 1e6 * w.total_tokens() / max(work_tokens, 1), 1),
        "parity_max_abs_err_vs_gpu_fp32_out": max(errs) if errs else None,
    }


# --------------------------------------------------------------------------


def main(argv=None) -> int:
    args = parse_args(argv)
    global SETTLE_S
    SETTLE_S = max(0.0, args.settle_s)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the paged-decode path has no "
                                   "cross-GPU step here (see the sharding notes); run with --gpus 1"}),
              flush=True)
        return 2

    log("importing torch")
    import torch

    import paged_kv_cache_443_amd as pa
    from paged_kv_cache_443_amd import _lib, perfmodel
    from workloads import CONFIGS

    if not torch.cuda.is_available():
        log("no GPU visible")
        return 1
    _lib.lib()  # fails loudly when the HIP library is not built
    peak = perfmodel.HBM_PEAK_GBPS
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    flush = Flush(torch, pa, args.flush_mib, dev)
    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)  # plain copy: copy_probe_mib MiB read, the same written
        torch.cuda.synchronize()
        del src, dst

    others = [int(c) for c in args.others.split(",") if c.strip()] if args.others else []
    others = [c for c in others if c != args.config]
    runs = [args.config] + others

    # read-bandwidth probe for every workload's tile pattern
    probe = {}
    if args.probe_mib > 0:
        pats = [probe_pattern(CONFIGS[c]) for c in runs]
        if 5 in runs:
            pats.append(probe_pattern(type(CONFIGS[5])(**{**CONFIGS[5].__dict__, "kv_dtype": "i4"})))
        probe = run_probe(torch, pa, args.probe_mib, min(args.steps, 20), flush, pats)

    # headline workload
    case = Case(args.config, args.seed, torch, pa, perfmodel)
    log(f"timing cfg{args.config}: {args.warmup} warmup + {args.steps} steps")
    t = time_case(case, args.steps, args.warmup, flush)
    head = summarise(case, t, peak, probe)
    log(f"cfg{args.config}: {head['us_per_step']} us/step (median), {head['step_GBps']} GB/s "
        f"({100 * head['step_frac_of_peak']:.1f}% of {peak:.0f}); dominant kernel "
        f"{head['roofline']['achieved']} GB/s")
    out32 = case.decode_f32().cpu().numpy()
    copy_stats = time_copy_blocks(case, args.steps, args.warmup, flush)
    log(f"copy_blocks: {copy_stats}")
    swap_stats = time_swap(case, min(args.steps, 10), min(args.warmup, 2))
    log(f"swap_blocks: {swap_stats}")
    # causal multi-query decode: quantised and bf16 caches (not the KV-split or fp32 workloads)
    multi = not case.split and case.s.kv_dtype != "f32"
    multi_stats = time_multi(case, args.steps, args.warmup, flush, perfmodel) if multi else {}
    log(f"decode_multi: {multi_stats}")

    s = case.s
    line = {
        "metric": METRIC,
        "value": head["step_GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us_per_step"] / 1e3, 5),
        "us_per_step": head["us_per_step"],
        "step_us_stats": head["step_us_stats"],
        "frac_of_hbm_peak": head["step_frac_of_peak"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.kv_dtype,
        "data": "synthetic",
        "config": {
            "workload": s.name,
            "batch": s.B, "q_heads": s.Hq, "kv_heads": s.Hkv, "head_dim": s.D, "block_size": s.bs,
            "kv_dtype": s.kv_dtype, "q_out_dtype": s.q_dtype, "cached_tokens": case.w.total_tokens(),
            "partition_size": s.partition_size, "seed": case.w.seed,
        },
        "kernel_mean_us": head["kernel_mean_us"],
        "kernel_median_us": head["kernel_median_us"],
        "bytes_per_step": head["bytes"],
        "roofline": head["roofline"],
        "probe": probe,
        "copy_blocks": copy_stats,
        "swap_blocks": swap_stats,
        "decode_multi": multi_stats,
    }

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds, perfmodel, out32)
    case.free()
    del case
    torch.cuda.empty_cache()

    if not args.no_multi_shapes:
        shapes = {}
        for shape in MULTI_SHAPES:
            shapes[shape[0]] = time_multi_shape(torch, pa, perfmodel, shape, args.steps, args.warmup, flush)
            log(f"decode_multi {shape[0]}: {shapes[shape[0]]}")
        multi_stats["shapes"] = shapes
        mqa = {}
        for shape in MQA_SHAPES:
            mqa[shape[0]] = time_decode_shape(torch, pa, perfmodel, shape, args.steps, args.warmup, flush)
            log(f"decode {shape[0]}: {mqa[shape[0]]}")
        line["decode_mqa"] = mqa
    if not args.no_mla:
        line["mla_decode"] = time_mla(torch, pa, perfmodel, args.steps, args.warmup, flush)
        log(f"mla_decode: {line['mla_decode']}")

    other = {}
    extra = [(c, {}) for c in others]
    if 5 in runs:
        # the int8 workload's shapes with an int4 cache (the other quantised KV format)
        extra.append((5, {"kv_dtype": "i4", "name": "int4kv-gqa-append"}))
    for c, kw in extra:
        key = f"cfg{c}" + ("-int4" if kw else "")
        oc = Case(c, None, torch, pa, perfmodel, **kw)
        log(f"timing {key}")
        ot = time_case(oc, args.steps, args.warmup, flush)
        other[key] = summarise(oc, ot, peak, probe)
        log(f"{key}: {other[key]['us_per_step']} us/step, {other[key]['step_GBps']} GB/s, dominant kernel "
            f"{other[key]['roofline']['frac']:.3f} of peak")
        oc.free()
        del oc
        torch.cuda.empty_cache()
    if other:
        line["other_workloads"] = other

    text = json.dumps(line)
    print(text, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(text + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
