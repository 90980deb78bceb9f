"""Seeded generators for the paged-decode workloads.

Everything here is an input draw.  A workload is described *logically*:
per-sequence token K/V values by position, the block table each sequence
uses, the query vectors and the one new token each sequence appends in a
decode step.  How a block is laid out in memory, how tokens are written
into it, quantisation and attention itself are not in this module.

Recipe (all draws from numpy ``Generator(PCG64(...))``):

* stream ``[seed, cfg, 0]``: lengths, then the pool permutation;
* stream ``[seed, cfg, 1]``: the query vectors, N(0,1);
* stream ``[seed, cfg, 2, b]``: sequence ``b``'s K then V values, N(0,1),
  drawn as float32 arrays ``[L, Hkv, D]``; for the long-context workload
  the 1 % "peaked" positions follow (chosen without replacement, K scaled
  by 8 before rounding to the storage type).
* bf16 storage values are the round-to-nearest-even bf16 of the float32
  draw.

Beam pairs (prefix sharing): the second member of a pair has the first
member's length and the same token values at every position except the
last one (its own newly appended token, drawn from its own stream).  Its
block table repeats the first member's first ``S = min(ceil(L/32),
nblocks-1)`` entries -- the physically shared prefix blocks -- and the rest
of its blocks are private copies, so the last block (the copy-on-write
block holding the new token) always differs.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

# --------------------------------------------------------------------------
# bf16 storage helpers (storage-type rounding of synthetic draws)
# --------------------------------------------------------------------------


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    r = ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_from_bits(b: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 values (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest-even bf16 value, returned as float32."""
    return bf16_from_bits(bf16_bits(x))


def blocks_needed(length: int, block_size: int) -> int:
    """Blocks an allocator hands a sequence of ``length`` tokens (partial last block)."""
    return -(-int(length) // int(block_size))


# --------------------------------------------------------------------------
# workload descriptions
# --------------------------------------------------------------------------


@dataclass(frozen=True)
class WorkloadSpec:
    cfg: int
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    bs: int
    kv_dtype: str  # "f32" | "bf16" | "i8" | "i4"
    q_dtype: str  # "f32" | "bf16"
    scale: float
    max_len: int  # table width = ceil(max_len / bs)
    partition_size: Optional[int] = None
    pool_blocks: Optional[int] = None  # fixed pool size (else ceil(pool_factor * needed))
    pool_factor: float = 1.2
    beam_pair_frac: float = 0.0
    peak_frac: float = 0.0
    peak_scale: float = 8.0
    lengths: Optional[Tuple[int, ...]] = None  # explicit lengths
    len_dist: str = "explicit"  # "explicit" | "uniform" | "lognormal" | "fixed"
    len_lo: int = 0
    len_hi: int = 0
    ln_median: float = 512.0
    ln_sigma: float = 0.9
    v_scale: float = 1.0  # V draws multiplied by this (a power of two keeps them exact in bf16)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def max_blocks(self) -> int:
        return blocks_needed(self.max_len, self.bs)


CONFIGS: Dict[int, WorkloadSpec] = {
    1: WorkloadSpec(
        cfg=1, name="tiny-mha-f32", B=4, Hq=4, Hkv=4, D=64, bs=16,
        kv_dtype="f32", q_dtype="f32", scale=1.0 / math.sqrt(64), max_len=64,
        pool_blocks=16, lengths=(7, 16, 33, 40), len_dist="explicit",
    ),
    2: WorkloadSpec(
        cfg=2, name="llama13b-mha-bf16", B=64, Hq=40, Hkv=40, D=128, bs=16,
        kv_dtype="bf16", q_dtype="bf16", scale=1.0 / math.sqrt(128), max_len=2048,
        len_dist="uniform", len_lo=128, len_hi=2048,
    ),
    3: WorkloadSpec(
        cfg=3, name="70b-gqa-bf16-beams", B=128, Hq=64, Hkv=8, D=128, bs=16,
        kv_dtype="bf16", q_dtype="bf16", scale=1.0 / math.sqrt(128), max_len=4096,
        len_dist="lognormal", len_lo=32, len_hi=4096, ln_median=512.0, ln_sigma=0.9,
        beam_pair_frac=0.25,
    ),
    4: WorkloadSpec(
        cfg=4, name="longctx-gqa-bf16-split", B=8, Hq=32, Hkv=8, D=128, bs=64,
        kv_dtype="bf16", q_dtype="bf16", scale=1.0 / math.sqrt(128), max_len=32768,
        partition_size=512, len_dist="fixed", len_lo=32768, len_hi=32768,
        peak_frac=0.01, peak_scale=8.0,
    ),
    5: WorkloadSpec(
        cfg=5, name="int8kv-gqa-append", B=256, Hq=32, Hkv=8, D=128, bs=16,
        kv_dtype="i8", q_dtype="bf16", scale=1.0 / math.sqrt(128), max_len=8192,
        len_dist="uniform", len_lo=1024, len_hi=8192,
    ),
}

# Reduced-size variants with the same structure, for oracle-speed parity tests.
SMALL: Dict[int, dict] = {
    1: {},
    2: dict(B=6, max_len=700, len_lo=128, len_hi=700),
    3: dict(B=16, max_len=1024, len_hi=1024, ln_median=256.0),
    4: dict(B=2, max_len=4096, len_lo=4096, len_hi=4096, partition_size=512),
    5: dict(B=6, max_len=2048, len_lo=1024, len_hi=2048),
}


def default_seed(cfg: int) -> int:
    return 1000 + int(cfg)


# --------------------------------------------------------------------------
# the workload object
# --------------------------------------------------------------------------


@dataclass
class Workload:
    spec: WorkloadSpec
    seed: int
    context_lens: np.ndarray  # int32 [B]
    block_tables: np.ndarray  # int32 [B, max_blocks], -1 beyond the used entries
    num_blocks: int
    q: np.ndarray  # float32 [B, Hq, D], values exact in q dtype
    pair_of: Dict[int, int] = field(default_factory=dict)  # second member -> first member
    shared_blocks: Dict[int, int] = field(default_factory=dict)  # second member -> S

    # ---- convenience -----------------------------------------------------
    @property
    def B(self) -> int:
        return self.spec.B

    def _rng(self, *key: int) -> np.random.Generator:
        return np.random.Generator(np.random.PCG64([self.seed, self.spec.cfg, *key]))

    def _store(self, x: np.ndarray) -> np.ndarray:
        """Round float32 draws to the values the cache's source tensors hold."""
        if self.spec.kv_dtype == "f32":
            return x.astype(np.float32, copy=False)
        return bf16_round(x)

    def _draw_own(self, b: int, L: int) -> Tuple[np.ndarray, np.ndarray]:
        s = self.spec
        rng = self._rng(2, b)
        K = rng.standard_normal((L, s.Hkv, s.D), dtype=np.float32)
        V = rng.standard_normal((L, s.Hkv, s.D), dtype=np.float32)
        if s.peak_frac > 0.0 and L > 0:
            n_peak = int(round(s.peak_frac * L))
            pos = rng.choice(L, size=n_peak, replace=False)
            K[pos] *= np.float32(s.peak_scale)
        if s.v_scale != 1.0:
            V *= np.float32(s.v_scale)
        return self._store(K), self._store(V)

    def tokens(self, b: int) -> Tuple[np.ndarray, np.ndarray]:
        """All K/V token values of sequence ``b``: float32 ``[L, Hkv, D]`` each."""
        L = int(self.context_lens[b])
        if b in self.pair_of:
            K, V = self.tokens(self.pair_of[b])
            K = K.copy()
            V = V.copy()
            if L > 0:
                rng = self._rng(2, b)
                s = self.spec
                kn = rng.standard_normal((s.Hkv, s.D), dtype=np.float32)
                vn = rng.standard_normal((s.Hkv, s.D), dtype=np.float32) * np.float32(s.v_scale)
                K[L - 1] = self._store(kn)
                V[L - 1] = self._store(vn)
            return K, V
        return self._draw_own(b, L)

    def slots(self, b: int, start: int = 0, stop: Optional[int] = None) -> np.ndarray:
        """Slot ids (physical_block * bs + offset) of positions [start, stop) of ``b``."""
        L = int(self.context_lens[b])
        stop = L if stop is None else stop
        t = np.arange(start, stop, dtype=np.int64)
        bs = self.spec.bs
        return (self.block_tables[b, t // bs].astype(np.int64) * bs + t % bs).astype(np.int32)

    def new_tokens(self) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """The token each sequence appends this step (its position L-1).

        Returns K ``[B, Hkv, D]``, V ``[B, Hkv, D]`` (float32 values) and
        slots ``[B]`` (-1 for an empty sequence).
        """
        s = self.spec
        Kn = np.zeros((s.B, s.Hkv, s.D), np.float32)
        Vn = np.zeros((s.B, s.Hkv, s.D), np.float32)
        sl = np.full((s.B,), -1, np.int32)
        for b in range(s.B):
            L = int(self.context_lens[b])
            if L == 0:
                continue
            K, V = self.tokens(b)
            Kn[b], Vn[b] = K[L - 1], V[L - 1]
            sl[b] = self.slots(b, L - 1, L)[0]
        return Kn, Vn, sl

    def query_counts(self, max_q: int) -> np.ndarray:
        """New tokens per sequence for a multi-query step: uniform in
        [1, min(max_q, L)] (0 for an empty sequence), seeded."""
        rng = self._rng(3)
        hi = np.minimum(self.context_lens.astype(np.int64), int(max_q))
        n = rng.integers(1, np.maximum(hi, 1) + 1)
        return np.where(hi > 0, n, 0).astype(np.int32)

    def multi_queries(self, counts: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
        """Queries of a multi-query step: ``q_start [B + 1]`` (int32, the
        exclusive prefix sum of ``counts``) and ``q [total, Hq, D]`` (float32
        values exact in the q dtype), standard normal like ``q``."""
        s = self.spec
        counts = np.asarray(counts, np.int64)
        assert counts.shape == (s.B,) and np.all(counts >= 0)
        q_start = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        rng = self._rng(4)
        q = rng.standard_normal((int(q_start[-1]), s.Hq, s.D), dtype=np.float32)
        if s.q_dtype == "bf16":
            q = bf16_round(q)
        return q_start, q

    def used_blocks(self) -> np.ndarray:
        """Distinct physical blocks referenced by the valid table entries."""
        ids = [self.block_tables[b, : blocks_needed(int(L), self.spec.bs)] for b, L in enumerate(self.context_lens)]
        return np.unique(np.concatenate(ids)) if ids else np.zeros((0,), np.int32)

    def total_tokens(self) -> int:
        return int(np.sum(self.context_lens, dtype=np.int64))


# --------------------------------------------------------------------------
# construction
# --------------------------------------------------------------------------


def _draw_lengths(spec: WorkloadSpec, rng: np.random.Generator) -> np.ndarray:
    if spec.len_dist == "explicit":
        L = np.asarray(spec.lengths, dtype=np.int64)
        assert L.shape == (spec.B,)
    elif spec.len_dist == "fixed":
        L = np.full((spec.B,), spec.len_lo, dtype=np.int64)
    elif spec.len_dist == "uniform":
        L = rng.integers(spec.len_lo, spec.len_hi, endpoint=True, size=spec.B)
    elif spec.len_dist == "lognormal":
        z = rng.standard_normal(spec.B)
        L = np.rint(np.exp(math.log(spec.ln_median) + spec.ln_sigma * z)).astype(np.int64)
        L = np.clip(L, spec.len_lo, spec.len_hi)
    else:
        raise ValueError(spec.len_dist)
    assert L.max(initial=0) <= spec.max_len
    return L.astype(np.int32)


def _build(spec: WorkloadSpec, seed: int) -> Workload:
    rng = np.random.Generator(np.random.PCG64([seed, spec.cfg, 0]))
    lens = _draw_lengths(spec, rng)

    # beam pairs: (0,1), (2,3), ... over the first beam_pair_frac of the batch
    pair_of: Dict[int, int] = {}
    n_pair_seqs = int(round(spec.beam_pair_frac * spec.B)) // 2 * 2
    for a in range(0, n_pair_seqs, 2):
        pair_of[a + 1] = a
        lens[a + 1] = lens[a]

    nb = [blocks_needed(int(L), spec.bs) for L in lens]
    shared: Dict[int, int] = {}
    for b2, a in pair_of.items():
        shared[b2] = min(blocks_needed(int(lens[a]), 32), nb[a] - 1) if nb[a] > 0 else 0
    needed = sum(nb) - sum(shared.values())
    pool = spec.pool_blocks if spec.pool_blocks is not None else int(math.ceil(spec.pool_factor * needed))
    pool = max(pool, 1)
    assert pool >= needed, (pool, needed)
    perm = rng.permutation(pool).astype(np.int32)

    tables = np.full((spec.B, spec.max_blocks), -1, dtype=np.int32)
    nxt = 0
    for b in range(spec.B):
        S = shared.get(b, 0)
        if S:
            tables[b, :S] = tables[pair_of[b], :S]
        for j in range(S, nb[b]):
            tables[b, j] = perm[nxt]
            nxt += 1
    assert nxt == needed

    qrng = np.random.Generator(np.random.PCG64([seed, spec.cfg, 1]))
    q = qrng.standard_normal((spec.B, spec.Hq, spec.D), dtype=np.float32)
    if spec.q_dtype == "bf16":
        q = bf16_round(q)
    return Workload(spec=spec, seed=seed, context_lens=lens, block_tables=tables,
                    num_blocks=pool, q=q, pair_of=pair_of, shared_blocks=shared)


def make_workload(cfg: int, seed: Optional[int] = None, small: bool = False, **overrides) -> Workload:
    """Workload ``cfg`` (1..5) with its default seed ``1000 + cfg``.

    ``small=True`` keeps the structure (head counts, head_dim, block size,
    dtypes, sharing, peaks, split) but cuts batch and lengths so the fp64
    oracle runs in well under a second.
    """
    spec = CONFIGS[int(cfg)]
    kw = dict(SMALL[int(cfg)]) if small else {}
    kw.update(overrides)
    if kw:
        spec = WorkloadSpec(**{**spec.__dict__, **kw})
    return _build(spec, default_seed(cfg) if seed is None else int(seed))


def make_custom(*, B: int, Hq: int, Hkv: int, D: int, bs: int, kv_dtype: str, q_dtype: Optional[str] = None,
                lengths: Sequence[int], seed: int = 7, scale: Optional[float] = None, max_len: Optional[int] = None,
                pool_factor: float = 1.2, pool_blocks: Optional[int] = None, beam_pair_frac: float = 0.0,
                peak_frac: float = 0.0, partition_size: Optional[int] = None, cfg: int = 99,
                v_scale: float = 1.0) -> Workload:
    """A workload with explicit lengths and shapes (edge cases, sweeps)."""
    q_dtype = q_dtype or ("f32" if kv_dtype == "f32" else "bf16")
    lengths = tuple(int(x) for x in lengths)
    spec = WorkloadSpec(
        cfg=cfg, name="custom", B=B, Hq=Hq, Hkv=Hkv, D=D, bs=bs, kv_dtype=kv_dtype, q_dtype=q_dtype,
        scale=(1.0 / math.sqrt(D)) if scale is None else float(scale),
        max_len=max(max_len or 0, max(lengths, default=0), 1), partition_size=partition_size,
        pool_blocks=pool_blocks, pool_factor=pool_factor, beam_pair_frac=beam_pair_frac,
        peak_frac=peak_frac, lengths=lengths, len_dist="explicit", v_scale=float(v_scale),
    )
    return _build(spec, seed)
