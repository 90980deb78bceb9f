"""Seeded synthetic decode batches over an MLA latent cache.

MLA (multi-head latent attention) caches one compressed vector c per token
instead of per-head K and V; the heads' keys and values are recovered from
it by learned up-projections at inference (page "字节跳动 AI Infra (2)",
question on KV-cache principles, the MLA paragraph: c = X W_down into 512
dimensions, K = c W_up_K into num_heads x head_dim).  There are no trained
weights here: the up-projections are seeded draws like everything else.

This module only draws inputs (lengths, a block pool with block tables,
latent rows, queries and the two up-projection matrices); it holds none of
the attention arithmetic and no cache layout.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence, Tuple

import numpy as np

from .gen import bf16_round, blocks_needed


@dataclass(frozen=True)
class MlaSpec:
    name: str
    B: int
    H: int                # query heads
    d_h: int              # head_dim of the recovered K and V
    d_c: int              # latent width (the cached vector)
    bs: int               # tokens per block
    max_len: int
    len_dist: str = "uniform"  # "uniform" | "explicit"
    len_lo: int = 0
    len_hi: int = 0
    lengths: Tuple[int, ...] = field(default_factory=tuple)
    pool_factor: float = 1.2
    partition_size: int = 512  # tokens per attention piece (the fastest of 256..1024 on the benchmark batch)
    cfg: int = 6          # seed stream key (after the five K/V workloads)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d_h)

    @property
    def max_blocks(self) -> int:
        return blocks_needed(self.max_len, self.bs)


# One GPU's decode batch of an MLA layer: 16 query heads of head_dim 128 over
# the 512-wide latent the pages name, 128 sequences of 1024-8192 tokens.
MLA_CONFIG = MlaSpec(name="mla-latent-gqa16", B=128, H=16, d_h=128, d_c=512, bs=16, max_len=8192,
                     len_lo=1024, len_hi=8192)
MLA_SMALL = dict(B=5, max_len=1500, len_lo=300, len_hi=1500)


@dataclass
class MlaWorkload:
    spec: MlaSpec
    seed: int
    context_lens: np.ndarray  # int32 [B]
    block_tables: np.ndarray  # int32 [B, max_blocks], -1 beyond the used entries
    num_blocks: int
    q: np.ndarray             # float32 [B, H, d_h], bf16 values
    w_uk: np.ndarray          # float32 [d_c, H * d_h], bf16 values: K = c W_uk
    w_uv: np.ndarray          # float32 [d_c, H * d_h], bf16 values: V = c W_uv

    @property
    def B(self) -> int:
        return self.spec.B

    def _rng(self, *key: int) -> np.random.Generator:
        return np.random.Generator(np.random.PCG64([self.seed, self.spec.cfg, *key]))

    def latent(self, b: int) -> np.ndarray:
        """Latent rows of every cached token of sequence ``b``: float32 ``[L, d_c]`` (bf16 values)."""
        L = int(self.context_lens[b])
        c = self._rng(2, b).standard_normal((L, self.spec.d_c), dtype=np.float32)
        return bf16_round(c)

    def slots(self, b: int, start: int = 0, stop: Optional[int] = None) -> np.ndarray:
        """Slot ids (physical_block * bs + offset) of positions [start, stop) of ``b``."""
        L = int(self.context_lens[b])
        stop = L if stop is None else stop
        t = np.arange(start, stop, dtype=np.int64)
        bs = self.spec.bs
        return (self.block_tables[b, t // bs].astype(np.int64) * bs + t % bs).astype(np.int32)

    def used_blocks(self) -> np.ndarray:
        ids = [self.block_tables[b, : blocks_needed(int(L), self.spec.bs)] for b, L in enumerate(self.context_lens)]
        return np.unique(np.concatenate(ids)) if ids else np.zeros((0,), np.int32)

    def total_tokens(self) -> int:
        return int(np.sum(self.context_lens, dtype=np.int64))


def make_mla(seed: int = 1006, small: bool = False, **overrides) -> MlaWorkload:
    """The MLA decode batch (``small``: a few short sequences with the same head shapes)."""
    kw = dict(MLA_SMALL) if small else {}
    kw.update(overrides)
    spec = replace(MLA_CONFIG, **kw) if kw else MLA_CONFIG
    return build_mla(spec, seed)


def make_mla_custom(*, H: int, d_h: int, d_c: int, bs: int, lengths: Sequence[int], seed: int = 9,
                    partition_size: int = 1024, max_len: Optional[int] = None,
                    pool_factor: float = 1.2) -> MlaWorkload:
    lengths = tuple(int(x) for x in lengths)
    spec = MlaSpec(name="mla-custom", B=len(lengths), H=H, d_h=d_h, d_c=d_c, bs=bs,
                   max_len=max(max_len or 0, max(lengths, default=0), 1), len_dist="explicit", lengths=lengths,
                   partition_size=partition_size, pool_factor=pool_factor)
    return build_mla(spec, seed)


def build_mla(spec: MlaSpec, seed: int) -> MlaWorkload:
    rng = np.random.Generator(np.random.PCG64([seed, spec.cfg, 0]))
    if spec.len_dist == "explicit":
        lens = np.asarray(spec.lengths, np.int64)
        assert lens.shape == (spec.B,)
    else:
        lens = rng.integers(spec.len_lo, spec.len_hi, endpoint=True, size=spec.B)
    assert lens.max(initial=0) <= spec.max_len
    lens = lens.astype(np.int32)
    nb = [blocks_needed(int(L), spec.bs) for L in lens]
    needed = sum(nb)
    pool = max(int(math.ceil(spec.pool_factor * needed)), 1)
    perm = rng.permutation(pool).astype(np.int32)
    tables = np.full((spec.B, spec.max_blocks), -1, dtype=np.int32)
    nxt = 0
    for b in range(spec.B):
        tables[b, : nb[b]] = perm[nxt: nxt + nb[b]]
        nxt += nb[b]
    qrng = np.random.Generator(np.random.PCG64([seed, spec.cfg, 1]))
    q = bf16_round(qrng.standard_normal((spec.B, spec.H, spec.d_h), dtype=np.float32))
    # up-projections with unit-variance outputs for unit-variance latents
    wrng = np.random.Generator(np.random.PCG64([seed, spec.cfg, 3]))
    s = np.float32(1.0 / math.sqrt(spec.d_c))
    w_uk = bf16_round(wrng.standard_normal((spec.d_c, spec.H * spec.d_h), dtype=np.float32) * s)
    w_uv = bf16_round(wrng.standard_normal((spec.d_c, spec.H * spec.d_h), dtype=np.float32) * s)
    return MlaWorkload(spec=spec, seed=seed, context_lens=lens, block_tables=tables, num_blocks=pool, q=q,
                       w_uk=w_uk, w_uv=w_uv)
