"""Helpers for the GPU tests: move workloads and oracle caches onto the device.

Inputs always come from ``workloads`` or from the oracle (never from the
GPU path); outputs are compared with the oracle on the host.
"""
from __future__ import annotations

import sys
from concurrent.futures import ThreadPoolExecutor
from typing import Iterable, Optional

import numpy as np
import torch

import paged_kv_cache_443_amd as pa
from workloads import bf16_bits

DEV = "cuda:0"
TOL = {"f32": 2e-3, "bf16": 1.5e-2, "i8": 1.5e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _bf16_tensor(x: np.ndarray) -> torch.Tensor:
    """float32 values (exact in bf16) -> bf16 device tensor with the same values."""
    return torch.from_numpy(bf16_bits(x).view(np.int16)).to(DEV).view(torch.bfloat16)


def to_dev_values(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV)
    return _bf16_tensor(np.ascontiguousarray(x, np.float32))


def poisoned_cache(w) -> pa.KVCache:
    """Device pool of the workload's size, every element poison."""
    s = w.spec
    c = pa.KVCache.allocate(w.num_blocks, s.Hkv, s.bs, s.D, s.kv_dtype, DEV)
    fill_poison(c)
    return c


def fill_poison(c: pa.KVCache) -> None:
    if c.kv_dtype == "f32":
        c.k_cache.fill_(float("nan"))
        c.v_cache.fill_(float("nan"))
    elif c.kv_dtype == "bf16":
        c.k_cache.view(torch.int16).fill_(0x7FC0)
        c.v_cache.view(torch.int16).fill_(0x7FC0)
    else:
        c.k_cache.fill_(-128)
        c.v_cache.fill_(-128)
        c.k_scale.fill_(float("nan"))
        c.v_scale.fill_(float("nan"))


def upload_oracle_cache(oc) -> pa.KVCache:
    """Device copy of an oracle-built host cache (same layout, same bits)."""
    kv = oc.kv_dtype
    if kv == "bf16":
        k = torch.from_numpy(oc.k.view(np.int16)).to(DEV).view(torch.bfloat16)
        v = torch.from_numpy(oc.v.view(np.int16)).to(DEV).view(torch.bfloat16)
    else:
        k = torch.from_numpy(oc.k).to(DEV)
        v = torch.from_numpy(oc.v).to(DEV)
    ks = vs = None
    if kv == "i8":
        ks = torch.from_numpy(oc.k_scale).to(DEV)
        vs = torch.from_numpy(oc.v_scale).to(DEV)
    return pa.KVCache(k.contiguous(), v.contiguous(), ks, vs, oc.num_blocks, oc.Hkv, oc.bs, oc.D, kv)


def download_cache(c: pa.KVCache):
    """Host numpy copies of the pools in the oracle's storage dtypes."""
    if c.kv_dtype == "bf16":
        k = c.k_cache.view(torch.int16).cpu().numpy().view(np.uint16)
        v = c.v_cache.view(torch.int16).cpu().numpy().view(np.uint16)
    else:
        k = c.k_cache.cpu().numpy()
        v = c.v_cache.cpu().numpy()
    ks = vs = None
    if c.kv_dtype == "i8":
        ks = c.k_scale.cpu().numpy()
        vs = c.v_scale.cpu().numpy()
    return k, v, ks, vs


def meta(w):
    """Device q (in the workload's q dtype), block tables and context lengths."""
    s = w.spec
    q = to_dev_values(w.q, s.q_dtype)
    tables = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    return q, tables, lens


def gpu_append_tokens(w, cache: pa.KVCache, include_last: bool = True, seqs: Optional[Iterable[int]] = None,
                      workers: int = 8) -> None:
    """Write the workload's token values into ``cache`` through pa_reshape_and_cache."""
    s = w.spec
    seqs = list(range(s.B) if seqs is None else seqs)

    def host(b):
        L = int(w.context_lens[b])
        n = L if include_last else max(L - 1, 0)
        start = w.shared_blocks.get(b, 0) * s.bs if b in w.pair_of else 0
        if n <= start:
            return None
        K, V = w.tokens(b)
        return K[start:n], V[start:n], w.slots(b, start, n)

    with ThreadPoolExecutor(max_workers=workers) as ex:
        for r in ex.map(host, seqs):
            if r is None:
                continue
            K, V, sl = r
            kd = to_dev_values(K, "f32" if s.kv_dtype == "f32" else "bf16")
            vd = to_dev_values(V, "f32" if s.kv_dtype == "f32" else "bf16")
            pa.reshape_and_cache(kd, vd, torch.from_numpy(sl).to(DEV), cache)


def max_err(got: torch.Tensor, want: np.ndarray) -> float:
    g = got.float().cpu().numpy().astype(np.float64)
    return float(np.max(np.abs(g - want))) if g.size else 0.0


def bf16_rne_of(t32: torch.Tensor) -> torch.Tensor:
    """Round-to-nearest-even bf16 of an fp32 device tensor, via host integer math."""
    b = bf16_bits(t32.cpu().numpy())
    return torch.from_numpy(b.view(np.int16))
