"""Helpers for the GPU tests: move workloads and oracle caches onto the device.

Inputs always come from ``workloads`` or from the oracle (never from the
GPU path); outputs are compared with the oracle on the host.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import paged_kv_cache_443_amd as pa
from workloads import bf16_bits
from workloads.device import (DEV, append_tokens, fill_poison, meta, poisoned_cache,  # noqa: F401
                              to_dev_values)

gpu_append_tokens = append_tokens

TOL = {"f32": 2e-3, "bf16": 1.5e-2, "i8": 1.5e-2, "i4": 1.5e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_pools(oc):
    """The pools of an oracle-built cache in the library's memory order
    (bf16 bits, int8 codes, int4 bytes), through the oracle's storage codec."""
    return oracle.storage.pools(oc)


def upload_oracle_cache(oc) -> pa.KVCache:
    """Device copy of an oracle-built host cache (the library's layout, same bits)."""
    kv = oc.kv_dtype
    kp, vp = oracle_pools(oc)
    if kv == "bf16":
        k = torch.from_numpy(kp.view(np.int16)).to(DEV).view(torch.bfloat16)
        v = torch.from_numpy(vp.view(np.int16)).to(DEV).view(torch.bfloat16)
    else:  # fp32 values, int8 codes, int4 bytes (two codes each)
        k = torch.from_numpy(kp).to(DEV)
        v = torch.from_numpy(vp).to(DEV)
    ks = vs = None
    if kv in ("i8", "i4"):
        ks = torch.from_numpy(oc.k_scale).to(DEV)
        vs = torch.from_numpy(oc.v_scale).to(DEV)
    return pa.KVCache(k.contiguous(), v.contiguous(), ks, vs, oc.num_blocks, oc.Hkv, oc.bs, oc.D, kv)


def download_cache(c: pa.KVCache):
    """Host numpy copies of the pools in the oracle's storage dtypes (int4: the stored bytes)."""
    if c.kv_dtype == "bf16":
        k = c.k_cache.view(torch.int16).cpu().numpy().view(np.uint16)
        v = c.v_cache.view(torch.int16).cpu().numpy().view(np.uint16)
    else:
        k = c.k_cache.cpu().numpy()
        v = c.v_cache.cpu().numpy()
    ks = vs = None
    if c.kv_dtype in ("i8", "i4"):
        ks = c.k_scale.cpu().numpy()
        vs = c.v_scale.cpu().numpy()
    return k, v, ks, vs


def max_err(got: torch.Tensor, want: np.ndarray) -> float:
    g = got.float().cpu().numpy().astype(np.float64)
    return float(np.max(np.abs(g - want))) if g.size else 0.0


def bf16_rne_of(t32: torch.Tensor) -> torch.Tensor:
    """Round-to-nearest-even bf16 of an fp32 device tensor, via host integer math."""
    b = bf16_bits(t32.cpu().numpy())
    return torch.from_numpy(b.view(np.int16))
