"""Pure-Python (no numpy arithmetic) paged decode, for tiny inputs only.

TEST INFRASTRUCTURE (see ``oracle/__init__``).  Written independently of
``paged.decode``: scalar loops, explicit index arithmetic into the flat
storage of the pools, ``math.exp``.  It is the brute-force check that pins
the vectorised oracle.
"""
from __future__ import annotations

import math
import struct


def _bf16_to_float(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def decode_bruteforce(q, k_flat, v_flat, k_scale_flat, v_scale_flat, kv_dtype: str, Hkv: int, bs: int, D: int,
                      block_tables, context_lens, scale: float):
    """Same result as ``paged.decode`` from flat Python lists of the pools.

    ``q`` is a nested list ``[B][Hq][D]`` of floats; ``k_flat``/``v_flat`` are
    the pools flattened in storage order (ints for bf16 bit patterns and
    int8 codes, floats for fp32; for int4 the stored bytes, two codes each);
    scales likewise (floats) or None.
    """
    x = 16 if kv_dtype == "i4" else 16 // {"f32": 4, "bf16": 2, "i8": 1}[kv_dtype]
    quantised = kv_dtype in ("i8", "i4")
    B = len(q)
    Hq = len(q[0])
    G = Hq // Hkv

    def load(flat, idx):
        if kv_dtype == "i4":
            # element idx of the unpacked order is nibble idx % 2 (low first)
            # of byte idx // 2; a 4-bit two's-complement code
            nib = (int(flat[idx // 2]) >> (4 * (idx % 2))) & 0xF
            return float(nib - 16 if nib >= 8 else nib)
        raw = flat[idx]
        if kv_dtype == "bf16":
            return _bf16_to_float(raw)
        return float(raw)

    def k_at(pb, h, t, d):
        # K pool [nb][Hkv][D/x][bs][x]; bf16 tiles hold offset t at the slot
        # whose bits 2 and 3 are those of t exchanged
        slot = t
        if kv_dtype == "bf16":
            b2, b3 = (t >> 2) & 1, (t >> 3) & 1
            slot = t - 4 * b2 - 8 * b3 + 8 * b2 + 4 * b3
        idx = (((pb * Hkv + h) * (D // x) + d // x) * bs + slot) * x + d % x
        val = load(k_flat, idx)
        if quantised:
            val *= float(k_scale_flat[(pb * Hkv + h) * bs + t])
        return val

    def v_at(pb, h, t, d):
        # V pool [nb][Hkv][bs/x][D][x]
        idx = (((pb * Hkv + h) * (bs // x) + t // x) * D + d) * x + t % x
        val = load(v_flat, idx)
        if quantised:
            val *= float(v_scale_flat[(pb * Hkv + h) * bs + t])
        return val

    out = [[[0.0] * D for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        L = int(context_lens[b])
        for h in range(Hq):
            kv = h // G
            logits = []
            for t in range(L):
                pb = int(block_tables[b][t // bs])
                off = t % bs
                acc = 0.0
                for d in range(D):
                    acc += q[b][h][d] * k_at(pb, kv, off, d)
                logits.append(scale * acc)
            if L == 0:
                continue
            mx = max(logits)
            weights = [math.exp(s - mx) for s in logits]
            total = sum(weights)
            for d in range(D):
                num = 0.0
                for t in range(L):
                    pb = int(block_tables[b][t // bs])
                    num += weights[t] * v_at(pb, kv, t % bs, d)
                out[b][h][d] = num / total
    return out
