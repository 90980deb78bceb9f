"""The library's storage order of a paged cache: a codec between the
oracle's logical blocks and the bytes of the pools.

TEST INFRASTRUCTURE (see ``oracle/__init__``).  Nothing in the oracle's
arithmetic goes through this module: tests use it to hand an oracle-built
cache to the library (``pools``) and to read a library-written cache back
(``from_pools``).  Written from the storage contract stated in ``pa.h``:

* ``x`` = elements in one 16-byte vector (fp32: 4, bf16: 8, int8: 16); int4:
  16 codes in one 8-byte vector;
* K pool ``[num_blocks][Hkv][D/x][bs][x]``: K of (block pb, kv head h,
  in-block offset t, channel d) is ``K[pb, h, d // x, slot(t), d % x]``,
  where ``slot(t) = t`` except for bf16, whose slot is ``t`` with bits 2
  and 3 exchanged (in every 16 offsets the order 0-3, 8-11, 4-7, 12-15);
* V pool ``[num_blocks][Hkv][bs/x][D][x]``: V of (pb, h, t, d) is
  ``V[pb, h, t // x, d, t % x]``;
* int4: two 4-bit two's-complement codes per byte, the even element of a
  pair in the low nibble (a K vector: 16 channels of one token; a V vector:
  16 tokens of one channel);
* int8 / int4 scales: fp16 ``[num_blocks][Hkv][bs]``, as the oracle holds
  them.

Each (block, kv head) owns ``bs * D`` contiguous elements of each pool, so
block ``pb`` of a single-head cache starts at element ``pb * bs * D``: the
address the kernel sketch on page "字节跳动 AI Infra (2)" (PagedAttention
question) computes from the physical block id.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .layout import PagedCache

_ELEM_BYTES = {"f32": 4, "bf16": 2, "i8": 1}


def x_per_16b(kv_dtype: str) -> int:
    """Elements per storage vector (16 bytes; int4: 8 bytes of 16 codes)."""
    return 16 if kv_dtype == "i4" else 16 // _ELEM_BYTES[kv_dtype]


def k_slot(offs, kv_dtype: str):
    """Position on a K tile's token axis of in-block offset(s) ``offs``.

    Identity except for bf16 caches, which exchange bits 2 and 3.
    """
    if kv_dtype != "bf16":
        return offs
    o = np.asarray(offs)
    return (o & ~12) | ((o & 4) << 1) | ((o & 8) >> 1)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """int4 codes ``[..., 2n]`` in [-8, 7] -> bytes ``[..., n]``, even element in the low nibble."""
    c = np.asarray(codes).astype(np.int16) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(b: np.ndarray) -> np.ndarray:
    """Inverse of ``pack_nibbles``: bytes ``[..., n]`` -> int8 codes ``[..., 2n]``."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int16)
    lo, hi = b & 0xF, b >> 4
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.int16)
    out[..., 0::2], out[..., 1::2] = lo, hi
    return np.where(out >= 8, out - 16, out).astype(np.int8)


def pools(cache: PagedCache) -> Tuple[np.ndarray, np.ndarray]:
    """The K and V pools of ``cache`` in the library's memory order (bf16 as
    uint16 bits, int4 as the packed bytes); the scales need no reordering."""
    kv, bs, D = cache.kv_dtype, cache.bs, cache.D
    x = x_per_16b(kv)
    nb, H = cache.num_blocks, cache.Hkv
    if D % x or bs % x:
        raise ValueError("head_dim and block_size must be multiples of the vector width")
    # K: [nb][H][bs][D] -> [nb][H][D/x][bs][x], offset t at slot(t)
    k = cache.k.reshape(nb, H, bs, D // x, x).transpose(0, 1, 3, 2, 4)
    kp = np.empty_like(k)
    kp[:, :, :, k_slot(np.arange(bs), kv), :] = k
    # V: [nb][H][bs][D] -> [nb][H][bs/x][D][x]
    vp = np.ascontiguousarray(cache.v.reshape(nb, H, bs // x, x, D).transpose(0, 1, 2, 4, 3))
    if kv == "i4":
        return pack_nibbles(kp), pack_nibbles(vp)
    return kp, vp


def from_pools(kv_dtype: str, k_pool: np.ndarray, v_pool: np.ndarray, k_scale: Optional[np.ndarray],
               v_scale: Optional[np.ndarray], num_blocks: int, Hkv: int, bs: int, D: int) -> PagedCache:
    """The logical cache held by pools in the library's memory order (the
    inverse of ``pools``)."""
    x = x_per_16b(kv_dtype)
    kp = np.asarray(k_pool)
    vp = np.asarray(v_pool)
    if kv_dtype == "i4":
        kp, vp = unpack_nibbles(kp), unpack_nibbles(vp)
    kp = kp.reshape(num_blocks, Hkv, D // x, bs, x)
    vp = vp.reshape(num_blocks, Hkv, bs // x, D, x)
    k = kp[:, :, :, k_slot(np.arange(bs), kv_dtype), :].transpose(0, 1, 3, 2, 4).reshape(num_blocks, Hkv, bs, D)
    v = vp.transpose(0, 1, 2, 4, 3).reshape(num_blocks, Hkv, bs, D)
    ks = None if k_scale is None else np.array(k_scale, copy=True)
    vs = None if v_scale is None else np.array(v_scale, copy=True)
    return PagedCache(kv_dtype, num_blocks, Hkv, bs, D, np.ascontiguousarray(k), np.ascontiguousarray(v), ks, vs)
