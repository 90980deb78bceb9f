"""The paged KV cache as host arrays, read and written element by element.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

Storage contract of the library (one pool for K, one for V, shared by all
sequences; a sequence reaches its blocks through its block table):

* ``x`` = number of elements in 16 bytes (fp32: 4, bf16: 8, int8: 16);
* K pool ``[num_blocks][Hkv][D/x][bs][x]``: K of (block pb, kv head h,
  in-block offset t, channel d) is ``K[pb, h, d // x, slot(t), d % x]``,
  where ``slot(t) = t`` for fp32 and int8 caches and, for bf16 caches,
  ``t`` with bits 2 and 3 exchanged (inside every group of 16 offsets the
  order is 0-3, 8-11, 4-7, 12-15);
* V pool ``[num_blocks][Hkv][bs/x][D][x]``: V of (pb, h, t, d) is
  ``V[pb, h, t // x, d, t % x]``;
* int8 only: fp16 scales ``[num_blocks][Hkv][bs]`` for K and for V.
* int4: the int8 layout with x = 16 codes per 8-byte vector: two 4-bit
  two's-complement codes per byte, the even element of a pair in the low
  nibble.  A K vector holds 16 channels of one token, a V vector 16 tokens
  of one channel; the fp16 scales are those of int8.  Here the codes are
  held unpacked (one int8 per code, same indexing as int8 with x = 16);
  ``packed_k`` / ``packed_v`` give the stored bytes.

Each (block, kv head) therefore owns ``bs * D`` contiguous elements of each
pool, and block ``pb`` of a single-head cache starts at element
``pb * bs * D`` -- the address the kernel sketch on page "字节跳动 AI Infra (2)"
(PagedAttention question) computes from the physical block id.

bf16 values are held as their uint16 bit patterns; this module converts
them to float64 itself (exactly).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

_ELEM_BYTES = {"f32": 4, "bf16": 2, "i8": 1}
_BF16_NAN = np.uint16(0x7FC0)
QUANTISED = ("i8", "i4")


def x_per_16b(kv_dtype: str) -> int:
    """Elements per storage vector (16 bytes; int4: 8 bytes of 16 codes)."""
    return 16 if kv_dtype == "i4" else 16 // _ELEM_BYTES[kv_dtype]


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """int4 codes ``[..., 2n]`` in [-8, 7] -> bytes ``[..., n]``, even element in the low nibble."""
    c = np.asarray(codes).astype(np.int16) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def k_slot(offs, kv_dtype: str):
    """Position inside a K tile's token axis of in-block offset(s) ``offs``.

    Identity for fp32 and int8 caches; bf16 caches exchange bits 2 and 3 of
    the offset.
    """
    if kv_dtype != "bf16":
        return offs
    o = np.asarray(offs)
    return (o & ~12) | ((o & 4) << 1) | ((o & 8) >> 1)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact float64 values."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f32_to_bf16_bits_exact(v: np.ndarray) -> np.ndarray:
    """float values that are exactly representable in bf16 -> bit patterns.

    Raises if any value would need rounding: the cache stores the source
    tensor's bf16 values unchanged, so its inputs must already be bf16.
    """
    f = np.ascontiguousarray(v, dtype=np.float32)
    u = f.view(np.uint32)
    if np.any((u & np.uint32(0xFFFF)) != 0):
        raise ValueError("value not representable in bf16")
    return (u >> np.uint32(16)).astype(np.uint16)


@dataclass
class PagedCache:
    kv_dtype: str
    num_blocks: int
    Hkv: int
    bs: int
    D: int
    k: np.ndarray
    v: np.ndarray
    k_scale: Optional[np.ndarray] = None
    v_scale: Optional[np.ndarray] = None

    @property
    def x(self) -> int:
        return x_per_16b(self.kv_dtype)

    @classmethod
    def empty(cls, kv_dtype: str, num_blocks: int, Hkv: int, bs: int, D: int, poison: bool = True) -> "PagedCache":
        """A pool whose every element is poison (NaN, or int8 -128 with NaN scales)."""
        x = x_per_16b(kv_dtype)
        assert D % x == 0 and bs % x == 0
        ks = (num_blocks, Hkv, D // x, bs, x)
        vs = (num_blocks, Hkv, bs // x, D, x)
        if kv_dtype == "f32":
            fill = np.float32(np.nan) if poison else np.float32(0)
            return cls(kv_dtype, num_blocks, Hkv, bs, D, np.full(ks, fill, np.float32), np.full(vs, fill, np.float32))
        if kv_dtype == "bf16":
            fill = _BF16_NAN if poison else np.uint16(0)
            return cls(kv_dtype, num_blocks, Hkv, bs, D, np.full(ks, fill, np.uint16), np.full(vs, fill, np.uint16))
        if kv_dtype in QUANTISED:
            # poison codes are outside what the quantiser writes (-128 / -8)
            fill = np.int8(-128 if kv_dtype == "i8" else -8) if poison else np.int8(0)
            sfill = np.float16(np.nan) if poison else np.float16(0)
            return cls(kv_dtype, num_blocks, Hkv, bs, D, np.full(ks, fill, np.int8), np.full(vs, fill, np.int8),
                       np.full((num_blocks, Hkv, bs), sfill, np.float16), np.full((num_blocks, Hkv, bs), sfill, np.float16))
        raise ValueError(kv_dtype)

    # ---- element access (float64) ---------------------------------------
    def k_rows(self, pbs: np.ndarray, h: int, offs: np.ndarray) -> np.ndarray:
        """K of tokens (pbs[i], offs[i]) of kv head h as float64 ``[n, D]``."""
        raw = self.k[pbs, h, :, k_slot(offs, self.kv_dtype), :].reshape(len(pbs), self.D)  # [n, D/x, x] -> [n, D]
        return self._to_f64(raw, self.k_scale, pbs, h, offs)

    def v_rows(self, pbs: np.ndarray, h: int, offs: np.ndarray) -> np.ndarray:
        """V of tokens (pbs[i], offs[i]) of kv head h as float64 ``[n, D]``."""
        x = self.x
        raw = self.v[pbs, h, offs // x, :, offs % x]  # [n, D]
        return self._to_f64(raw, self.v_scale, pbs, h, offs)

    def _to_f64(self, raw, scale, pbs, h, offs) -> np.ndarray:
        if self.kv_dtype == "f32":
            return raw.astype(np.float64)
        if self.kv_dtype == "bf16":
            return bf16_bits_to_f64(raw)
        s = scale[pbs, h, offs].astype(np.float64)  # fp16 -> f64 exact
        return raw.astype(np.float64) * s[:, None]

    # ---- element store ----------------------------------------------------
    def store(self, pbs: np.ndarray, offs: np.ndarray, kraw: np.ndarray, vraw: np.ndarray,
              kscale: Optional[np.ndarray] = None, vscale: Optional[np.ndarray] = None) -> None:
        """Store storage-typed rows ``[n, Hkv, D]`` at tokens (pbs[i], offs[i])."""
        n = len(pbs)
        x = self.x
        H = self.Hkv
        hh = np.arange(H)[None, :]
        P = pbs[:, None]
        O = offs[:, None]
        # K[pb, h, d//x, slot(t), d%x]
        self.k[P, hh, :, k_slot(O, self.kv_dtype), :] = kraw.reshape(n, H, self.D // x, x)
        # V[pb, h, t//x, d, t%x]
        self.v[P, hh, O // x, :, O % x] = vraw
        if self.kv_dtype in QUANTISED:
            self.k_scale[P, hh, O] = kscale
            self.v_scale[P, hh, O] = vscale

    # ---- int4 storage bytes ---------------------------------------------
    def packed_k(self) -> np.ndarray:
        """int4 K pool as stored: ``[num_blocks][Hkv][D/16][bs][8]`` bytes."""
        assert self.kv_dtype == "i4"
        return pack_nibbles(self.k)

    def packed_v(self) -> np.ndarray:
        """int4 V pool as stored: ``[num_blocks][Hkv][bs/16][D][8]`` bytes."""
        assert self.kv_dtype == "i4"
        return pack_nibbles(self.v)
