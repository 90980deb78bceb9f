"""The paged KV cache as host arrays, read and written element by element.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

One pool of physical blocks holds every sequence's K and V; a sequence
reaches its blocks through its block table (page "字节跳动 AI Infra (2)",
PagedAttention question: block pool and block table).  The oracle holds the
pool logically, in the plainest order:

* K and V ``[num_blocks][Hkv][bs][D]``: element (block pb, kv head h,
  in-block offset t, channel d) at ``[pb, h, t, d]``, in the storage type:
  fp32 values, bf16 bit patterns (uint16), int8 codes, or int4 codes (one
  int8 per code, in [-8, 7]);
* int8 / int4 only: fp16 scales ``[num_blocks][Hkv][bs]`` for K and for V
  (one per token and kv head).

How the library orders these elements in memory is a separate codec
(``oracle.storage``, written from the storage contract in ``pa.h``); the
decode arithmetic here never sees it.  bf16 values are held as their uint16
bit patterns; this module converts them to float64 itself (exactly).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

_BF16_NAN = np.uint16(0x7FC0)
QUANTISED = ("i8", "i4")
_DTYPES = ("f32", "bf16", "i8", "i4")


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

    @classmethod
    def empty(cls, kv_dtype: str, num_blocks: int, Hkv: int, bs: int, D: int, poison: bool = True) -> "PagedCache":
        """A pool whose every element is poison (NaN, or int8 -128 with NaN scales)."""
        if kv_dtype not in _DTYPES:
            raise ValueError(kv_dtype)
        ks = vs = (num_blocks, Hkv, bs, D)
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
        raw = self.k[pbs, h, offs, :]  # [n, D]
        return self._to_f64(raw, self.k_scale, pbs, h, offs)

    def v_rows(self, pbs: np.ndarray, h: int, offs: np.ndarray) -> np.ndarray:
        """V of tokens (pbs[i], offs[i]) of kv head h as float64 ``[n, D]``."""
        raw = self.v[pbs, h, offs, :]  # [n, D]
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
        hh = np.arange(self.Hkv)[None, :]
        P = pbs[:, None]
        O = offs[:, None]
        self.k[P, hh, O, :] = kraw
        self.v[P, hh, O, :] = vraw
        if self.kv_dtype in QUANTISED:
            self.k_scale[P, hh, O] = kscale
            self.v_scale[P, hh, O] = vscale
