"""Symmetric int8 and int4 quantisation of one (token, kv head) row, fp16 scale.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

The pages name INT8 KV-cache quantisation (page "字节跳动 AI Infra (2)",
KV-cache optimisation table: INT8 halves KV memory; page "LLM推理优化",
section 1.3: K and V quantised from 16-bit floats to INT8) but fix no
rounding rule.  The reading used here (symmetric, one scale per row):

1. ``a`` = max over the row of |x| (x is a bf16 value, exact in float32);
2. ``s32`` = a / 127 as an IEEE float32 division;
3. ``s16`` = s32 rounded to fp16, nearest-even; this is the stored scale;
4. if ``s16`` is 0 every code is 0; otherwise each code is
   round-half-to-even(float32(x / float32(s16))), clamped to [-127, 127];
5. dequantised value = code * s16 (exact in float32).

The divisions that decide the integer codes are taken in float32, the
precision the kernel uses; tests pin that this equals rounding the exact
quotient for every bf16 x and fp16 scale in range.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def quantize_int8(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Quantise rows ``[..., D]`` of float32 values; return (codes int8, scales fp16)."""
    xf = np.asarray(x, dtype=np.float32)
    a = np.max(np.abs(xf), axis=-1)  # float32, exact
    s32 = (a / np.float32(127.0)).astype(np.float32)  # IEEE float32 divide
    s16 = s32.astype(np.float16)  # nearest-even
    sf = s16.astype(np.float32)
    nz = sf != 0
    safe = np.where(nz, sf, np.float32(1.0))
    qf = np.rint((xf / safe[..., None]).astype(np.float32))  # float32 quotient, ties-to-even
    qf = np.clip(qf, -127, 127)
    qf = np.where(nz[..., None], qf, 0)
    return qf.astype(np.int8), s16


def quantize_int4(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """INT4 rows (page "LLM推理优化", section 1.3, names INT4 next to INT8 for
    the KV cache and fixes nothing else).  The same reading as int8 with the
    symmetric 4-bit range: ``s32`` = a / 7, ``s16`` = fp16(s32), codes
    round-half-to-even(float32(x / s16)) clamped to [-7, 7], all 0 when s16 is
    0.  Returns (codes int8 in [-7, 7], scales fp16)."""
    xf = np.asarray(x, dtype=np.float32)
    a = np.max(np.abs(xf), axis=-1)
    s32 = (a / np.float32(7.0)).astype(np.float32)
    s16 = s32.astype(np.float16)
    sf = s16.astype(np.float32)
    nz = sf != 0
    safe = np.where(nz, sf, np.float32(1.0))
    qf = np.rint((xf / safe[..., None]).astype(np.float32))
    qf = np.clip(qf, -7, 7)
    qf = np.where(nz[..., None], qf, 0)
    return qf.astype(np.int8), s16


def dequantize_int8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """code * scale, float64 (exact)."""
    return codes.astype(np.float64) * scales.astype(np.float64)[..., None]
