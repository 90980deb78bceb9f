"""Paged-attention decode for AMD MI355X (gfx950): Python binding.

Thin marshalling layer over the C ABI of ``libpa.so`` (include/pa.h): each
function takes torch tensors, checks that they are contiguous device
tensors of the expected dtypes and shapes, and passes raw pointers, sizes
and the current HIP stream to the library entry point of the same name.
All computation happens in the library's HIP kernels; there is no CPU or
PyTorch fallback.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import PA_BF16, PA_F32, PA_I4, PA_I8, PaKvCache, PaLatentCache

__all__ = [
    "PAError",
    "KVCache",
    "reshape_and_cache",
    "decode",
    "append_decode",
    "append_decode_split",
    "decode_multi",
    "decode_split",
    "decode_split_noalloc",
    "reduce",
    "split_workspace_bytes",
    "probe_read",
    "LatentCache",
    "mla_append",
    "mla_workspace_bytes",
    "mla_decode",
    "max_partitions",
    "copy_blocks",
    "swap_blocks",
    "BlockManager",
    "OutOfBlocks",
]

_DT = {torch.float32: PA_F32, torch.bfloat16: PA_BF16, torch.int8: PA_I8}
_KV_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "i8": torch.int8, "i4": torch.uint8}
_ELEM = {"f32": 4, "bf16": 2, "i8": 1}
_QUANT = ("i8", "i4")


class PAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = _lib.status_string(status)
        if status == _lib.PA_ERR_HIP:
            msg += f" (hipError {_lib.lib().pa_last_hip_error()})"
        super().__init__(f"{fn}: {msg}")


def _check(fn: str, st: int) -> None:
    if st != _lib.PA_OK:
        raise PAError(fn, st)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, shape=None, host_ok: bool = False) -> None:
    if not (t.is_cuda or (host_ok and t.device.type == "cpu" and t.is_pinned())):
        raise ValueError(f"{name} must be a GPU tensor" + (" or pinned host memory" if host_ok else ""))
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


@dataclass
class KVCache:
    """One layer's paged KV cache: the two block pools (+ int8 scales).

    Shapes (x = elements per 16 bytes):
      k_cache [num_blocks, Hkv, head_dim // x, block_size, x]
      v_cache [num_blocks, Hkv, block_size // x, head_dim, x]
      k_scale, v_scale (int8 only): float16 [num_blocks, Hkv, block_size]
    bf16 K tiles keep in-block offset t at slot t with bits 2 and 3
    exchanged; write them through ``reshape_and_cache``.
    """

    k_cache: torch.Tensor
    v_cache: torch.Tensor
    k_scale: Optional[torch.Tensor]
    v_scale: Optional[torch.Tensor]
    num_blocks: int
    num_kv_heads: int
    block_size: int
    head_dim: int
    kv_dtype: str  # "f32" | "bf16" | "i8" | "i4"

    @property
    def x(self) -> int:
        """Elements per storage vector (int4: 16 codes in 8 bytes)."""
        return 16 if self.kv_dtype == "i4" else 16 // _ELEM[self.kv_dtype]

    @staticmethod
    def shapes(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int, kv_dtype: str):
        if kv_dtype == "i4":  # uint8 pools, two codes per byte
            return ((num_blocks, num_kv_heads, head_dim // 16, block_size, 8),
                    (num_blocks, num_kv_heads, block_size // 16, head_dim, 8),
                    (num_blocks, num_kv_heads, block_size))
        x = 16 // _ELEM[kv_dtype]
        return ((num_blocks, num_kv_heads, head_dim // x, block_size, x),
                (num_blocks, num_kv_heads, block_size // x, head_dim, x),
                (num_blocks, num_kv_heads, block_size))

    @classmethod
    def allocate(cls, num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int, kv_dtype: str,
                 device="cuda") -> "KVCache":
        """Uninitialised pools (torch.empty) of the library's layout.  ``device="cpu"``
        gives pinned host pools (the host side of ``swap_blocks``)."""
        ks, vs, ss = cls.shapes(num_blocks, num_kv_heads, block_size, head_dim, kv_dtype)
        dt = _KV_TORCH[kv_dtype]
        pin = torch.device(device).type == "cpu"
        k = torch.empty(ks, dtype=dt, device=device, pin_memory=pin)
        v = torch.empty(vs, dtype=dt, device=device, pin_memory=pin)
        sk = sv = None
        if kv_dtype in _QUANT:
            sk = torch.empty(ss, dtype=torch.float16, device=device, pin_memory=pin)
            sv = torch.empty(ss, dtype=torch.float16, device=device, pin_memory=pin)
        return cls(k, v, sk, sv, num_blocks, num_kv_heads, block_size, head_dim, kv_dtype)

    def descriptor(self, host_ok: bool = False) -> PaKvCache:
        """The C descriptor.  Pools must be on the GPU, or pinned host memory
        where ``host_ok`` (the swap)."""
        ks, vs, ss = self.shapes(self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim, self.kv_dtype)
        dt = _KV_TORCH[self.kv_dtype]
        _need(self.k_cache, "k_cache", dt, ks, host_ok)
        _need(self.v_cache, "v_cache", dt, vs, host_ok)
        if self.kv_dtype in _QUANT:
            _need(self.k_scale, "k_scale", torch.float16, ss, host_ok)
            _need(self.v_scale, "v_scale", torch.float16, ss, host_ok)
        return PaKvCache(_ptr(self.k_cache), _ptr(self.v_cache), _ptr(self.k_scale), _ptr(self.v_scale),
                         self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim,
                         {"f32": PA_F32, "bf16": PA_BF16, "i8": PA_I8, "i4": PA_I4}[self.kv_dtype])


def reshape_and_cache(key: torch.Tensor, value: torch.Tensor, slot_mapping: torch.Tensor, cache: KVCache) -> None:
    """Write tokens' K/V rows ``[T, Hkv, D]`` into slots ``slot_mapping[T]`` (int32, -1 skips)."""
    T = key.shape[0]
    src = torch.float32 if cache.kv_dtype == "f32" else torch.bfloat16
    _need(key, "key", src, (T, cache.num_kv_heads, cache.head_dim))
    _need(value, "value", src, (T, cache.num_kv_heads, cache.head_dim))
    _need(slot_mapping, "slot_mapping", torch.int32, (T,))
    desc = cache.descriptor()
    st = _lib.lib().pa_reshape_and_cache(_ptr(key), _ptr(value), _DT[src], _ptr(slot_mapping), T,
                                         ctypes.byref(desc), _stream(key.device))
    _check("pa_reshape_and_cache", st)


def _decode_args(q, cache, block_tables, context_lens):
    B, Hq, D = q.shape
    if D != cache.head_dim:
        raise ValueError("q head_dim differs from the cache's")
    _need(q, "q", (torch.float32, torch.bfloat16))
    _need(block_tables, "block_tables", torch.int32)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    _need(context_lens, "context_lens", torch.int32, (B,))
    return B, Hq, D


def decode(q: torch.Tensor, cache: KVCache, block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
           out: torch.Tensor) -> torch.Tensor:
    """Single-pass paged decode attention; writes and returns ``out`` ``[B, Hq, D]``."""
    B, Hq, D = _decode_args(q, cache, block_tables, context_lens)
    _need(out, "out", (torch.float32, torch.bfloat16), (B, Hq, D))
    desc = cache.descriptor()
    st = _lib.lib().pa_decode(_ptr(q), _DT[q.dtype], B, Hq, ctypes.byref(desc), _ptr(block_tables),
                              block_tables.shape[1], _ptr(context_lens), float(scale), _ptr(out), _DT[out.dtype],
                              _stream(q.device))
    _check("pa_decode", st)
    return out


def append_decode(key: torch.Tensor, value: torch.Tensor, slot_mapping: torch.Tensor, q: torch.Tensor, cache: KVCache,
                  block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float, out: torch.Tensor) -> torch.Tensor:
    """One decode step: write each sequence's new token (``key``/``value`` ``[B, Hkv, D]``, slots ``[B]``),
    then decode every sequence into ``out`` ``[B, Hq, D]``.  One kernel where the library fuses them."""
    B, Hq, D = _decode_args(q, cache, block_tables, context_lens)
    src = torch.float32 if cache.kv_dtype == "f32" else torch.bfloat16
    _need(key, "key", src, (B, cache.num_kv_heads, D))
    _need(value, "value", src, (B, cache.num_kv_heads, D))
    _need(slot_mapping, "slot_mapping", torch.int32, (B,))
    _need(out, "out", (torch.float32, torch.bfloat16), (B, Hq, D))
    desc = cache.descriptor()
    st = _lib.lib().pa_append_decode(_ptr(key), _ptr(value), _DT[src], _ptr(slot_mapping), _ptr(q), _DT[q.dtype], B, Hq,
                                     ctypes.byref(desc), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
                                     float(scale), _ptr(out), _DT[out.dtype], _stream(q.device))
    _check("pa_append_decode", st)
    return out


def append_decode_split(key: torch.Tensor, value: torch.Tensor, slot_mapping: torch.Tensor, q: torch.Tensor,
                        cache: KVCache, block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                        partition_size: int, part_out: torch.Tensor, part_lse: torch.Tensor) -> None:
    """One KV-split decode step: write each sequence's new token, then the split pass into
    ``part_out`` / ``part_lse`` (merge them with ``reduce``).  One kernel where the library fuses them."""
    B, Hq, D = _decode_args(q, cache, block_tables, context_lens)
    src = torch.float32 if cache.kv_dtype == "f32" else torch.bfloat16
    _need(key, "key", src, (B, cache.num_kv_heads, D))
    _need(value, "value", src, (B, cache.num_kv_heads, D))
    _need(slot_mapping, "slot_mapping", torch.int32, (B,))
    if part_out.dim() != 4:
        raise ValueError("part_out must be [num_seqs, num_heads, max_num_partitions, head_dim]")
    Pmax = part_out.shape[2]
    _need(part_out, "part_out", torch.float32, (B, Hq, Pmax, D))
    _need(part_lse, "part_lse", torch.float32, (B, Hq, Pmax))
    desc = cache.descriptor()
    st = _lib.lib().pa_append_decode_split(_ptr(key), _ptr(value), _DT[src], _ptr(slot_mapping), _ptr(q),
                                           _DT[q.dtype], B, Hq, ctypes.byref(desc), _ptr(block_tables),
                                           block_tables.shape[1], _ptr(context_lens), float(scale),
                                           int(partition_size), Pmax, _ptr(part_out), _ptr(part_lse),
                                           _stream(q.device))
    _check("pa_append_decode_split", st)


def decode_multi(q: torch.Tensor, q_start: torch.Tensor, max_q_len: int, cache: KVCache, block_tables: torch.Tensor,
                 context_lens: torch.Tensor, scale: float, out: torch.Tensor) -> torch.Tensor:
    """Causal paged attention of several new tokens per sequence.

    ``q`` and ``out`` are ``[num_queries, Hq, D]``; the new tokens of sequence
    b are rows ``q_start[b] .. q_start[b + 1] - 1`` (int32 ``[B + 1]``, device)
    and the last of its ``context_lens[b]`` cached positions.  ``max_q_len``
    bounds every sequence's count of new tokens.  Writes and returns ``out``.
    """
    NQ, Hq, D = q.shape
    if D != cache.head_dim:
        raise ValueError("q head_dim differs from the cache's")
    _need(q, "q", (torch.float32, torch.bfloat16))
    _need(block_tables, "block_tables", torch.int32)
    if block_tables.dim() != 2:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    B = block_tables.shape[0]
    _need(context_lens, "context_lens", torch.int32, (B,))
    _need(q_start, "q_start", torch.int32, (B + 1,))
    _need(out, "out", (torch.float32, torch.bfloat16), (NQ, Hq, D))
    desc = cache.descriptor()
    st = _lib.lib().pa_decode_multi(_ptr(q), _DT[q.dtype], B, Hq, _ptr(q_start), NQ, int(max_q_len),
                                    ctypes.byref(desc), _ptr(block_tables), block_tables.shape[1],
                                    _ptr(context_lens), float(scale), _ptr(out), _DT[out.dtype], _stream(q.device))
    _check("pa_decode_multi", st)
    return out


def max_partitions(max_blocks_per_seq: int, block_size: int, partition_size: int) -> int:
    """Smallest max_num_partitions pa_decode_split accepts for a table width."""
    return -(-(max_blocks_per_seq * block_size) // partition_size)


def decode_split(q: torch.Tensor, cache: KVCache, block_tables: torch.Tensor, context_lens: torch.Tensor,
                 scale: float, partition_size: int, part_out: torch.Tensor, part_lse: torch.Tensor) -> None:
    """KV-split first pass: ``part_out [B, Hq, Pmax, D]`` and ``part_lse [B, Hq, Pmax]`` (fp32)."""
    B, Hq, D = _decode_args(q, cache, block_tables, context_lens)
    if part_out.dim() != 4:
        raise ValueError("part_out must be [num_seqs, num_heads, max_num_partitions, head_dim]")
    Pmax = part_out.shape[2]
    _need(part_out, "part_out", torch.float32, (B, Hq, Pmax, D))
    _need(part_lse, "part_lse", torch.float32, (B, Hq, Pmax))
    desc = cache.descriptor()
    st = _lib.lib().pa_decode_split(_ptr(q), _DT[q.dtype], B, Hq, ctypes.byref(desc), _ptr(block_tables),
                                    block_tables.shape[1], _ptr(context_lens), float(scale), int(partition_size),
                                    Pmax, _ptr(part_out), _ptr(part_lse), _stream(q.device))
    _check("pa_decode_split", st)


def decode_split_noalloc(q: torch.Tensor, cache: KVCache, block_tables: torch.Tensor, context_lens: torch.Tensor,
                         scale: float, partition_size: int, out: torch.Tensor) -> torch.Tensor:
    """KV-split decode (split pass + merge) into ``out`` ``[B, Hq, D]`` with the partials in the library's
    own fixed device scratch (32 MiB per GPU): no workspace argument and no allocation.  Calls that
    overlap on one GPU race on that scratch."""
    B, Hq, D = _decode_args(q, cache, block_tables, context_lens)
    _need(out, "out", (torch.float32, torch.bfloat16), (B, Hq, D))
    desc = cache.descriptor()
    st = _lib.lib().pa_decode_split_noalloc(_ptr(q), _DT[q.dtype], B, Hq, ctypes.byref(desc), _ptr(block_tables),
                                            block_tables.shape[1], _ptr(context_lens), float(scale),
                                            int(partition_size), _ptr(out), _DT[out.dtype], _stream(q.device))
    _check("pa_decode_split_noalloc", st)
    return out


def reduce(part_out: torch.Tensor, part_lse: torch.Tensor, context_lens: torch.Tensor, partition_size: int,
           out: torch.Tensor) -> torch.Tensor:
    """KV-split second pass (log-sum-exp merge) into ``out`` ``[B, Hq, D]``."""
    B, Hq, Pmax, D = part_out.shape
    _need(part_out, "part_out", torch.float32)
    _need(part_lse, "part_lse", torch.float32, (B, Hq, Pmax))
    _need(context_lens, "context_lens", torch.int32, (B,))
    _need(out, "out", (torch.float32, torch.bfloat16), (B, Hq, D))
    st = _lib.lib().pa_reduce(_ptr(part_out), _ptr(part_lse), B, Hq, D, Pmax, _ptr(context_lens), int(partition_size),
                              _ptr(out), _DT[out.dtype], _stream(out.device))
    _check("pa_reduce", st)
    return out


@dataclass
class LatentCache:
    """One layer's paged MLA latent cache: ``latent`` bf16 ``[num_blocks, block_size, latent_dim]``."""

    latent: torch.Tensor
    num_blocks: int
    block_size: int
    latent_dim: int

    @classmethod
    def allocate(cls, num_blocks: int, block_size: int, latent_dim: int = 512, device="cuda") -> "LatentCache":
        t = torch.empty((num_blocks, block_size, latent_dim), dtype=torch.bfloat16, device=device)
        return cls(t, num_blocks, block_size, latent_dim)

    def descriptor(self) -> PaLatentCache:
        _need(self.latent, "latent", torch.bfloat16, (self.num_blocks, self.block_size, self.latent_dim))
        return PaLatentCache(_ptr(self.latent), self.num_blocks, self.block_size, self.latent_dim)


def mla_append(rows: torch.Tensor, slot_mapping: torch.Tensor, cache: LatentCache) -> None:
    """Write latent rows ``[T, latent_dim]`` (bf16) into slots ``slot_mapping[T]`` (int32, -1 skips)."""
    T = rows.shape[0]
    _need(rows, "rows", torch.bfloat16, (T, cache.latent_dim))
    _need(slot_mapping, "slot_mapping", torch.int32, (T,))
    desc = cache.descriptor()
    _check("pa_mla_append", _lib.lib().pa_mla_append(_ptr(rows), _ptr(slot_mapping), T, ctypes.byref(desc),
                                                     _stream(rows.device)))


def mla_workspace_bytes(num_seqs: int, num_heads: int, cache: LatentCache, max_blocks_per_seq: int,
                        partition_size: int) -> int:
    return int(_lib.lib().pa_mla_workspace_bytes(num_seqs, num_heads, cache.latent_dim, max_blocks_per_seq,
                                                 cache.block_size, partition_size))


def mla_decode(q: torch.Tensor, w_uk: torch.Tensor, w_uv: torch.Tensor, cache: LatentCache,
               block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float, partition_size: int,
               workspace: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    """Decode over an MLA latent cache: ``q`` bf16 ``[B, H, head_dim]``, up-projections ``w_uk`` / ``w_uv``
    bf16 ``[latent_dim, H * head_dim]``, a device ``workspace`` of at least ``mla_workspace_bytes`` bytes;
    writes and returns ``out`` ``[B, H, head_dim]`` (fp32 or bf16)."""
    B, H, D = q.shape
    _need(q, "q", torch.bfloat16)
    _need(w_uk, "w_uk", torch.bfloat16, (cache.latent_dim, H * D))
    _need(w_uv, "w_uv", torch.bfloat16, (cache.latent_dim, H * D))
    _need(block_tables, "block_tables", torch.int32)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    _need(context_lens, "context_lens", torch.int32, (B,))
    _need(workspace, "workspace")
    _need(out, "out", (torch.float32, torch.bfloat16), (B, H, D))
    desc = cache.descriptor()
    st = _lib.lib().pa_mla_decode(_ptr(q), B, H, D, _ptr(w_uk), _ptr(w_uv), ctypes.byref(desc), _ptr(block_tables),
                                  block_tables.shape[1], _ptr(context_lens), float(scale), int(partition_size),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out),
                                  _DT[out.dtype], _stream(q.device))
    _check("pa_mla_decode", st)
    return out


PROBE_MODES = {"seq": 0, "seq_nt": 1, "tiles": 2, "tiles_nt": 3}


def probe_read(buf: torch.Tensor, mode: str, sink: torch.Tensor, tile_bytes: int = 4096) -> int:
    """Read ``buf`` (a contiguous GPU tensor) once with the library's HBM read probe; returns the bytes read.

    ``mode``: "seq" / "seq_nt" (one sequential pass, ordinary / non-temporal loads) or "tiles" /
    "tiles_nt" (whole ``tile_bytes`` tiles in a scattered order, the largest power-of-two count that
    fits).  ``sink`` is a one-element int32 GPU tensor that keeps the loads live."""
    _need(buf, "buf")
    _need(sink, "sink", torch.int32)
    nbytes = buf.numel() * buf.element_size() // 16 * 16
    st = _lib.lib().pa_probe_read(_ptr(buf), nbytes, PROBE_MODES[mode], int(tile_bytes), _ptr(sink),
                                  _stream(buf.device))
    _check("pa_probe_read", st)
    if mode.startswith("seq"):
        return nbytes
    n = 1
    while n * 2 * tile_bytes <= nbytes:
        n *= 2
    return n * tile_bytes


def split_workspace_bytes(num_seqs: int, num_heads: int, head_dim: int, max_num_partitions: int) -> int:
    return int(_lib.lib().pa_split_workspace_bytes(num_seqs, num_heads, head_dim, max_num_partitions))


def copy_blocks(cache: KVCache, block_pairs: torch.Tensor) -> None:
    """Copy whole physical blocks: ``block_pairs`` int32 ``[n, 2]`` (source, destination) on the device."""
    _need(block_pairs, "block_pairs", torch.int32)
    if block_pairs.dim() != 2 or block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be [num_pairs, 2]")
    desc = cache.descriptor()
    st = _lib.lib().pa_copy_blocks(ctypes.byref(desc), _ptr(block_pairs), block_pairs.shape[0],
                                   _stream(block_pairs.device))
    _check("pa_copy_blocks", st)


def swap_blocks(src: KVCache, dst: KVCache, block_pairs: torch.Tensor, stream_device="cuda") -> None:
    """Copy whole blocks from pool ``src`` to pool ``dst`` (the same layout; either
    may be a pinned host pool from ``KVCache.allocate(..., device="cpu")``).
    ``block_pairs`` int32 ``[n, 2]`` (id in src, id in dst), on the GPU or
    pinned.  Runs on the current stream of ``stream_device``; synchronise
    before reading a host destination."""
    _need(block_pairs, "block_pairs", torch.int32, host_ok=True)
    if block_pairs.dim() != 2 or block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be [num_pairs, 2]")
    ds, dd = src.descriptor(host_ok=True), dst.descriptor(host_ok=True)
    st = _lib.lib().pa_swap_blocks(ctypes.byref(ds), ctypes.byref(dd), _ptr(block_pairs), block_pairs.shape[0],
                                   _stream(torch.device(stream_device)))
    _check("pa_swap_blocks", st)


class OutOfBlocks(PAError):
    pass


def _i32_array(values):
    n = len(values)
    arr = (ctypes.c_int32 * max(n, 1))(*values)
    return arr, n


class BlockManager:
    """Host bookkeeping of a block pool through the library's C++ block manager.

    Reference counts, on-demand allocation (lowest free id first), fork and
    copy-on-write; ``append_slot`` returns the slot for a sequence's next
    token and the (source, destination) block copies to run first
    (``copy_blocks``).  Tables are Python lists of block ids.
    """

    def __init__(self, num_blocks: int, block_size: int):
        self._h = ctypes.c_void_p()
        self.block_size = int(block_size)
        st = _lib.lib().pa_bm_create(int(num_blocks), int(block_size), ctypes.byref(self._h))
        _check("pa_bm_create", st)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            _lib.lib().pa_bm_destroy(h)
            self._h = None

    @staticmethod
    def _raise(fn: str, st: int) -> None:
        if st == _lib.PA_ERR_OUT_OF_BLOCKS:
            raise OutOfBlocks(fn, st)
        _check(fn, st)

    def num_free(self) -> int:
        return int(_lib.lib().pa_bm_num_free(self._h))

    def refcount(self, block: int) -> int:
        return int(_lib.lib().pa_bm_refcount(self._h, int(block)))

    def allocate(self, n: int):
        arr, _ = _i32_array([0] * n)
        self._raise("pa_bm_allocate", _lib.lib().pa_bm_allocate(self._h, int(n), arr))
        return [int(arr[i]) for i in range(n)]

    def free(self, ids) -> None:
        arr, n = _i32_array(list(ids))
        self._raise("pa_bm_free", _lib.lib().pa_bm_free(self._h, arr, n))

    def fork(self, table):
        arr, n = _i32_array(list(table))
        self._raise("pa_bm_fork", _lib.lib().pa_bm_fork(self._h, arr, n))
        return list(table)

    def append_slot(self, table: list, length: int):
        """Room for the token at position ``length``; ``table`` is updated in place.
        Returns (slot, copies) with copies a list of (source, destination)."""
        cap = len(table) + 1
        arr, _ = _i32_array(list(table) + [0])
        tlen = ctypes.c_int32(len(table))
        slot = ctypes.c_int32(0)
        pair = (ctypes.c_int32 * 2)()
        self._raise("pa_bm_append_slot", _lib.lib().pa_bm_append_slot(
            self._h, arr, ctypes.byref(tlen), cap, int(length), ctypes.byref(slot), pair))
        table[:] = [int(arr[i]) for i in range(tlen.value)]
        copies = [(int(pair[0]), int(pair[1]))] if pair[0] >= 0 else []
        return int(slot.value), copies
