"""ctypes view of ``libpa.so`` (the C ABI in include/pa.h).  No fallback:
if the library is missing or fails to load, every call raises."""
from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int, c_int32, c_size_t, c_void_p

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpa.so")

PA_OK = 0
PA_ERR_NULL_PTR = 1
PA_ERR_BAD_SHAPE = 2
PA_ERR_UNSUPPORTED = 3
PA_ERR_MISALIGNED = 4
PA_ERR_BAD_WORKSPACE = 5
PA_ERR_HIP = 6
PA_ERR_OUT_OF_BLOCKS = 7
PA_ERR_INVALID_BLOCK = 8

PA_F32 = 0
PA_BF16 = 1
PA_I8 = 2
PA_I4 = 3

EXPORTED = (
    "pa_reshape_and_cache",
    "pa_decode",
    "pa_append_decode",
    "pa_append_decode_split",
    "pa_decode_multi",
    "pa_decode_split",
    "pa_decode_split_noalloc",
    "pa_reduce",
    "pa_copy_blocks",
    "pa_swap_blocks",
    "pa_bm_create",
    "pa_bm_destroy",
    "pa_bm_num_free",
    "pa_bm_refcount",
    "pa_bm_allocate",
    "pa_bm_free",
    "pa_bm_fork",
    "pa_bm_append_slot",
    "pa_split_workspace_bytes",
    "pa_probe_read",
    "pa_mla_append",
    "pa_mla_workspace_bytes",
    "pa_mla_decode",
    "pa_status_string",
    "pa_last_hip_error",
)


class PaKvCache(ctypes.Structure):
    """Mirror of ``pa_kv_cache``."""

    _fields_ = [
        ("k_cache", c_void_p),
        ("v_cache", c_void_p),
        ("k_scale", c_void_p),
        ("v_scale", c_void_p),
        ("num_blocks", c_int32),
        ("num_kv_heads", c_int32),
        ("block_size", c_int32),
        ("head_dim", c_int32),
        ("kv_dtype", c_int),
    ]


class PaLatentCache(ctypes.Structure):
    """Mirror of ``pa_latent_cache``."""

    _fields_ = [
        ("latent", c_void_p),
        ("num_blocks", c_int32),
        ("block_size", c_int32),
        ("latent_dim", c_int32),
    ]


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded library, with argument types declared."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} not built: run `python -m paged_kv_cache_443_amd.build` "
                           "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(PaKvCache)
    L.pa_reshape_and_cache.argtypes = [c_void_p, c_void_p, c_int, c_void_p, c_int32, P, c_void_p]
    L.pa_reshape_and_cache.restype = c_int
    L.pa_decode.argtypes = [c_void_p, c_int, c_int32, c_int32, P, c_void_p, c_int32, c_void_p, c_float, c_void_p,
                            c_int, c_void_p]
    L.pa_decode.restype = c_int
    L.pa_append_decode.argtypes = [c_void_p, c_void_p, c_int, c_void_p, c_void_p, c_int, c_int32, c_int32, P,
                                   c_void_p, c_int32, c_void_p, c_float, c_void_p, c_int, c_void_p]
    L.pa_append_decode.restype = c_int
    L.pa_append_decode_split.argtypes = [c_void_p, c_void_p, c_int, c_void_p, c_void_p, c_int, c_int32, c_int32, P,
                                         c_void_p, c_int32, c_void_p, c_float, c_int32, c_int32, c_void_p, c_void_p,
                                         c_void_p]
    L.pa_append_decode_split.restype = c_int
    L.pa_decode_multi.argtypes = [c_void_p, c_int, c_int32, c_int32, c_void_p, c_int32, c_int32, P, c_void_p,
                                  c_int32, c_void_p, c_float, c_void_p, c_int, c_void_p]
    L.pa_decode_multi.restype = c_int
    L.pa_decode_split.argtypes = [c_void_p, c_int, c_int32, c_int32, P, c_void_p, c_int32, c_void_p, c_float,
                                  c_int32, c_int32, c_void_p, c_void_p, c_void_p]
    L.pa_decode_split.restype = c_int
    L.pa_decode_split_noalloc.argtypes = [c_void_p, c_int, c_int32, c_int32, P, c_void_p, c_int32, c_void_p, c_float,
                                          c_int32, c_void_p, c_int, c_void_p]
    L.pa_decode_split_noalloc.restype = c_int
    L.pa_reduce.argtypes = [c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p, c_int32, c_void_p,
                            c_int, c_void_p]
    L.pa_reduce.restype = c_int
    L.pa_copy_blocks.argtypes = [P, c_void_p, c_int32, c_void_p]
    L.pa_copy_blocks.restype = c_int
    L.pa_swap_blocks.argtypes = [P, P, c_void_p, c_int32, c_void_p]
    L.pa_swap_blocks.restype = c_int
    I32P = ctypes.POINTER(c_int32)
    L.pa_bm_create.argtypes = [c_int32, c_int32, ctypes.POINTER(c_void_p)]
    L.pa_bm_create.restype = c_int
    L.pa_bm_destroy.argtypes = [c_void_p]
    L.pa_bm_destroy.restype = None
    L.pa_bm_num_free.argtypes = [c_void_p]
    L.pa_bm_num_free.restype = c_int32
    L.pa_bm_refcount.argtypes = [c_void_p, c_int32]
    L.pa_bm_refcount.restype = c_int32
    L.pa_bm_allocate.argtypes = [c_void_p, c_int32, I32P]
    L.pa_bm_allocate.restype = c_int
    L.pa_bm_free.argtypes = [c_void_p, I32P, c_int32]
    L.pa_bm_free.restype = c_int
    L.pa_bm_fork.argtypes = [c_void_p, I32P, c_int32]
    L.pa_bm_fork.restype = c_int
    L.pa_bm_append_slot.argtypes = [c_void_p, I32P, I32P, c_int32, c_int32, I32P, I32P]
    L.pa_bm_append_slot.restype = c_int
    L.pa_split_workspace_bytes.argtypes = [c_int32, c_int32, c_int32, c_int32]
    L.pa_split_workspace_bytes.restype = c_size_t
    L.pa_probe_read.argtypes = [c_void_p, c_size_t, c_int32, c_int32, c_void_p, c_void_p]
    L.pa_probe_read.restype = c_int
    LP = ctypes.POINTER(PaLatentCache)
    L.pa_mla_append.argtypes = [c_void_p, c_void_p, c_int32, LP, c_void_p]
    L.pa_mla_append.restype = c_int
    L.pa_mla_workspace_bytes.argtypes = [c_int32, c_int32, c_int32, c_int32, c_int32, c_int32]
    L.pa_mla_workspace_bytes.restype = c_size_t
    L.pa_mla_decode.argtypes = [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p, LP, c_void_p, c_int32,
                                c_void_p, c_float, c_int32, c_void_p, c_size_t, c_void_p, c_int, c_void_p]
    L.pa_mla_decode.restype = c_int
    L.pa_status_string.argtypes = [c_int]
    L.pa_status_string.restype = ctypes.c_char_p
    L.pa_last_hip_error.argtypes = []
    L.pa_last_hip_error.restype = c_int32
    _LIB = L
    return L


def status_string(code: int) -> str:
    return lib().pa_status_string(code).decode()
