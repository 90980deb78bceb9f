"""The C ABI library on the host: it loads, exports every declared symbol,
and rejects invalid arguments before any launch (no GPU needed: every call
here fails validation, so nothing reaches the HIP runtime)."""
import ctypes
import os
import re

import pytest

from paged_kv_cache_443_amd import _lib
from paged_kv_cache_443_amd._lib import (PA_BF16, PA_ERR_BAD_SHAPE, PA_ERR_BAD_WORKSPACE, PA_ERR_MISALIGNED,
                                         PA_ERR_NULL_PTR, PA_ERR_UNSUPPORTED, PA_F32, PA_I4, PA_I8, PA_OK, PaKvCache,
                                         PaLatentCache)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

# fake, never-dereferenced device addresses with chosen alignment
A = 0x7F0000000000
A16 = [A + 0x1000 * i for i in range(1, 16)]


def _cache(kv=PA_BF16, nb=8, H=2, bs=16, D=128, k=A16[0], v=A16[1], ks=None, vs=None):
    if kv in (PA_I8, PA_I4) and ks is None:
        ks, vs = A16[2], A16[3]
    return PaKvCache(k, v, ks, vs, nb, H, bs, D, kv)


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_exports_every_declared_symbol(L):
    text = "".join(open(h, encoding="utf-8").read() for h in HEADERS)
    declared = set(re.findall(r"^(?:pa_status|size_t|const char \*|int32_t|void)\s*(pa_\w+)\(", text, re.M))
    assert declared == set(_lib.EXPORTED)
    for name in declared:
        assert hasattr(L, name), name


def test_status_strings(L):
    for code in range(9):
        s = _lib.status_string(code)
        assert s and s != "unknown status"
    assert _lib.status_string(99) == "unknown status"
    assert L.pa_last_hip_error() == 0


def test_workspace_bytes(L):
    n = L.pa_split_workspace_bytes(8, 32, 128, 64)
    out_bytes = 8 * 32 * 64 * 128 * 4
    assert n == (out_bytes + 255) // 256 * 256 + 8 * 32 * 64 * 4
    assert L.pa_split_workspace_bytes(0, 1, 64, 1) == 256 * 0 + 0
    assert L.pa_split_workspace_bytes(-1, 1, 64, 1) == 0


def _decode(L, cache, q=A16[4], qdt=PA_BF16, B=4, Hq=8, tables=A16[5], mbps=8, lens=A16[6], scale=0.1,
            out=A16[7], odt=PA_F32):
    return L.pa_decode(q, qdt, B, Hq, ctypes.byref(cache), tables, mbps, lens, scale, out, odt, None)


def test_decode_rejections(L):
    c = _cache()
    assert _decode(L, c, q=None) == PA_ERR_NULL_PTR
    assert _decode(L, c, tables=None) == PA_ERR_NULL_PTR
    assert _decode(L, c, lens=None) == PA_ERR_NULL_PTR
    assert _decode(L, c, out=None) == PA_ERR_NULL_PTR
    assert L.pa_decode(A16[4], PA_BF16, 4, 8, None, A16[5], 8, A16[6], 0.1, A16[7], PA_F32, None) == PA_ERR_NULL_PTR
    assert _decode(L, _cache(k=None)) == PA_ERR_NULL_PTR
    assert _decode(L, _cache(ks=A16[2])) == PA_ERR_NULL_PTR  # scales on a bf16 cache
    assert _decode(L, PaKvCache(A16[0], A16[1], None, None, 8, 2, 16, 128, PA_I8)) == PA_ERR_NULL_PTR  # int8 without scales
    assert _decode(L, PaKvCache(A16[0], A16[1], None, None, 8, 2, 16, 128, PA_I4)) == PA_ERR_NULL_PTR  # int4 without scales
    assert _decode(L, _cache(kv=PA_I4), qdt=PA_F32) == PA_ERR_UNSUPPORTED  # f32 q with an int4 cache
    assert _decode(L, _cache(kv=PA_I4), odt=PA_I4) == PA_ERR_UNSUPPORTED
    assert _decode(L, _cache(kv=4)) == PA_ERR_UNSUPPORTED  # no such dtype
    assert _decode(L, c, B=-1) == PA_ERR_BAD_SHAPE
    assert _decode(L, c, Hq=0) == PA_ERR_BAD_SHAPE
    assert _decode(L, c, Hq=7) == PA_ERR_BAD_SHAPE  # not a multiple of Hkv
    assert _decode(L, c, mbps=0) == PA_ERR_BAD_SHAPE
    assert _decode(L, c, scale=float("nan")) == PA_ERR_BAD_SHAPE
    assert _decode(L, c, mbps=2 ** 30) == PA_ERR_BAD_SHAPE  # max length overflows int32
    assert _decode(L, _cache(nb=0)) == PA_ERR_BAD_SHAPE
    assert _decode(L, _cache(bs=8)) == PA_ERR_UNSUPPORTED
    assert _decode(L, _cache(D=96)) == PA_ERR_UNSUPPORTED
    assert _decode(L, _cache(kv=7)) == PA_ERR_UNSUPPORTED
    assert _decode(L, c, qdt=PA_I8) == PA_ERR_UNSUPPORTED
    assert _decode(L, c, qdt=PA_F32) == PA_ERR_UNSUPPORTED  # f32 q with a bf16 cache
    assert _decode(L, _cache(kv=PA_F32), odt=PA_BF16, qdt=PA_F32) == PA_ERR_UNSUPPORTED
    assert _decode(L, c, odt=PA_I8) == PA_ERR_UNSUPPORTED
    # dtype arguments outside the enumerators (C callers pass plain ints)
    assert _decode(L, c, qdt=9) == PA_ERR_UNSUPPORTED
    assert _decode(L, c, odt=-1) == PA_ERR_UNSUPPORTED
    assert _decode(L, c, q=A16[4] + 8) == PA_ERR_MISALIGNED
    assert _decode(L, c, out=A16[7] + 4) == PA_ERR_MISALIGNED
    assert _decode(L, c, tables=A16[5] + 2) == PA_ERR_MISALIGNED
    assert _decode(L, _cache(k=A16[0] + 8)) == PA_ERR_MISALIGNED
    assert _decode(L, _cache(kv=PA_I8, ks=A16[2] + 4, vs=A16[3])) == PA_ERR_MISALIGNED
    # zero sequences is a no-op that never touches the (null) pointers
    assert L.pa_decode(None, PA_BF16, 0, 8, ctypes.byref(c), None, 8, None, 0.1, None, PA_F32, None) == PA_OK


def _multi(L, cache, qs=A16[10], nq=6, mq=3, B=4, Hq=8, q=A16[4], out=A16[7], odt=PA_F32):
    return L.pa_decode_multi(q, PA_BF16, B, Hq, qs, nq, mq, ctypes.byref(cache), A16[5], 8, A16[6], 0.1, out, odt,
                             None)


def test_multi_rejections(L):
    c = _cache()
    assert _multi(L, c, qs=None) == PA_ERR_NULL_PTR
    assert _multi(L, c, q=None) == PA_ERR_NULL_PTR
    assert _multi(L, c, out=None) == PA_ERR_NULL_PTR
    assert _multi(L, _cache(kv=PA_F32)) == PA_ERR_UNSUPPORTED  # bf16 q with an f32 cache
    assert _multi(L, c, mq=0) == PA_ERR_BAD_SHAPE
    assert _multi(L, c, nq=-1) == PA_ERR_BAD_SHAPE
    assert _multi(L, c, nq=13, mq=3) == PA_ERR_BAD_SHAPE  # more rows than num_seqs * max_q_len
    assert _multi(L, c, mq=2 ** 30, nq=6) == PA_ERR_BAD_SHAPE  # rows per kv head overflow int32
    assert _multi(L, c, qs=A16[10] + 2) == PA_ERR_MISALIGNED
    assert _multi(L, c, odt=PA_I8) == PA_ERR_UNSUPPORTED
    assert _multi(L, c, Hq=7) == PA_ERR_BAD_SHAPE
    # no rows, or no sequences: a no-op that never touches the (null) pointers
    assert _multi(L, c, nq=0, qs=None, out=None) == PA_OK
    assert L.pa_decode_multi(None, PA_BF16, 0, 8, None, 0, 1, ctypes.byref(c), None, 8, None, 0.1, None, PA_F32,
                             None) == PA_OK


def test_swap_rejections(L):
    g, h = _cache(nb=8), _cache(nb=3, k=A16[11], v=A16[12])

    def swap(src=g, dst=h, pairs=A16[13], n=2):
        return L.pa_swap_blocks(ctypes.byref(src), ctypes.byref(dst), pairs, n, None)

    assert swap(pairs=None) == PA_ERR_NULL_PTR
    assert swap(pairs=A16[13] + 2) == PA_ERR_MISALIGNED
    assert swap(n=-1) == PA_ERR_BAD_SHAPE
    assert swap(dst=_cache(nb=3, k=A16[11], v=A16[12], bs=32)) == PA_ERR_BAD_SHAPE  # layouts differ
    assert swap(dst=_cache(nb=3, k=A16[11], v=A16[12], D=64)) == PA_ERR_BAD_SHAPE
    assert swap(dst=_cache(nb=3, k=A16[11], v=A16[12], H=4)) == PA_ERR_BAD_SHAPE
    assert swap(dst=_cache(kv=PA_I8, nb=3, k=A16[11], v=A16[12])) == PA_ERR_BAD_SHAPE
    assert swap(dst=_cache(nb=3, k=None)) == PA_ERR_NULL_PTR
    assert swap(src=_cache(k=A16[0] + 8)) == PA_ERR_MISALIGNED
    assert L.pa_swap_blocks(None, ctypes.byref(h), A16[13], 2, None) == PA_ERR_NULL_PTR
    assert swap(pairs=None, n=0) == PA_OK  # no pairs: a no-op


def _split(L, cache, P=512, Pmax=1, po=A16[8], pl=A16[9], mbps=8, B=4):
    return L.pa_decode_split(A16[4], PA_BF16, B, 8, ctypes.byref(cache), A16[5], mbps, A16[6], 0.1, P, Pmax, po, pl,
                             None)


def test_split_rejections(L):
    c = _cache(bs=64)
    assert _split(L, c, P=0) == PA_ERR_BAD_SHAPE
    assert _split(L, c, P=96) == PA_ERR_BAD_SHAPE  # not a multiple of block_size
    assert _split(L, c, Pmax=0) == PA_ERR_BAD_SHAPE
    assert _split(L, c, P=128, Pmax=3) == PA_ERR_BAD_WORKSPACE  # 8*64 tokens need 4 partitions of 128
    assert _split(L, c, P=128, Pmax=4, po=None) == PA_ERR_NULL_PTR
    assert _split(L, c, P=128, Pmax=4, pl=None) == PA_ERR_NULL_PTR
    assert _split(L, c, P=128, Pmax=4, po=A16[8] + 4) == PA_ERR_MISALIGNED
    assert _split(L, c, P=128, Pmax=4, pl=A16[9] + 2) == PA_ERR_MISALIGNED
    assert _split(L, c, P=128, Pmax=4, B=0) == PA_OK  # no-op


def _noalloc(L, cache, B=4, Hq=8, mbps=8, P=512, out=A16[7], odt=PA_F32):
    return L.pa_decode_split_noalloc(A16[4], PA_BF16, B, Hq, ctypes.byref(cache), A16[5], mbps, A16[6], 0.1, P, out,
                                     odt, None)


def test_split_noalloc_rejections(L):
    c = _cache(bs=64)
    assert _noalloc(L, c, P=0) == PA_ERR_BAD_SHAPE
    assert _noalloc(L, c, P=96) == PA_ERR_BAD_SHAPE  # not a multiple of block_size
    assert _noalloc(L, c, out=None) == PA_ERR_NULL_PTR
    assert _noalloc(L, c, out=A16[7] + 4) == PA_ERR_MISALIGNED
    assert _noalloc(L, c, odt=PA_I8) == PA_ERR_UNSUPPORTED
    # partials beyond the 32 MiB scratch: 64 seqs x 64 heads x 64 partitions x (128 + 1) floats
    assert _noalloc(L, _cache(bs=64, H=8), B=64, Hq=64, mbps=512, P=512) == PA_ERR_BAD_WORKSPACE
    assert _noalloc(L, c, B=0, out=None) == PA_OK  # no-op


def _reduce(L, po=A16[8], pl=A16[9], B=4, Hq=8, D=128, Pmax=4, lens=A16[6], P=512, out=A16[7], odt=PA_BF16):
    return L.pa_reduce(po, pl, B, Hq, D, Pmax, lens, P, out, odt, None)


def test_reduce_rejections(L):
    assert _reduce(L, po=None) == PA_ERR_NULL_PTR
    assert _reduce(L, out=None) == PA_ERR_NULL_PTR
    assert _reduce(L, lens=None) == PA_ERR_NULL_PTR
    assert _reduce(L, B=-2) == PA_ERR_BAD_SHAPE
    assert _reduce(L, Pmax=0) == PA_ERR_BAD_SHAPE
    assert _reduce(L, P=0) == PA_ERR_BAD_SHAPE
    assert _reduce(L, D=80) == PA_ERR_UNSUPPORTED
    assert _reduce(L, odt=PA_I8) == PA_ERR_UNSUPPORTED
    assert _reduce(L, odt=17) == PA_ERR_UNSUPPORTED
    assert _reduce(L, po=A16[8] + 4) == PA_ERR_MISALIGNED
    assert _reduce(L, B=0, po=None, out=None) == PA_OK


def _append(L, cache, key=A16[10], value=A16[11], sdt=PA_BF16, slots=A16[12], T=3):
    return L.pa_reshape_and_cache(key, value, sdt, slots, T, ctypes.byref(cache), None)


def test_append_rejections(L):
    c = _cache()
    assert _append(L, c, key=None) == PA_ERR_NULL_PTR
    assert _append(L, c, slots=None) == PA_ERR_NULL_PTR
    assert _append(L, c, T=-1) == PA_ERR_BAD_SHAPE
    assert _append(L, c, sdt=PA_F32) == PA_ERR_UNSUPPORTED
    assert _append(L, _cache(kv=PA_F32), sdt=PA_BF16) == PA_ERR_UNSUPPORTED
    assert _append(L, _cache(kv=PA_I8), sdt=PA_F32) == PA_ERR_UNSUPPORTED
    assert _append(L, _cache(kv=PA_I4), sdt=PA_F32) == PA_ERR_UNSUPPORTED
    assert _append(L, c, sdt=5) == PA_ERR_UNSUPPORTED
    assert _append(L, _cache(kv=-3)) == PA_ERR_UNSUPPORTED
    assert _append(L, c, key=A16[10] + 4) == PA_ERR_MISALIGNED
    assert _append(L, c, slots=A16[12] + 1) == PA_ERR_MISALIGNED
    assert _append(L, c, T=0, key=None, value=None, slots=None) == PA_OK


def test_python_wrappers_refuse_cpu_tensors():
    import torch
    import paged_kv_cache_443_amd as pa
    cache = pa.KVCache(torch.zeros(2, 1, 16, 16, 8, dtype=torch.bfloat16), torch.zeros(2, 1, 2, 128, 8, dtype=torch.bfloat16),
                       None, None, 2, 1, 16, 128, "bf16")
    with pytest.raises(ValueError):
        pa.decode(torch.zeros(1, 1, 128, dtype=torch.bfloat16), cache, torch.zeros(1, 1, dtype=torch.int32),
                  torch.ones(1, dtype=torch.int32), 0.1, torch.zeros(1, 1, 128))


def test_probe_rejections(L):
    sink = A16[3]

    def probe(buf=A16[0], nbytes=1 << 20, mode=0, tile=4096, snk=sink):
        return L.pa_probe_read(buf, nbytes, mode, tile, snk, None)

    assert probe(buf=None) == PA_ERR_NULL_PTR
    assert probe(snk=None) == PA_ERR_NULL_PTR
    assert probe(mode=4) == PA_ERR_UNSUPPORTED
    assert probe(mode=-1) == PA_ERR_UNSUPPORTED
    assert probe(nbytes=0) == PA_ERR_BAD_SHAPE
    assert probe(nbytes=100) == PA_ERR_BAD_SHAPE  # not a multiple of 16
    assert probe(mode=2, tile=24) == PA_ERR_BAD_SHAPE
    assert probe(mode=3, tile=0) == PA_ERR_BAD_SHAPE
    assert probe(mode=2, tile=2 << 20) == PA_ERR_BAD_SHAPE  # a tile larger than the buffer
    assert probe(buf=A16[0] + 8) == PA_ERR_MISALIGNED
    assert probe(snk=sink + 2) == PA_ERR_MISALIGNED


def test_mla_rejections(L):
    def lc(nb=64, bs=16, dc=512, ptr=A16[0]):
        return PaLatentCache(ptr, nb, bs, dc)

    def dec(cache=None, q=A16[4], B=4, H=16, D=128, wk=A16[1], wv=A16[2], tables=A16[5], mbps=8, lens=A16[6],
            scale=0.1, P=1024, ws=A16[8], wsb=1 << 24, out=A16[7], odt=PA_BF16):
        c = cache if cache is not None else lc()
        return L.pa_mla_decode(q, B, H, D, wk, wv, ctypes.byref(c), tables, mbps, lens, scale, P, ws, wsb, out, odt,
                               None)

    need = L.pa_mla_workspace_bytes(4, 16, 512, 8, 16, 1024)
    assert need == 4 * 16 * 512 * 4 + 4 * 16 * 1 * 512 * 4 + 256  # q_lat, one partition of partials, lse padded
    assert dec(q=None) == PA_ERR_NULL_PTR
    assert dec(wk=None) == PA_ERR_NULL_PTR
    assert dec(ws=None) == PA_ERR_NULL_PTR
    assert dec(cache=lc(ptr=None)) == PA_ERR_NULL_PTR
    assert dec(cache=lc(dc=256)) == PA_ERR_UNSUPPORTED
    assert dec(cache=lc(bs=8)) == PA_ERR_UNSUPPORTED
    assert dec(cache=lc(nb=0)) == PA_ERR_BAD_SHAPE
    assert dec(D=96) == PA_ERR_UNSUPPORTED
    assert dec(H=0) == PA_ERR_BAD_SHAPE
    assert dec(B=4097) == PA_ERR_BAD_SHAPE
    assert dec(P=96) == PA_ERR_BAD_SHAPE       # not a multiple of 64
    assert dec(P=8192) == PA_ERR_BAD_SHAPE     # longer than 4096
    assert dec(cache=lc(bs=64), P=96) == PA_ERR_BAD_SHAPE  # not a multiple of the block size either
    assert dec(scale=float("inf")) == PA_ERR_BAD_SHAPE
    assert dec(wsb=need - 1) == PA_ERR_BAD_WORKSPACE
    assert dec(odt=PA_I8) == PA_ERR_UNSUPPORTED
    assert dec(ws=A16[8] + 16) == PA_ERR_MISALIGNED  # workspace must be 256-byte aligned
    assert dec(q=A16[4] + 8) == PA_ERR_MISALIGNED
    assert dec(B=0, q=None, out=None, ws=None) == PA_OK  # no-op
    app = lambda rows=A16[9], slots=A16[10], T=3, cache=None: L.pa_mla_append(  # noqa: E731
        rows, slots, T, ctypes.byref(cache if cache is not None else lc()), None)
    assert app(rows=None) == PA_ERR_NULL_PTR
    assert app(T=-1) == PA_ERR_BAD_SHAPE
    assert app(slots=A16[10] + 2) == PA_ERR_MISALIGNED
    assert app(cache=lc(dc=128)) == PA_ERR_UNSUPPORTED
    assert app(T=0, rows=None, slots=None) == PA_OK
