"""int4 KV cache on the GPU vs the oracle, through the C ABI (needs an MI355X):
append bit for bit (stored bytes and scales), decode, split + merge,
multi-query, block copy and swap."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_443_amd as pa
from gpu_util import (DEV, TOL, bf16_rne_of, download_cache, fill_poison, gpu_append_tokens, max_err, meta,
                      oracle_pools, poisoned_cache, say, to_dev_values, upload_oracle_cache)
from workloads import bf16_round, make_custom, make_workload

pytestmark = pytest.mark.gpu

SENTINEL = -123.25


def _same_as_oracle(c: pa.KVCache, oc) -> None:
    k, v, ks, vs = download_cache(c)
    okp, ovp = oracle_pools(oc)
    assert np.array_equal(k, okp), "K bytes"
    assert np.array_equal(v, ovp), "V bytes"
    assert np.array_equal(ks.view(np.uint16), oc.k_scale.view(np.uint16)), "K scales"
    assert np.array_equal(vs.view(np.uint16), oc.v_scale.view(np.uint16)), "V scales"


# (Hq, Hkv, D, bs, lengths): one call writes every token of a sequence, so
# neighbouring tokens' V nibbles (one byte) are written concurrently
APPEND_SHAPES = [
    (32, 8, 128, 16, [1, 15, 16, 17, 100, 513]),
    (8, 8, 64, 32, [31, 33, 64, 200]),
    (12, 4, 128, 64, [65, 128, 7]),
]


@pytest.mark.parametrize("shape", range(len(APPEND_SHAPES)))
def test_int4_append_bit_exact(shape):
    Hq, Hkv, D, bs, lens = APPEND_SHAPES[shape]
    w = make_custom(B=len(lens), Hq=Hq, Hkv=Hkv, D=D, bs=bs, kv_dtype="i4", lengths=lens, seed=60 + shape)
    say(f"[int4 append] Hkv={Hkv} D={D} bs={bs}")
    cache = poisoned_cache(w)
    gpu_append_tokens(w, cache)
    torch.cuda.synchronize()
    _same_as_oracle(cache, oracle.build_cache(w))


def test_int4_append_edge_rows():
    """Quantiser corner cases (ties, zero rows, subnormal scales, clamping) bit for bit."""
    say("[int4 append] edge rows")
    rng = np.random.default_rng(6)
    D = 128
    base = np.array([7.0, 3.5, -3.5, 2.5, 0.5, -0.5, 1.0, -7.0] * 16)
    rows = [np.zeros(D), np.full(D, 2.0 ** -20), base, base * 2.0 ** -18, -base * 5.0,
            np.tile([14.0, 5.0, -3.0, 1.0], 32)]
    rows += [rng.standard_normal(D) * 10 ** rng.uniform(-6, 3) for _ in range(58)]
    X = bf16_round(np.stack(rows).astype(np.float32))
    T = X.shape[0]
    K = X.reshape(T, 1, D)
    V = -K[::-1].copy()
    oc = oracle.PagedCache.empty("i4", 8, 1, 16, D)
    slots = np.arange(T, dtype=np.int32) + 3
    oracle.append(oc, K, V, slots)
    c = pa.KVCache.allocate(8, 1, 16, D, "i4", DEV)
    fill_poison(c)
    pa.reshape_and_cache(to_dev_values(K, "bf16"), to_dev_values(V, "bf16"), torch.from_numpy(slots).to(DEV), c)
    torch.cuda.synchronize()
    _same_as_oracle(c, oc)


DECODE_SHAPES = [
    ("cfg5", None),
    ("gqa8-bs16", (64, 8, 128, 16, [0, 1, 15, 16, 17, 63, 64, 65, 300, 1100])),
    ("mha-d64-bs32", (8, 8, 64, 32, [31, 32, 33, 129, 500])),
    ("mqa40-bs64", (40, 1, 128, 64, [64, 65, 700, 3])),
]


def _decode_case(name, shape, seed):
    if shape is None:
        return make_workload(5, small=True, kv_dtype="i4")
    Hq, Hkv, D, bs, lens = shape
    return make_custom(B=len(lens), Hq=Hq, Hkv=Hkv, D=D, bs=bs, kv_dtype="i4", lengths=lens, seed=seed)


@pytest.mark.parametrize("case", range(len(DECODE_SHAPES)))
def test_int4_decode_and_split_match_oracle(case):
    name, shape = DECODE_SHAPES[case]
    w = _decode_case(name, shape, 70 + case)
    s = w.spec
    say(f"[int4 decode] {name} B={w.B}")
    oc = oracle.build_cache(w)
    want = oracle.decode(w.q, oc, w.block_tables, w.context_lens, s.scale)
    cache = upload_oracle_cache(oc)
    q, tables, lens = meta(w)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    pa.decode(q, cache, tables, lens, s.scale, out)
    ob = torch.empty(q.shape, dtype=torch.bfloat16, device=DEV)
    pa.decode(q, cache, tables, lens, s.scale, ob)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(out))
    err = max_err(out, want)
    say(f"  decode max abs err {err:.3e}")
    assert err <= TOL["i4"]
    assert torch.equal(ob.view(torch.int16).cpu(), bf16_rne_of(out))
    # split + merge
    P = 2 * s.bs
    pmax = pa.max_partitions(tables.shape[1], s.bs, P)
    po = torch.full((w.B, s.Hq, pmax, s.D), SENTINEL, dtype=torch.float32, device=DEV)
    pl = torch.full((w.B, s.Hq, pmax), SENTINEL, dtype=torch.float32, device=DEV)
    pa.decode_split(q, cache, tables, lens, s.scale, P, po, pl)
    outs = torch.empty_like(out)
    pa.reduce(po, pl, lens, P, outs)
    torch.cuda.synchronize()
    assert max_err(outs, want) <= TOL["i4"]
    want_po, want_pl = oracle.decode_partials(w.q, oc, w.block_tables, w.context_lens, s.scale, P, pmax)
    gl = pl.cpu().numpy().astype(np.float64)
    for b, L in enumerate(w.context_lens):
        n = -(-int(L) // P)
        assert np.all(gl[b, :, n:] == SENTINEL)
        if n:
            assert np.max(np.abs(gl[b, :, :n] - want_pl[b, :, :n])) <= 1e-3


def test_int4_multi_query_matches_oracle():
    w = make_custom(B=5, Hq=32, Hkv=8, D=128, bs=16, kv_dtype="i4", lengths=[40, 9, 300, 16, 130], seed=81)
    counts = w.query_counts(6)
    q_start, q = w.multi_queries(counts)
    say(f"[int4 multi] counts={counts.tolist()}")
    oc = oracle.build_cache(w)
    want = oracle.decode_multi(q, q_start, oc, w.block_tables, w.context_lens, w.spec.scale)
    cache = upload_oracle_cache(oc)
    _, tables, lens = meta(w)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    pa.decode_multi(to_dev_values(q, "bf16"), torch.from_numpy(q_start).to(DEV), 6, cache, tables, lens,
                    w.spec.scale, out)
    torch.cuda.synchronize()
    assert max_err(out, want) <= TOL["i4"]


def test_int4_copy_and_swap_bit_exact():
    w = make_custom(B=2, Hq=8, Hkv=2, D=64, bs=16, kv_dtype="i4", lengths=[40, 70], seed=82, pool_factor=3.0)
    say("[int4 copy/swap]")
    oc = oracle.build_cache(w)
    cache = upload_oracle_cache(oc)
    used = [int(b) for b in w.used_blocks()]
    free = sorted(set(range(w.num_blocks)) - set(used))
    pairs = [(used[0], free[0]), (used[3], free[1])]
    pa.copy_blocks(cache, torch.tensor(pairs, dtype=torch.int32, device=DEV))
    oracle.copy_blocks(oc, pairs)
    torch.cuda.synchronize()
    _same_as_oracle(cache, oc)
    host = pa.KVCache.allocate(4, 2, 16, 64, "i4", device="cpu")
    fill_poison(host)
    ohost = oracle.PagedCache.empty("i4", 4, 2, 16, 64)
    out_pairs = [(used[1], 2), (used[2], 0)]
    pa.swap_blocks(cache, host, torch.tensor(out_pairs, dtype=torch.int32, device=DEV))
    oracle.swap_blocks(oc, ohost, out_pairs)
    torch.cuda.synchronize()
    _same_as_oracle(host, ohost)
