"""Checks that pin the oracle to facts outside its own code path.

Each ``check_*`` takes the function under test as an argument so the same
checks run against the real oracle (tests/test_oracle_pins.py, must pass)
and against oracles with a planted mistake (tests/test_oracle_mutants.py,
each must fail at least one check).  Failures raise AssertionError.
"""
from __future__ import annotations

import json
import math
import os
from typing import Callable, List, Sequence, Tuple

import numpy as np

import oracle
from oracle import PagedCache

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


# --------------------------------------------------------------------------
# building small paged caches from dense per-sequence K/V
# --------------------------------------------------------------------------


def dyadic(rng: np.random.Generator, shape, step: float = 0.125, lim: float = 4.0) -> np.ndarray:
    """Values on a coarse binary grid: sums and shifts stay exact in fp32 and bf16."""
    return np.clip(np.rint(rng.standard_normal(shape) / step) * step, -lim, lim).astype(np.float32)


def paged_from_dense(Ks: Sequence[np.ndarray], Vs: Sequence[np.ndarray], bs: int, kv_dtype: str = "f32",
                     rng: np.random.Generator = None, spare: int = 3, width: int = None):
    """Scatter dense ``[L_b, Hkv, D]`` K/V of each sequence into a shuffled pool.

    Returns (cache, block_tables, context_lens); unused table entries are -1
    and the pool is NaN-poisoned outside the written slots.
    """
    rng = rng or np.random.default_rng(0)
    Hkv, D = Ks[0].shape[1], Ks[0].shape[2]
    lens = np.array([k.shape[0] for k in Ks], np.int32)
    nbs = [oracle.blocks_for(L, bs) for L in lens]
    pool = sum(nbs) + spare
    perm = rng.permutation(pool).astype(np.int32)
    width = width or max(max(nbs, default=1), 1) + 1
    tables = np.full((len(Ks), width), -1, np.int32)
    cache = PagedCache.empty(kv_dtype, pool, Hkv, bs, D)
    nxt = 0
    for b, (K, V) in enumerate(zip(Ks, Vs)):
        for j in range(nbs[b]):
            tables[b, j] = perm[nxt]
            nxt += 1
        L = int(lens[b])
        if L:
            t = np.arange(L)
            slots = tables[b, t // bs].astype(np.int64) * bs + t % bs
            oracle.append(cache, K, V, slots)
    return cache, tables, lens


def rand_case(rng, B=3, Hq=4, Hkv=2, D=16, bs=4, lens=(5, 9, 12), kv_dtype="f32"):
    Ks = [dyadic(rng, (L, Hkv, D)) for L in lens]
    Vs = [dyadic(rng, (L, Hkv, D)) for L in lens]
    q = dyadic(rng, (len(lens), Hq, D))
    cache, tables, cl = paged_from_dense(Ks, Vs, bs, kv_dtype, rng)
    return q, Ks, Vs, cache, tables, cl


DecodeFn = Callable[..., np.ndarray]


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# --------------------------------------------------------------------------
# decode pins
# --------------------------------------------------------------------------


def check_closed_forms(decode: DecodeFn) -> None:
    rng = np.random.default_rng(11)
    Hq, Hkv, D, bs = 4, 2, 16, 4
    # (a) identical keys -> the mean of the V rows
    L = 11
    k = dyadic(rng, (1, Hkv, D))
    K = np.repeat(k, L, axis=0)
    V = dyadic(rng, (L, Hkv, D))
    q = dyadic(rng, (1, Hq, D))
    cache, tb, cl = paged_from_dense([K], [V], bs, rng=rng)
    out = decode(q, cache, tb, cl, 0.7)
    G = Hq // Hkv
    want = np.stack([V[:, h // G].astype(np.float64).mean(axis=0) for h in range(Hq)])
    _close(out[0], want, 1e-12, "identical keys")

    # (b) one dominant key (logit gap >= 40) -> its V row
    L = 13
    K = dyadic(rng, (L, Hkv, D), lim=1.0)
    V = dyadic(rng, (L, Hkv, D))
    q = dyadic(rng, (1, Hq, D), lim=1.0)
    q[0, :, 0] = 1.0
    tstar = 6
    K[tstar, :, :] = 0.0
    K[tstar, :, 0] = 64.0  # logit 64*scale vs |others| <= D*1*1*scale
    scale = 1.0
    cache, tb, cl = paged_from_dense([K], [V], bs, rng=rng)
    out = decode(q, cache, tb, cl, scale)
    want = np.stack([V[tstar, h // G].astype(np.float64) for h in range(Hq)])
    # every other logit is at most 16 + (-1 * ... ) <= 16 + 15 below 64 -> gap >= 33; bound L*e^-33*max|v|
    _close(out[0], want, L * math.exp(-33.0) * 4.0 + 1e-15, "dominant key")

    # (c) a single cached token -> that token's V row exactly
    K = dyadic(rng, (1, Hkv, D))
    V = dyadic(rng, (1, Hkv, D))
    q = dyadic(rng, (1, Hq, D))
    cache, tb, cl = paged_from_dense([K], [V], bs, rng=rng)
    out = decode(q, cache, tb, cl, 0.3)
    want = np.stack([V[0, h // G].astype(np.float64) for h in range(Hq)])
    _close(out[0], want, 0.0, "L=1")

    # (d) scale 0 -> uniform weights -> mean of V
    L = 9
    K = dyadic(rng, (L, Hkv, D))
    V = dyadic(rng, (L, Hkv, D))
    q = dyadic(rng, (1, Hq, D))
    cache, tb, cl = paged_from_dense([K], [V], bs, rng=rng)
    out = decode(q, cache, tb, cl, 0.0)
    want = np.stack([V[:, h // G].astype(np.float64).mean(axis=0) for h in range(Hq)])
    _close(out[0], want, 1e-12, "scale 0")

    # (e) an empty sequence next to a non-empty one -> zero row
    Ks = [np.zeros((0, Hkv, D), np.float32), dyadic(rng, (5, Hkv, D))]
    Vs = [np.zeros((0, Hkv, D), np.float32), dyadic(rng, (5, Hkv, D))]
    q = dyadic(rng, (2, Hq, D))
    cache, tb, cl = paged_from_dense(Ks, Vs, bs, rng=rng)
    out = decode(q, cache, tb, cl, 0.5)
    assert np.all(out[0] == 0.0), "L=0 must give zeros"
    assert np.all(np.isfinite(out[1]))


def check_shift_invariances(decode: DecodeFn) -> None:
    """Weights sum to one (V + c -> out + c); softmax ignores a common logit
    offset (K + c -> same out)."""
    rng = np.random.default_rng(12)
    q, Ks, Vs, cache, tb, cl = rand_case(rng)
    base = decode(q, cache, tb, cl, 0.5)
    c = dyadic(rng, (1, Ks[0].shape[1], Ks[0].shape[2]), lim=1.0)
    cache2, tb2, cl2 = paged_from_dense(Ks, [v + c for v in Vs], 4, rng=np.random.default_rng(5))
    out = decode(q, cache2, tb2, cl2, 0.5)
    G = q.shape[1] // Ks[0].shape[1]
    shift = np.stack([c[0, h // G] for h in range(q.shape[1])]).astype(np.float64)
    _close(out, base + shift[None], 1e-12, "V + c")
    cache3, tb3, cl3 = paged_from_dense([k + c for k in Ks], Vs, 4, rng=np.random.default_rng(6))
    out = decode(q, cache3, tb3, cl3, 0.5)
    _close(out, base, 1e-12, "K + c")
    # a positive scale on V scales the output
    cache4, tb4, cl4 = paged_from_dense(Ks, [2.0 * v for v in Vs], 4, rng=np.random.default_rng(7))
    _close(decode(q, cache4, tb4, cl4, 0.5), 2.0 * base, 1e-12, "2V")


def check_token_permutation(decode: DecodeFn) -> None:
    """Attention is a set operation over the cached tokens: permuting token
    positions (moving each token's K and V together) leaves the output fixed."""
    rng = np.random.default_rng(13)
    q, Ks, Vs, cache, tb, cl = rand_case(rng, lens=(7, 13))
    base = decode(q, cache, tb, cl, 0.5)
    perms = [rng.permutation(k.shape[0]) for k in Ks]
    cache2, tb2, cl2 = paged_from_dense([k[p] for k, p in zip(Ks, perms)], [v[p] for v, p in zip(Vs, perms)], 4,
                                        rng=np.random.default_rng(8))
    _close(decode(q, cache2, tb2, cl2, 0.5), base, 1e-12, "token permutation")


def check_block_relabel(decode: DecodeFn) -> None:
    """Moving blocks to other physical ids (and rewriting the tables) changes nothing."""
    rng = np.random.default_rng(14)
    q, Ks, Vs, cache, tb, cl = rand_case(rng, lens=(6, 17, 40), bs=16, kv_dtype="bf16")
    base = decode(q, cache, tb, cl, 0.5)
    perm = rng.permutation(cache.num_blocks)  # new id of old block i is perm[i]
    c2 = PagedCache.empty(cache.kv_dtype, cache.num_blocks, cache.Hkv, cache.bs, cache.D)
    c2.k[perm] = cache.k
    c2.v[perm] = cache.v
    tb2 = np.where(tb >= 0, perm[np.maximum(tb, 0)], -1).astype(np.int32)
    _close(decode(q, c2, tb2, cl, 0.5), base, 1e-12, "block relabel")


def check_gqa_vs_mha(decode: DecodeFn) -> None:
    """GQA equals MHA whose K/V head h is a copy of GQA K/V head h // G."""
    rng = np.random.default_rng(15)
    Hq, Hkv, D, bs = 6, 2, 16, 4
    G = Hq // Hkv
    lens = (5, 11)
    Ks = [dyadic(rng, (L, Hkv, D)) for L in lens]
    Vs = [dyadic(rng, (L, Hkv, D)) for L in lens]
    q = dyadic(rng, (2, Hq, D))
    cache, tb, cl = paged_from_dense(Ks, Vs, bs, rng=rng)
    g = decode(q, cache, tb, cl, 0.4)
    rep = [h // G for h in range(Hq)]
    cache2, tb2, cl2 = paged_from_dense([k[:, rep] for k in Ks], [v[:, rep] for v in Vs], bs, rng=rng)
    m = decode(q, cache2, tb2, cl2, 0.4)
    _close(g, m, 1e-12, "GQA vs replicated MHA")
    # and the heads of one group really differ from another group's
    assert np.max(np.abs(g[:, 0] - g[:, G])) > 1e-3


def check_cow(decode: DecodeFn) -> None:
    """Two beams with the same tokens: one shares prefix blocks physically with
    the other and owns a copied last block; the other layout gives every
    block privately.  Both must produce equal outputs."""
    rng = np.random.default_rng(16)
    Hq, Hkv, D, bs = 4, 2, 16, 4
    L = 11  # 3 blocks
    K = dyadic(rng, (L, Hkv, D))
    V = dyadic(rng, (L, Hkv, D))
    q = dyadic(rng, (1, Hq, D))
    q2 = np.concatenate([q, q])
    cache, tb, cl = paged_from_dense([K, K], [V, V], bs, rng=rng, spare=2)  # private copies
    priv = decode(q2, cache, tb, cl, 0.5)
    shared = tb.copy()
    shared[1, :2] = tb[0, :2]  # beam 2 now points at beam 1's first two blocks
    sh = decode(q2, cache, shared, cl, 0.5)
    _close(sh, priv, 0.0, "COW sharing")
    _close(sh[0], sh[1], 0.0, "beams")


def check_bruteforce(decode: DecodeFn) -> None:
    """Against pure-Python scalar loops over the flat pool storage (the
    oracle's logical cache through its storage codec: pins the codec too)."""
    rng = np.random.default_rng(17)
    for kv_dtype, bs, Hq, Hkv, D, lens in [
        ("f32", 16, 4, 4, 64, (7, 16, 33, 40)),
        ("bf16", 16, 4, 2, 16, (1, 15, 17, 32)),
        ("i8", 16, 8, 2, 32, (3, 16, 21)),
        ("bf16", 32, 2, 1, 16, (40,)),
    ]:
        Ks = [dyadic(rng, (L, Hkv, D)) for L in lens]
        Vs = [dyadic(rng, (L, Hkv, D)) for L in lens]
        q = rng.standard_normal((len(lens), Hq, D)).astype(np.float32)
        cache, tb, cl = paged_from_dense(Ks, Vs, bs, kv_dtype, rng)
        got = decode(q, cache, tb, cl, 1.0 / math.sqrt(D))
        ksf = cache.k_scale.ravel().astype(np.float64).tolist() if cache.k_scale is not None else None
        vsf = cache.v_scale.ravel().astype(np.float64).tolist() if cache.v_scale is not None else None
        kp, vp = oracle.storage.pools(cache)  # the pools in memory order, as pa.h states it
        want = oracle.decode_bruteforce(q.astype(np.float64).tolist(), kp.ravel().tolist(), vp.ravel().tolist(),
                                        ksf, vsf, kv_dtype, Hkv, bs, D, tb.tolist(), cl.tolist(), 1.0 / math.sqrt(D))
        _close(got, np.array(want), 1e-12, f"brute force {kv_dtype} bs{bs}")


def check_dense_library(decode: DecodeFn) -> None:
    """Against torch's CPU scaled_dot_product_attention (float64) on the
    de-paged, contiguous K/V of each sequence: the textbook
    softmax(q K^T * scale) V computed by a library routine, with K/V heads
    repeated G times for GQA."""
    import torch

    rng = np.random.default_rng(23)
    for Hq, Hkv, D, bs, lens in [(4, 4, 64, 16, (7, 16, 33, 40)), (8, 2, 32, 8, (1, 9, 30)),
                                 (6, 1, 16, 4, (13, 5))]:
        Ks = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in lens]
        Vs = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in lens]
        q = rng.standard_normal((len(lens), Hq, D)).astype(np.float32)
        cache, tb, cl = paged_from_dense(Ks, Vs, bs, "f32", rng)
        scale = 1.0 / math.sqrt(D)
        got = decode(q, cache, tb, cl, scale)
        G = Hq // Hkv
        for b, L in enumerate(lens):
            k = torch.from_numpy(Ks[b]).double().permute(1, 0, 2).repeat_interleave(G, dim=0)  # [Hq, L, D]
            v = torch.from_numpy(Vs[b]).double().permute(1, 0, 2).repeat_interleave(G, dim=0)
            qq = torch.from_numpy(q[b]).double().unsqueeze(1)  # [Hq, 1, D]
            want = torch.nn.functional.scaled_dot_product_attention(qq, k, v, scale=scale)[:, 0].numpy()
            _close(got[b], want, 1e-12, f"dense library Hq{Hq} Hkv{Hkv} seq{b}")


ALL_DECODE_CHECKS = [check_closed_forms, check_shift_invariances, check_token_permutation, check_block_relabel,
                     check_gqa_vs_mha, check_cow, check_bruteforce, check_dense_library]


# --------------------------------------------------------------------------
# split / merge pins
# --------------------------------------------------------------------------


def check_split(partials, merge, decode: DecodeFn) -> None:
    rng = np.random.default_rng(18)
    q, Ks, Vs, cache, tb, cl = rand_case(rng, Hq=4, Hkv=2, D=16, bs=4, lens=(1, 8, 13, 0, 24))
    base = decode(q, cache, tb, cl, 0.5)
    for P in (4, 8, 12, 24, 64):
        pmax = max(1, -(-int(cl.max()) // P))
        po, pl = partials(q, cache, tb, cl, 0.5, P, pmax)
        _close(merge(po, pl, cl, P), base, 1e-12, f"merge(partials) P={P}")
        # empty ranges carry zero output and -inf lse
        for b, L in enumerate(cl):
            n = -(-int(L) // P)
            assert np.all(po[b, :, n:] == 0.0) and np.all(np.isneginf(pl[b, :, n:]))
    # P >= L: a single partition whose output is the decode output and whose
    # lse is log sum_t exp(s_t), checked against a direct sum here
    P = 64
    po, pl = partials(q, cache, tb, cl, 0.5, P, 1)
    _close(po[:, :, 0], base, 1e-12, "single partition")
    b, h = 2, 3
    K, _ = oracle.gather_sequence(cache, tb[b], int(cl[b]), h // 2)
    s = 0.5 * (K @ q[b, h].astype(np.float64))
    assert abs(pl[b, h, 0] - math.log(sum(math.exp(v) for v in s))) < 1e-12


# --------------------------------------------------------------------------
# quantiser pins
# --------------------------------------------------------------------------


def check_quant_golden(quantize, name: str = "int8_worked.json") -> None:
    for case in golden(name)["cases"]:
        x = np.array(case["x"], np.float32)[None, :]
        codes, scale = quantize(x)
        assert float(scale[0]) == case["scale"], (case, float(scale[0]))
        assert codes[0].tolist() == case["codes"], (case, codes[0].tolist())


def check_quant_invariants(quantize, qmax: int = 127) -> None:
    rng = np.random.default_rng(19)
    from workloads import bf16_round
    x = bf16_round((rng.standard_normal((4000, 64)) * rng.uniform(1e-3, 50, (4000, 1))).astype(np.float32))
    codes, s16 = quantize(x)
    s = s16.astype(np.float64)
    # the largest-magnitude element maps to +-qmax
    i = np.argmax(np.abs(x), axis=1)
    top = codes[np.arange(len(x)), i].astype(np.int64)
    assert np.all(np.abs(top) == qmax)
    assert np.all(np.sign(top) == np.sign(x[np.arange(len(x)), i]))
    # reconstruction error at most half a step
    err = np.abs(codes.astype(np.float64) * s[:, None] - x.astype(np.float64))
    assert np.all(err <= s[:, None] / 2 * (1 + 1e-12))
    # the scale is the fp16 nearest to absmax/127 (checked with exact rationals)
    from fractions import Fraction
    for r in range(0, 4000, 397):
        a = Fraction(float(np.max(np.abs(x[r])))) / qmax
        got = Fraction(float(s16[r]))
        # neighbours of got in fp16
        up = Fraction(float(np.nextafter(s16[r], np.float16(np.inf))))
        dn = Fraction(float(np.nextafter(s16[r], np.float16(0))))
        assert abs(got - a) <= abs(up - a) and abs(got - a) <= abs(dn - a)
    # codes never use the most negative value of the type (-128 / -8)
    assert codes.min() >= -qmax and codes.max() <= qmax


def check_quant_rounding_exact(quantize, n: int = 20000, qmax: int = 127) -> None:
    """The float32 quotient rounds to the same integer as the exact quotient
    (so taking the decision in float32 equals the exact rule)."""
    from fractions import Fraction
    rng = np.random.default_rng(20)
    from workloads import bf16_round
    x = bf16_round((rng.standard_normal((n, 8)) * rng.uniform(1e-2, 10, (n, 1))).astype(np.float32))
    # force exact .5 ties into some rows: x = (k + 1/2) * s for the row's scale s
    codes, s16 = quantize(x)
    for r in range(0, n, 41):
        s = Fraction(float(s16[r]))
        if s == 0:
            continue
        for d in range(8):
            qx = Fraction(float(x[r, d])) / s
            fl = qx.numerator // qx.denominator
            rem = qx - fl
            want = fl + 1 if rem > Fraction(1, 2) else fl if rem < Fraction(1, 2) else (fl if fl % 2 == 0 else fl + 1)
            want = max(-qmax, min(qmax, want))
            assert int(codes[r, d]) == want, (r, d, float(x[r, d]), float(s16[r]))
