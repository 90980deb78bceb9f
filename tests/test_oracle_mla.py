"""Pins of the oracle's MLA latent-cache decode (``oracle.mla``), CPU only.

The MLA paragraph of page "字节跳动 AI Infra (2)" (question on KV-cache
principles) fixes what is computed: the cache holds one latent row c per
token, K = c W_up_K recovers the heads' keys (d_compress -> num_heads x
head_dim), V the same way with W_up_V (our reading), and attention then runs
as over full-width K/V.  None of these checks re-uses the oracle's own
expansion or attention code:

* the recovered per-head K/V, computed here head by head with explicit
  column slices, written into an ordinary fp32 paged K/V cache and decoded
  by ``oracle.decode`` (itself pinned elsewhere), equal ``mla_decode``;
* the absorbed form (the query moved into the latent space, W_up_K^T q,
  and the value projection applied after the softmax sum) is the same
  result by associativity of the products;
* closed forms: one cached token returns its recovered V row; a zero key
  projection gives the mean of the recovered V rows; physical block
  relabelling changes nothing;
* a pure-Python brute force (scalar loops, no numpy) on tiny shapes;
* planted mistakes in the oracle (transposed head slicing, the K matrix
  used for V, no scale) each fail at least one of these.
"""
import math

import numpy as np
import pytest

import oracle
import oracle.mla as omla
from workloads import make_mla, make_mla_custom


def _expanded_mha_cache(w):
    """fp32 MHA paged cache (kv heads = query heads) holding K_t[h] = c_t W_uk[:, h block],
    V_t[h] = c_t W_uv[:, h block], computed head by head with explicit slices."""
    s = w.spec
    cache = oracle.PagedCache.empty("f32", w.num_blocks, s.H, s.bs, s.d_h)
    for b in range(s.B):
        L = int(w.context_lens[b])
        if not L:
            continue
        C = w.latent(b).astype(np.float64)
        K = np.zeros((L, s.H, s.d_h))
        V = np.zeros((L, s.H, s.d_h))
        for h in range(s.H):
            cols = slice(h * s.d_h, (h + 1) * s.d_h)
            K[:, h, :] = C @ w.w_uk[:, cols].astype(np.float64)
            V[:, h, :] = C @ w.w_uv[:, cols].astype(np.float64)
        oracle.append(cache, K.astype(np.float32), V.astype(np.float32), w.slots(b))
    return cache


def _mla(w, cache=None, **kw):
    cache = oracle.mla_build_cache(w) if cache is None else cache
    args = dict(q=w.q, cache=cache, w_uk=w.w_uk, w_uv=w.w_uv, block_tables=w.block_tables,
                context_lens=w.context_lens, scale=w.spec.scale)
    args.update(kw)
    return oracle.mla_decode(**args)


def check_expanded_equals_mha(w):
    got = _mla(w)
    want = oracle.decode(w.q, _expanded_mha_cache(w), w.block_tables, w.context_lens, w.spec.scale)
    # the expanded K/V are held in fp32: ~1e-7 relative
    assert np.max(np.abs(got - want)) < 2e-5, np.max(np.abs(got - want))


def check_absorbed_form(w):
    s = w.spec
    cache = oracle.mla_build_cache(w)
    got = _mla(w, cache)
    for b in range(s.B):
        L = int(w.context_lens[b])
        if not L:
            assert np.all(got[b] == 0)
            continue
        C = cache.c[w.block_tables[b, np.arange(L) // s.bs], np.arange(L) % s.bs]
        for h in range(s.H):
            cols = slice(h * s.d_h, (h + 1) * s.d_h)
            q_lat = w.w_uk[:, cols].astype(np.float64) @ w.q[b, h].astype(np.float64)  # [d_c]
            sc = s.scale * (C @ q_lat)
            p = np.exp(sc - sc.max())
            o_lat = (p @ C) / p.sum()
            want = o_lat @ w.w_uv[:, cols].astype(np.float64)
            assert np.max(np.abs(got[b, h] - want)) < 1e-9, (b, h)


def check_closed_forms(w):
    s = w.spec
    cache = oracle.mla_build_cache(w)
    # one cached token: the output is that token's recovered V row
    one = np.minimum(w.context_lens, 1)
    got = _mla(w, cache, context_lens=one)
    for b in range(s.B):
        if one[b]:
            c0 = cache.c[w.block_tables[b, 0], 0]
            for h in range(s.H):
                want = c0 @ w.w_uv[:, h * s.d_h:(h + 1) * s.d_h].astype(np.float64)
                assert np.max(np.abs(got[b, h] - want)) < 1e-12
    # zero key projection: every score is 0, the output is the mean recovered V
    got = _mla(w, cache, w_uk=np.zeros_like(w.w_uk))
    for b in range(s.B):
        L = int(w.context_lens[b])
        if L:
            C = cache.c[w.block_tables[b, np.arange(L) // s.bs], np.arange(L) % s.bs]
            for h in range(s.H):
                want = C.mean(axis=0) @ w.w_uv[:, h * s.d_h:(h + 1) * s.d_h].astype(np.float64)
                assert np.max(np.abs(got[b, h] - want)) < 1e-10


def check_block_relabelling(w):
    cache = oracle.mla_build_cache(w, poison=False)
    base = _mla(w, cache)
    perm = np.random.default_rng(3).permutation(cache.num_blocks)
    moved = oracle.LatentCache(np.empty_like(cache.c))
    moved.c[perm] = cache.c
    tables = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    got = _mla(w, moved, block_tables=tables)
    assert np.max(np.abs(got - base)) < 1e-12


def brute_mla(q, c_rows_per_seq, w_uk, w_uv, H, d_h, scale):
    """Pure-Python scalar loops: recover K, V per token and head, softmax, weighted sum."""
    out = []
    for b, rows in enumerate(c_rows_per_seq):
        ob = []
        for h in range(H):
            K, V = [], []
            for c in rows:
                K.append([sum(c[i] * w_uk[i][h * d_h + d] for i in range(len(c))) for d in range(d_h)])
                V.append([sum(c[i] * w_uv[i][h * d_h + d] for i in range(len(c))) for d in range(d_h)])
            if not rows:
                ob.append([0.0] * d_h)
                continue
            s = [scale * sum(q[b][h][d] * k[d] for d in range(d_h)) for k in K]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = sum(e)
            ob.append([sum(e[t] * V[t][d] for t in range(len(rows))) / z for d in range(d_h)])
        out.append(ob)
    return out


def check_brute(w):
    s = w.spec
    got = _mla(w)
    rows = [w.latent(b).astype(np.float64).tolist() for b in range(s.B)]
    want = brute_mla(w.q.astype(np.float64).tolist(), rows, w.w_uk.astype(np.float64).tolist(),
                     w.w_uv.astype(np.float64).tolist(), s.H, s.d_h, s.scale)
    assert np.max(np.abs(got - np.array(want))) < 1e-12


def _tiny():
    return make_mla_custom(H=3, d_h=4, d_c=8, bs=4, lengths=[5, 1, 0, 9], seed=41)


CHECKS = [check_expanded_equals_mha, check_absorbed_form, check_closed_forms, check_block_relabelling, check_brute]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_pins_tiny(check):
    check(_tiny())


@pytest.mark.parametrize("check", [check_expanded_equals_mha, check_absorbed_form, check_block_relabelling],
                         ids=lambda c: c.__name__)
def test_pins_mla_workload_shapes(check):
    # the benchmark workload's head shapes (16 heads of 128 over a 512-wide latent), short sequences
    w = make_mla(small=True, B=3, max_len=300, len_lo=40, len_hi=300)
    check(w)


# ---- planted mistakes --------------------------------------------------


def _expand_interleaved(c_rows, w_up, H, d_h):  # column d * H + h instead of h * d_h + d
    full = np.asarray(c_rows, np.float64) @ np.asarray(w_up, np.float64)
    return full.reshape(full.shape[0], d_h, H).transpose(0, 2, 1)


def test_mutant_interleaved_heads_is_caught(monkeypatch):
    monkeypatch.setattr(omla, "mla_expand", _expand_interleaved)
    with pytest.raises(AssertionError):
        check_expanded_equals_mha(_tiny())
    with pytest.raises(AssertionError):
        check_brute(_tiny())


def test_mutant_k_projection_for_v_is_caught(monkeypatch):
    real = omla.mla_decode

    def wrong(q, cache, w_uk, w_uv, block_tables, context_lens, scale):
        return real(q, cache, w_uk, w_uk, block_tables, context_lens, scale)

    monkeypatch.setattr(oracle, "mla_decode", wrong)
    with pytest.raises(AssertionError):
        check_closed_forms(_tiny())
    with pytest.raises(AssertionError):
        check_brute(_tiny())


def test_mutant_no_scale_is_caught(monkeypatch):
    real = omla.mla_decode
    monkeypatch.setattr(oracle, "mla_decode",
                        lambda q, cache, w_uk, w_uv, block_tables, context_lens, scale:
                        real(q, cache, w_uk, w_uv, block_tables, context_lens, 1.0))
    with pytest.raises(AssertionError):
        check_brute(_tiny())
    with pytest.raises(AssertionError):
        check_expanded_equals_mha(_tiny())
