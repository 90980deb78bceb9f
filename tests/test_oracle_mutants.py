"""Plant plausible mistakes in the oracle (on the CPU) and show the pins catch each.

Every mutant below must make at least one pin check fail; if a mutant
passes every check, the pins have a blind spot.
"""
import numpy as np
import pytest

import oracle
import oracle.layout as olayout
import oracle.paged as opaged
import pinlib


def _fails_some(checks, *args):
    failed = []
    for chk in checks:
        try:
            chk(*args)
        except (AssertionError, IndexError, ValueError, FloatingPointError, ZeroDivisionError):
            failed.append(chk.__name__)
    return failed


# ---- decode mutants (monkeypatched into the oracle modules) -------------


def _m_gqa_mod(mp):
    mp.setattr(opaged, "kv_head_for", lambda h, Hq, Hkv: h % Hkv)


def _m_no_scale(mp):
    mp.setattr(opaged, "_scores", lambda q, K, scale: K @ q)


def _m_neg_sign(mp):
    mp.setattr(opaged, "_scores", lambda q, K, scale: -float(scale) * (K @ q))


def _m_no_normalise(mp):
    def f(s, V):
        w = np.exp(s - s.max())
        return (w @ V) / len(s), float(s.max() + np.log(w.sum()))
    mp.setattr(opaged, "_softmax_apply", f)


def _m_offset_shift(mp):
    orig = opaged.gather_sequence

    def g(cache, row, length, kv, start=0, stop=None):
        stop = length if stop is None else stop
        t = np.arange(start, stop, dtype=np.int64)
        pbs = row[t // cache.bs].astype(np.int64)
        offs = (cache.bs - 1) - t % cache.bs
        return cache.k_rows(pbs, kv, offs), cache.v_rows(pbs, kv, offs)
    mp.setattr(opaged, "gather_sequence", g)


def _m_drop_last(mp):
    orig = opaged.gather_sequence

    def g(cache, row, length, kv, start=0, stop=None):
        stop = length if stop is None else stop
        return orig(cache, row, length, kv, start, max(start, stop - 1) if stop - start > 1 else stop)
    mp.setattr(opaged, "gather_sequence", g)


def _m_v_channels_reversed(mp):
    orig = olayout.PagedCache.v_rows
    mp.setattr(olayout.PagedCache, "v_rows", lambda self, pbs, h, offs: orig(self, pbs, h, offs)[:, ::-1])


def _m_k_transposed(mp):
    # channels read as 8-wide vectors transposed (a vector-layout mix-up)
    def k_rows(self, pbs, h, offs):
        raw = self.k[pbs, h, offs, :].reshape(len(pbs), self.D // 8, 8).transpose(0, 2, 1).reshape(len(pbs), self.D)
        return self._to_f64(raw, self.k_scale, pbs, h, offs)
    mp.setattr(olayout.PagedCache, "k_rows", k_rows)


def _m_v_reads_k(mp):
    def v_rows(self, pbs, h, offs):
        raw = self.k[pbs, h, offs, :]
        return self._to_f64(raw, self.k_scale, pbs, h, offs)
    mp.setattr(olayout.PagedCache, "v_rows", v_rows)


def _m_scale_from_v(mp):
    def k_rows(self, pbs, h, offs):
        raw = self.k[pbs, h, offs, :]
        return self._to_f64(raw, self.v_scale, pbs, h, offs)
    mp.setattr(olayout.PagedCache, "k_rows", k_rows)


DECODE_MUTANTS = [_m_gqa_mod, _m_no_scale, _m_neg_sign, _m_no_normalise, _m_offset_shift, _m_drop_last,
                  _m_v_channels_reversed, _m_k_transposed, _m_v_reads_k, _m_scale_from_v]


@pytest.mark.parametrize("mutant", DECODE_MUTANTS, ids=lambda f: f.__name__)
def test_decode_mutant_is_caught(mutant, monkeypatch):
    mutant(monkeypatch)
    failed = _fails_some(pinlib.ALL_DECODE_CHECKS, oracle.decode)
    assert failed, f"{mutant.__name__} passed every decode pin"


# ---- split / merge mutants -------------------------------------------------


def _merge_unweighted(po, pl, cl, P):
    B, Hq, Pm, D = po.shape
    out = np.zeros((B, Hq, D))
    for b, L in enumerate(cl):
        n = -(-int(L) // P)
        if n:
            out[b] = po[b, :, :n].mean(axis=1)
    return out


def _partials_lse_without_max(q, cache, tb, cl, scale, P, pmax):
    po, pl = oracle.decode_partials(q, cache, tb, cl, scale, P, pmax)
    # planted: forget the running max in the log-sum-exp
    B, Hq = pl.shape[:2]
    for b in range(B):
        for h in range(Hq):
            L = int(cl[b])
            for p in range(-(-L // P)):
                K, _ = oracle.gather_sequence(cache, tb[b], L, oracle.kv_head_for(h, Hq, cache.Hkv), p * P,
                                              min((p + 1) * P, L))
                s = scale * (K @ np.asarray(q[b, h], np.float64))
                pl[b, h, p] = np.log(np.exp(s - s.max()).sum())
    return po, pl


def _partials_off_by_one_range(q, cache, tb, cl, scale, P, pmax):
    return oracle.decode_partials(q, cache, tb, np.maximum(np.asarray(cl) - 1, 0), scale, P, pmax)


@pytest.mark.parametrize("partials,merge", [
    (oracle.decode_partials, _merge_unweighted),
    (_partials_lse_without_max, oracle.merge_partials),
    (_partials_off_by_one_range, oracle.merge_partials),
], ids=["merge-unweighted", "lse-no-max", "partials-short-range"])
def test_split_mutant_is_caught(partials, merge):
    assert _fails_some([pinlib.check_split], partials, merge, oracle.decode)


# ---- quantiser mutants -------------------------------------------------------


def _q_half_away(x):
    xf = np.asarray(x, np.float32)
    s16 = (np.max(np.abs(xf), -1) / np.float32(127)).astype(np.float32).astype(np.float16)
    sf = np.where(s16 == 0, 1, s16).astype(np.float32)
    v = (xf / sf[..., None]).astype(np.float32)
    qv = np.sign(v) * np.floor(np.abs(v) + 0.5)
    qv = np.where(s16[..., None] == 0, 0, np.clip(qv, -127, 127))
    return qv.astype(np.int8), s16


def _q_fp32_scale(x):
    codes, s16 = oracle.quantize_int8(x)
    xf = np.asarray(x, np.float32)
    s32 = (np.max(np.abs(xf), -1) / np.float32(127)).astype(np.float32)
    return codes, s32  # planted: stores the unrounded scale


def _q_div128(x):
    xf = np.asarray(x, np.float32)
    s16 = (np.max(np.abs(xf), -1) / np.float32(128)).astype(np.float32).astype(np.float16)
    sf = np.where(s16 == 0, 1, s16).astype(np.float32)
    qv = np.where(s16[..., None] == 0, 0, np.clip(np.rint(xf / sf[..., None]), -127, 127))
    return qv.astype(np.int8), s16


def _q_truncate(x):
    xf = np.asarray(x, np.float32)
    s16 = (np.max(np.abs(xf), -1) / np.float32(127)).astype(np.float32).astype(np.float16)
    sf = np.where(s16 == 0, 1, s16).astype(np.float32)
    qv = np.where(s16[..., None] == 0, 0, np.clip(np.trunc(xf / sf[..., None]), -127, 127))
    return qv.astype(np.int8), s16


def _q_no_clamp(x):
    xf = np.asarray(x, np.float32)
    s16 = (np.max(np.abs(xf), -1) / np.float32(127)).astype(np.float32).astype(np.float16)
    sf = np.where(s16 == 0, 1, s16).astype(np.float32)
    qv = np.where(s16[..., None] == 0, 0, np.rint(xf / sf[..., None]))
    return qv.astype(np.int64).astype(np.int8), s16  # wraps instead of clamping


@pytest.mark.parametrize("mutant", [_q_half_away, _q_fp32_scale, _q_div128, _q_truncate, _q_no_clamp],
                         ids=lambda f: f.__name__)
def test_quant_mutant_is_caught(mutant):
    checks = [pinlib.check_quant_golden, pinlib.check_quant_invariants, pinlib.check_quant_rounding_exact]
    assert _fails_some(checks, mutant), f"{mutant.__name__} passed every quantiser pin"
