"""Pins of the oracle's int4 KV cache: the quantiser, the nibble packing and
decode over packed storage (no GPU)."""
import numpy as np
import pytest

import oracle
import pinlib
from oracle.storage import pack_nibbles, unpack_nibbles


def test_int4_golden_rows_and_bytes():
    """Hand-worked rows: scales, codes, and the stored bytes."""
    pinlib.check_quant_golden(oracle.quantize_int4, "int4_worked.json")
    for case in pinlib.golden("int4_worked.json")["cases"]:
        codes, _ = oracle.quantize_int4(np.array(case["x"], np.float32)[None, :])
        assert pack_nibbles(codes[0]).tolist() == case["bytes"], case


def test_int4_invariants():
    pinlib.check_quant_invariants(oracle.quantize_int4, qmax=7)


def test_int4_rounding_equals_exact_rule():
    pinlib.check_quant_rounding_exact(oracle.quantize_int4, qmax=7)


def test_nibble_packing_round_trips_every_code():
    codes = np.array([[a, b] for a in range(-8, 8) for b in range(-8, 8)], np.int8)
    packed = pack_nibbles(codes)[:, 0]
    assert len(set(packed.tolist())) == 256  # every byte once
    lo = (packed & 0xF).astype(np.int16)
    hi = (packed >> 4).astype(np.int16)
    assert np.array_equal(np.where(lo >= 8, lo - 16, lo), codes[:, 0])
    assert np.array_equal(np.where(hi >= 8, hi - 16, hi), codes[:, 1])
    assert np.array_equal(unpack_nibbles(pack_nibbles(codes)), codes)


def _int4_cache(rng, lens, Hkv=2, D=32, bs=16):
    Ks = [pinlib.dyadic(rng, (L, Hkv, D)) for L in lens]
    Vs = [pinlib.dyadic(rng, (L, Hkv, D)) for L in lens]
    cache, tb, cl = pinlib.paged_from_dense(Ks, Vs, bs, "i4", rng)
    return Ks, Vs, cache, tb, cl


def test_int4_decode_matches_bruteforce_over_packed_bytes():
    """The vectorised decode on unpacked codes equals a scalar decode that
    reads the stored bytes (low nibble = even element) and scales."""
    rng = np.random.default_rng(44)
    lens = [5, 16, 33, 0]
    Hq, Hkv, D, bs = 4, 2, 32, 16
    _, _, cache, tb, cl = _int4_cache(rng, lens, Hkv, D, bs)
    q = pinlib.dyadic(rng, (len(lens), Hq, D))
    got = oracle.decode(q, cache, tb, cl, 0.25)
    kp, vp = oracle.storage.pools(cache)  # the stored bytes
    want = oracle.decode_bruteforce(q.astype(np.float64).tolist(), kp.ravel().tolist(),
                                    vp.ravel().tolist(), cache.k_scale.ravel().tolist(),
                                    cache.v_scale.ravel().tolist(), "i4", Hkv, bs, D, tb.tolist(), cl.tolist(), 0.25)
    assert np.max(np.abs(got - np.array(want))) < 1e-12


def test_int4_decode_equals_dense_attention_on_dequantised_values():
    """Decode over the int4 cache equals dense attention (a library routine)
    over the dequantised K/V, and the dequantised values are within half a
    step of the inputs."""
    rng = np.random.default_rng(45)
    lens = [7, 40, 17]
    Hq, Hkv, D, bs = 4, 2, 32, 16
    Ks, Vs, cache, tb, cl = _int4_cache(rng, lens, Hkv, D, bs)
    q = pinlib.dyadic(rng, (len(lens), Hq, D))
    got = oracle.decode(q, cache, tb, cl, 0.3)
    deq_K, deq_V = [], []
    for b, L in enumerate(lens):
        kq, ks = oracle.quantize_int4(Ks[b])
        vq, vs = oracle.quantize_int4(Vs[b])
        deq_K.append(oracle.dequantize_int8(kq, ks))
        deq_V.append(oracle.dequantize_int8(vq, vs))
        assert np.all(np.abs(deq_K[-1] - Ks[b]) <= ks.astype(np.float64)[..., None] / 2 + 1e-12)
    import torch
    G = Hq // Hkv
    for b in range(len(lens)):
        k = torch.from_numpy(deq_K[b]).permute(1, 0, 2).repeat_interleave(G, dim=0)  # [Hq, L, D] float64
        v = torch.from_numpy(deq_V[b]).permute(1, 0, 2).repeat_interleave(G, dim=0)
        qq = torch.from_numpy(q[b]).double().unsqueeze(1)
        want = torch.nn.functional.scaled_dot_product_attention(qq, k, v, scale=0.3)[:, 0].numpy()
        assert np.max(np.abs(got[b] - want)) < 1e-12


def _pack_high_first(codes):
    c = np.asarray(codes).astype(np.int16) & 0xF
    return (c[..., 1::2] | (c[..., 0::2] << 4)).astype(np.uint8)


def test_nibble_order_mutant_is_caught(monkeypatch):
    """Packing the odd element into the low nibble breaks the brute-force pin."""
    import oracle.storage as storage
    monkeypatch.setattr(storage, "pack_nibbles", _pack_high_first)
    with pytest.raises(AssertionError):
        test_int4_decode_matches_bruteforce_over_packed_bytes()
