"""The vector-ALU decode (PA_DECODE_VALU=1) against the oracle (needs an MI355X).

pa_decode runs its single-token bf16 units on v_dot2_f32_bf16 instead of the
matrix cores when the environment variable PA_DECODE_VALU is "1"; the path
exists to measure which arithmetic unit pays, and must compute the same
attention: ragged and empty sequences, every block size, G = 1 .. 16
(padded groups), several table windows, NaN-poisoned pools, bf16 and fp32
outputs.
"""
import pytest
import torch

import oracle
import paged_kv_cache_443_amd as pa
from gpu_util import DEV, TOL, max_err, meta, say, upload_oracle_cache
from workloads import make_custom

pytestmark = pytest.mark.gpu


def _decode(w, cache, out_dtype=torch.float32):
    q, tables, lens = meta(w)
    out = torch.full(q.shape, -5.0, dtype=out_dtype, device=DEV)
    pa.decode(q, cache, tables, lens, w.spec.scale, out)
    torch.cuda.synchronize()
    return out


CASES = []
for bs in (16, 32, 64):
    for Hq, Hkv in ((8, 8), (16, 8), (12, 4), (40, 5), (64, 8), (16, 1)):
        CASES.append((bs, Hq, Hkv))


@pytest.mark.parametrize("bs,Hq,Hkv", CASES)
def test_valu_decode_matches_oracle(monkeypatch, bs, Hq, Hkv):
    lens = [0, 1, 2, 31, 32, 33, bs - 1, bs + 1, 64, 65, 127, 129, 500, 1000]
    w = make_custom(B=len(lens), Hq=Hq, Hkv=Hkv, D=128, bs=bs, kv_dtype="bf16", lengths=lens, seed=300 + bs + Hq)
    oc = oracle.build_cache(w)
    want = oracle.decode(w.q, oc, w.block_tables, w.context_lens, w.spec.scale)
    cache = upload_oracle_cache(oc)
    mfma = _decode(w, cache)
    monkeypatch.setenv("PA_DECODE_VALU", "1")
    valu = _decode(w, cache)
    valu16 = _decode(w, cache, torch.bfloat16)
    monkeypatch.delenv("PA_DECODE_VALU")
    err = max_err(valu, want)
    say(f"[valu] bs={bs} Hq={Hq} Hkv={Hkv}: max abs err {err:.3e} (matrix cores {max_err(mfma, want):.3e})")
    assert err <= TOL["bf16"]
    assert torch.all(valu[0] == 0)  # empty sequence
    assert max_err(valu16, want) <= TOL["bf16"]


def test_valu_decode_spans_table_windows(monkeypatch):
    """A sequence longer than one staged table window (1024 entries)."""
    lens = [1024 * 16 + 77, 3, 4000]
    w = make_custom(B=3, Hq=2, Hkv=1, D=128, bs=16, kv_dtype="bf16", lengths=lens, seed=331)
    oc = oracle.build_cache(w)
    want = oracle.decode(w.q, oc, w.block_tables, w.context_lens, w.spec.scale)
    cache = upload_oracle_cache(oc)
    monkeypatch.setenv("PA_DECODE_VALU", "1")
    out = _decode(w, cache)
    err = max_err(out, want)
    say(f"[valu windows] max abs err {err:.3e}")
    assert err <= TOL["bf16"]


def test_valu_not_taken_where_it_does_not_apply(monkeypatch):
    """int8 caches, head_dim 64 and groups above 16 keep the matrix cores
    (their results still match the oracle with the variable set)."""
    monkeypatch.setenv("PA_DECODE_VALU", "1")
    for kv, D, Hq, Hkv in (("i8", 128, 8, 2), ("bf16", 64, 8, 2), ("bf16", 128, 32, 1)):
        w = make_custom(B=4, Hq=Hq, Hkv=Hkv, D=D, bs=16, kv_dtype=kv, lengths=[5, 100, 0, 333], seed=340)
        oc = oracle.build_cache(w)
        want = oracle.decode(w.q, oc, w.block_tables, w.context_lens, w.spec.scale)
        out = _decode(w, upload_oracle_cache(oc))
        assert max_err(out, want) <= TOL[kv], (kv, D, Hq, Hkv)
