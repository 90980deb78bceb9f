"""pa_mla_decode / pa_mla_append (decode over an MLA latent cache) vs the
fp64 oracle, through the C ABI (needs an MI355X).

Inputs come from ``workloads.mla`` (seeded latent rows, queries and
up-projections); expected values from ``oracle.mla_*`` only."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_443_amd as pa
from gpu_util import DEV, TOL, bf16_rne_of, max_err, say
from workloads import bf16_bits, make_mla, make_mla_custom
from workloads.device import mla_fill

pytestmark = pytest.mark.gpu


def _bf16_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(bf16_bits(np.asarray(x, np.float32)).view(np.int16)).to(DEV).view(torch.bfloat16)


def _upload(oc: "oracle.LatentCache") -> pa.LatentCache:
    t = _bf16_dev(oc.c)  # poison NaN stays NaN
    return pa.LatentCache(t.contiguous(), oc.num_blocks, oc.bs, oc.d_c)


def _gpu_fill(w) -> pa.LatentCache:
    """Device latent pool, every element NaN, every cached token written by pa_mla_append."""
    return mla_fill(w, DEV)


def _decode(w, cache, P, out_dtype=torch.float32, tables=None):
    s = w.spec
    tbl = torch.from_numpy(w.block_tables if tables is None else tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    q = _bf16_dev(w.q)
    wk, wv = _bf16_dev(w.w_uk), _bf16_dev(w.w_uv)
    nbytes = pa.mla_workspace_bytes(s.B, s.H, cache, tbl.shape[1], P)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    out = torch.full(q.shape, float("nan"), dtype=out_dtype, device=DEV)
    pa.mla_decode(q, wk, wv, cache, tbl, lens, s.scale, P, ws, out)
    torch.cuda.synchronize()
    return out


def _want(w, oc=None):
    oc = oracle.mla_build_cache(w) if oc is None else oc
    return oracle.mla_decode(w.q, oc, w.w_uk, w.w_uv, w.block_tables, w.context_lens, w.spec.scale)


def test_mla_append_is_bit_exact():
    w = make_mla(small=True)
    say(f"[mla append] B={w.B} tokens={w.total_tokens()}")
    c = _gpu_fill(w)
    torch.cuda.synchronize()
    got = c.latent.view(torch.int16).cpu().numpy().view(np.uint16)
    want = bf16_bits(oracle.mla_build_cache(w).c.astype(np.float32))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("P", [64, 256, 1024])
def test_mla_decode_matches_oracle(P):
    w = make_mla(small=True)
    say(f"[mla decode] B={w.B} H={w.spec.H} P={P}")
    cache = _gpu_fill(w)
    out = _decode(w, cache, P)
    err = max_err(out, _want(w))
    say(f"  max abs err {err:.3e}")
    assert np.all(np.isfinite(out.cpu().numpy()))
    assert err <= TOL["bf16"]
    ob = _decode(w, cache, P, torch.bfloat16)
    assert torch.equal(ob.view(torch.int16).cpu(), bf16_rne_of(out)), "bf16 out must be RNE of the fp32 out"


EDGE = [
    # (H, d_h, bs, lengths, P): empty and one-token sequences, chunk and block edges,
    # a head count below one group, two groups with a ragged second, head_dim 64
    (16, 128, 16, [0, 1, 63, 64, 65, 129, 1000], 256),
    (1, 128, 16, [7, 200], 128),
    (20, 128, 32, [33, 64, 500], 192),
    (32, 64, 64, [64, 65, 640, 1], 640),
    (8, 64, 16, [2000, 3, 1024], 1024),
]


@pytest.mark.parametrize("case", range(len(EDGE)))
def test_mla_edge_shapes(case):
    H, d_h, bs, lens, P = EDGE[case]
    w = make_mla_custom(H=H, d_h=d_h, d_c=512, bs=bs, lengths=lens, seed=50 + case, partition_size=P)
    say(f"[mla edge] H={H} d_h={d_h} bs={bs} lens={lens} P={P}")
    oc = oracle.mla_build_cache(w)
    out = _decode(w, _upload(oc), P)
    err = max_err(out, _want(w, oc))
    say(f"  max abs err {err:.3e}")
    assert err <= TOL["bf16"]
    for b, L in enumerate(lens):
        if L == 0:
            assert bool(torch.all(out[b] == 0))


def test_mla_block_relabelling_is_bitwise_invariant():
    w = make_mla(small=True)
    oc = oracle.mla_build_cache(w, poison=False)
    base = _decode(w, _upload(oc), 256)
    perm = np.random.default_rng(7).permutation(oc.num_blocks)
    moved = oracle.LatentCache(np.empty_like(oc.c))
    moved.c[perm] = oc.c
    tables = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    got = _decode(w, _upload(moved), 256, tables=tables)
    assert torch.equal(got, base)


def test_mla_refuses_a_short_workspace():
    w = make_mla(small=True)
    s = w.spec
    cache = _gpu_fill(w)
    tbl = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    nbytes = pa.mla_workspace_bytes(s.B, s.H, cache, tbl.shape[1], 1024)
    ws = torch.empty(nbytes - 256, dtype=torch.uint8, device=DEV)
    out = torch.full((s.B, s.H, s.d_h), 3.0, dtype=torch.float32, device=DEV)
    with pytest.raises(pa.PAError):
        pa.mla_decode(_bf16_dev(w.q), _bf16_dev(w.w_uk), _bf16_dev(w.w_uv), cache, tbl, lens, s.scale, 1024, ws, out)
    torch.cuda.synchronize()
    assert bool(torch.all(out == 3.0))


def test_mla_full_size_every_sequence():
    """The benchmark's MLA batch (128 sequences of 1024-8192 tokens, 16 heads over
    a 512-wide latent) in the benchmark's launch, every sequence against the oracle."""
    w = make_mla()
    s = w.spec
    say(f"[mla full] B={w.B} tokens={w.total_tokens()} P={s.partition_size}")
    cache = _gpu_fill(w)
    out = _decode(w, cache, s.partition_size).cpu().numpy().astype(np.float64)
    oc = oracle.mla_build_cache(w)
    worst = 0.0
    for b0 in range(0, w.B, 16):
        sl = slice(b0, b0 + 16)
        want = oracle.mla_decode(w.q[sl], oc, w.w_uk, w.w_uv, w.block_tables[sl], w.context_lens[sl], s.scale)
        worst = max(worst, float(np.max(np.abs(out[sl] - want))))
    say(f"  max abs err over all {w.B} sequences {worst:.3e}")
    assert worst <= TOL["bf16"]
