"""Causal multi-query paged attention (pa_decode_multi) vs the fp64 oracle,
through the C ABI (needs an MI355X)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_443_amd as pa
from gpu_util import DEV, TOL, bf16_rne_of, max_err, meta, say, to_dev_values, upload_oracle_cache
from workloads import make_custom, make_workload

pytestmark = pytest.mark.gpu

SENTINEL = -123.25


def _multi_gpu(w, cache, q_start, q, max_q, out_dtype=torch.float32, out=None):
    _, tables, lens = meta(w)
    qd = to_dev_values(q, w.spec.q_dtype)
    qs = torch.from_numpy(q_start).to(DEV)
    if out is None:
        out = torch.full(q.shape, SENTINEL, dtype=out_dtype, device=DEV)
    pa.decode_multi(qd, qs, max_q, cache, tables, lens, w.spec.scale, out)
    torch.cuda.synchronize()
    return out


# (kv dtype, Hq, Hkv, D, bs, max new tokens, lengths): ragged lengths, a
# sequence that is all new tokens, empty sequences, row groups of 16 that
# straddle query tokens (G = 3, 5), MHA with many row groups, MQA.
CASES = [
    ("bf16", 64, 8, 128, 16, 5, [37, 1, 300, 5, 0, 129, 64, 17, 1000, 2]),
    ("bf16", 8, 8, 128, 16, 20, [20, 45, 7, 400, 33, 0]),
    ("bf16", 12, 4, 64, 64, 6, [6, 130, 64, 65, 700, 3]),
    ("bf16", 10, 2, 128, 32, 4, [31, 32, 33, 250, 4, 1]),
    ("i8", 16, 4, 128, 32, 7, [7, 90, 257, 33, 1, 512]),
    ("i8", 8, 1, 64, 16, 3, [3, 48, 49, 600, 0, 2]),
    ("i8", 40, 8, 128, 16, 9, [100, 9, 16, 17, 800]),
    # chunked-prefill sized chunks: up to 100 new tokens, hundreds of rows per kv head
    ("bf16", 16, 2, 128, 16, 100, [150, 300, 100, 40]),
    ("i8", 8, 8, 64, 32, 64, [64, 200, 129]),
    # wide units (two row groups per wavefront): bf16 head_dim 64, int8, int4
    ("bf16", 8, 8, 64, 32, 300, [300, 420, 77]),
    ("i8", 16, 2, 128, 16, 40, [40, 250, 90, 17]),
    ("i4", 24, 4, 128, 64, 30, [30, 200, 333]),
    ("bf16", 32, 8, 128, 16, 70, [70, 1100, 5, 300]),
    # fp32 caches (vector ALUs, one wavefront per query row and head)
    ("f32", 8, 2, 64, 16, 5, [37, 1, 300, 5, 0, 129]),
    ("f32", 4, 4, 128, 32, 9, [9, 70, 33, 250]),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_multi_matches_oracle(case):
    kv, Hq, Hkv, D, bs, mq, lens = CASES[case]
    w = make_custom(B=len(lens), Hq=Hq, Hkv=Hkv, D=D, bs=bs, kv_dtype=kv, lengths=lens, seed=40 + case)
    counts = w.query_counts(mq)
    counts[np.argmax(w.context_lens)] = min(mq, int(np.max(w.context_lens)))  # at least one at the bound
    q_start, q = w.multi_queries(counts)
    say(f"[multi] case {case}: {kv} Hq={Hq} Hkv={Hkv} D={D} bs={bs} max_q={mq} counts={counts.tolist()}")
    oc = oracle.build_cache(w)
    want = oracle.decode_multi(q, q_start, oc, w.block_tables, w.context_lens, w.spec.scale)
    cache = upload_oracle_cache(oc)
    out = _multi_gpu(w, cache, q_start, q, mq)
    assert torch.all(torch.isfinite(out))
    err = max_err(out, want)
    say(f"  max abs err {err:.3e} (tol {TOL[kv]})")
    assert err <= TOL[kv]
    if kv != "f32":  # fp32 caches write fp32 rows only
        ob = _multi_gpu(w, cache, q_start, q, mq, torch.bfloat16)
        assert torch.equal(ob.view(torch.int16).cpu(), bf16_rne_of(out)), "bf16 out must be RNE of the fp32 out"
    # a looser max_q_len bound launches more row groups per unit (another
    # split of the tokens between wavefronts): the same values up to fp32
    # summation order
    out2 = _multi_gpu(w, cache, q_start, q, mq + 17)
    assert torch.all(out2 != SENTINEL)
    assert torch.max(torch.abs(out2 - out)).item() <= 1e-5
    assert max_err(out2, want) <= TOL[kv]


# Launches with enough (sequence, kv head) pairs to fill the GPU (>= 256
# units): a few row groups per kv head are served two per work-group, held by
# every wavefront.  Row groups straddle query tokens (G = 3, 5), sequences
# shorter than their new tokens, empty ones and one new token mix with full
# ones.
BIG = [
    ("bf16", 64, 8, 128, 16, 8, 32),
    ("bf16", 12, 4, 64, 32, 6, 64),
    ("bf16", 40, 8, 128, 64, 5, 40),
    ("i8", 64, 8, 128, 16, 8, 32),
    ("i8", 24, 4, 64, 32, 6, 64),
    ("i4", 64, 8, 128, 16, 8, 32),
]


@pytest.mark.parametrize("case", range(len(BIG)))
def test_many_units_match_oracle(case):
    kv, Hq, Hkv, D, bs, mq, B = BIG[case]
    rng = np.random.default_rng(900 + case)
    lens = rng.integers(1, 400, size=B)
    lens[:4] = [0, 1, mq - 1, mq]
    w = make_custom(B=B, Hq=Hq, Hkv=Hkv, D=D, bs=bs, kv_dtype=kv, lengths=lens.tolist(), seed=60 + case)
    counts = w.query_counts(mq)
    counts[5::3] = np.minimum(mq, w.context_lens[5::3])  # a third at the bound
    q_start, q = w.multi_queries(counts)
    say(f"[multi many] case {case}: {kv} Hq={Hq} Hkv={Hkv} D={D} bs={bs} max_q={mq} B={B}")
    oc = oracle.build_cache(w)
    want = oracle.decode_multi(q, q_start, oc, w.block_tables, w.context_lens, w.spec.scale)
    cache = upload_oracle_cache(oc)
    out = _multi_gpu(w, cache, q_start, q, mq)
    assert torch.all(torch.isfinite(out))
    err = max_err(out, want)
    say(f"  max abs err {err:.3e} (tol {TOL[kv]})")
    assert err <= TOL[kv]
    ob = _multi_gpu(w, cache, q_start, q, mq, torch.bfloat16)
    assert torch.equal(ob.view(torch.int16).cpu(), bf16_rne_of(out)), "bf16 out must be RNE of the fp32 out"


@pytest.mark.parametrize("cfg", [1, 2, 3, 5, "mqa"])
def test_one_new_token_is_decode_bitwise(cfg):
    """With one new token per sequence (max_q_len 1) the multi-query path is
    pa_decode, bit for bit."""
    if cfg == "mqa":  # 40 query heads on one kv head: three row groups per unit
        w = make_custom(B=5, Hq=40, Hkv=1, D=128, bs=16, kv_dtype="bf16", lengths=[1, 77, 300, 16, 513], seed=5)
    else:
        w = make_workload(cfg, small=True)
    say(f"[multi=decode] cfg{cfg} small B={w.B}")
    oc = oracle.build_cache(w)
    cache = upload_oracle_cache(oc)
    counts = (w.context_lens > 0).astype(np.int32)
    q_start = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    live = np.flatnonzero(counts)
    out = _multi_gpu(w, cache, q_start, w.q[live], 1)
    q, tables, lens = meta(w)
    ref = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    pa.decode(q, cache, tables, lens, w.spec.scale, ref)
    torch.cuda.synchronize()
    assert torch.equal(out, ref[torch.from_numpy(live).to(DEV)])


def test_rows_are_causal():
    """Changing the K/V of a sequence's last position changes only the query
    rows that see it (the last row of that sequence)."""
    lens = [40, 70, 25]
    w = make_custom(B=3, Hq=16, Hkv=4, D=128, bs=16, kv_dtype="bf16", lengths=lens, seed=77)
    counts = np.array([4, 6, 3], np.int32)
    q_start, q = w.multi_queries(counts)
    say("[multi] causality")
    oc = oracle.build_cache(w)
    cache = upload_oracle_cache(oc)
    out = _multi_gpu(w, cache, q_start, q, 6)
    # replace position L-1 of sequence 1 with a large key/value in every kv head
    L = lens[1]
    blk = int(w.block_tables[1, (L - 1) // 16])
    oc2 = oracle.build_cache(w)
    K = np.full((1, 4, 128), 3.0, np.float32)
    oracle.append(oc2, K, -K, np.array([blk * 16 + (L - 1) % 16], np.int32))
    cache2 = upload_oracle_cache(oc2)
    out2 = _multi_gpu(w, cache2, q_start, q, 6)
    last = int(q_start[2]) - 1
    changed = torch.any((out2 != out).flatten(1), dim=1).cpu().numpy()
    assert changed[last] and changed.sum() == 1, np.flatnonzero(changed)
    want = oracle.decode_multi(q, q_start, oc2, w.block_tables, w.context_lens, w.spec.scale)
    assert max_err(out2, want) <= TOL["bf16"]


def test_out_of_range_q_start_is_skipped():
    """A sequence whose q_start entries leave [0, num_queries] is skipped; the
    others are served."""
    lens = [30, 50, 20]
    w = make_custom(B=3, Hq=8, Hkv=2, D=128, bs=16, kv_dtype="bf16", lengths=lens, seed=78)
    q_start, q = w.multi_queries(np.array([2, 3, 1], np.int32))
    oc = oracle.build_cache(w)
    want = oracle.decode_multi(q, q_start, oc, w.block_tables, w.context_lens, w.spec.scale)
    cache = upload_oracle_cache(oc)
    bad = q_start.copy()
    bad[3] = 99  # the last sequence claims rows past the end
    say("[multi] q_start past num_queries")
    out = _multi_gpu(w, cache, bad, q, 3)
    assert max_err(out[:5], want[:5]) <= TOL["bf16"]
    assert torch.all(out[5:] == SENTINEL)


def test_full_size_chunk_sampled():
    """The 13B MHA decode workload at full size with 4 new tokens per
    sequence (the multi-query step the benchmark times); sampled sequences
    against the oracle."""
    w = make_workload(2)
    s = w.spec
    from workloads.device import append_tokens
    say(f"[multi full] cfg2 B={w.B} tokens={w.total_tokens()}")
    cache = pa.KVCache.allocate(w.num_blocks, s.Hkv, s.bs, s.D, s.kv_dtype, DEV)
    append_tokens(w, cache)
    counts = np.minimum(w.context_lens, 4).astype(np.int32)
    q_start, q = w.multi_queries(counts)
    out = _multi_gpu(w, cache, q_start, q, 4)
    assert torch.all(torch.isfinite(out))
    picks = sorted({0, int(np.argmax(w.context_lens)), w.B // 2, w.B - 1})
    oc = oracle.build_cache(w, seqs=picks)
    sub_counts = counts[picks]
    sub_start = np.concatenate([[0], np.cumsum(sub_counts)]).astype(np.int32)
    sub_q = np.concatenate([q[q_start[b]:q_start[b + 1]] for b in picks])
    want = oracle.decode_multi(sub_q, sub_start, oc, w.block_tables[picks], w.context_lens[picks], s.scale)
    rows = np.concatenate([np.arange(q_start[b], q_start[b + 1]) for b in picks])
    err = max_err(out[torch.from_numpy(rows).to(DEV)], want)
    say(f"  sampled seqs {picks}: max abs err {err:.3e}")
    assert err <= TOL[s.kv_dtype]
