"""Whole full-size batches against the oracle (needs an MI355X).

Each workload at the size the benchmark times: the cache is written by the
GPU append, then the benchmark's step runs (pa_append_decode, or
pa_append_decode_split + pa_reduce for the KV-split workload) and EVERY
sequence's output is compared with the oracle's fp64 decode, computed in
worker processes (``oracle_pool``).  The long multi-query chunks that take
the wide units are checked on every sequence, one query row in eight.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_443_amd as pa
from gpu_util import DEV, TOL, max_err, meta, poisoned_cache, say
from oracle_pool import rows_decode, whole_batch_decode
from workloads import make_custom, make_workload
from workloads.device import append_tokens, new_token_batch, to_dev_values

pytestmark = pytest.mark.gpu

SENTINEL = -123.25

# (config, overrides): the benchmark's four timed workloads and the int8
# workload's shapes with an int4 cache
FULL = [(2, {}), (3, {}), (4, {}), (5, {}), (5, {"kv_dtype": "i4"})]


@pytest.mark.parametrize("case", range(len(FULL)), ids=["cfg2", "cfg3", "cfg4", "cfg5", "cfg5-int4"])
def test_full_batch_step_matches_oracle(case):
    cfg, kw = FULL[case]
    w = make_workload(cfg, **kw)
    s = w.spec
    say(f"[full batch] cfg{cfg} {kw} B={w.B} tokens={w.total_tokens()} pool={w.num_blocks}")
    cache = poisoned_cache(w)
    append_tokens(w, cache, include_last=False)
    kn, vn, sl = new_token_batch(w)
    q, tables, lens = meta(w)
    out = torch.full(q.shape, SENTINEL, dtype=torch.float32, device=DEV)
    if s.partition_size:
        pmax = pa.max_partitions(tables.shape[1], s.bs, s.partition_size)
        B, Hq, D = q.shape
        po = torch.full((B, Hq, pmax, D), SENTINEL, dtype=torch.float32, device=DEV)
        pl = torch.full((B, Hq, pmax), SENTINEL, dtype=torch.float32, device=DEV)
        pa.append_decode_split(kn, vn, sl, q, cache, tables, lens, s.scale, s.partition_size, po, pl)
        pa.reduce(po, pl, lens, s.partition_size, out)
    else:
        pa.append_decode(kn, vn, sl, q, cache, tables, lens, s.scale, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    del out, cache
    torch.cuda.empty_cache()
    want = whole_batch_decode(cfg, kw, w.context_lens)
    err = np.abs(got - want).max(axis=(1, 2))
    worst = int(np.argmax(err))
    say(f"  all {w.B} sequences: max abs err {err.max():.3e} (sequence {worst}, length "
        f"{int(w.context_lens[worst])}), median over sequences {np.median(err):.3e}")
    assert np.all(np.isfinite(got))
    assert err.max() <= TOL[s.kv_dtype]


# long chunks that take the wide units (enough rows for two groups per
# wavefront and enough (sequence, kv head) pairs to fill the GPU):
# (kv dtype, Hq, Hkv, cached tokens, new tokens, sequences, block size)
WIDE = [
    ("bf16", 40, 40, 2048, 512, 8, 16),
    ("bf16", 64, 8, 1500, 300, 8, 32),
    ("bf16", 32, 8, 1100, 200, 8, 64),
    ("i8", 32, 8, 2048, 256, 8, 16),
    ("i4", 32, 8, 1024, 128, 16, 64),
]


@pytest.mark.parametrize("case", range(len(WIDE)))
def test_wide_units_every_sequence(case):
    """Every sequence of the chunk, query rows i = b mod 8 + 8 j (so each
    row position mod 8 is hit across the batch) plus the first and last new
    token, every head, against the oracle's decode on the context cut at the
    row's own position."""
    kv, Hq, Hkv, L, n, B, bs = WIDE[case]
    custom = dict(B=B, Hq=Hq, Hkv=Hkv, D=128, bs=bs, kv_dtype=kv, lengths=[L - 37 * i for i in range(B)],
                  seed=90 + case)
    w = make_custom(**custom)
    s = w.spec
    say(f"[multi wide] {kv} Hq={Hq} Hkv={Hkv} L<={L} n={n} B={B} bs={bs}")
    cache = pa.KVCache.allocate(w.num_blocks, Hkv, bs, 128, kv, DEV)
    append_tokens(w, cache)
    counts = np.full(B, n, np.int32)
    q_start, q = w.multi_queries(counts)
    _, tables, lens = meta(w)
    out = torch.full((int(q_start[-1]), Hq, 128), SENTINEL, dtype=torch.float32, device=DEV)
    pa.decode_multi(to_dev_values(q, s.q_dtype), torch.from_numpy(q_start).to(DEV), n, cache, tables, lens, s.scale,
                    out)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(out))
    rows = sorted({(b, i) for b in range(B) for i in [*range(b % 8, n, 8), 0, n - 1]})
    want = rows_decode(custom, n, rows, w.context_lens)
    idx = torch.tensor([int(q_start[b]) + i for b, i in rows], device=DEV)
    err = max_err(out[idx], want)
    say(f"  {len(rows)} rows over all {B} sequences: max abs err {err:.3e}")
    assert err <= TOL[kv]


def test_wide_units_negative_scale():
    """A negative softmax scale on the bf16 wide units (they fold the scale
    into the exponent and take the query's sign instead): sampled rows
    against the oracle, and the output equals the launch with the query
    negated and the scale's magnitude, bit for bit."""
    B, Hq, Hkv, L, n, bs = 8, 64, 8, 1200, 300, 16
    custom = dict(B=B, Hq=Hq, Hkv=Hkv, D=128, bs=bs, kv_dtype="bf16", lengths=[L - 41 * i for i in range(B)],
                  seed=97, scale=-0.7 / np.sqrt(128))
    w = make_custom(**custom)
    s = w.spec
    say(f"[multi wide, scale {s.scale:.4f}] Hq={Hq} Hkv={Hkv} L<={L} n={n} B={B}")
    cache = pa.KVCache.allocate(w.num_blocks, Hkv, bs, 128, "bf16", DEV)
    append_tokens(w, cache)
    q_start, q = w.multi_queries(np.full(B, n, np.int32))
    _, tables, lens = meta(w)
    qs = torch.from_numpy(q_start).to(DEV)

    def run(qv, scale):
        out = torch.full((int(q_start[-1]), Hq, 128), SENTINEL, dtype=torch.float32, device=DEV)
        pa.decode_multi(to_dev_values(qv, s.q_dtype), qs, n, cache, tables, lens, scale, out)
        torch.cuda.synchronize()
        return out

    out = run(q, s.scale)
    assert torch.all(torch.isfinite(out))
    assert torch.equal(out, run(-q, -s.scale))
    rows = sorted({(b, i) for b in range(B) for i in (0, 7 * b + 3, n - 1)})
    want = rows_decode(custom, n, rows, w.context_lens)
    idx = torch.tensor([int(q_start[b]) + i for b, i in rows], device=DEV)
    err = max_err(out[idx], want)
    say(f"  {len(rows)} rows: max abs err {err:.3e}")
    assert err <= TOL["bf16"]
