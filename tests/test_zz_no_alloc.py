"""pa_decode_split_noalloc (KV-split decode with the partials in the
library's own fixed device scratch) against pa_decode_split + pa_reduce with
a caller workspace, through the C ABI (needs an MI355X).

Two calls in a row share the one scratch array: the second, smaller call
must not see the first one's partials.  Results are compared bit for bit
with the workspace form (same kernels, same max_num_partitions) and with
the oracle within the workload tolerance."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_443_amd as pa
from gpu_util import DEV, TOL, max_err, meta, say, upload_oracle_cache
from workloads import make_custom, make_workload

pytestmark = pytest.mark.gpu


def _with_workspace(w, cache, P, out_dtype):
    q, tables, lens = meta(w)
    pmax = pa.max_partitions(tables.shape[1], w.spec.bs, P)
    B, Hq, D = q.shape
    po = torch.empty((B, Hq, pmax, D), dtype=torch.float32, device=DEV)
    pl = torch.empty((B, Hq, pmax), dtype=torch.float32, device=DEV)
    pa.decode_split(q, cache, tables, lens, w.spec.scale, P, po, pl)
    out = torch.empty(q.shape, dtype=out_dtype, device=DEV)
    pa.reduce(po, pl, lens, P, out)
    return out


def _noalloc(w, cache, P, out_dtype):
    q, tables, lens = meta(w)
    out = torch.full(q.shape, float("nan"), dtype=out_dtype, device=DEV)
    pa.decode_split_noalloc(q, cache, tables, lens, w.spec.scale, P, out)
    return out


def _cases(kv):
    big = make_workload(4, small=True) if kv == "bf16" else make_workload(5, small=True)
    bs = big.spec.bs
    small = make_custom(B=3, Hq=big.spec.Hq, Hkv=big.spec.Hkv, D=128, bs=bs, kv_dtype=kv,
                        lengths=[5 * bs + 3, bs, 1], seed=31)
    P = 512 if kv == "bf16" else 256
    return [(big, P), (small, 2 * bs)]


@pytest.mark.parametrize("kv", ["bf16", "i8"])
def test_noalloc_two_calls_match_workspace_form(kv):
    cases = _cases(kv)
    caches = []
    for w, P in cases:
        oc = oracle.build_cache(w)
        caches.append((oc, upload_oracle_cache(oc)))
    for odt in (torch.float32, torch.bfloat16):
        # two calls in a row on one stream, the second smaller; then the references
        got = [_noalloc(w, c, P, odt) for (w, P), (_, c) in zip(cases, caches)]
        torch.cuda.synchronize()
        ref = [_with_workspace(w, c, P, odt) for (w, P), (_, c) in zip(cases, caches)]
        torch.cuda.synchronize()
        for i, ((w, P), (oc, _)) in enumerate(zip(cases, caches)):
            say(f"[noalloc] {kv} call {i}: B={w.B} Hq={w.spec.Hq} P={P} out={odt}")
            assert torch.equal(got[i].view(torch.int16 if odt == torch.bfloat16 else torch.int32),
                               ref[i].view(torch.int16 if odt == torch.bfloat16 else torch.int32)), i
            if odt == torch.float32:
                want = oracle.decode(w.q, oc, w.block_tables, w.context_lens, w.spec.scale)
                err = max_err(got[i], want)
                say(f"  max abs err vs oracle {err:.3e}")
                assert err <= TOL[kv]


def test_noalloc_refuses_more_than_its_scratch():
    # 64 sequences x 64 heads x 64 partitions x (128 + 1) floats > 32 MiB
    w = make_custom(B=64, Hq=64, Hkv=8, D=128, bs=64, kv_dtype="bf16", lengths=[64] * 64, max_len=64 * 512,
                    seed=5)
    oc = oracle.build_cache(w)
    cache = upload_oracle_cache(oc)
    q, tables, lens = meta(w)
    assert pa.max_partitions(tables.shape[1], 64, 512) == 64
    out = torch.full(q.shape, 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(pa.PAError, match="max_num_partitions|workspace|partitions"):
        pa.decode_split_noalloc(q, cache, tables, lens, w.spec.scale, 512, out)
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0))
    # the same batch fits with longer partitions (8 of them)
    pa.decode_split_noalloc(q, cache, tables, lens, w.spec.scale, 4096, out)
    torch.cuda.synchronize()
    want = oracle.decode(w.q, oc, w.block_tables, w.context_lens, w.spec.scale)
    assert max_err(out, want) <= TOL["bf16"]
