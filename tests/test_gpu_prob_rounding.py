"""Error bound of the paths that round the softmax weights to bf16 once
(needs an MI355X).

The int4 decode and the wide multi-query units multiply V by the weights
p_t (times the token's V scale for a quantised cache) rounded to bf16 once;
the other paths split each weight into a bf16 high part and a bf16
remainder and multiply both.  One rounding moves each term p_t v_t by at most
2^-9 of itself, so an output element is off by at most

    2^-9 * sum_t p_t |v_t|  <=  2^-9 * max_t |v_t|

beyond fp32 accumulation (far smaller); the split form leaves about 2^-17 of
that.  An absolute tolerance therefore only holds for bounded |v|.  These
tests draw V 64 times larger than the benchmark workloads (|v| up to ~300)
and check each (row, head) against 2^-8 * max|v| of its sequence (the
bound with a 2x margin) on the single-rounding paths, and against 2^-13 *
max|v| on the split paths.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_443_amd as pa
from gpu_util import DEV, meta, say, to_dev_values
from oracle_pool import rows_decode
from workloads import make_custom
from workloads.device import append_tokens

pytestmark = pytest.mark.gpu

V_SCALE = 64.0
SINGLE = 2.0 ** -8  # single bf16 rounding of p (bound 2^-9, 2x margin)
SPLIT = 2.0 ** -13  # hi + lo split of p


def _vmax(w) -> np.ndarray:
    """max |v| over each sequence's tokens and kv heads (float64 [B])."""
    return np.array([float(np.max(np.abs(w.tokens(b)[1]))) if int(w.context_lens[b]) else 0.0
                     for b in range(w.B)])


@pytest.mark.parametrize("kv,rel", [("i4", SINGLE), ("bf16", SPLIT), ("i8", SPLIT)])
def test_single_token_decode_error_scales_with_v(kv, rel):
    lens = [1, 17, 300, 1024, 2048, 4000]
    w = make_custom(B=len(lens), Hq=32, Hkv=8, D=128, bs=16, kv_dtype=kv, lengths=lens, seed=211,
                    v_scale=V_SCALE)
    cache = pa.KVCache.allocate(w.num_blocks, 8, 16, 128, kv, DEV)
    append_tokens(w, cache)
    q, tables, lens_d = meta(w)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    pa.decode(q, cache, tables, lens_d, w.spec.scale, out)
    torch.cuda.synchronize()
    oc = oracle.build_cache(w)
    want = oracle.decode(w.q, oc, w.block_tables, w.context_lens, w.spec.scale)
    err = np.abs(out.cpu().numpy().astype(np.float64) - want).max(axis=2)  # [B, Hq]
    vmax = _vmax(w)
    ratio = err / vmax[:, None]
    say(f"[p rounding] {kv} decode: max |v| {vmax.max():.1f}, max abs err {err.max():.3e}, "
        f"max err / max|v| {ratio.max():.3e} (bound {rel:.3e})")
    assert np.all(ratio <= rel)


# (kv dtype, Hq, Hkv, cached tokens, new tokens, sequences, block size):
# chunks long enough to take the wide units
WIDE = [("bf16", 64, 8, 1500, 300, 8, 32), ("i8", 32, 8, 2048, 256, 8, 16), ("i4", 32, 8, 1024, 128, 16, 64)]


@pytest.mark.parametrize("case", range(len(WIDE)))
def test_wide_units_error_scales_with_v(case):
    kv, Hq, Hkv, L, n, B, bs = WIDE[case]
    custom = dict(B=B, Hq=Hq, Hkv=Hkv, D=128, bs=bs, kv_dtype=kv, lengths=[L - 29 * i for i in range(B)],
                  seed=230 + case, v_scale=V_SCALE)
    w = make_custom(**custom)
    cache = pa.KVCache.allocate(w.num_blocks, Hkv, bs, 128, kv, DEV)
    append_tokens(w, cache)
    q_start, q = w.multi_queries(np.full(B, n, np.int32))
    _, tables, lens = meta(w)
    out = torch.empty((int(q_start[-1]), Hq, 128), dtype=torch.float32, device=DEV)
    pa.decode_multi(to_dev_values(q, w.spec.q_dtype), torch.from_numpy(q_start).to(DEV), n, cache, tables, lens,
                    w.spec.scale, out)
    torch.cuda.synchronize()
    rows = sorted({(b, i) for b in range(B) for i in (0, b % 16, n // 2, n - 1)})
    want = rows_decode(custom, n, rows, w.context_lens)
    idx = torch.tensor([int(q_start[b]) + i for b, i in rows], device=DEV)
    err = np.abs(out[idx].cpu().numpy().astype(np.float64) - want).max(axis=2)  # [rows, Hq]
    vmax = _vmax(w)[[b for b, _ in rows]]
    ratio = err / vmax[:, None]
    say(f"[p rounding] wide {kv}: max |v| {vmax.max():.1f}, max abs err {err.max():.3e}, "
        f"max err / max|v| {ratio.max():.3e} (bound {SINGLE:.3e})")
    assert np.all(ratio <= SINGLE)
