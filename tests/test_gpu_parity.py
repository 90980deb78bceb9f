"""HIP path vs the fp64 oracle, through the C ABI (needs an MI355X)."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_443_amd as pa
from gpu_util import (DEV, TOL, bf16_rne_of, download_cache, fill_poison, gpu_append_tokens, max_err, meta,
                      oracle_pools, poisoned_cache, say, upload_oracle_cache)
from workloads import make_custom, make_workload

pytestmark = pytest.mark.gpu

SENTINEL = -123.25


def _decode_gpu(w, cache, out_dtype=torch.float32):
    q, tables, lens = meta(w)
    out = torch.empty(q.shape, dtype=out_dtype, device=DEV)
    pa.decode(q, cache, tables, lens, w.spec.scale, out)
    torch.cuda.synchronize()
    return out


def _split_gpu(w, cache, P, out_dtype=torch.float32):
    q, tables, lens = meta(w)
    pmax = pa.max_partitions(tables.shape[1], w.spec.bs, P)
    B, Hq, D = q.shape
    # sentinels: partitions past a sequence's end must be left untouched
    po = torch.full((B, Hq, pmax, D), SENTINEL, dtype=torch.float32, device=DEV)
    pl = torch.full((B, Hq, pmax), SENTINEL, dtype=torch.float32, device=DEV)
    pa.decode_split(q, cache, tables, lens, w.spec.scale, P, po, pl)
    out = torch.empty(q.shape, dtype=out_dtype, device=DEV)
    pa.reduce(po, pl, lens, P, out)
    torch.cuda.synchronize()
    return po, pl, out, pmax


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_decode_matches_oracle(cfg):
    w = make_workload(cfg, small=True)
    say(f"[decode] cfg{cfg} small B={w.B} tokens={w.total_tokens()}")
    oc = oracle.build_cache(w)
    want = oracle.decode(w.q, oc, w.block_tables, w.context_lens, w.spec.scale)
    cache = upload_oracle_cache(oc)
    out = _decode_gpu(w, cache)
    err = max_err(out, want)
    say(f"  max abs err {err:.3e} (tol {TOL[w.spec.kv_dtype]})")
    assert np.all(np.isfinite(out.cpu().numpy()))
    assert err <= TOL[w.spec.kv_dtype]
    if w.spec.kv_dtype != "f32":
        ob = _decode_gpu(w, cache, torch.bfloat16)
        assert torch.equal(ob.view(torch.int16).cpu(), bf16_rne_of(out)), "bf16 out must be RNE of the fp32 out"


@pytest.mark.parametrize("cfg,P", [(2, 512), (3, 256), (4, 512), (5, 1024), (1, 16)])
def test_split_matches_oracle(cfg, P):
    w = make_workload(cfg, small=True)
    say(f"[split] cfg{cfg} P={P}")
    oc = oracle.build_cache(w)
    cache = upload_oracle_cache(oc)
    po, pl, out, pmax = _split_gpu(w, cache, P)
    want_po, want_pl = oracle.decode_partials(w.q, oc, w.block_tables, w.context_lens, w.spec.scale, P, pmax)
    tol = TOL[w.spec.kv_dtype]
    # partials of partitions past a sequence's end are not part of the contract
    # (only their lse, -inf, is); compare the used ones
    gpo = po.cpu().numpy().astype(np.float64)
    for b, L in enumerate(w.context_lens):
        n = -(-int(L) // P)
        if n:
            assert np.max(np.abs(gpo[b, :, :n] - want_po[b, :, :n])) <= tol, b
    gl = pl.cpu().numpy().astype(np.float64)
    for b, L in enumerate(w.context_lens):
        n = -(-int(L) // P)
        assert np.all(gl[b, :, n:] == SENTINEL) and np.all(gpo[b, :, n:] == SENTINEL), ("touched", b)
        if n:
            assert np.all(np.isfinite(want_pl[b, :, :n]))
            assert np.max(np.abs(gl[b, :, :n] - want_pl[b, :, :n])) <= 1e-3, b
    want = oracle.decode(w.q, oc, w.block_tables, w.context_lens, w.spec.scale)
    err = max_err(out, want)
    say(f"  merged max abs err {err:.3e}")
    assert err <= tol


@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
def test_append_bit_exact(cfg):
    w = make_workload(cfg, small=True)
    say(f"[append] cfg{cfg}")
    cache = poisoned_cache(w)
    gpu_append_tokens(w, cache)
    torch.cuda.synchronize()
    oc = oracle.build_cache(w)
    k, v, ks, vs = download_cache(cache)
    okp, ovp = oracle_pools(oc)
    assert np.array_equal(k.view(np.uint8), okp.view(np.uint8))
    assert np.array_equal(v.view(np.uint8), ovp.view(np.uint8))
    if w.spec.kv_dtype == "i8":
        assert np.array_equal(ks.view(np.uint16), oc.k_scale.view(np.uint16))
        assert np.array_equal(vs.view(np.uint16), oc.v_scale.view(np.uint16))


def test_append_int8_edge_rows():
    """Quantiser corner cases (ties, zero rows, subnormal scales, clamping) bit-exact."""
    say("[append] int8 edge rows")
    rng = np.random.default_rng(5)
    D = 128
    rows = [np.zeros(D), np.full(D, 2.0 ** -17 * 1.390625)]
    base = np.array([127.0, 63.5, -1.0, 0.0, 62.5, -62.5, 0.5, -0.5] * 16)
    rows += [base, base * 2.0 ** -20, -base * 3.0]
    rows += [rng.standard_normal(D) * 10 ** rng.uniform(-6, 3) for _ in range(59)]
    X = np.stack(rows).astype(np.float32)
    from workloads import bf16_round
    X = bf16_round(X)
    T = X.shape[0]
    K = X.reshape(T, 1, D)
    V = -K
    oc = oracle.PagedCache.empty("i8", 8, 1, 16, D)
    slots = np.arange(T, dtype=np.int32) + 3
    oracle.append(oc, K, V, slots)
    c = pa.KVCache.allocate(8, 1, 16, D, "i8", DEV)
    fill_poison(c)
    from gpu_util import to_dev_values
    pa.reshape_and_cache(to_dev_values(K, "bf16"), to_dev_values(V, "bf16"), torch.from_numpy(slots).to(DEV), c)
    torch.cuda.synchronize()
    k, v, ks, vs = download_cache(c)
    okp, ovp = oracle_pools(oc)
    assert np.array_equal(k, okp) and np.array_equal(v, ovp)
    assert np.array_equal(ks.view(np.uint16), oc.k_scale.view(np.uint16))
    assert np.array_equal(vs.view(np.uint16), oc.v_scale.view(np.uint16))


EDGE = []
for kv in ("bf16", "i8", "f32"):
    for bs in (16, 32, 64):
        for D in (64, 128):
            EDGE.append((kv, bs, D))


@pytest.mark.parametrize("kv,bs,D", EDGE)
def test_edge_lengths_and_groups(kv, bs, D):
    """Lengths around block and chunk boundaries, empty sequences, several GQA groups."""
    lens = [0, 1, bs - 1, bs, bs + 1, 31, 32, 33, 63, 64, 65, 129, 200]
    for Hq, Hkv in ((8, 8), (8, 2), (16, 1), (32, 1), (12, 4), (40, 1), (80, 1)):
        w = make_custom(B=len(lens), Hq=Hq, Hkv=Hkv, D=D, bs=bs, kv_dtype=kv, lengths=lens, seed=bs * D + Hq)
        say(f"[edge] kv={kv} bs={bs} D={D} Hq={Hq} Hkv={Hkv}")
        oc = oracle.build_cache(w)
        want = oracle.decode(w.q, oc, w.block_tables, w.context_lens, w.spec.scale)
        cache = upload_oracle_cache(oc)
        out = _decode_gpu(w, cache)
        assert max_err(out, want) <= TOL[kv], (Hq, Hkv)
        assert torch.all(out[0] == 0)  # empty sequence
        P = 2 * bs
        po, pl, outs, pmax = _split_gpu(w, cache, P)
        assert max_err(outs, want) <= TOL[kv], ("split", Hq, Hkv)


@pytest.mark.parametrize("B,Hq,kv", [(300, 64, "bf16"), (300, 64, "i8"), (600, 64, "i8"), (200, 32, "bf16"),
                                      (64, 128, "bf16")])
def test_mqa_batches_both_unit_shapes(B, Hq, kv):
    """One kv head: units of one or two row groups, chosen from the GPU's
    work-group slots (large batches take two per unit, small ones one, the
    units of a sequence sharing its lines); both against the oracle."""
    rng = np.random.default_rng(B + Hq)
    lens = rng.integers(0, 300, size=B).tolist()
    w = make_custom(B=B, Hq=Hq, Hkv=1, D=128, bs=16, kv_dtype=kv, lengths=lens, seed=B * Hq)
    say(f"[mqa] B={B} Hq={Hq} kv={kv}")
    oc = oracle.build_cache(w)
    want = oracle.decode(w.q, oc, w.block_tables, w.context_lens, w.spec.scale)
    cache = upload_oracle_cache(oc)
    out = _decode_gpu(w, cache)
    err = max_err(out, want)
    say(f"  max abs err {err:.3e}")
    assert err <= TOL[kv]


def test_block_relabel_is_bitwise_invariant():
    w = make_workload(3, small=True)
    say("[relabel] cfg3 small")
    oc = oracle.build_cache(w)
    out1 = _decode_gpu(w, upload_oracle_cache(oc))
    rng = np.random.default_rng(9)
    perm = rng.permutation(oc.num_blocks)
    oc2 = oracle.PagedCache.empty(oc.kv_dtype, oc.num_blocks, oc.Hkv, oc.bs, oc.D)
    oc2.k[perm] = oc.k
    oc2.v[perm] = oc.v
    w.block_tables = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    out2 = _decode_gpu(w, upload_oracle_cache(oc2))
    assert torch.equal(out1, out2)


def test_repeatable_bitwise():
    w = make_workload(5, small=True)
    say("[repeat] cfg5 small")
    cache = upload_oracle_cache(oracle.build_cache(w))
    a = _decode_gpu(w, cache)
    b = _decode_gpu(w, cache)
    assert torch.equal(a, b)
    po1, pl1, o1, _ = _split_gpu(w, cache, 512)
    po2, pl2, o2, _ = _split_gpu(w, cache, 512)
    assert torch.equal(o1, o2) and torch.equal(pl1, pl2)


def test_cow_beams_equal_bitwise():
    """Beam pairs that share prefix blocks give identical rows for identical queries."""
    w = make_workload(3, small=True)
    say("[cow] cfg3 small")
    oc = oracle.build_cache(w, include_last=False)
    w.context_lens = np.maximum(w.context_lens - 1, 0).astype(np.int32)
    for b2, a in w.pair_of.items():
        w.q[b2] = w.q[a]
    out = _decode_gpu(w, upload_oracle_cache(oc))
    for b2, a in w.pair_of.items():
        assert torch.equal(out[a], out[b2])


def test_split_partition_sweep_agrees():
    w = make_workload(4, small=True)
    say("[sweep] cfg4 small partitions")
    oc = oracle.build_cache(w)
    want = oracle.decode(w.q, oc, w.block_tables, w.context_lens, w.spec.scale)
    cache = upload_oracle_cache(oc)
    for P in (64, 128, 512, 4096):
        _, _, out, _ = _split_gpu(w, cache, P)
        assert max_err(out, want) <= TOL["bf16"], P


def test_int8_full_cache_fill_bit_exact():
    """The whole int8 workload (about 1.1 M tokens x 8 kv heads) written by
    pa_reshape_and_cache equals the oracle's quantised cache bit for bit."""
    w = make_workload(5)
    say(f"[fill] cfg5 full B={w.B} tokens={w.total_tokens()} pool={w.num_blocks}")
    cache = poisoned_cache(w)
    gpu_append_tokens(w, cache)
    torch.cuda.synchronize()
    k, v, ks, vs = download_cache(cache)
    del cache
    torch.cuda.empty_cache()
    oc = oracle.build_cache(w, poison=True)
    used = w.used_blocks()
    say(f"  comparing {len(used)} used blocks")
    okp, ovp = oracle_pools(oc)
    assert np.array_equal(k[used], okp[used])
    assert np.array_equal(v[used], ovp[used])
    assert np.array_equal(ks[used].view(np.uint16), oc.k_scale[used].view(np.uint16))
    assert np.array_equal(vs[used].view(np.uint16), oc.v_scale[used].view(np.uint16))


def test_invalid_calls_touch_nothing():
    """A call the host validation rejects returns its status and launches
    nothing: sentinel outputs and caches stay as they were."""
    from paged_kv_cache_443_amd import _lib
    import ctypes
    say("[abi] invalid calls on device buffers")
    w = make_workload(3, small=True)
    cache = upload_oracle_cache(oracle.build_cache(w))
    q, tables, lens = meta(w)
    out = torch.full(q.shape, SENTINEL, dtype=torch.float32, device=DEV)
    L = _lib.lib()
    desc = cache.descriptor()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    B, Hq, D = q.shape
    # num_heads not a multiple of num_kv_heads
    st = L.pa_decode(q.data_ptr(), _lib.PA_BF16, B, Hq - 1, ctypes.byref(desc), tables.data_ptr(), tables.shape[1],
                     lens.data_ptr(), 0.1, out.data_ptr(), _lib.PA_F32, stream)
    assert st == _lib.PA_ERR_BAD_SHAPE
    # out misaligned by 4 bytes
    st = L.pa_decode(q.data_ptr(), _lib.PA_BF16, B, Hq, ctypes.byref(desc), tables.data_ptr(), tables.shape[1],
                     lens.data_ptr(), 0.1, out.data_ptr() + 4, _lib.PA_F32, stream)
    assert st == _lib.PA_ERR_MISALIGNED
    # fp32 queries against a bf16 cache
    st = L.pa_decode(q.data_ptr(), _lib.PA_F32, B, Hq, ctypes.byref(desc), tables.data_ptr(), tables.shape[1],
                     lens.data_ptr(), 0.1, out.data_ptr(), _lib.PA_F32, stream)
    assert st == _lib.PA_ERR_UNSUPPORTED
    # append with the wrong source dtype must not write the cache
    before = cache.k_cache.clone()
    kn = torch.zeros((2, w.spec.Hkv, w.spec.D), dtype=torch.float32, device=DEV)
    sl = torch.zeros((2,), dtype=torch.int32, device=DEV)
    st = L.pa_reshape_and_cache(kn.data_ptr(), kn.data_ptr(), _lib.PA_F32, sl.data_ptr(), 2, ctypes.byref(desc),
                                stream)
    assert st == _lib.PA_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(out == SENTINEL)
    assert torch.equal(before.view(torch.int16), cache.k_cache.view(torch.int16))  # bitwise: the pool holds NaN poison


def test_side_stream_matches_default_stream():
    """The binding launches on torch's current stream: a decode issued on a
    side stream gives the same bits as on the default stream."""
    w = make_workload(2, small=True)
    say("[stream] cfg2 small on a side stream")
    cache = upload_oracle_cache(oracle.build_cache(w))
    ref = _decode_gpu(w, cache)
    q, tables, lens = meta(w)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
        pa.decode(q, cache, tables, lens, w.spec.scale, out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("cfg", [3, 4])
@pytest.mark.parametrize("fused", [False, True])
def test_graph_replays_match_eager(cfg, fused):
    """A decode step (append + decode, or append + split + merge; as separate
    calls or as the fused calls) captured in a HIP graph replays to the eager
    result every time, with eager work between the replays."""
    w = make_workload(cfg, small=True)
    s = w.spec
    say(f"[graph] cfg{cfg} small fused={fused}")
    cache = poisoned_cache(w)
    gpu_append_tokens(w, cache, include_last=False)
    from workloads.device import new_token_batch
    kn, vn, sl = new_token_batch(w)
    q, tables, lens = meta(w)
    P = s.partition_size or 256
    pmax = pa.max_partitions(tables.shape[1], s.bs, P)
    B, Hq, D = q.shape
    po = torch.zeros((B, Hq, pmax, D), dtype=torch.float32, device=DEV)
    pl = torch.zeros((B, Hq, pmax), dtype=torch.float32, device=DEV)
    out = torch.zeros(q.shape, dtype=torch.float32, device=DEV)

    def step():
        if fused and s.partition_size:
            pa.append_decode_split(kn, vn, sl, q, cache, tables, lens, s.scale, P, po, pl)
            pa.reduce(po, pl, lens, P, out)
        elif fused:
            pa.append_decode(kn, vn, sl, q, cache, tables, lens, s.scale, out)
        else:
            pa.reshape_and_cache(kn, vn, sl, cache)
            if s.partition_size:
                pa.decode_split(q, cache, tables, lens, s.scale, P, po, pl)
                pa.reduce(po, pl, lens, P, out)
            else:
                pa.decode(q, cache, tables, lens, s.scale, out)

    step()
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for i in range(3):
        out.fill_(float("nan"))
        _decode_gpu(w, cache)  # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i}"


def test_graph_replays_multi_query_and_int4():
    """Captured HIP graphs of a multi-query step (append + pa_decode_multi)
    and of an int4 step (append with nibble atomics + decode) replay to the
    eager result every time, with eager work between the replays."""
    from workloads.device import new_token_batch
    # int4 step
    w = make_workload(5, small=True, kv_dtype="i4")
    s = w.spec
    say("[graph] int4 step")
    cache = poisoned_cache(w)
    gpu_append_tokens(w, cache, include_last=False)
    kn, vn, sl = new_token_batch(w)
    q, tables, lens = meta(w)
    out = torch.zeros(q.shape, dtype=torch.float32, device=DEV)
    # multi-query step on a bf16 cache (4 new tokens per sequence, causal)
    wm = make_custom(B=4, Hq=16, Hkv=4, D=128, bs=16, kv_dtype="bf16", lengths=[40, 90, 17, 300], seed=95)
    cm = poisoned_cache(wm)
    gpu_append_tokens(wm, cm)
    qs_np, qm_np = wm.multi_queries(np.full(4, 4, np.int32))
    from gpu_util import to_dev_values
    qm = to_dev_values(qm_np, "bf16")
    qs = torch.from_numpy(qs_np).to(DEV)
    _, tm, lm = meta(wm)
    outm = torch.zeros(qm.shape, dtype=torch.float32, device=DEV)

    def step():
        pa.reshape_and_cache(kn, vn, sl, cache)
        pa.decode(q, cache, tables, lens, s.scale, out)
        pa.decode_multi(qm, qs, 4, cm, tm, lm, wm.spec.scale, outm)

    step()
    torch.cuda.synchronize()
    ref, refm = out.clone(), outm.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for i in range(3):
        out.fill_(float("nan"))
        outm.fill_(float("nan"))
        _decode_gpu(w, cache)  # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"int4 replay {i}"
        assert torch.equal(outm, refm), f"multi replay {i}"
    # the int4 step writes the same bytes every replay (the nibble atomics are idempotent)
    oc = oracle.build_cache(w)
    k, v, ks, vs = download_cache(cache)
    okp, ovp = oracle_pools(oc)
    assert np.array_equal(k, okp) and np.array_equal(v, ovp)
