"""pa_append_decode (one decode step in one call) vs pa_reshape_and_cache +
pa_decode, and pa_append_decode_split vs pa_reshape_and_cache +
pa_decode_split, bit for bit, and both vs the oracle, through the C ABI
(needs an MI355X)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_443_amd as pa
from gpu_util import DEV, TOL, download_cache, gpu_append_tokens, max_err, meta, poisoned_cache, say
from workloads import make_custom, make_workload
from workloads.device import new_token_batch

pytestmark = pytest.mark.gpu


def _two_ways(w, out_dtype=torch.float32):
    s = w.spec
    q, tables, lens = meta(w)
    kn, vn, sl = new_token_batch(w)
    fused = poisoned_cache(w)
    gpu_append_tokens(w, fused, include_last=False)
    apart = poisoned_cache(w)
    gpu_append_tokens(w, apart, include_last=False)
    out_f = torch.full(q.shape, float("nan"), dtype=out_dtype, device=DEV)
    out_a = torch.full(q.shape, float("nan"), dtype=out_dtype, device=DEV)
    pa.append_decode(kn, vn, sl, q, fused, tables, lens, s.scale, out_f)
    pa.reshape_and_cache(kn, vn, sl, apart)
    pa.decode(q, apart, tables, lens, s.scale, out_a)
    torch.cuda.synchronize()
    return fused, apart, out_f, out_a


def _same_pools(a: pa.KVCache, b: pa.KVCache) -> bool:
    ka, va, ksa, vsa = download_cache(a)
    kb, vb, ksb, vsb = download_cache(b)
    ok = np.array_equal(ka.view(np.uint8), kb.view(np.uint8)) and np.array_equal(va.view(np.uint8), vb.view(np.uint8))
    if ksa is not None:
        ok = ok and np.array_equal(ksa.view(np.uint16), ksb.view(np.uint16))
        ok = ok and np.array_equal(vsa.view(np.uint16), vsb.view(np.uint16))
    return ok


CASES = [
    ("cfg2", lambda: make_workload(2, small=True)),
    ("cfg3 beams", lambda: make_workload(3, small=True)),
    ("cfg5 int8", lambda: make_workload(5, small=True)),
    ("cfg5 int4", lambda: make_workload(5, small=True, kv_dtype="i4")),
    ("mha d64 bs32", lambda: make_custom(B=6, Hq=8, Hkv=8, D=64, bs=32, kv_dtype="bf16",
                                         lengths=[1, 31, 32, 33, 200, 0], seed=21)),
    # the last chunk's wavefront writes the new row: a second table window
    # (more than 1024 blocks), blocks spanning two chunks (bs 64), int8 at bs 32
    ("gqa two windows", lambda: make_custom(B=3, Hq=8, Hkv=2, D=128, bs=16, kv_dtype="bf16",
                                            lengths=[16400, 16384, 33], seed=23)),
    ("gqa bs64", lambda: make_custom(B=5, Hq=16, Hkv=2, D=128, bs=64, kv_dtype="bf16",
                                     lengths=[64, 65, 130, 1, 0], seed=24)),
    ("int8 d64 bs32", lambda: make_custom(B=4, Hq=8, Hkv=2, D=64, bs=32, kv_dtype="i8",
                                          lengths=[32, 33, 97, 2], seed=25)),
    ("int4 bs64", lambda: make_custom(B=4, Hq=8, Hkv=2, D=128, bs=64, kv_dtype="i4",
                                      lengths=[64, 129, 3, 700], seed=26)),
    # no fused kernel: fp32 cache, and 32 query heads per kv head (two launches)
    ("cfg1 f32", lambda: make_workload(1)),
    ("mqa 32 heads", lambda: make_custom(B=4, Hq=32, Hkv=1, D=128, bs=16, kv_dtype="bf16",
                                         lengths=[5, 70, 16, 300], seed=22)),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_fused_step_equals_two_calls_and_oracle(case):
    name, make = CASES[case]
    w = make()
    say(f"[fused] {name} B={w.B}")
    fused, apart, out_f, out_a = _two_ways(w)
    assert torch.equal(out_f, out_a), "the fused step must give the two calls' output bit for bit"
    assert _same_pools(fused, apart), "and the same cache"
    want = oracle.decode(w.q, oracle.build_cache(w), w.block_tables, w.context_lens, w.spec.scale)
    err = max_err(out_f, want)
    say(f"  max abs err {err:.3e}")
    assert err <= TOL[w.spec.kv_dtype]


@pytest.mark.parametrize("cfg", [2, 3, 5, "5-int4"])
def test_fused_step_full_size_bitwise(cfg):
    """The benchmark's workloads at full size: fused step = two calls, bit for bit."""
    w = make_workload(5, kv_dtype="i4") if cfg == "5-int4" else make_workload(cfg)
    say(f"[fused full] cfg{cfg} B={w.B} tokens={w.total_tokens()}")
    fused, apart, out_f, out_a = _two_ways(w, torch.bfloat16)
    assert torch.equal(out_f.view(torch.int16), out_a.view(torch.int16))
    assert _same_pools(fused, apart)


@pytest.mark.parametrize("kv", ["bf16", "i8", "i4"])
def test_fused_step_with_skipped_appends(kv):
    """Sequences whose new token is not appended (slot -1, or past the pool)
    read position L - 1 from the cache, as pa_decode does after a skipped
    append: their key/value rows must not reach the output."""
    w = make_custom(B=6, Hq=16, Hkv=2, D=128, bs=16, kv_dtype=kv, lengths=[40, 17, 300, 1, 64, 129], seed=27)
    s = w.spec
    say(f"[fused skipped] {kv} B={w.B}")
    q, tables, lens = meta(w)
    kn, vn, sl = new_token_batch(w)
    sl = sl.clone()
    sl[1] = -1
    sl[3] = w.num_blocks * s.bs + 5  # past the pool: the append skips it
    sl[4] = -1
    # rows that would change the output if they were used
    kn = kn * 50
    vn = vn * 50
    fused = poisoned_cache(w)
    gpu_append_tokens(w, fused, include_last=True)
    apart = poisoned_cache(w)
    gpu_append_tokens(w, apart, include_last=True)
    out_f = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
    out_a = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
    pa.append_decode(kn, vn, sl, q, fused, tables, lens, s.scale, out_f)
    pa.reshape_and_cache(kn, vn, sl, apart)
    pa.decode(q, apart, tables, lens, s.scale, out_a)
    torch.cuda.synchronize()
    assert torch.equal(out_f, out_a)
    assert _same_pools(fused, apart)
    # the skipped sequences still see their original last token
    want = oracle.decode(w.q, oracle.build_cache(w), w.block_tables, w.context_lens, s.scale)
    skipped = [1, 3, 4]
    err = float(np.max(np.abs(out_f[skipped].cpu().numpy().astype(np.float64) - want[skipped])))
    say(f"  skipped sequences: max abs err {err:.3e}")
    assert err <= TOL[kv]


SPLIT_CASES = [
    ("cfg4 long context", lambda: make_workload(4, small=True), None),
    ("gqa bf16 bs16 P32", lambda: make_custom(B=5, Hq=16, Hkv=2, D=128, bs=16, kv_dtype="bf16",
                                              lengths=[1, 31, 32, 33, 700], seed=28), 32),
    ("gqa int8 bs16 P64", lambda: make_custom(B=4, Hq=8, Hkv=2, D=128, bs=16, kv_dtype="i8",
                                              lengths=[64, 65, 300, 2], seed=29), 64),
    ("mha int8 d64 bs32 P32", lambda: make_custom(B=3, Hq=4, Hkv=4, D=64, bs=32, kv_dtype="i8",
                                                  lengths=[32, 95, 0], seed=30), 32),
    # not fused: int4 cache, and 32 query heads per kv head (two launches)
    ("int4 bs16 P32", lambda: make_custom(B=3, Hq=8, Hkv=2, D=128, bs=16, kv_dtype="i4",
                                          lengths=[40, 3, 200], seed=31), 32),
    ("mqa 32 heads P32", lambda: make_custom(B=3, Hq=32, Hkv=1, D=128, bs=16, kv_dtype="bf16",
                                             lengths=[40, 3, 200], seed=32), 32),
]


@pytest.mark.parametrize("case", range(len(SPLIT_CASES)))
def test_fused_split_step_equals_two_calls_and_oracle(case):
    """pa_append_decode_split = pa_reshape_and_cache + pa_decode_split, bit for
    bit (partials, lse and cache), and the merged result matches the oracle."""
    name, make, P = SPLIT_CASES[case]
    w = make()
    s = w.spec
    P = P or s.partition_size
    say(f"[fused split] {name} B={w.B} P={P}")
    q, tables, lens = meta(w)
    kn, vn, sl = new_token_batch(w)
    pmax = pa.max_partitions(tables.shape[1], s.bs, P)
    B, Hq, D = q.shape
    res = []
    for fused in (True, False):
        c = poisoned_cache(w)
        gpu_append_tokens(w, c, include_last=False)
        po = torch.full((B, Hq, pmax, D), float("nan"), dtype=torch.float32, device=DEV)
        pl = torch.full((B, Hq, pmax), float("nan"), dtype=torch.float32, device=DEV)
        if fused:
            pa.append_decode_split(kn, vn, sl, q, c, tables, lens, s.scale, P, po, pl)
        else:
            pa.reshape_and_cache(kn, vn, sl, c)
            pa.decode_split(q, c, tables, lens, s.scale, P, po, pl)
        torch.cuda.synchronize()
        res.append((c, po, pl))
    (cf, pof, plf), (ca, poa, pla) = res
    assert torch.equal(pof.view(torch.int32), poa.view(torch.int32)), "partials must equal the two calls' bit for bit"
    assert torch.equal(plf.view(torch.int32), pla.view(torch.int32))
    assert _same_pools(cf, ca)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    pa.reduce(pof, plf, lens, P, out)
    torch.cuda.synchronize()
    want = oracle.decode(w.q, oracle.build_cache(w), w.block_tables, w.context_lens, s.scale)
    err = max_err(out, want)
    say(f"  max abs err {err:.3e}")
    assert err <= TOL[s.kv_dtype]


def test_fused_split_step_full_size_bitwise():
    """The long-context workload at full size: fused split step = two calls, bit for bit."""
    w = make_workload(4)
    s = w.spec
    say(f"[fused split full] cfg4 B={w.B} tokens={w.total_tokens()}")
    q, tables, lens = meta(w)
    kn, vn, sl = new_token_batch(w)
    pmax = pa.max_partitions(tables.shape[1], s.bs, s.partition_size)
    B, Hq, D = q.shape
    res = []
    for fused in (True, False):
        c = poisoned_cache(w)
        gpu_append_tokens(w, c, include_last=False)
        po = torch.full((B, Hq, pmax, D), float("nan"), dtype=torch.float32, device=DEV)
        pl = torch.full((B, Hq, pmax), float("nan"), dtype=torch.float32, device=DEV)
        if fused:
            pa.append_decode_split(kn, vn, sl, q, c, tables, lens, s.scale, s.partition_size, po, pl)
        else:
            pa.reshape_and_cache(kn, vn, sl, c)
            pa.decode_split(q, c, tables, lens, s.scale, s.partition_size, po, pl)
        torch.cuda.synchronize()
        res.append((c, po, pl))
        del c
    (cf, pof, plf), (ca, poa, pla) = res
    assert torch.equal(pof.view(torch.int32), poa.view(torch.int32))
    assert torch.equal(plf.view(torch.int32), pla.view(torch.int32))
    assert _same_pools(cf, ca)


@pytest.mark.parametrize("kv", ["bf16", "i8"])
def test_fused_split_step_with_skipped_appends(kv):
    """pa_append_decode_split with some appends skipped (slot -1, or past the
    pool): those sequences read position L - 1 from the cache; partials equal
    the two calls' bit for bit and the merge matches the oracle."""
    w = make_custom(B=6, Hq=16, Hkv=2, D=128, bs=16, kv_dtype=kv, lengths=[40, 17, 300, 1, 64, 129], seed=33)
    s = w.spec
    P = 32
    say(f"[fused split skipped] {kv} B={w.B}")
    q, tables, lens = meta(w)
    kn, vn, sl = new_token_batch(w)
    sl = sl.clone()
    sl[1] = -1
    sl[3] = w.num_blocks * s.bs + 5
    sl[4] = -1
    kn = kn * 50
    vn = vn * 50
    pmax = pa.max_partitions(tables.shape[1], s.bs, P)
    B, Hq, D = q.shape
    res = []
    for fused in (True, False):
        c = poisoned_cache(w)
        gpu_append_tokens(w, c, include_last=True)
        po = torch.full((B, Hq, pmax, D), float("nan"), dtype=torch.float32, device=DEV)
        pl = torch.full((B, Hq, pmax), float("nan"), dtype=torch.float32, device=DEV)
        if fused:
            pa.append_decode_split(kn, vn, sl, q, c, tables, lens, s.scale, P, po, pl)
        else:
            pa.reshape_and_cache(kn, vn, sl, c)
            pa.decode_split(q, c, tables, lens, s.scale, P, po, pl)
        torch.cuda.synchronize()
        res.append((c, po, pl))
    (cf, pof, plf), (ca, poa, pla) = res
    assert torch.equal(pof.view(torch.int32), poa.view(torch.int32))
    assert torch.equal(plf.view(torch.int32), pla.view(torch.int32))
    assert _same_pools(cf, ca)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    pa.reduce(pof, plf, lens, P, out)
    torch.cuda.synchronize()
    want = oracle.decode(w.q, oracle.build_cache(w), w.block_tables, w.context_lens, s.scale)
    skipped = [1, 3, 4]
    err = float(np.max(np.abs(out[skipped].cpu().numpy().astype(np.float64) - want[skipped])))
    say(f"  skipped sequences: max abs err {err:.3e}")
    assert err <= TOL[kv]


@pytest.mark.parametrize("kv", ["bf16", "i8", "i4"])
def test_fused_step_with_a_slot_that_is_not_position_l_minus_1(kv):
    """A slot that is not the table's slot of position L - 1 (a free block, or
    a later offset of the last block): the fused step must not splice the row
    in at L - 1 but read that position from the cache, as the two calls do."""
    w = make_custom(B=5, Hq=16, Hkv=2, D=128, bs=16, kv_dtype=kv, lengths=[40, 17, 300, 70, 129], seed=28)
    s = w.spec
    say(f"[fused slot mismatch] {kv} B={w.B}")
    q, tables, lens = meta(w)
    kn, vn, sl = new_token_batch(w)
    free = sorted(set(range(w.num_blocks)) - set(int(b) for b in w.used_blocks()))
    assert free
    sl = sl.clone()
    sl[0] = free[0] * s.bs + 7                      # a block no sequence reads
    L2 = int(w.context_lens[2])
    assert (L2 - 1) % s.bs != s.bs - 1
    sl[2] = int(w.block_tables[2][(L2 - 1) // s.bs]) * s.bs + (L2 - 1) % s.bs + 1  # a tail slot of the last block
    sl[3] = free[-1] * s.bs + (int(w.context_lens[3]) - 1) % s.bs  # L - 1's offset in a free block
    kn = kn * 50  # rows that would change the output if spliced in
    vn = vn * 50
    fused = poisoned_cache(w)
    gpu_append_tokens(w, fused, include_last=True)
    apart = poisoned_cache(w)
    gpu_append_tokens(w, apart, include_last=True)
    out_f = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
    out_a = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
    pa.append_decode(kn, vn, sl, q, fused, tables, lens, s.scale, out_f)
    pa.reshape_and_cache(kn, vn, sl, apart)
    pa.decode(q, apart, tables, lens, s.scale, out_a)
    torch.cuda.synchronize()
    assert torch.equal(out_f, out_a)
    assert _same_pools(fused, apart)
    # the sequences with mismatched slots decode over the cache as it was
    want = oracle.decode(w.q, oracle.build_cache(w), w.block_tables, w.context_lens, w.spec.scale)
    err = max_err(out_f[[0, 2, 3]], want[[0, 2, 3]])
    say(f"  max abs err (mismatched rows) {err:.3e}")
    assert err <= TOL[kv]
    if kv == "i4":
        return  # the int4 split step is two launches
    # the fused split pass takes the same check
    P = 64
    pmax = pa.max_partitions(tables.shape[1], s.bs, P)
    B, Hq, D = q.shape
    res = []
    for fuse in (True, False):
        c = poisoned_cache(w)
        gpu_append_tokens(w, c, include_last=True)
        po = torch.full((B, Hq, pmax, D), float("nan"), dtype=torch.float32, device=DEV)
        pl = torch.full((B, Hq, pmax), float("nan"), dtype=torch.float32, device=DEV)
        if fuse:
            pa.append_decode_split(kn, vn, sl, q, c, tables, lens, s.scale, P, po, pl)
        else:
            pa.reshape_and_cache(kn, vn, sl, c)
            pa.decode_split(q, c, tables, lens, s.scale, P, po, pl)
        res.append((c, po, pl))
    torch.cuda.synchronize()
    (cf, pof, plf), (ca, poa, pla) = res
    assert torch.equal(pof.view(torch.int32), poa.view(torch.int32))
    assert torch.equal(plf.view(torch.int32), pla.view(torch.int32))
    assert _same_pools(cf, ca)
