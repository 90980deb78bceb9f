"""Copy-on-write on the GPU: pa_copy_blocks and a beam-search scenario
driven by the C++ block manager, against the oracle (needs an MI355X)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_443_amd as pa
from gpu_util import DEV, TOL, download_cache, max_err, oracle_pools, say, to_dev_values, upload_oracle_cache
from workloads import bf16_round

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv,bs", [("f32", 16), ("bf16", 16), ("bf16", 64), ("i8", 16), ("i8", 32)])
def test_copy_blocks_bit_exact(kv, bs):
    say(f"[copy] kv={kv} bs={bs}")
    rng = np.random.default_rng(bs)
    nb, H, D = 24, 4, 128
    oc = oracle.PagedCache.empty(kv, nb, H, bs, D)
    K = rng.standard_normal((nb * bs, H, D)).astype(np.float32)
    V = rng.standard_normal((nb * bs, H, D)).astype(np.float32)
    if kv != "f32":
        K, V = bf16_round(K), bf16_round(V)
    oracle.append(oc, K[: 20 * bs], V[: 20 * bs], np.arange(20 * bs))  # blocks 20..23 stay poison
    cache = upload_oracle_cache(oc)
    pairs = [(3, 21), (7, 0), (19, 22), (0 + 1, 23), (5, 40), (-1, 2)]  # the last two are skipped (out of range)
    dev_pairs = torch.tensor(pairs, dtype=torch.int32, device=DEV)
    pa.copy_blocks(cache, dev_pairs)
    torch.cuda.synchronize()
    oracle.copy_blocks(oc, [p for p in pairs if 0 <= min(p) and max(p) < nb])
    k, v, ks, vs = download_cache(cache)
    okp, ovp = oracle_pools(oc)
    assert np.array_equal(k.view(np.uint8), okp.view(np.uint8))
    assert np.array_equal(v.view(np.uint8), ovp.view(np.uint8))
    if kv == "i8":
        assert np.array_equal(ks.view(np.uint16), oc.k_scale.view(np.uint16))
        assert np.array_equal(vs.view(np.uint16), oc.v_scale.view(np.uint16))


def test_beam_search_with_copy_on_write_matches_oracle():
    """Prompts are written, each sequence forks into beams, and every beam
    appends its own tokens for several steps; the C++ block manager decides
    slots and copy-on-write copies, the GPU runs copy_blocks, append and
    decode.  The oracle does the same with its own manager, copy and append."""
    say("[beams] copy-on-write scenario")
    rng = np.random.default_rng(11)
    Hq, Hkv, D, bs, nb = 8, 2, 128, 16, 96
    prompts = [40, 16, 33, 7]
    beams = 3
    steps = 20
    scale = 1.0 / np.sqrt(D)

    def tok():
        return bf16_round(rng.standard_normal((Hkv, D)).astype(np.float32))

    ours, ref = pa.BlockManager(nb, bs), oracle.BlockManager(nb, bs)
    cache = pa.KVCache.allocate(nb, Hkv, bs, D, "bf16", DEV)
    cache.k_cache.view(torch.int16).fill_(0x7FC0)
    cache.v_cache.view(torch.int16).fill_(0x7FC0)
    oc = oracle.PagedCache.empty("bf16", nb, Hkv, bs, D)

    t_ours, t_ref, lens = [], [], []
    for L in prompts:
        a, b = [], []
        K = np.stack([tok() for _ in range(L)])
        V = np.stack([tok() for _ in range(L)])
        slots = []
        for pos in range(L):
            s1, c1 = ours.append_slot(a, pos)
            s2, c2 = ref.append_slot(b, pos)
            assert (s1, c1) == (s2, c2) and not c1
            slots.append(s1)
        sl = np.array(slots, np.int32)
        pa.reshape_and_cache(to_dev_values(K, "bf16"), to_dev_values(V, "bf16"), torch.from_numpy(sl).to(DEV), cache)
        oracle.append(oc, K, V, sl)
        for _ in range(beams):  # the prompt's table is shared by its beams, then released
            t_ours.append(ours.fork(a))
            t_ref.append(ref.fork(b))
            lens.append(L)
        ours.free(a)
        ref.free(b)

    B = len(t_ours)
    for step in range(steps):
        Kn = np.stack([tok() for _ in range(B)])
        Vn = np.stack([tok() for _ in range(B)])
        slots, pairs = [], []
        for i in range(B):
            s1, c1 = ours.append_slot(t_ours[i], lens[i])
            s2, c2 = ref.append_slot(t_ref[i], lens[i])
            assert (s1, c1) == (s2, c2), (step, i)
            slots.append(s1)
            pairs += c1
            lens[i] += 1
        if pairs:
            pa.copy_blocks(cache, torch.tensor(pairs, dtype=torch.int32, device=DEV))
            oracle.copy_blocks(oc, pairs)
        sl = np.array(slots, np.int32)
        pa.reshape_and_cache(to_dev_values(Kn, "bf16"), to_dev_values(Vn, "bf16"), torch.from_numpy(sl).to(DEV), cache)
        oracle.append(oc, Kn, Vn, sl)

        width = max(len(t) for t in t_ours)
        tables = np.full((B, width), -1, np.int32)
        for i, t in enumerate(t_ours):
            tables[i, : len(t)] = t
        q = bf16_round(rng.standard_normal((B, Hq, D)).astype(np.float32))
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
        pa.decode(to_dev_values(q, "bf16"), cache, torch.from_numpy(tables).to(DEV),
                  torch.tensor(lens, dtype=torch.int32, device=DEV), scale, out)
        torch.cuda.synchronize()
        want = oracle.decode(q, oc, tables, np.array(lens, np.int32), scale)
        assert max_err(out, want) <= TOL["bf16"], step
    k, v, _, _ = download_cache(cache)
    okp, ovp = oracle_pools(oc)
    used = sorted({b for t in t_ours for b in t})
    assert np.array_equal(k[used], okp[used]) and np.array_equal(v[used], ovp[used])
    assert ours.num_free() == ref.num_free()
