"""Automatic prefix caching on the GPU: requests that share a system prompt
map its cached blocks instead of writing them again, and decode the same as a
request that wrote everything itself.

dev.to, "Why LLMs Run Out of VRAM: KV Cache Fragmentation and How
PagedAttention Fixes It", §5 "Zero-Copy Forking" (a shared system prompt is
stored once and mapped by every request that starts with it), and vLLM's
"Automatic Prefix Caching" design page (a full block is found again by its
parent block and its own tokens).  A token's K and V depend on every token
before it, so the test draws them from a generator seeded by the whole prefix
up to that token: two requests that agree on a prefix agree on its cache
content, as they would in a model.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_255_amd as pa
import workloads
from oracle import alloc_model as am
from tests.scenario import check_close, poisoned_device_cache, poisoned_host_cache, to_f64

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


class _W:
    def __init__(self, nb, hkv, d, kv, bs):
        self.num_blocks, self.num_kv_heads, self.head_dim, self.kv_dtype = nb, hkv, d, kv
        self.block_size = bs


def _prefix_seed(tokens, i, which):
    return zlib.crc32(np.asarray(tokens[: i + 1], dtype=np.int32).tobytes() + which) & 0x7FFFFFFF


def _kv_rows(tokens, lo, hi, Hkv, D, qd):
    """K and V of tokens lo..hi-1 of a prompt, each seeded by its prefix."""
    k = [workloads.normal((Hkv, D), _prefix_seed(tokens, i, b"k"), qd) for i in range(lo, hi)]
    v = [workloads.normal((Hkv, D), _prefix_seed(tokens, i, b"v"), qd) for i in range(lo, hi)]
    return torch.stack(k).cuda(), torch.stack(v).cuda()


@pytest.mark.parametrize("kv,kernel,part,bs", [("bf16", pa.KERNEL_MFMA, pa.PARTITION_BALANCED, 16),
                                               ("bf16", pa.KERNEL_VALU, 0, 16),
                                               ("e4m3", pa.KERNEL_MFMA, pa.PARTITION_BALANCED, 16),
                                               ("bf16", pa.KERNEL_MFMA, pa.PARTITION_BALANCED, 32)])
def test_prefix_matched_requests_decode_like_fully_written_ones(kv, kernel, part, bs):
    say(f"[case] prefix cache kv={kv} kernel={kernel} partition={part} block_size={bs}")
    Hq, Hkv, D, NB = 8, 2, 128, 48  # group 4: both kernels
    qd = "bf16"
    rng = np.random.default_rng(77)
    system = [int(x) for x in rng.integers(0, 1000, size=40)]
    prompt_a = system + [int(x) for x in rng.integers(0, 1000, size=10)]  # 50 tokens
    prompt_b = system + [int(x) for x in rng.integers(0, 1000, size=13)]  # 53 tokens
    prompt_d = prompt_a[:48]                                               # only full cached blocks

    pool = pa.pa_block_pool_init(NB, Hkv, D, kv, block_size=bs, shuffle_seed=99)
    model = am.PoolModel(NB, bs, 99)
    desc = pa.kv_desc(Hq, Hkv, D, NB, qd, kv, block_size=bs, kernel=kernel)
    shape = _W(NB, Hkv, D, kv, bs)
    kc, vc = poisoned_device_cache(shape), poisoned_device_cache(shape)
    hk, hv = poisoned_host_cache(shape), poisoned_host_cache(shape)
    k_scale = v_scale = (1.0 / 64 if kv == "e4m3" else 1.0)
    common = dict(num_kv_heads=Hkv, head_dim=D, block_size=bs, num_blocks=NB, kv_dtype=kv,
                  in_dtype=qd, k_scale=k_scale, v_scale=v_scale)
    written = []

    def admit(tokens, use_cache=True):
        """A request: map what the cache holds, write the rest, register."""
        s, m = pa.pa_seq_create(pool), model.seq_create()
        hit = 0
        if use_cache:
            hit = pa.pa_prefix_match(pool, s, tokens)
            assert (am.OK, hit) == model.prefix_match(m, tokens)
        n = len(tokens) - hit
        slots = pa.pa_seq_append_slots(pool, s, n)
        assert list(slots) == model.append_slots(m, n)[1]
        if n:
            k, v = _kv_rows(tokens, hit, len(tokens), Hkv, D, qd)
            d_slots = torch.from_numpy(np.asarray(slots, dtype=np.int32)).cuda()
            pa.pa_cache_append(k, v, kc, vc, d_slots, desc, k_scale, v_scale)
            oracle.cache_append(workloads.storage(k), workloads.storage(v), hk, hv,
                                np.asarray(slots, dtype=np.int32), **common)
        written.append(n)
        if use_cache:
            assert pa.pa_prefix_register(pool, s, tokens) == model.prefix_register(m, tokens)[1]
        return s, m, hit

    a, ma, hit_a = admit(prompt_a)
    b, mb, hit_b = admit(prompt_b)
    c, mc, _ = admit(prompt_b, use_cache=False)
    d, md, hit_d = admit(prompt_d)
    # full blocks inside the 40 shared tokens; d's 48 tokens are all a's
    hb, hd = (40 // bs) * bs, (48 // bs) * bs
    assert (hit_a, hit_b, hit_d) == (0, hb, hd)
    assert written == [50, 53 - hb, 53, 48 - hd]
    n_cached = 50 // bs + 53 // bs - hb // bs  # a's full blocks, then b's beyond the match
    assert pa.pa_pool_get_stats(pool)["cached_blocks"] == model.stats()["cached_blocks"] == n_cached
    assert len(pa.pa_pool_take_copies(pool)) == 0

    # every request takes one more token (decode with the fused append)
    seqs, mseqs = [a, b, d], [ma, mb, md]
    slots = pa.pa_seq_append_slots_batch(pool, seqs, 1)
    assert list(slots) == model.append_slots_batch(mseqs, 1)[1]
    slots_c = pa.pa_seq_append_slots(pool, c, 1)
    assert list(slots_c) == model.append_slots(mc, 1)[1]
    assert len(pa.pa_pool_take_copies(pool)) == 0  # matched blocks are full: no copy
    maxb = -(-54 // bs)
    tables, lens = pa.pa_export_block_tables(pool, seqs, maxb)
    np.testing.assert_array_equal(tables, np.array(model.export(mseqs, maxb)[1], dtype=np.int32))
    tables_c, lens_c = pa.pa_export_block_tables(pool, [a, c, d], maxb)
    assert list(lens) == list(lens_c) == [51, 54, 49]
    np.testing.assert_array_equal(tables_c, np.array(model.export([ma, mc, md], maxb)[1],
                                                     dtype=np.int32))
    assert list(tables[1][:hb // bs]) == list(tables[0][:hb // bs])
    assert list(tables[2][:hd // bs]) == list(tables[0][:hd // bs])
    assert not (set(tables[1]) & set(tables_c[1])) - {-1}  # c shares nothing with b

    B = 3
    q = workloads.normal((B, Hq, D), 501, qd, "cuda")
    k_new = workloads.normal((B, Hkv, D), 502, qd, "cuda")
    v_new = workloads.normal((B, Hkv, D), 503, qd, "cuda")
    scale = float(np.float32(D ** -0.5))
    ws = None
    if part:
        ws = torch.empty(pa.pa_decode_workspace_bytes(desc, B, 64, part), dtype=torch.uint8,
                         device="cuda")
    outs = []
    for tb, ln, sl in ((tables, lens, slots), (tables_c, lens_c,
                                               np.array([slots[0], slots_c[0], slots[2]]))):
        out = torch.full_like(q, 7.0)
        pa.pa_decode_append(q, k_new, v_new, torch.from_numpy(np.asarray(sl, dtype=np.int32)).cuda(),
                            kc, vc, torch.from_numpy(tb).cuda(), torch.from_numpy(ln).cuda(), 64,
                            scale, out, desc, k_scale, v_scale, workspace=ws, partition_size=part)
        torch.cuda.synchronize()
        outs.append(out.clone())
    # same content and same lengths: the prefix-mapped request gives the same bits
    assert torch.equal(outs[0], outs[1])

    oracle.cache_append(workloads.storage(k_new), workloads.storage(v_new), hk, hv,
                        np.asarray(slots, dtype=np.int32), **common)
    oracle.cache_append(workloads.storage(k_new[1:2]), workloads.storage(v_new[1:2]), hk, hv,
                        np.asarray(slots_c, dtype=np.int32), **common)
    np.testing.assert_array_equal(kc.view(torch.uint8).cpu().numpy(), hk.view(np.uint8))
    np.testing.assert_array_equal(vc.view(torch.uint8).cpu().numpy(), hv.view(np.uint8))
    ref = oracle.decode(workloads.storage(q), hk, hv, tables, lens, num_q_heads=Hq,
                        num_kv_heads=Hkv, head_dim=D, block_size=bs, num_blocks=NB,
                        q_dtype=qd, kv_dtype=kv, scale=scale, k_scale=k_scale, v_scale=v_scale)
    check_close(to_f64(outs[0]), ref, kv, qd)

    # eviction leaves mapped blocks alone: every cached block is still in a table
    assert pa.pa_prefix_evict(pool, NB) == model.prefix_evict(NB) == 0
    for s, m in ((a, ma), (b, mb), (c, mc), (d, md)):
        pa.pa_seq_free(pool, s)
        model.free_seq(m)
    st = pa.pa_pool_get_stats(pool)
    assert st["cached_blocks"] == n_cached and st["free_blocks"] == NB - n_cached
    # once no table maps them they go, leaves first
    assert pa.pa_prefix_evict(pool, NB) == model.prefix_evict(NB) == n_cached
    st = pa.pa_pool_get_stats(pool)
    assert st["cached_blocks"] == 0 and st["free_blocks"] == NB == model.stats()["free_blocks"]
