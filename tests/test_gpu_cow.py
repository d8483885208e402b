"""Copy on write on the GPU: the block-copy kernel, and forked sequences that
append into a shared partly filled block, checked against the oracle.

dev.to, "Why LLMs Run Out of VRAM: KV Cache Fragmentation and How
PagedAttention Fixes It", §5 "Zero-Copy Forking", "Parallel Sampling & Tree
Search": branches map the prompt's blocks (reference counts); a branch's
first new token goes to a private block.  The library pool queues the copy
(shared -> private) and pa_copy_blocks makes it; the oracle side runs the
allocator model and copies the blocks of its host caches with numpy.
"""
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


@pytest.mark.parametrize("kv,bs", [("bf16", 16), ("e4m3", 16), ("bf16", 256)])
def test_copy_blocks_kernel(kv, bs):
    say(f"[case] copy_blocks kv={kv} block_size={bs}")
    NB, Hkv, D = 40, 4, 128
    desc = pa.kv_desc(8, Hkv, D, NB, "bf16", kv, block_size=bs)
    eb = 1 if kv == "e4m3" else 2
    nbytes = NB * Hkv * bs * D * eb
    g = torch.Generator().manual_seed(11)
    k = torch.randint(0, 256, (nbytes,), generator=g, dtype=torch.uint8)
    v = torch.randint(0, 256, (nbytes,), generator=g, dtype=torch.uint8)
    kd, vd = k.cuda(), v.cuda()
    # sources and destinations disjoint; one source copied twice; one bad pair
    pairs = np.array([[3, 10], [3, 11], [17, 2], [39, 0], [5, 40]], dtype=np.int32)
    pa.pa_copy_blocks(kd, vd, torch.from_numpy(pairs).cuda(), desc)
    torch.cuda.synchronize()
    blk = Hkv * bs * D * eb
    wk, wv = k.numpy().reshape(NB, blk).copy(), v.numpy().reshape(NB, blk).copy()
    for s, d in pairs:
        if 0 <= s < NB and 0 <= d < NB:
            wk[d], wv[d] = wk[s], wv[s]
    np.testing.assert_array_equal(kd.cpu().numpy().reshape(NB, blk), wk)
    np.testing.assert_array_equal(vd.cpu().numpy().reshape(NB, blk), wv)


@pytest.mark.parametrize("kv,kernel,part,bs", [("bf16", pa.KERNEL_MFMA, pa.PARTITION_BALANCED, 16),
                                               ("bf16", pa.KERNEL_VALU, 0, 16),
                                               ("e4m3", pa.KERNEL_MFMA, 0, 16),
                                               ("bf16", pa.KERNEL_MFMA, pa.PARTITION_BALANCED, 64),
                                               ("e4m3", pa.KERNEL_VALU, 64, 64)])
def test_branches_append_into_a_shared_partial_block(kv, kernel, part, bs):
    """A 20-token prompt (second block partly filled) forked into three
    branches; each step appends one token to every sequence.  The pool's
    tables, slots and copies match the model's; after the copies and appends
    the caches match the oracle's byte for byte and the decode matches the
    oracle's output."""
    say(f"[case] copy-on-write branches kv={kv} kernel={kernel} partition={part} bs={bs}")
    Hq, Hkv, D, NB = 8, 2, 128, 24
    qd = "bf16"
    pool = pa.pa_block_pool_init(NB, Hkv, D, kv, block_size=bs, shuffle_seed=4242)
    model = am.PoolModel(NB, bs, 4242)
    desc = pa.kv_desc(Hq, Hkv, D, NB, qd, kv, block_size=bs, kernel=kernel)

    def tensor(shape, seed):
        return workloads.normal(shape, seed, qd, "cuda")

    shape = _W(NB, Hkv, D, kv, bs)
    kc, vc = poisoned_device_cache(shape), poisoned_device_cache(shape)
    hk, hv = poisoned_host_cache(shape), poisoned_host_cache(shape)
    k_scale = v_scale = (1.0 / 64 if kv == "e4m3" else 1.0)
    common = dict(num_kv_heads=Hkv, head_dim=D, block_size=bs, num_blocks=NB, kv_dtype=kv,
                  in_dtype=qd, k_scale=k_scale, v_scale=v_scale)

    def write(slots, k, v):
        d_slots = torch.from_numpy(np.asarray(slots, dtype=np.int32)).cuda()
        pa.pa_cache_append(k, v, kc, vc, d_slots, desc, k_scale, v_scale)
        oracle.cache_append(workloads.storage(k), workloads.storage(v), hk, hv,
                            np.asarray(slots, dtype=np.int32), **common)

    def copies():
        got = pa.pa_pool_take_copies(pool)
        want = np.array(model.take_copies(), dtype=np.int32).reshape(-1, 2)
        np.testing.assert_array_equal(got, want)
        if len(got):
            pa.pa_copy_blocks(kc, vc, torch.from_numpy(got).cuda(), desc)
            blk_k = hk.view(np.uint8).reshape(NB, -1)
            blk_v = hv.view(np.uint8).reshape(NB, -1)
            for s, d in got:
                blk_k[d], blk_v[d] = blk_k[s].copy(), blk_v[s].copy()
        return len(got)

    root, mroot = pa.pa_seq_create(pool), model.seq_create()
    slots = pa.pa_seq_append_slots(pool, root, 20)
    assert list(slots) == model.append_slots(mroot, 20)[1]
    write(slots, tensor((20, Hkv, D), 901), tensor((20, Hkv, D), 902))
    seqs, mseqs = [root], [mroot]
    for _ in range(3):
        seqs.append(pa.pa_seq_fork(pool, root))
        mseqs.append(model.fork(mroot)[1])
    n_copies = 0
    for step in range(5):
        slots = pa.pa_seq_append_slots_batch(pool, seqs, 1)
        st, mslots = model.append_slots_batch(mseqs, 1)
        assert st == am.OK and list(slots) == mslots
        n_copies += copies()
        B = len(seqs)
        write(slots, tensor((B, Hkv, D), 1000 + step), tensor((B, Hkv, D), 2000 + step))
    assert n_copies == 3  # three of the four sharers get a private copy; the last writes in place
    maxb = 4
    tables, lens = pa.pa_export_block_tables(pool, seqs, maxb)
    st, mt, ml = model.export(mseqs, maxb)
    np.testing.assert_array_equal(tables, np.array(mt, dtype=np.int32))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(kc.view(torch.uint8).cpu().numpy(), hk.view(np.uint8))
    np.testing.assert_array_equal(vc.view(torch.uint8).cpu().numpy(), hv.view(np.uint8))

    B = len(seqs)
    q = tensor((B, Hq, D), 3000)
    out = torch.full_like(q, 7.0)
    ws = None
    if part:
        ws = torch.empty(pa.pa_decode_workspace_bytes(desc, B, 64, part), dtype=torch.uint8,
                         device="cuda")
    scale = float(np.float32(D ** -0.5))
    pa.pa_decode(q, kc, vc, torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(), 64,
                 scale, out, desc, k_scale, v_scale, workspace=ws, partition_size=part)
    torch.cuda.synchronize()
    ref = oracle.decode(workloads.storage(q), hk, hv, tables, lens, num_q_heads=Hq,
                        num_kv_heads=Hkv, head_dim=D, block_size=bs, num_blocks=NB,
                        q_dtype=qd, kv_dtype=kv, scale=scale, k_scale=k_scale, v_scale=v_scale)
    check_close(to_f64(out), ref, kv, qd)


class _W:
    """The cache shape fields poisoned_*_cache read."""

    def __init__(self, nb, hkv, d, kv, bs=16):
        self.num_blocks, self.num_kv_heads, self.head_dim, self.kv_dtype = nb, hkv, d, kv
        self.block_size = bs
