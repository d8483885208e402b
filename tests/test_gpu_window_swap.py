"""Sliding windows and block swapping on the GPU, against the oracle.

vaibhawkumar.in, "Why LLMs run out of VRAM: KV cache fragmentation and the
PagedAttention fix", "PagedAttention: the idea": sliding the window hands the
oldest whole pages back; a cut inside the first kept page only moves its
start.  hyperinfer.ai, "KV cache & paged attention deep dive", "What 16-token
blocks buy you": swapping to CPU memory goes block by block.

The decode kernels take window starts and leave the tokens before them out;
the pool releases the blocks a window leaves behind; pa_swap_blocks moves
whole blocks between the device caches and pinned host memory.  The oracle
side runs the allocator model and mirrors every transfer on host arrays.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_255_amd as pa
import workloads
from oracle import alloc_model as am
from tests.scenario import (GpuStep, Inputs, OracleStep, check_close, poisoned_device_cache,
                            poisoned_host_cache, to_f64)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def _starts(lens, bs, seed):
    """Window starts covering the edge cases: none, empty, one token, inside
    the first block, past whole blocks, anywhere."""
    rng = np.random.default_rng(seed)
    out = []
    for i, n in enumerate(lens):
        n = int(n)
        pick = [0, n, max(n - 1, 0), min(3, n), min(bs + 5, n), n // 2,
                int(rng.integers(0, n + 1))][i % 7]
        out.append(pick)
    return np.array(out, dtype=np.int32)


def _window_cases():
    out = []
    for bs in (16, 64):
        for cid in (2, 3, 5):
            for kernel, part in ((pa.KERNEL_MFMA, pa.PARTITION_BALANCED), (pa.KERNEL_MFMA, 0),
                                 (pa.KERNEL_MFMA, 64), (pa.KERNEL_VALU, 0)):
                out.append((bs, cid, kernel, part))
    return out


@pytest.mark.parametrize("bs,cid,kernel,part", _window_cases())
def test_windowed_decode_matches_oracle(bs, cid, kernel, part):
    w = workloads.config(cid, "small", block_size=bs)
    G = w.num_q_heads // w.num_kv_heads
    if kernel == pa.KERNEL_VALU and not (G in (1, 2, 4) or (G == 8 and w.head_dim == 64)):
        pytest.skip("shape not built for this kernel")
    say(f"[case] window block_size={bs} cfg{cid} kernel={kernel} partition={part}")
    inp = Inputs(w)
    g = GpuStep(w, 0, inp, partition=part, kernel=kernel)
    o = OracleStep(w, 0, inp)
    g.append_prefill()
    g.append_step()
    starts = _starts(g.lens, bs, cid * 10 + bs)
    out = to_f64(g.decode(seq_starts=starts))
    torch.cuda.synchronize()
    ref = o.decode(seq_starts=starts)
    err = check_close(out, ref, w.kv_dtype, w.q_dtype)
    for b, (s, n) in enumerate(zip(starts, g.lens)):
        if s == n:
            assert np.all(out[b] == 0.0)  # an empty window gives a zero row
    say(f"[ok] err={err:.3g}")


def test_windowed_decode_append_equals_append_then_decode():
    """The appending decode with windows: same bits and cache bytes as the
    separate append followed by the windowed decode."""
    w = workloads.config(2, "small")
    inp = Inputs(w)
    a = GpuStep(w, 0, inp, partition=pa.PARTITION_BALANCED, kernel=pa.KERNEL_MFMA)
    b = GpuStep(w, 0, inp, partition=pa.PARTITION_BALANCED, kernel=pa.KERNEL_MFMA)
    a.append_prefill()
    b.append_prefill()
    starts = _starts(a.lens, 16, 5)
    say(f"[case] windowed decode_append starts={starts.tolist()}")
    a.append_step()
    ref = a.decode(seq_starts=starts).clone()
    got = b.decode_append(seq_starts=starts).clone()
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    assert torch.equal(a.k_cache.view(torch.uint8), b.k_cache.view(torch.uint8))
    assert torch.equal(a.v_cache.view(torch.uint8), b.v_cache.view(torch.uint8))


def test_bad_window_start_gives_nan_rows():
    w = workloads.config(2, "small")
    inp = Inputs(w)
    g = GpuStep(w, 0, inp, partition=pa.PARTITION_BALANCED, kernel=pa.KERNEL_MFMA)
    g.append_prefill()
    g.append_step()
    starts = np.zeros(w.num_seqs, dtype=np.int32)
    starts[1] = int(g.lens[1]) + 1
    starts[3] = -1
    out = to_f64(g.decode(seq_starts=starts))
    torch.cuda.synchronize()
    assert np.all(np.isnan(out[1])) and np.all(np.isnan(out[3]))
    assert np.all(np.isfinite(out[[0, 2, 4]]))


class _W:
    def __init__(self, nb, hkv, d, kv, bs):
        self.num_blocks, self.num_kv_heads, self.head_dim, self.kv_dtype = nb, hkv, d, kv
        self.block_size = bs


@pytest.mark.parametrize("kv,bs,kernel,part", [("bf16", 16, pa.KERNEL_MFMA, pa.PARTITION_BALANCED),
                                               ("e4m3", 16, pa.KERNEL_MFMA, 0),
                                               ("bf16", 64, pa.KERNEL_VALU, 0),
                                               ("bf16", 32, pa.KERNEL_MFMA, 64)])
def test_slides_and_swaps_through_a_serving_run(kv, bs, kernel, part):
    """Eight sequences decode for 40 steps.  Each step: the copy-on-write
    copies, window slides (the released blocks go back to the pool and are
    reused), swaps out to pinned host memory and back in, one appended token
    per resident sequence, then the windowed decode of every resident
    sequence.  The library's tables, lengths, starts and swap pairs equal the
    model's; cache and swap-space bytes equal the oracle side's; the decode
    matches the oracle."""
    say(f"[case] serving run kv={kv} bs={bs} kernel={kernel} partition={part}")
    rng = np.random.default_rng(1234 + bs)
    Hq, Hkv, D, qd = 8, 2, 128, "bf16"
    per_seq = -(-(4 * bs + 41) // bs)  # blocks of the longest sequence
    NB = NH = 9 * per_seq + 20
    pool = pa.pa_block_pool_init(NB, Hkv, D, kv, block_size=bs, shuffle_seed=7,
                                 num_host_blocks=NH)
    model = am.PoolModel(NB, bs, 7, num_host_blocks=NH)
    desc = pa.kv_desc(Hq, Hkv, D, NB, qd, kv, block_size=bs, kernel=kernel)
    shape = _W(NB, Hkv, D, kv, bs)
    kc, vc = poisoned_device_cache(shape), poisoned_device_cache(shape)
    hk, hv = poisoned_host_cache(shape), poisoned_host_cache(shape)
    host = _W(NH, Hkv, D, kv, bs)
    # swap space: pinned host memory on the GPU side, numpy on the oracle side
    sk = torch.full((pa.pa_block_bytes(pool) * NH,), 0xFF, dtype=torch.uint8, pin_memory=True)
    sv = torch.full((pa.pa_block_bytes(pool) * NH,), 0xFF, dtype=torch.uint8, pin_memory=True)
    mk, mv = poisoned_host_cache(host), poisoned_host_cache(host)
    blk_bytes = pa.pa_block_bytes(pool)
    k_scale = v_scale = (1.0 / 64 if kv == "e4m3" else 1.0)
    common = dict(num_kv_heads=Hkv, head_dim=D, block_size=bs, num_blocks=NB, kv_dtype=kv,
                  in_dtype=qd, k_scale=k_scale, v_scale=v_scale)

    def rows(n, seed):
        return (workloads.normal((n, Hkv, D), seed, qd, "cuda"),
                workloads.normal((n, Hkv, D), seed + 1, qd, "cuda"))

    def write(slots, k, v):
        pa.pa_cache_append(k, v, kc, vc, torch.from_numpy(np.asarray(slots, np.int32)).cuda(),
                           desc, k_scale, v_scale)
        oracle.cache_append(workloads.storage(k), workloads.storage(v), hk, hv,
                            np.asarray(slots, dtype=np.int32), **common)

    def blocks(a):
        return a.view(np.uint8).reshape(-1, blk_bytes)

    def copies():
        got = pa.pa_pool_take_copies(pool)
        np.testing.assert_array_equal(got, np.array(model.take_copies(), np.int32).reshape(-1, 2))
        if len(got):
            pa.pa_copy_blocks(kc, vc, torch.from_numpy(got).cuda(), desc)
            for s, d in got:
                blocks(hk)[d], blocks(hv)[d] = blocks(hk)[s].copy(), blocks(hv)[s].copy()

    seqs = []  # (lib id, model id)
    for i in range(8):
        s, m = pa.pa_seq_create(pool), model.seq_create()
        n = int(rng.integers(1, 4 * bs))
        slots = pa.pa_seq_append_slots(pool, s, n)
        assert list(slots) == model.append_slots(m, n)[1]
        write(slots, *rows(n, 100 + 2 * i))
        seqs.append((s, m))
    fork = (pa.pa_seq_fork(pool, seqs[0][0]), model.fork(seqs[0][1])[1])
    seqs.append(fork)

    n_out = n_in = n_rel = 0
    for step in range(40):
        copies()
        for s, m in seqs:
            if m in model.swapped:
                continue
            if rng.random() < 0.3:
                win = int(rng.integers(0, 3 * bs))
                rel = pa.pa_seq_slide_window(pool, s, win)
                assert (am.OK, rel) == model.slide_window(m, win)
                n_rel += rel
        for s, m in seqs:
            r = rng.random()
            if m not in model.swapped and r < 0.1:
                st, mp = model.swap_out(m)
                if st != am.OK:
                    continue
                got = pa.pa_seq_swap_out(pool, s)
                np.testing.assert_array_equal(got, np.array(mp, np.int32).reshape(-1, 2))
                if len(got):
                    pa.pa_swap_blocks(kc, vc, sk, sv, torch.from_numpy(got).cuda(), desc,
                                      to_host=True)
                    for d, h in got:
                        blocks(mk)[h], blocks(mv)[h] = blocks(hk)[d].copy(), blocks(hv)[d].copy()
                n_out += 1
            elif m in model.swapped and r < 0.4:
                st, mp = model.swap_in(m)
                if st != am.OK:
                    continue
                got = pa.pa_seq_swap_in(pool, s)
                np.testing.assert_array_equal(got, np.array(mp, np.int32).reshape(-1, 2))
                if len(got):
                    pa.pa_swap_blocks(kc, vc, sk, sv, torch.from_numpy(got).cuda(), desc,
                                      to_host=False)
                    for h, d in got:
                        blocks(hk)[d], blocks(hv)[d] = blocks(mk)[h].copy(), blocks(mv)[h].copy()
                n_in += 1
        res = [(s, m) for s, m in seqs if m not in model.swapped]
        if not res:
            continue
        st, mslots = model.append_slots_batch([m for _, m in res], 1)
        assert st == am.OK
        slots = pa.pa_seq_append_slots_batch(pool, [s for s, _ in res], 1)
        assert list(slots) == mslots
        copies()  # a fork's first token may need a private copy
        write(slots, *rows(len(res), 1000 + 2 * step))
        maxb = per_seq + 1
        tables, lens, starts = pa.pa_export_block_tables(pool, [s for s, _ in res], maxb,
                                                         with_starts=True)
        st, mt, ml, mw = model.export([m for _, m in res], maxb, with_starts=True)
        np.testing.assert_array_equal(tables, np.array(mt, np.int32))
        np.testing.assert_array_equal(lens, ml)
        np.testing.assert_array_equal(starts, mw)
        B = len(res)
        q = workloads.normal((B, Hq, D), 5000 + step, qd, "cuda")
        out = torch.full_like(q, 7.0)
        ws = None
        if part:
            ws = torch.empty(pa.pa_decode_workspace_bytes(desc, B, maxb * bs, part),
                             dtype=torch.uint8, device="cuda")
        pa.pa_decode(q, kc, vc, torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(),
                     maxb * bs, 0.088, out, desc, k_scale, v_scale, workspace=ws,
                     partition_size=part, seq_starts=torch.from_numpy(starts).cuda())
        torch.cuda.synchronize()
        ref = oracle.decode(workloads.storage(q), hk, hv, tables, lens, num_q_heads=Hq,
                            num_kv_heads=Hkv, head_dim=D, block_size=bs, num_blocks=NB,
                            q_dtype=qd, kv_dtype=kv, scale=float(np.float32(0.088)),
                            k_scale=k_scale, v_scale=v_scale, seq_starts=starts)
        check_close(to_f64(out), ref, kv, qd)
        # every block a resident table maps, and the whole swap space, byte for byte
        mapped = sorted({int(b) for row in tables for b in row if b >= 0})
        for cache, mirror in ((kc, hk), (vc, hv)):
            got = cache.view(torch.uint8).cpu().numpy().reshape(-1, blk_bytes)
            np.testing.assert_array_equal(got[mapped], blocks(mirror)[mapped])
        swapped_host = sorted({h for _, m in seqs if m in model.swapped
                               for h in model.tables[m]})
        np.testing.assert_array_equal(sk.numpy().reshape(-1, blk_bytes)[swapped_host],
                                      blocks(mk)[swapped_host])
        np.testing.assert_array_equal(sv.numpy().reshape(-1, blk_bytes)[swapped_host],
                                      blocks(mv)[swapped_host])
    say(f"[ok] swaps out {n_out}, in {n_in}, blocks released by windows {n_rel}")
    assert n_out >= 5 and n_in >= 3 and n_rel >= 5
