"""Every shape the kernels take, against the oracle.

The five workloads fix a few shapes; this sweep covers the rest of what the
decode entry points accept: each (q, KV) storage pair, query groups of 1 to
16 heads per KV head (dev.to, "Why LLMs Run Out of VRAM...", §2 "Example 2":
grouped-query attention), head_dim 64 and 128, both kernels and every
partition mode, over lengths that end anywhere in a tile (0, 1, 15, 16, 17,
...).  Each case builds its pool with the library, fills the caches with the
append kernel on the GPU and the oracle's append on the CPU, checks the
cache bytes, and compares the decode with the oracle's.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_255_amd as pa
import workloads
from tests.scenario import check_close, poisoned_device_cache, poisoned_host_cache, to_f64

pytestmark = pytest.mark.gpu

LENS = [0, 1, 15, 16, 17, 33, 250, 701]
PAIRS = [("bf16", "bf16"), ("f16", "f16"), ("bf16", "e4m3"), ("f16", "e4m3"), ("f32", "f32")]


def say(*a):
    print(*a, flush=True)


class _W:
    def __init__(self, nb, hkv, d, kv):
        self.num_blocks, self.num_kv_heads, self.head_dim, self.kv_dtype = nb, hkv, d, kv
        self.block_size = 16


def _supported(kernel, q, kv, G, D):
    if kernel == pa.KERNEL_MFMA:
        return q in ("bf16", "f16") and G <= 16
    return G in (1, 2, 4) or (G == 8 and D == 64)


def _cases():
    out = []
    for q, kv in PAIRS:
        for G in (1, 2, 4, 8, 16):
            for D in (64, 128):
                for kernel, part in ((pa.KERNEL_MFMA, pa.PARTITION_BALANCED),
                                     (pa.KERNEL_MFMA, 0), (pa.KERNEL_MFMA, 48),
                                     (pa.KERNEL_VALU, 0), (pa.KERNEL_VALU, 64)):
                    if _supported(kernel, q, kv, G, D):
                        out.append((q, kv, G, D, kernel, part))
    return out


@pytest.mark.parametrize("q,kv,G,D,kernel,part", _cases())
def test_shape_matches_oracle(q, kv, G, D, kernel, part):
    say(f"[case] q={q} kv={kv} G={G} D={D} kernel={kernel} partition={part}")
    Hkv = 1 if G == 16 else 2
    Hq = G * Hkv
    B = len(LENS)
    NB = sum(-(-n // 16) for n in LENS) + 7
    seed = zlib.crc32(f"{q}/{kv}/{G}/{D}".encode()) & 0xFFFF
    pool = pa.pa_block_pool_init(NB, Hkv, D, kv, shuffle_seed=seed + 1)
    seqs = [pa.pa_seq_create(pool) for _ in LENS]
    slots = np.concatenate([pa.pa_seq_append_slots(pool, s, n) for s, n in zip(seqs, LENS)])
    maxb = max(-(-n // 16) for n in LENS)
    tables, lens = pa.pa_export_block_tables(pool, seqs, maxb)
    T = int(sum(LENS))
    k = workloads.normal((T, Hkv, D), seed + 2, q, "cuda")
    v = workloads.normal((T, Hkv, D), seed + 3, q, "cuda")
    k_scale = v_scale = 1.0
    if kv == "e4m3":
        k_scale, v_scale = workloads.fp8_scale(k), workloads.fp8_scale(v)
    desc = pa.kv_desc(Hq, Hkv, D, NB, q, kv, kernel=kernel)
    shape = _W(NB, Hkv, D, kv)
    kc, vc = poisoned_device_cache(shape), poisoned_device_cache(shape)
    hk, hv = poisoned_host_cache(shape), poisoned_host_cache(shape)
    pa.pa_cache_append(k, v, kc, vc, torch.from_numpy(slots.astype(np.int32)).cuda(), desc,
                       k_scale, v_scale)
    oracle.cache_append(workloads.storage(k), workloads.storage(v), hk, hv, slots,
                        num_kv_heads=Hkv, head_dim=D, block_size=16, num_blocks=NB, kv_dtype=kv,
                        in_dtype=q, k_scale=k_scale, v_scale=v_scale)
    qt = workloads.normal((B, Hq, D), seed + 4, q, "cuda")
    out = torch.full_like(qt, 7.0)
    max_len = maxb * 16
    ws = None
    if part:
        ws = torch.empty(pa.pa_decode_workspace_bytes(desc, B, max_len, part), dtype=torch.uint8,
                         device="cuda")
    scale = float(np.float32(D ** -0.5))
    pa.pa_decode(qt, kc, vc, torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(),
                 max_len, scale, out, desc, k_scale, v_scale, workspace=ws, partition_size=part)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(kc.view(torch.uint8).cpu().numpy(), hk.view(np.uint8))
    np.testing.assert_array_equal(vc.view(torch.uint8).cpu().numpy(), hv.view(np.uint8))
    ref = oracle.decode(workloads.storage(qt), hk, hv, tables, lens, num_q_heads=Hq,
                        num_kv_heads=Hkv, head_dim=D, block_size=16, num_blocks=NB, q_dtype=q,
                        kv_dtype=kv, scale=scale, k_scale=k_scale, v_scale=v_scale)
    got = to_f64(out)
    assert np.all(got[0] == 0.0)  # the zero-length sequence
    err = check_close(got, ref, kv, q)
    say(f"[ok] err={err:.3g}")
