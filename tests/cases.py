"""Random small paged-attention problems for the oracle's CPU pins.

Builds storage arrays, block tables (random injective placement of each
sequence's blocks in the pool) and lengths from a numpy seed.  It contains
no attention arithmetic.  Cache shapes: K [blocks][Hkv][bs][D]; V
[blocks][Hkv][bs/16][16 D] (16-token tiles; the order inside a tile is
undone by bruteforce.v_token_major).
"""
import numpy as np
import torch

BS = 16


def random_storage(rng, shape, dtype, scale=1.0):
    x = rng.standard_normal(shape).astype(np.float32) * scale
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype == "e4m3":
        # arbitrary finite codes (0x7F / 0xFF are NaN)
        codes = rng.integers(0, 256, size=shape, dtype=np.int64)
        codes = np.where((codes & 0x7F) == 0x7F, codes - 1, codes)
        return codes.astype(np.uint8)
    raise ValueError(dtype)


def v_shape(NB, Hkv, D, bs):
    return (NB, Hkv, bs // 16, 16 * D)


def random_case(seed, *, B=3, Hq=4, Hkv=2, D=32, q_dtype="f32", kv_dtype="f32",
                lens=None, extra_blocks=5, max_len=90, bs=BS):
    rng = np.random.default_rng(seed)
    if lens is None:
        lens = rng.integers(1, max_len, size=B)
    lens = np.asarray(lens, dtype=np.int32)
    nblk = [-(-int(n) // bs) for n in lens]
    NB = sum(nblk) + extra_blocks
    perm = rng.permutation(NB)
    maxb = max(max(nblk), 1)
    tables = np.full((len(lens), maxb), -1, dtype=np.int32)
    pos = 0
    for b, k in enumerate(nblk):
        tables[b, :k] = perm[pos:pos + k]
        pos += k
    q = random_storage(rng, (len(lens), Hq, D), q_dtype)
    k = random_storage(rng, (NB, Hkv, bs, D), kv_dtype)
    v = random_storage(rng, v_shape(NB, Hkv, D, bs), kv_dtype)
    return dict(q=q, k=k, v=v, tables=tables, lens=lens, NB=NB, Hq=Hq, Hkv=Hkv, D=D, bs=bs,
                q_dtype=q_dtype, kv_dtype=kv_dtype, scale=float(np.float32(1 / np.sqrt(D))))
