"""Brute-force contiguous attention in numpy, used to pin the oracle.

Written separately from the oracle: stored values are decoded with library
routines (numpy float16, torch bfloat16 / float8_e4m3fn views), each
sequence's K and V are gathered into contiguous [n][D] arrays with
np.concatenate over its block table, and softmax(q K^T * scale) V is then
evaluated with whole-array numpy operations (dev.to, "Why LLMs Run Out of
VRAM...", §1 attention formula; §4 block table).
"""
import numpy as np
import torch

ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1}


def decode_storage(a, dtype):
    """Stored values -> float64, via library conversions."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(a, dtype=np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        t = torch.from_numpy(np.asarray(a, dtype=np.uint16).view(np.int16).copy())
        return t.view(torch.bfloat16).to(torch.float64).numpy()
    if dtype == "e4m3":
        t = torch.from_numpy(np.asarray(a, dtype=np.uint8).copy())
        return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    raise ValueError(dtype)


def gather(cache_vals, table, n, bs):
    """Contiguous [n][Hkv][D] rows of one sequence from a paged cache given as
    float64 [blocks][Hkv][bs][D]."""
    nblk = -(-n // bs)
    parts = [cache_vals[table[j]].transpose(1, 0, 2) for j in range(nblk)]
    return np.concatenate(parts, axis=0)[:n]


def v_token_major(v_vals, num_kv_heads, head_dim, bs, elem_bytes):
    """The V cache as [blocks][Hkv][bs][D].  It is stored per block and KV
    head as bs/16 tiles of 16 tokens, each tile a run of 16-byte pieces: with
    p = 4 / elem_bytes, piece (q, a, c) (q < D/16p, a < 4, c < 16) holds the
    p x 4 values (i, r) of dim 16 (p q + i) + c and token 4 a + r.  Works on
    any array (storage codes or decoded values)."""
    p = 4 // elem_bytes
    t = np.asarray(v_vals).reshape(-1, num_kv_heads, bs // 16, head_dim // (16 * p), 4, 16, p, 4)
    # axes: block, head, tile, q, a, c, i, r -> block, head, (tile, a, r), (q, i, c)
    t = t.transpose(0, 1, 2, 4, 7, 3, 6, 5)
    return t.reshape(-1, num_kv_heads, bs, head_dim)


def v_from_token_major(v_tok, elem_bytes):
    """Inverse of v_token_major: [blocks][Hkv][bs][D] -> V storage order
    [blocks][Hkv][bs/16][16 D]."""
    NB, H, bs, D = v_tok.shape
    p = 4 // elem_bytes
    t = np.asarray(v_tok).reshape(NB, H, bs // 16, 4, 4, D // (16 * p), p, 16)
    # axes: block, head, tile, a, r, q, i, c -> block, head, tile, q, a, c, i, r
    return np.ascontiguousarray(t.transpose(0, 1, 2, 5, 3, 7, 6, 4)).reshape(NB, H, bs // 16, 16 * D)


def attention(q, k_cache, v_cache, tables, lens, *, num_q_heads, num_kv_heads, head_dim,
              block_size, q_dtype, kv_dtype, scale, k_scale=1.0, v_scale=1.0, seq_starts=None):
    """seq_starts: optional window starts; the rows before them are cut off
    the gathered K and V before the softmax."""
    B = len(lens)
    G = num_q_heads // num_kv_heads
    qv = decode_storage(q, q_dtype).reshape(B, num_q_heads, head_dim)
    kv = decode_storage(k_cache, kv_dtype).reshape(-1, num_kv_heads, block_size, head_dim)
    vv = v_token_major(decode_storage(v_cache, kv_dtype), num_kv_heads, head_dim, block_size,
                       ELEM_BYTES[kv_dtype])
    out = np.zeros((B, num_q_heads, head_dim))
    for b in range(B):
        n = int(lens[b])
        w = 0 if seq_starts is None else int(seq_starts[b])
        if n == w:
            continue
        K = gather(kv, tables[b], n, block_size)[w:] * k_scale  # [n - w][Hkv][D]
        V = gather(vv, tables[b], n, block_size)[w:] * v_scale
        for h in range(num_q_heads):
            g = h // G
            s = K[:, g, :] @ qv[b, h] * scale
            w = np.exp(s - s.max())
            out[b, h] = (w[:, None] * V[:, g, :]).sum(0) / w.sum()
    return out
