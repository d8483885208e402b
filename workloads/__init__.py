"""Seeded synthetic inputs for the paged-KV decode path.

This module only draws inputs: sequence lengths, the order of pool
operations that build the block tables, random tensors and the per-tensor
FP8 scale.  It holds none of the method's arithmetic (no addressing, no
quantisation, no attention), so both the GPU library and the CPU oracle can
consume what it produces without sharing any of the computation.

Workload shapes follow the pages' worked examples:
  * dev.to, "Why LLMs Run Out of VRAM: KV Cache Fragmentation and How
    PagedAttention Fixes It", §2 "The Concrete Math of KV Cache Growth":
    Example 1 (Llama-2-13B: 40 layers, 40 KV heads, head_dim 128, fp16, 8
    users at 4,096 tokens) and Example 2 (Llama-3-8B GQA: 32 query heads
    sharing 8 KV heads, head_dim 128, batch 32); §3 (a 350-token output),
    §4 (16-token blocks), §5 (prompt blocks shared by reference count).
  * hyperinfer.ai, "KV cache & paged attention deep dive", "Why this matters
    for long context" (a 128K-token request on a 70B model) and "KV
    quantization cuts memory in half" (FP8 KV).
No public dataset is involved: the pages describe serving traffic (chat,
agents, long context) and these seeded N(0,1) inputs stand in for it.

A workload is a *plan*: a list of pool operations in order
  ("create",)            new sequence (ids count up from 0 in plan order)
  ("fork", parent)       new sequence sharing parent's blocks
  ("free", seq)          release a sequence
  ("prefill", seq, n)    reserve n token slots; their K/V come from the
                         prefill tensors, in plan order
followed by one decode step: one new token is appended to each sequence of
`decode_seqs` (in that order), and every one of them is decoded.
"""
from dataclasses import dataclass, field
import math

import numpy as np

BLOCK_SIZE = 16
TORCH_DTYPES = {"f32": "float32", "f16": "float16", "bf16": "bfloat16", "e4m3": "uint8"}


@dataclass
class Workload:
    name: str
    config_id: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    q_dtype: str          # dtype of q, out and the new tokens' K/V
    kv_dtype: str         # storage dtype of the cache
    num_blocks: int       # physical blocks per layer pool
    ops: list
    decode_seqs: list
    num_layers: int = 1
    block_size: int = BLOCK_SIZE
    seed: int = 0
    partition_size: int = -1  # launch configuration bench.py times (-1: balanced split)
    shuffle_seeds: list = field(default_factory=list)  # one per layer

    @property
    def num_seqs(self):
        return len(self.decode_seqs)

    @property
    def group(self):
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self):
        """1/sqrt(d_k) as an fp32 value (dev.to §1, attention formula)."""
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    def prefill_lengths(self):
        """Tokens stored per plan sequence before the decode step."""
        lens = {}
        nseq = 0
        for op in self.ops:
            if op[0] == "create":
                lens[nseq] = 0
                nseq += 1
            elif op[0] == "fork":
                lens[nseq] = lens[op[1]]
                nseq += 1
            elif op[0] == "prefill":
                lens[op[1]] += op[2]
            elif op[0] == "free":
                pass
        return lens

    def decode_lengths(self):
        pre = self.prefill_lengths()
        return [pre[s] + 1 for s in self.decode_seqs]

    def prefill_tokens(self):
        return sum(op[2] for op in self.ops if op[0] == "prefill")

    def max_seq_len(self):
        return max(self.decode_lengths())

    def max_blocks_per_seq(self):
        return -(-self.max_seq_len() // self.block_size)

    def kv_read_bytes(self):
        """K and V bytes one decode step must read: every valid (token, KV
        head) row of K and of V once, per layer."""
        eb = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1}[self.kv_dtype]
        return (sum(self.decode_lengths()) * self.num_kv_heads * self.head_dim * eb * 2
                * self.num_layers)

    def tensor_seed(self, layer, what):
        tags = {"q": 1, "k_new": 2, "v_new": 3, "k_pre": 4, "v_pre": 5}
        return (self.seed * 1000 + layer * 10 + tags[what]) & 0x7FFFFFFF


def _pool_blocks(lengths, slack, bs):
    need = sum(-(-n // bs) for n in lengths)
    return int(math.ceil(slack * need))


def _independent(name, cid, lens_pre, nblocks_slack, **kw):
    ops = []
    for i, n in enumerate(lens_pre):
        ops.append(("create",))
        ops.append(("prefill", i, int(n)))
    lens_dec = [int(n) + 1 for n in lens_pre]
    nb = kw.pop("num_blocks", None) or _pool_blocks(lens_dec, nblocks_slack, kw["block_size"])
    return Workload(name=name, config_id=cid, num_blocks=nb, ops=ops,
                    decode_seqs=list(range(len(lens_pre))), **kw)


def _shared_prefix(name, cid, prefix_len, suffixes, slack, **kw):
    ops = [("create",), ("prefill", 0, prefix_len)]
    children = []
    for _ in suffixes:
        ops.append(("fork", 0))
        children.append(len(children) + 1)
    ops.append(("free", 0))
    for c, s in zip(children, suffixes):
        ops.append(("prefill", c, int(s)))
    bs = kw["block_size"]
    need = -(-prefix_len // bs) + sum(
        -(-(prefix_len + int(s) + 1) // bs) - prefix_len // bs for s in suffixes)
    nb = int(math.ceil(slack * need))
    return Workload(name=name, config_id=cid, num_blocks=nb, ops=ops, decode_seqs=children,
                    **kw)


def config(cid, size="full", block_size=BLOCK_SIZE):
    """The five workloads; size="small" gives a reduced variant of the same
    shape that the oracle finishes in seconds (several tiles, ragged tails).
    block_size (16 by default, as in the pages' workloads) changes only how
    many tokens a physical block holds; lengths and tensors stay the same."""
    seed = 1000 + cid + (0 if size == "full" else 500)
    rng = np.random.default_rng(seed)
    bs = block_size
    if cid == 1:
        # Tiny fp32 MHA step: 4 heads, head_dim 64, lengths {17,33,64,100}
        # before the append, blocks permuted in a 64-block pool (the same
        # 1024 slots at other block sizes, at least 4 spare blocks).
        nb = max(64 * 16 // bs, _pool_blocks([18, 34, 65, 101], 1.0, bs) + 4)
        w = _independent("tiny-fp32-mha", 1, [17, 33, 64, 100], 1.0, num_blocks=nb,
                         num_q_heads=4, num_kv_heads=4, head_dim=64, q_dtype="f32",
                         kv_dtype="f32", seed=seed, partition_size=0, block_size=bs)
    elif cid == 2:
        # Llama-3-8B layer (dev.to §2 Example 2): 32 q heads on 8 KV heads,
        # head_dim 128, bf16; lengths uniform in [512, 4096], pool 1.25x.
        B, lo, hi = (32, 512, 4096) if size == "full" else (5, 20, 700)
        lens = rng.integers(lo, hi + 1, size=B)
        w = _independent("llama3-8b-gqa-bf16", 2, lens, 1.25, num_q_heads=32, num_kv_heads=8,
                         head_dim=128, q_dtype="bf16", kv_dtype="bf16", seed=seed,
                         block_size=bs)
    elif cid == 3:
        # Llama-2-13B MHA (dev.to §2 Example 1): 40 heads, head_dim 128, fp16,
        # 8 sequences at exactly 4096 tokens, all 40 layers, a pool per layer
        # with its own block permutation.
        B, n, L = (8, 4096, 40) if size == "full" else (3, 300, 2)
        w = _independent("llama2-13b-mha-fp16", 3, [n - 1] * B, 1.0, num_q_heads=40,
                         num_kv_heads=40, head_dim=128, q_dtype="f16", kv_dtype="f16",
                         seed=seed, num_layers=L, block_size=bs)
    elif cid == 4:
        # 256 sequences sharing a 2048-token prefix by reference count
        # (dev.to §5), each with its own suffix, geometric with mean 350
        # (the dev.to §3 output length) capped at 2048.
        B, P, mean = (256, 2048, 350) if size == "full" else (6, 64, 40)
        suf = np.minimum(rng.geometric(1.0 / mean, size=B), 2048)
        w = _shared_prefix("prefix-sharing-bf16", 4, P, suf, 1.25, num_q_heads=32,
                           num_kv_heads=8, head_dim=128, q_dtype="bf16", kv_dtype="bf16",
                           seed=seed, block_size=bs)
    elif cid == 5:
        # Long context (hyperinfer.ai "Why this matters for long context"):
        # 70B-shaped layer, 64 q heads on 8 KV heads, FP8 E4M3 KV, bf16 q,
        # 4 sequences at exactly 131072 tokens.
        B, n = (4, 131072) if size == "full" else (2, 1500)
        w = _independent("long-context-fp8-70b", 5, [n - 1] * B, 1.0, num_q_heads=64,
                         num_kv_heads=8, head_dim=128, q_dtype="bf16", kv_dtype="e4m3",
                         seed=seed, block_size=bs)
    else:
        raise ValueError(cid)
    w.shuffle_seeds = [seed * 7919 + layer + 1 for layer in range(w.num_layers)]
    return w


# -- tensors ---------------------------------------------------------------
def _torch():
    import torch
    return torch


def normal(shape, seed, dtype, device="cpu"):
    """N(0,1) samples from torch's seeded generator, rounded to `dtype`
    ("f32", "f16" or "bf16")."""
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return x.to(getattr(torch, TORCH_DTYPES[dtype]))


def step_tensors(w, layer=0, device="cpu"):
    """q [B][Hq][D], and the new token's k, v [B][Hkv][D], in w.q_dtype."""
    B, Hq, Hkv, D = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim
    q = normal((B, Hq, D), w.tensor_seed(layer, "q"), w.q_dtype, device)
    k = normal((B, Hkv, D), w.tensor_seed(layer, "k_new"), w.q_dtype, device)
    v = normal((B, Hkv, D), w.tensor_seed(layer, "v_new"), w.q_dtype, device)
    return q, k, v


def prefill_tensors(w, layer=0, device="cpu"):
    """K and V of every prefill token, [T][Hkv][D] in w.q_dtype, in plan order."""
    T, Hkv, D = w.prefill_tokens(), w.num_kv_heads, w.head_dim
    k = normal((T, Hkv, D), w.tensor_seed(layer, "k_pre"), w.q_dtype, device)
    v = normal((T, Hkv, D), w.tensor_seed(layer, "v_pre"), w.q_dtype, device)
    return k, v


def fp8_scale(x):
    """Per-tensor scale amax(|x|)/448 (448 = largest finite E4M3 value), as an
    fp32 number: the calibration of the stored FP8 data."""
    amax = float(x.abs().max().float().item())
    return float(np.float32(np.float32(amax) / np.float32(448.0))) if amax > 0 else 1.0


def storage(t):
    """Host numpy array holding a tensor's raw storage (uint16 for 16-bit
    floats, uint8 for FP8 bytes)."""
    torch = _torch()
    t = t.detach().contiguous().cpu()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.uint8:
        return t.numpy()
    if t.dtype == torch.int32:
        return t.numpy()
    raise TypeError(t.dtype)
