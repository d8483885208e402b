"""Blocks of 32 to 256 tokens on the GPU, against the oracle.

The pages use 16-token blocks and also name 32 (a vLLM option) and pages of
256 or more tokens (dev.to, "Why LLMs Run Out of VRAM...", §4 and §6;
vaibhawkumar.in, "Why LLMs run out of VRAM...", paged-cache sketch).  The
kernels work on 16-token tiles and a block of bs tokens is bs/16 of them, so
the block size changes the table walk and the addresses, not the
arithmetic: with the same lengths the balanced split cuts the same tiles,
and outputs are bit-identical to the 16-token layout.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_255_amd as pa
import workloads
from tests.scenario import GpuStep, Inputs, OracleStep, check_close, compare_cache_blocks, to_f64

pytestmark = pytest.mark.gpu

BLOCK_SIZES = [32, 64, 128, 256]


def say(*a):
    print(*a, flush=True)


def _cases():
    out = []
    for bs in BLOCK_SIZES:
        for cid in (1, 2, 3, 4, 5):
            if cid == 4 and bs > 64:
                continue  # the small prefix (64 tokens) would end inside a shared block
            for kernel, part in ((pa.KERNEL_MFMA, pa.PARTITION_BALANCED), (pa.KERNEL_MFMA, 0),
                                 (pa.KERNEL_MFMA, 64), (pa.KERNEL_VALU, 0),
                                 (pa.KERNEL_VALU, 64)):
                out.append((bs, cid, kernel, part))
    return out


def _supported(kernel, w):
    G = w.num_q_heads // w.num_kv_heads
    if kernel == pa.KERNEL_VALU:
        return G in (1, 2, 4) or (G == 8 and w.head_dim == 64)
    return w.q_dtype in ("bf16", "f16") and G <= 16


@pytest.mark.parametrize("bs,cid,kernel,part", _cases())
def test_parity_block_sizes(bs, cid, kernel, part):
    w = workloads.config(cid, "full" if cid == 1 else "small", block_size=bs)
    if not _supported(kernel, w):
        pytest.skip("shape not built for this kernel")
    say(f"[case] block_size={bs} cfg{cid} kernel={kernel} partition={part}")
    for layer in range(w.num_layers):
        inp = Inputs(w, layer)
        g = GpuStep(w, layer, inp, partition=part, kernel=kernel)
        o = OracleStep(w, layer, inp)
        np.testing.assert_array_equal(g.tables, o.tables)
        np.testing.assert_array_equal(g.step_slots, o.step_slots)
        g.append_prefill()
        g.append_step()
        torch.cuda.synchronize()
        compare_cache_blocks(g.k_cache, o.k_cache, w, None)
        compare_cache_blocks(g.v_cache, o.v_cache, w, None)
        out = to_f64(g.decode())
        err = check_close(out, o.decode(), w.kv_dtype, w.q_dtype)
        say(f"[ok] err={err:.3g}")


@pytest.mark.parametrize("bs", BLOCK_SIZES)
@pytest.mark.parametrize("cid,part", [(2, pa.PARTITION_BALANCED), (5, pa.PARTITION_BALANCED),
                                      (2, 64)])
def test_decode_append_block_sizes(bs, cid, part):
    """pa_decode_append (the step's token stored by the decode launch) leaves
    the same cache bytes and output bits as pa_cache_append + pa_decode."""
    say(f"[case] decode_append block_size={bs} cfg{cid} partition={part}")
    w = workloads.config(cid, "small", block_size=bs)
    inp = Inputs(w)
    a = GpuStep(w, 0, inp, partition=part, kernel=pa.KERNEL_MFMA)
    b = GpuStep(w, 0, inp, partition=part, kernel=pa.KERNEL_MFMA)
    a.append_prefill()
    b.append_prefill()
    a.append_step()
    ref = a.decode().clone()
    got = b.decode_append().clone()
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    assert torch.equal(a.k_cache.view(torch.uint8), b.k_cache.view(torch.uint8))
    assert torch.equal(a.v_cache.view(torch.uint8), b.v_cache.view(torch.uint8))


@pytest.mark.parametrize("cid", [2, 5])
def test_block_size_does_not_change_the_bits(cid):
    """The same tokens in pools of 16- and 64-..256-token blocks: the balanced
    split sees the same tiles, so every output bit agrees."""
    say(f"[case] bits across block sizes cfg{cid}")
    outs = []
    for bs in [16] + BLOCK_SIZES:
        w = workloads.config(cid, "small", block_size=bs)
        inp = Inputs(w)
        g = GpuStep(w, 0, inp, partition=pa.PARTITION_BALANCED, kernel=pa.KERNEL_MFMA)
        g.append_prefill()
        g.append_step()
        outs.append(g.decode().clone())
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
