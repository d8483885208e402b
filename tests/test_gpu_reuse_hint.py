"""The seq_shared hint on the GPU.

Requests that share a system prompt map the same prefix blocks (dev.to, "Why
LLMs Run Out of VRAM...", §5 "Zero-Copy Forking" and "Automatic Prefix
Caching"; hyperinfer.ai, "Prefix caching: share the system prompt"), so a
decode launch reads those blocks once per sequence.  pa_export_block_tables
counts, per sequence, the leading table entries that another exported table
also holds; the decode calls read those tiles with caching loads and the
rest with streaming loads.  The hint changes how bytes are fetched, never
which bytes: every output bit must equal the decode without it, which the
other GPU tests check against the oracle.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_255_amd as pa
import workloads
from tests.scenario import GpuStep, Inputs, OracleStep, check_close, to_f64

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def _shared(g, w):
    t, n, sh = pa.pa_export_block_tables(g.pool, g.dec, w.max_blocks_per_seq(),
                                         with_shared=True)
    np.testing.assert_array_equal(t, g.tables)
    np.testing.assert_array_equal(n, g.lens)
    return sh


def test_shared_counts_cover_the_prefix():
    """Config 4's decode sequences all map the 64-token prompt (4 blocks of 16
    tokens, the small size), and nothing after it."""
    w = workloads.config(4, "small")
    g = GpuStep(w, 0, Inputs(w), partition=pa.PARTITION_BALANCED, kernel=pa.KERNEL_MFMA)
    sh = _shared(g, w)
    assert np.all(sh == 64 // w.block_size), sh
    # a single sequence shares nothing with itself
    _, _, one = pa.pa_export_block_tables(g.pool, g.dec[:1], w.max_blocks_per_seq(),
                                          with_shared=True)
    assert one[0] == 0


@pytest.mark.parametrize("size", ["small", "full"])
@pytest.mark.parametrize("kernel,part", [(pa.KERNEL_MFMA, pa.PARTITION_BALANCED),
                                         (pa.KERNEL_MFMA, 0), (pa.KERNEL_MFMA, 64),
                                         (pa.KERNEL_VALU, 0)])
def test_hint_keeps_every_bit(size, kernel, part):
    """Config 4 with and without the hint: pa_decode and pa_decode_append give
    the same output bits and cache bytes; the full size matches the oracle on
    sampled rows too."""
    if size == "full" and kernel == pa.KERNEL_VALU:
        pytest.skip("the VALU kernel streams every block; the small size covers it")
    say(f"[case] reuse hint cfg4 {size} kernel={kernel} partition={part}")
    w = workloads.config(4, size)
    inp = Inputs(w)
    a = GpuStep(w, 0, inp, partition=part, kernel=kernel)
    b = GpuStep(w, 0, inp, partition=part, kernel=kernel)
    sh = _shared(a, w)
    assert sh.max() > 0
    a.append_prefill()
    b.append_prefill()
    a.append_step()
    ref = a.decode().clone()
    got = a.decode(out=torch.empty_like(ref), seq_shared=sh)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    # the appending decode, with the hint, against the two-call path without it
    got2 = b.decode_append(seq_shared=sh).clone()
    torch.cuda.synchronize()
    assert torch.equal(got2, ref)
    assert torch.equal(a.k_cache.view(torch.uint8), b.k_cache.view(torch.uint8))
    assert torch.equal(a.v_cache.view(torch.uint8), b.v_cache.view(torch.uint8))
    if size == "full":
        o = OracleStep(w, 0, inp)
        err = check_close(to_f64(got2), o.decode(), w.kv_dtype, w.q_dtype)
        say(f"[ok] every row err={err:.3g}")


def test_hint_counts_out_of_range_are_clamped():
    """Counts beyond the table (or negative) only choose the load policy of
    tiles that exist: the bits stay those of the decode without the hint."""
    w = workloads.config(4, "small")
    inp = Inputs(w)
    g = GpuStep(w, 0, inp, partition=pa.PARTITION_BALANCED, kernel=pa.KERNEL_MFMA)
    g.append_prefill()
    g.append_step()
    ref = g.decode().clone()
    B = len(g.dec)
    for fill in (-5, 1 << 30):
        got = g.decode(out=torch.empty_like(ref), seq_shared=np.full(B, fill, np.int32))
        torch.cuda.synchronize()
        assert torch.equal(got, ref), fill
