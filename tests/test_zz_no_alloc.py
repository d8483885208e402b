"""The allocation-free decode step (pa_decode_append_noalloc) against the
step with a caller workspace (pa_decode_append): the same output bits and
cache bytes, on two calls in a row, the second with a smaller batch, so the
scratch array holds the first call's states when the second starts.  Plus the
size limit, refused on the host before anything is launched.
"""
import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_255_amd as pa
import workloads
from tests.scenario import GpuStep, Inputs, OracleStep, check_close, to_f64

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def _noalloc(g, out):
    i, w = g.inputs, g.w
    slots = torch.from_numpy(np.ascontiguousarray(g.step_slots)).cuda()
    pa.pa_decode_append_noalloc(i.q, i.k_new, i.v_new, slots, g.k_cache, g.v_cache, g.d_tables,
                                g.d_lens, w.max_seq_len(), w.scale, out, g.desc, i.k_scale,
                                i.v_scale, partition_size=g.partition)
    return out


# (config 2 at full size in 64-token partitions would need about 34 MB of
# partial states, more than the scratch holds; the balanced split needs 2.7)
@pytest.mark.parametrize("first,second,part", [
    ((2, "full"), (2, "small"), pa.PARTITION_BALANCED),
    ((5, "small"), (4, "small"), pa.PARTITION_BALANCED),
    ((5, "small"), (4, "small"), 64)])
def test_noalloc_matches_workspace_step(first, second, part):
    for cid, size in (first, second):
        w = workloads.config(cid, size)
        say(f"[case] noalloc {w.name} {size} partition={part}")
        inp = Inputs(w, 0)
        ref = GpuStep(w, 0, inp, partition=part, kernel=pa.KERNEL_MFMA)
        ref.append_prefill()
        want = ref.decode_append(out=torch.full_like(inp.q, 7.0)).clone()
        got_step = GpuStep(w, 0, inp, partition=part, kernel=pa.KERNEL_MFMA)
        got_step.append_prefill()
        got = _noalloc(got_step, torch.full_like(inp.q, 3.0))
        torch.cuda.synchronize()
        assert torch.equal(want.view(torch.int16), got.view(torch.int16))
        assert torch.equal(ref.k_cache.view(torch.uint8), got_step.k_cache.view(torch.uint8))
        assert torch.equal(ref.v_cache.view(torch.uint8), got_step.v_cache.view(torch.uint8))
        if size == "small":
            o = OracleStep(w, 0, inp)
            err = check_close(to_f64(got), o.decode(), w.kv_dtype, w.q_dtype)
            say(f"[ok] oracle err={err:.3g}")


def test_noalloc_single_pass_needs_no_scratch():
    w = workloads.config(2, "small")
    inp = Inputs(w, 0)
    ref = GpuStep(w, 0, inp, partition=0, kernel=pa.KERNEL_MFMA)
    ref.append_prefill()
    want = ref.decode_append(out=torch.full_like(inp.q, 7.0)).clone()
    g = GpuStep(w, 0, inp, partition=0, kernel=pa.KERNEL_MFMA)
    g.append_prefill()
    got = _noalloc(g, torch.full_like(inp.q, 3.0))
    torch.cuda.synchronize()
    assert torch.equal(want.view(torch.int16), got.view(torch.int16))


def test_noalloc_refuses_more_than_its_scratch():
    """Config 5's four 131,072-token sequences in 16-token partitions need
    about 139 MB of partial states: refused with PA_ERR_CAPACITY before any
    pointer is used (the pointers here are placeholders)."""
    desc = pa.kv_desc(64, 8, 128, 32768, "bf16", "e4m3")
    need = pa.pa_decode_workspace_bytes(desc, 4, 131072, 16)
    assert need > pa.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(4096)
    st = pa._lib.pa_decode_append_noalloc(fake, fake, fake, fake, fake, fake, fake, 8192, fake,
                                          None, None, 4, 131072, 0.088, 1.0, 1.0, fake, 16,
                                          ctypes.byref(desc), None)
    assert st == pa.ERR_CAPACITY
    assert "allocation-free" in pa.pa_last_error()


def test_noalloc_with_a_share_plan():
    """A batch whose sequences share a prompt, with its share plan: the
    scratch has no room for the plan's prefix rows (their room is sized for
    W x 16 member slots, about 34 MB), so the allocation-free step reads the
    shared blocks with the plan's caching hint and gives the bits of
    pa_decode_append with the same plan and a workspace holding only the
    sequences' room; both match the oracle."""
    w = workloads.config(4, "small")
    say(f"[case] noalloc with a share plan {w.name}")
    inp = Inputs(w, 0)
    part = pa.PARTITION_BALANCED
    ref = GpuStep(w, 0, inp, partition=part, kernel=pa.KERNEL_MFMA)
    plan = ref.plan()
    assert plan[1] >= 1  # the batch has a group
    W = pa.pa_decode_balanced_waves(ref.desc)
    G = w.num_q_heads // w.num_kv_heads
    seq_room = (W + w.num_seqs * w.num_kv_heads) * G * (w.head_dim + 2) * 4
    assert seq_room < pa.pa_decode_workspace_bytes(ref.desc, w.num_seqs, w.max_seq_len(), part)
    ref.workspace = torch.empty(seq_room, dtype=torch.uint8, device="cuda")
    ref.append_prefill()
    want = ref.decode_append(out=torch.full_like(inp.q, 7.0), seq_shared=plan).clone()
    g = GpuStep(w, 0, inp, partition=part, kernel=pa.KERNEL_MFMA)
    g.append_prefill()
    i = g.inputs
    slots = torch.from_numpy(np.ascontiguousarray(g.step_slots)).cuda()
    got = torch.full_like(inp.q, 3.0)
    pa.pa_decode_append_noalloc(i.q, i.k_new, i.v_new, slots, g.k_cache, g.v_cache, g.d_tables,
                                g.d_lens, w.max_seq_len(), w.scale, got, g.desc, i.k_scale,
                                i.v_scale, partition_size=part,
                                seq_shared=torch.from_numpy(plan).cuda())
    torch.cuda.synchronize()
    assert torch.equal(want.view(torch.int16), got.view(torch.int16))
    assert torch.equal(ref.k_cache.view(torch.uint8), g.k_cache.view(torch.uint8))
    assert torch.equal(ref.v_cache.view(torch.uint8), g.v_cache.view(torch.uint8))
    err = check_close(to_f64(got), OracleStep(w, 0, inp).decode(), w.kv_dtype, w.q_dtype)
    say(f"[ok] oracle err={err:.3g}")
