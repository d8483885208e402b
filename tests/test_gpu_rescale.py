"""GPU parity on inputs that make the online softmax rescale its running sum
and accumulators by factors strictly between 0 and 1 (tests/rescale_case.py):
a plateau of thousands of tokens, then a token whose score beats it by 8.9
to 11.5 log2 units (inside a late tile of a range, in a later balanced run
and in a later fixed partition), the reverse order, and an appended token
that rescales the sequence's last tile.  Every launch mode of both kernels,
with the step's token appended by pa_cache_append before pa_decode and by
pa_decode_append, is compared with the oracle at the dtype's tolerance, and
the caches byte for byte.  test_rescale_inputs.py shows on the CPU that a
kernel which left out either multiplication of the rescale would miss these
tolerances by far.

Reference for what is computed: dev.to, "Why LLMs Run Out of VRAM: KV Cache
Fragmentation and How PagedAttention Fixes It", §1 (attention formula).
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_255_amd as pa
import workloads
from tests import rescale_case as rc
from tests.scenario import GpuStep, OracleStep, check_close, compare_cache_blocks, to_f64

pytestmark = pytest.mark.gpu

TORCH = {"bf16": torch.bfloat16, "f16": torch.float16}


def say(*a):
    print(*a, flush=True)


class _Inputs:
    """The planted values as device tensors in the activation dtype; FP8
    scales of 1 keep every planted value exact."""

    def __init__(self, c, q_dtype):
        dt = TORCH[q_dtype]
        dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda().to(dt)  # noqa: E731
        self.q = dev(c["q"])
        self.k_pre, self.v_pre = dev(c["k_pre"]), dev(c["v_pre"])
        self.k_new, self.v_new = dev(c["k_new"]), dev(c["v_new"])
        self.k_scale = self.v_scale = 1.0


def _workload(q_dtype, kv_dtype):
    w = workloads._independent("planted-rescale", 0, [n - 1 for n in rc.LENS], 1.25,
                               num_q_heads=rc.HQ, num_kv_heads=rc.HKV, head_dim=rc.D,
                               q_dtype=q_dtype, kv_dtype=kv_dtype, seed=0, block_size=16)
    w.shuffle_seeds = [20261203]
    return w


def _device_waves(w):
    """Runs of the balanced split on this device."""
    desc = pa.kv_desc(w.num_q_heads, w.num_kv_heads, w.head_dim, w.num_blocks, w.q_dtype,
                      w.kv_dtype)
    W = pa.pa_decode_balanced_waves(desc)
    assert 0 < W <= 1 << 16, W
    return W


@pytest.fixture(scope="module", params=[("bf16", "bf16"), ("f16", "f16"), ("bf16", "e4m3")],
                ids=lambda p: f"{p[0]}-{p[1]}")
def planted(request):
    w = _workload(*request.param)
    W = _device_waves(w)
    say(f"[setup] planted rescale {request.param} W={W} lengths={rc.LENS}")
    c = rc.build(W)
    inp = _Inputs(c, w.q_dtype)
    o = OracleStep(w, 0, inp)
    ref = o.decode()
    return w, inp, o, ref, W


CASES = [(0, pa.KERNEL_MFMA), (64, pa.KERNEL_MFMA), (512, pa.KERNEL_MFMA),
         (pa.PARTITION_BALANCED, pa.KERNEL_MFMA),
         (0, pa.KERNEL_VALU), (64, pa.KERNEL_VALU), (512, pa.KERNEL_VALU)]


@pytest.mark.parametrize("append", [False, True], ids=["append-then-decode", "decode-append"])
@pytest.mark.parametrize("mode,kernel", CASES)
def test_planted_rescale(planted, mode, kernel, append):
    w, inp, o, ref, W = planted
    say(f"[case] planted rescale {w.q_dtype}/{w.kv_dtype} mode={mode} kernel={kernel} "
        f"append={append}")
    g = GpuStep(w, 0, inp, partition=mode, kernel=kernel)
    np.testing.assert_array_equal(g.tables, o.tables)
    np.testing.assert_array_equal(g.lens, o.lens)
    np.testing.assert_array_equal(g.step_slots, o.step_slots)
    g.append_prefill()
    if append:
        out = g.decode_append()
    else:
        g.append_step()
        out = g.decode()
    torch.cuda.synchronize()
    got = to_f64(out)
    err = check_close(got, ref, w.kv_dtype, w.q_dtype)
    # the appended tokens' blocks, and with the folded append every block
    blocks = None if append else sorted({int(s) // 16 for s in o.step_slots})
    compare_cache_blocks(g.k_cache, o.k_cache, w, blocks)
    compare_cache_blocks(g.v_cache, o.v_cache, w, blocks)
    say(f"[ok] err={err:.3g}")
