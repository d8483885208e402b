"""The planted-score inputs of tests/rescale_case.py, on the CPU.

The GPU test (test_gpu_rescale.py) compares the kernels with the oracle on
these inputs.  Here a CPU model of the kernels' lazy online-softmax update
(tests/rescale_case.py: lazy_model) runs on the same values, for every launch
mode's work ranges, to show three things:
  * the model without a planted mistake agrees with the oracle (fp64), so the
    model is the update the kernels make;
  * in every mode some range rescales by a factor strictly between 0 and 1
    after it has summed many tokens;
  * with the sum's or the accumulator's multiplication left out of that
    rescale, the output moves by far more than the bf16 tolerance (1e-2), so
    the GPU test fails for a kernel with either mistake.
The balanced split is modelled with 1,024 runs, the count on an MI355X (256
CUs, one wave per SIMD); the GPU test places its tokens for the device's own
count.
"""
import numpy as np
import pytest
import torch

import oracle
from tests import rescale_case as rc

W_NOMINAL = 1024
MODES = [0, 64, 512, "balanced"]


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)


@pytest.fixture(scope="module")
def case():
    c = rc.build(W_NOMINAL)
    q = _bf16(c["q"])
    # stored values: every token of a sequence, the appended one last
    ks, vs, off = [], [], 0
    kp, vp = _bf16(c["k_pre"]), _bf16(c["v_pre"])
    kn, vn = _bf16(c["k_new"]), _bf16(c["v_new"])
    for b, n in enumerate(rc.LENS):
        ks.append(torch.cat([kp[off:off + n - 1], kn[b:b + 1]]))
        vs.append(torch.cat([vp[off:off + n - 1], vn[b:b + 1]]))
        off += n - 1
    # oracle: blocks in order, sequence after sequence
    nb = [rc.tiles(n) for n in rc.LENS]
    NB = sum(nb)
    first = np.concatenate([[0], np.cumsum(nb)])[:-1]
    tables = np.full((len(nb), max(nb)), -1, np.int32)
    for b in range(len(nb)):
        tables[b, :nb[b]] = np.arange(first[b], first[b] + nb[b])
    slots = np.concatenate([first[b] * 16 + np.arange(n) for b, n in enumerate(rc.LENS)])
    kc = np.zeros(NB * rc.HKV * 16 * rc.D, np.uint16)
    vc = np.zeros_like(kc)
    allk = torch.cat(ks).contiguous()
    allv = torch.cat(vs).contiguous()
    st = lambda t: t.view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    oracle.cache_append(st(allk), st(allv), kc, vc, slots.astype(np.int32),
                        num_kv_heads=rc.HKV, head_dim=rc.D, block_size=16, num_blocks=NB,
                        kv_dtype="bf16", in_dtype="bf16")
    scale = float(np.float32(1 / np.sqrt(rc.D)))
    ref = oracle.decode(st(q.contiguous()), kc, vc, tables, np.array(rc.LENS, np.int32),
                        num_q_heads=rc.HQ, num_kv_heads=rc.HKV, head_dim=rc.D, block_size=16,
                        num_blocks=NB, q_dtype="bf16", kv_dtype="bf16", scale=scale)
    qd = q.double().numpy()
    kd = [k.double().numpy() for k in ks]
    vd = [v.double().numpy() for v in vs]
    return dict(q=qd, k=kd, v=vd, ref=ref, scale=scale)


def _model(case, mode, **mut):
    out = np.zeros((len(rc.LENS), rc.HQ, rc.D))
    for b, n in enumerate(rc.LENS):
        for g in range(rc.HKV):
            rng = rc.ranges(mode, n, g, b, W_NOMINAL)
            out[b, g * rc.G:(g + 1) * rc.G] = rc.lazy_model(
                case["q"][b, g * rc.G:(g + 1) * rc.G], case["k"][b][:, g], case["v"][b][:, g],
                rng, case["scale"], **mut)
    return out


def test_placement():
    ts0, ts1, ts3 = rc.spike_tiles(W_NOMINAL)
    assert ts0 % 32 == 31 and ts0 > 32
    T, R, _, seg = rc.balanced_runs(rc.LENS, W_NOMINAL)
    assert rc.is_run_last(seg(0, 1) + ts1, T, R)
    assert not rc.is_run_first(seg(1, 1) + ts1, T, R)
    for g in range(rc.HKV):
        assert not rc.is_run_first(seg(g, 0) + ts0, T, R)
        # the spike's run is not the segment's first run
        assert rc.run_of(seg(g, 0) + ts0, T, R) > rc.run_of(seg(g, 0), T, R)
    # several tiles per balanced run, so "late in a run" means something
    assert T // R >= 8


@pytest.mark.parametrize("mode", MODES)
def test_model_is_the_oracle(case, mode):
    got = _model(case, mode)
    err = np.max(np.abs(got - case["ref"]))
    assert err < 1e-9, err


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("mutation", ["drop_l", "drop_acc"])
def test_a_rescale_left_out_is_caught(case, mode, mutation):
    got = _model(case, mode, **{mutation: True})
    err = np.abs(got - case["ref"]).max(axis=2)  # [B][HQ]
    # far beyond the bf16/fp16 tolerance (1e-2) and the FP8 one (2e-2)
    assert err.max() > 0.3, err.max()
    # for the rising sequences (0, 1, 3) in every head that rescales (c_h =
    # 8, 7, 9; the fourth head's step stays under the threshold), wherever
    # the highest token of the sequence is not the first tile of its range
    # (there the rescale factor is 0 and nothing is left to multiply)
    ts0, ts1, _ = rc.spike_tiles(W_NOMINAL)
    top = {0: ts0, 1: ts1, 3: rc.tiles(rc.LENS[3]) - 1}
    checked = 0
    for b, t in top.items():
        for g in range(rc.HKV):
            starts = [a // 16 for a, _ in rc.ranges(mode, rc.LENS[b], g, b, W_NOMINAL)]
            if t in starts:
                continue
            for h in range(g * rc.G, (g + 1) * rc.G):
                if rc.COEF[h % rc.G] != 6.0:
                    assert err[b, h] > 0.05, (b, h, err[b, h])
                    checked += 1
    assert checked >= 12, checked
