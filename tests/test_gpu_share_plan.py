"""The share plan (seq_shared) on the GPU.

Requests that share a system prompt map the same prefix blocks (dev.to, "Why
LLMs Run Out of VRAM...", §5 "Zero-Copy Forking" and "Automatic Prefix
Caching"; hyperinfer.ai, "Prefix caching: share the system prompt").  The
plan (pa_export_share_plan) names the groups of sequences that share their
leading blocks.  Two uses:

- a cache-policy hint: the leading entries other tables also hold are read
  with caching loads, the rest with streaming loads.  Bytes fetched change,
  never which bytes: every output bit equals the decode without the plan
  (fixed partitions, the VALU kernel, and the balanced split when the
  workspace has no room for prefix rows);
- prefix rows (balanced split with room for them): each group's shared
  blocks are read once per KV head for up to 4 x 16 / G members at a time,
  and the merge folds each member's row state with its own pieces.  The sum
  runs in another order, so the outputs are checked against the oracle, and
  against the decode that reads every sequence's blocks itself (the same
  tolerance), rather than bit for bit; bits must not depend on where the
  blocks sit in the pool, nor on whether the two launches run as one call.
"""
import dataclasses

import numpy as np
import pytest
import torch

import paged_kv_cache_255_amd as pa
import workloads
from tests.scenario import GpuStep, Inputs, OracleStep, check_close, to_f64

pytestmark = pytest.mark.gpu

BAL = pa.PARTITION_BALANCED


def say(*a):
    print(*a, flush=True)


def _base_workspace(g):
    """A workspace with room for the sequences' slots only: the balanced
    launch then reads every sequence's blocks itself."""
    w = g.w
    G = w.num_q_heads // w.num_kv_heads
    W = pa.pa_decode_balanced_waves(g.desc)
    assert W > 0
    return torch.empty((W + w.num_seqs * w.num_kv_heads) * G * (w.head_dim + 2) * 4,
                       dtype=torch.uint8, device="cuda")


def _hint_only_plan(g, fill):
    """A plan with no groups whose cache-policy counts are all `fill`."""
    B = len(g.dec)
    plan = np.zeros(pa.share_plan_words(B), np.int32)
    plan[0] = pa.SHARE_PLAN_MAGIC
    plan[2:2 + B] = fill
    plan[2 + B:2 + 2 * B] = -1
    return plan


def test_plan_covers_the_prefix():
    """Config 4's decode sequences all map the 64-token prompt (4 blocks of 16
    tokens, the small size), and nothing after it: one group of all of them."""
    w = workloads.config(4, "small")
    g = GpuStep(w, 0, Inputs(w), partition=BAL, kernel=pa.KERNEL_MFMA)
    plan = g.plan()
    B = len(g.dec)
    assert np.all(plan[2:2 + B] == 64 // w.block_size), plan
    assert plan[1] == 1 and plan[2 + 4 * B] == B and plan[2 + 5 * B] == 4


@pytest.mark.parametrize("size", ["small", "full"])
@pytest.mark.parametrize("kernel,part,room", [(pa.KERNEL_MFMA, BAL, False),
                                              (pa.KERNEL_MFMA, 0, True),
                                              (pa.KERNEL_MFMA, 64, True),
                                              (pa.KERNEL_VALU, 0, True)])
def test_plan_as_hint_keeps_every_bit(size, kernel, part, room):
    """Config 4 where the plan is a cache-policy hint only: pa_decode and
    pa_decode_append give the same output bits and cache bytes with and
    without it; the full size matches the oracle on every row too."""
    if size == "full" and kernel == pa.KERNEL_VALU:
        pytest.skip("the VALU kernel streams every block; the small size covers it")
    say(f"[case] plan as hint cfg4 {size} kernel={kernel} partition={part}")
    w = workloads.config(4, size)
    inp = Inputs(w)
    a = GpuStep(w, 0, inp, partition=part, kernel=kernel)
    b = GpuStep(w, 0, inp, partition=part, kernel=kernel)
    if not room:
        a.workspace = _base_workspace(a)
        b.workspace = _base_workspace(b)
    plan = a.plan()
    assert plan[1] > 0
    a.append_prefill()
    b.append_prefill()
    a.append_step()
    ref = a.decode().clone()
    got = a.decode(out=torch.empty_like(ref), seq_shared=plan)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    got2 = b.decode_append(seq_shared=plan).clone()
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
    tiles that exist: the bits stay those of the decode without the plan."""
    w = workloads.config(4, "small")
    inp = Inputs(w)
    g = GpuStep(w, 0, inp, partition=BAL, kernel=pa.KERNEL_MFMA)
    g.append_prefill()
    g.append_step()
    ref = g.decode().clone()
    for fill in (-5, 1 << 30):
        got = g.decode(out=torch.empty_like(ref), seq_shared=_hint_only_plan(g, fill))
        torch.cuda.synchronize()
        assert torch.equal(got, ref), fill


@pytest.mark.parametrize("kind", ["hint", "rows"])
def test_held_results_fill_the_area(kind):
    """1,500 sequences of 17 to 47 own tokens (with a 64-token shared prompt
    for "rows"): each balanced run meets a dozen pieces, so the LDS area that
    holds a run's outputs, partial states, segment records and appended
    tokens until the run ends (launches with a plan) fills and is stored
    before the run's end, more than once.  The appending decode with the plan
    still gives the bits and cache bytes of the two-call path (without the
    plan for "hint", with it for "rows") and matches the oracle on every
    row.  (At 17 tokens or more the outputs stay below 2.6 in magnitude, where
    a bf16 output's own rounding, up to 2^-9 of it, leaves room in the 1e-2
    tolerance.)"""
    say(f"[case] held results fill the area: {kind}")
    rng = np.random.default_rng(2024)
    own = rng.integers(17, 48, size=1500)
    kw = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, q_dtype="bf16", kv_dtype="bf16",
              seed=2024, block_size=16)
    if kind == "hint":
        w = workloads._independent("many-short-bf16", 0, own, 1.25, **kw)
    else:
        w = workloads._shared_prefix("many-short-prefix-bf16", 0, 64, own, 1.25, **kw)
    w.shuffle_seeds = [2024 * 7919 + 1]
    inp = Inputs(w)
    a = GpuStep(w, 0, inp, partition=BAL, kernel=pa.KERNEL_MFMA)
    b = GpuStep(w, 0, inp, partition=BAL, kernel=pa.KERNEL_MFMA)
    plan = _hint_only_plan(a, 0) if kind == "hint" else a.plan()
    if kind == "rows":
        assert plan[1] == 1
    a.append_prefill()
    b.append_prefill()
    a.append_step()
    ref = a.decode(seq_shared=None if kind == "hint" else plan).clone()
    got = b.decode_append(seq_shared=plan).clone()
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    assert torch.equal(a.k_cache.view(torch.uint8), b.k_cache.view(torch.uint8))
    assert torch.equal(a.v_cache.view(torch.uint8), b.v_cache.view(torch.uint8))
    err = check_close(to_f64(got), OracleStep(w, 0, inp).decode(), w.kv_dtype, w.q_dtype)
    say(f"[ok] every row err={err:.3g}")


@pytest.mark.parametrize("size", ["small", "full"])
def test_prefix_rows_match_oracle(size):
    """Config 4 with prefix rows: the appending decode matches the oracle on
    every row and writes the same cache bytes as the two-call path; pa_decode
    with the plan and without it (each sequence reading the prompt itself)
    both match the oracle, and their difference is recorded."""
    say(f"[case] prefix rows cfg4 {size}")
    w = workloads.config(4, size)
    inp = Inputs(w)
    a = GpuStep(w, 0, inp, partition=BAL, kernel=pa.KERNEL_MFMA)
    b = GpuStep(w, 0, inp, partition=BAL, kernel=pa.KERNEL_MFMA)
    plan = a.plan()
    a.append_prefill()
    b.append_prefill()
    a.append_step()
    dup = a.decode().clone()                     # no plan: every sequence reads the prompt
    rows = a.decode(out=torch.empty_like(dup), seq_shared=plan).clone()
    fused = b.decode_append(seq_shared=plan).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.k_cache.view(torch.uint8), b.k_cache.view(torch.uint8))
    assert torch.equal(a.v_cache.view(torch.uint8), b.v_cache.view(torch.uint8))
    assert torch.equal(rows, fused)
    o = OracleStep(w, 0, inp)
    ref = o.decode()
    e_rows = check_close(to_f64(rows), ref, w.kv_dtype, w.q_dtype)
    e_dup = check_close(to_f64(dup), ref, w.kv_dtype, w.q_dtype)
    diff = float((rows.float() - dup.float()).abs().max())
    say(f"[ok] rows err={e_rows:.3g} per-sequence err={e_dup:.3g} |rows - per-seq|={diff:.3g}")
    assert diff <= 1e-2


@pytest.mark.parametrize("size", ["small", "full"])
def test_prefix_rows_bits_do_not_depend_on_placement(size):
    """The same batch in a pool with another block permutation: the split and
    the plan depend on lengths and sharing only, so every bit repeats."""
    say(f"[case] prefix rows placement {size}")
    w = workloads.config(4, size)
    w2 = dataclasses.replace(w)
    w2.shuffle_seeds = [s + 12345 for s in w.shuffle_seeds]
    inp = Inputs(w)
    outs = []
    for ww in (w, w2):
        g = GpuStep(ww, 0, inp, partition=BAL, kernel=pa.KERNEL_MFMA)
        g.append_prefill()
        outs.append((g.decode_append(seq_shared=g.plan()).clone(), g.tables.copy()))
    torch.cuda.synchronize()
    assert not np.array_equal(outs[0][1], outs[1][1])
    assert torch.equal(outs[0][0], outs[1][0])


def test_prefix_rows_two_phase_bits():
    """pa_decode_partials then pa_decode_merge, given the plan, give
    pa_decode's bits with it (config 4 at full size)."""
    say("[case] prefix rows two-phase")
    w = workloads.config(4)
    inp = Inputs(w)
    g = GpuStep(w, 0, inp, partition=BAL, kernel=pa.KERNEL_MFMA)
    g.append_prefill()
    g.append_step()
    plan = g.plan()
    one = g.decode(seq_shared=plan).clone()
    two = torch.full_like(one, 7.0)
    dplan = torch.from_numpy(plan).cuda()
    pa.pa_decode_partials(inp.q, g.k_cache, g.v_cache, g.d_tables, g.d_lens, w.max_seq_len(),
                          w.scale, two, g.desc, g.workspace, BAL, inp.k_scale, inp.v_scale,
                          seq_shared=dplan)
    pa.pa_decode_merge(g.d_lens, g.d_tables.shape[1], w.max_seq_len(), two, g.desc, g.workspace,
                       BAL, seq_shared=dplan)
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), two.view(torch.int16))


def test_shared_vs_duplicated_blocks():
    """Config 4 (small) with the prompt's blocks copied per sequence into
    blocks of their own: nothing is shared, so the plan has no groups and
    every sequence reads its copy.  Both that decode and the shared one with
    prefix rows match the oracle (which gives the two identical results), and
    lie within the tolerance of each other."""
    say("[case] shared vs duplicated")
    w = workloads.config(4, "small")
    inp = Inputs(w)
    g = GpuStep(w, 0, inp, partition=BAL, kernel=pa.KERNEL_MFMA)
    g.append_prefill()
    g.append_step()
    shared = g.decode(seq_shared=g.plan()).clone()

    B, P = len(g.dec), 64 // w.block_size
    per_block = w.num_kv_heads * w.block_size * w.head_dim
    nb2 = w.num_blocks + B * P
    kc = torch.empty(nb2 * per_block, dtype=g.k_cache.dtype, device="cuda")
    vc = torch.empty_like(kc)
    kc[:w.num_blocks * per_block] = g.k_cache
    vc[:w.num_blocks * per_block] = g.v_cache
    tables = g.tables.copy()
    for b in range(B):
        for j in range(P):
            src, dst = int(tables[b, j]), w.num_blocks + b * P + j
            kc[dst * per_block:(dst + 1) * per_block] = g.k_cache[src * per_block:
                                                                  (src + 1) * per_block]
            vc[dst * per_block:(dst + 1) * per_block] = g.v_cache[src * per_block:
                                                                  (src + 1) * per_block]
            tables[b, j] = dst
    assert len(np.unique(tables[:, :P])) == B * P
    desc2 = pa.kv_desc(w.num_q_heads, w.num_kv_heads, w.head_dim, nb2, w.q_dtype, w.kv_dtype,
                       block_size=w.block_size, kernel=pa.KERNEL_MFMA)
    ws = torch.empty(pa.pa_decode_workspace_bytes(desc2, B, w.max_seq_len(), BAL),
                     dtype=torch.uint8, device="cuda")
    dup = torch.empty_like(shared)
    pa.pa_decode(inp.q, kc, vc, torch.from_numpy(tables).cuda(), g.d_lens, w.max_seq_len(),
                 w.scale, dup, desc2, inp.k_scale, inp.v_scale, workspace=ws,
                 partition_size=BAL)
    torch.cuda.synchronize()
    ref = OracleStep(w, 0, inp).decode()
    e_s = check_close(to_f64(shared), ref, w.kv_dtype, w.q_dtype)
    e_d = check_close(to_f64(dup), ref, w.kv_dtype, w.q_dtype)
    diff = float((shared.float() - dup.float()).abs().max())
    say(f"[ok] shared err={e_s:.3g} duplicated err={e_d:.3g} |diff|={diff:.3g}")
    assert diff <= 1e-2


@pytest.mark.parametrize("hq,hkv,kv,bs", [
    (32, 8, "bf16", 16),     # G = 4: 16 members a row
    (64, 8, "e4m3", 16),     # G = 8, FP8 KV: 8 members a row
    (32, 2, "bf16", 16),     # G = 16: 4 members a row
    (16, 8, "f16", 32),      # G = 2: 32 members a row; two tiles a block
])
def test_prefix_rows_shapes(hq, hkv, kv, bs):
    """Three prompts (96, 288 and 32 tokens) forked 20, 9 and 5 times; one
    child of the first grows 32 tokens and is forked 4 times more (its
    children share 2 more blocks than their group does), 6 loners; then each
    goes on with a suffix of its own.  Every row of the appending decode with
    prefix rows matches the oracle.  (Forks at block boundaries only: a fork
    inside a block would need the copy-on-write copy this harness does not
    run.)"""
    say(f"[case] prefix rows shape Hq={hq} Hkv={hkv} kv={kv} bs={bs}")
    rng = np.random.default_rng(hq * 100 + hkv)
    ops = []
    dec = []
    n = 0

    def new_seq(op):
        nonlocal n
        ops.append(op)
        n += 1
        return n - 1

    for prompt, count in ((96, 20), (288, 9), (32, 5)):
        parent = new_seq(("create",))
        ops.append(("prefill", parent, prompt))
        kids = [new_seq(("fork", parent)) for _ in range(count)]
        dec += kids
        if prompt == 96:
            ops.append(("prefill", kids[0], 32))
            dec += [new_seq(("fork", kids[0])) for _ in range(4)]
        ops.append(("free", parent))
    shared_members = list(dec)
    for _ in range(6):
        s = new_seq(("create",))
        ops.append(("prefill", s, int(rng.integers(1, 200))))
        dec.append(s)
    for s in shared_members:
        k = int(rng.integers(0, 90))
        if k:
            ops.append(("prefill", s, k))
    total = sum(o[2] for o in ops if o[0] == "prefill")
    nblocks = 2 * (total // bs + 2 * len(dec) + 16)
    w = workloads.Workload(name="prefix-shapes", config_id=4, num_blocks=nblocks, ops=ops,
                           decode_seqs=dec, num_q_heads=hq, num_kv_heads=hkv, head_dim=128,
                           q_dtype="f16" if kv == "f16" else "bf16", kv_dtype=kv,
                           seed=hq * 7 + hkv, block_size=bs)
    w.shuffle_seeds = [hq * 31 + hkv + 1]
    inp = Inputs(w)
    g = GpuStep(w, 0, inp, partition=BAL, kernel=pa.KERNEL_MFMA)
    plan = g.plan()
    B = len(dec)
    assert plan[1] == 3, plan[1]
    assert list(plan[2 + 4 * B:2 + 4 * B + 3]) == [24, 9, 5]
    assert list(plan[2 + 5 * B:2 + 5 * B + 3]) == [96 // bs, 288 // bs, 32 // bs]
    g.append_prefill()
    got = g.decode_append(seq_shared=plan).clone()
    torch.cuda.synchronize()
    err = check_close(to_f64(got), OracleStep(w, 0, inp).decode(), w.kv_dtype, w.q_dtype)
    say(f"[ok] err={err:.3g}")
