"""The integer arithmetic of the balanced work split, checked on the CPU.

The decode kernel cuts the T tiles of all (sequence, KV head) segments, in
order, into R = min(T, W) runs [i*T/R, (i+1)*T/R); each segment is charged
seg_cost virtual tiles before its real ones (kSegmentCostShared in a launch
that reads prefix rows, kSegmentCost in any other) (a wave that starts a new
segment inside its run pays a pipeline restart).  The merge finds the run of
a tile as ((x + 1) * R - 1) // T, and a run's partial state for a segment
goes to slot run + segment.  These tests restate those formulas and check the
properties the kernels rely on: every run is non-empty, the runs tile [0, T)
exactly, run_of_tile inverts the cut, the runs the decode gives a piece of a
segment are exactly the ones the merge reads, every real tile is decoded
once, and no two (run, segment) pairs share a slot.  (The device code is
checked end to end by the GPU parity tests; this pins the arithmetic itself,
including sizes no GPU test reaches.)
"""
import os
import random
import re

import pytest


def runs(T, W):
    return min(T, W)


def run_bounds(i, T, R):
    return i * T // R, (i + 1) * T // R


def run_of_tile(x, T, R):
    return ((x + 1) * R - 1) // T


@pytest.mark.parametrize("T,W", [(1, 1), (1, 3072), (7, 3), (3072, 3072), (3073, 3072),
                                 (43_712, 3072), (262_144, 3072), (10**9 + 7, 3072),
                                 (5, 2048), (2**31 - 1, 1 << 20)])
def test_runs_tile_the_range_and_invert(T, W):
    R = runs(T, W)
    assert 1 <= R <= T
    rng = random.Random(T * 31 + W)
    idx = {0, R - 1, R // 2} | {rng.randrange(R) for _ in range(200)}
    for i in sorted(idx):
        x0, x1 = run_bounds(i, T, R)
        assert x1 > x0, "empty run"
        if i > 0:
            assert run_bounds(i - 1, T, R)[1] == x0, "runs not adjacent"
        for x in {x0, x1 - 1, (x0 + x1) // 2}:
            assert run_of_tile(x, T, R) == i
    assert run_bounds(0, T, R)[0] == 0 and run_bounds(R - 1, T, R)[1] == T


def test_run_of_tile_exhaustive_small():
    for T in range(1, 120):
        for W in (1, 2, 3, 5, 8, 64, 200):
            R = runs(T, W)
            owner = []
            for i in range(R):
                x0, x1 = run_bounds(i, T, R)
                owner += [i] * (x1 - x0)
            assert len(owner) == T
            assert [run_of_tile(x, T, R) for x in range(T)] == owner


def _segment_costs():
    """kSegmentCost and kSegmentCostShared as work.hpp defines them (read
    from the header, so the model below cannot drift from the kernels)."""
    here = os.path.dirname(os.path.abspath(__file__))
    text = open(os.path.join(here, "..", "paged_kv_cache_255_amd", "csrc", "work.hpp")).read()
    return [int(re.search(r"constexpr int32_t %s = (\d+);" % name, text).group(1))
            for name in ("kSegmentCost", "kSegmentCostShared")]


SEGMENT_COSTS = _segment_costs()


def test_segment_costs_are_positive():
    assert all(c > 0 for c in SEGMENT_COSTS)


@pytest.mark.parametrize("SEGMENT_COST", SEGMENT_COSTS)
@pytest.mark.parametrize("seed", range(40))
def test_decode_pieces_match_merge_parts(seed, SEGMENT_COST):
    """The decode's walk (a run's virtual tiles meet each segment's start
    charge, then its real tiles) against the merge's run bounds."""
    rng = random.Random(seed)
    nseg = rng.randint(1, 300)
    real = [rng.choice([0, 1, 2, rng.randint(1, 400)]) for _ in range(nseg)]
    virt = [n + SEGMENT_COST if n > 0 else 0 for n in real]
    T = sum(virt)
    if T == 0:
        return
    W = rng.choice([1, 7, 256, 1024, 3072, T, 2 * T])
    R = runs(T, W)
    starts = [sum(virt[:s]) for s in range(nseg)]
    # decode side: run i walks [x0, x1)
    pieces = {}  # segment -> list of (run, j, je)
    for i in range(R):
        x0, x1 = run_bounds(i, T, R)
        s = next(k for k in range(nseg) if starts[k] + virt[k] > x0)  # segment holding x0
        x = x0
        while x < x1:
            r0 = starts[s] + SEGMENT_COST
            lo, hi = max(x, r0), min(x1, r0 + real[s])
            if hi > lo:
                pieces.setdefault(s, []).append((i, lo - r0, hi - r0))
            x = r0 + real[s]
            if x < x1:
                s = next(k for k in range(s + 1, nseg) if virt[k] > 0)
    used = set()
    for s in range(nseg):
        if real[s] == 0:
            assert s not in pieces
            continue
        got = pieces[s]
        # every real tile once, in order
        assert got[0][1] == 0 and got[-1][2] == real[s]
        assert all(got[k][2] == got[k + 1][1] for k in range(len(got) - 1))
        # merge side
        S0 = starts[s] + SEGMENT_COST
        i0, i1 = run_of_tile(S0, T, R), run_of_tile(S0 + real[s] - 1, T, R)
        assert [p[0] for p in got] == list(range(i0, i1 + 1))
        # one run holds it all exactly when the merge finds i0 == i1
        assert (len(got) == 1) == (i0 == i1)
        if i0 != i1:
            for i in range(i0, i1 + 1):
                slot = i + s
                assert slot not in used
                assert slot < R + nseg  # within the workspace's W + B*Hkv slots
                used.add(slot)
