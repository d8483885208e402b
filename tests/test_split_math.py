"""The integer arithmetic of the balanced work split, checked on the CPU.

The decode kernel cuts the T tiles of all (sequence, KV head) segments, in
order, into R = min(T, W) runs [i*T/R, (i+1)*T/R); the merge finds the run of
a tile as ((x + 1) * R - 1) // T, and a run's partial state for a segment
goes to slot run + segment.  These tests restate those three formulas and
check the properties the kernels rely on: every run is non-empty, the runs
tile [0, T) exactly, run_of_tile inverts the cut, and no two (run, segment)
pairs share a slot.  (The device code is checked end to end by the GPU
parity tests; this pins the arithmetic itself, including sizes no GPU test
reaches.)
"""
import random

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


@pytest.mark.parametrize("seed", range(20))
def test_partial_slots_are_unique(seed):
    rng = random.Random(seed)
    nseg = rng.randint(1, 300)
    seg_tiles = [rng.choice([0, 1, 2, rng.randint(1, 400)]) for _ in range(nseg)]
    T = sum(seg_tiles)
    if T == 0:
        return
    W = rng.choice([1, 7, 256, 3072, T, 2 * T])
    R = runs(T, W)
    used = set()
    start = 0
    for s, n in enumerate(seg_tiles):
        if n == 0:
            continue
        i0, i1 = run_of_tile(start, T, R), run_of_tile(start + n - 1, T, R)
        if i0 != i1:  # split segment: runs i0..i1 each leave a partial state
            for i in range(i0, i1 + 1):
                slot = i + s
                assert slot not in used
                assert slot < R + nseg  # within the workspace's W + B*Hkv slots
                used.add(slot)
        start += n
