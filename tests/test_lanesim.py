"""The decode and merge kernels' indexing, run on the CPU.

tests/lanesim/sim_decode.cpp compiles the library's device sources
(decode_mfma.hip, merge.hip and their headers, with the constant address
space removed) for the host, with every lane a thread, under AddressSanitizer
and UndefinedBehaviorSanitizer.  It runs the balanced decode kernel with the
append folded in, with and without the shared-block hint, then the segment
merge, on seeded tables, and checks that every output element is written
and that the merge reads only slots the decode runs wrote (the workspace
starts as NaN).
The arithmetic is not checked here (the GPU parity tests do that): this pins
the work split, the run placement, the slot arithmetic, the token store and
the LDS area that holds a run's results to stay inside their buffers for shapes the GPU tests do not reach, such as a
wave count that is not a multiple of 32.
"""
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_255_amd", "csrc")
SIM = os.path.join(ROOT, "tests", "lanesim")
CLANG = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang++")


@pytest.fixture(scope="module")
def sim(tmp_path_factory):
    if not os.path.exists(CLANG):
        pytest.skip("no ROCm clang++ to build the lane simulator")
    d = tmp_path_factory.mktemp("lanesim")
    src = d / "src"
    src.mkdir()
    for f in ("device.hpp", "work.hpp", "merge.hip", "decode_mfma.hip", "append.hpp"):
        text = open(os.path.join(CSRC, f)).read()
        for space in (1, 3, 4):
            text = text.replace(f"__attribute__((address_space({space})))", "")
        (src / f).write_text(text)
    exe = d / "sim"
    subprocess.check_call([CLANG, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                           "-I", SIM, "-I", str(src), "-I", os.path.join(ROOT, "include"),
                           "-x", "c++", os.path.join(SIM, "sim_decode.cpp"), "-o", str(exe),
                           "-lpthread"])
    return d, exe


def _plan(tables, lens, bs=16):
    """A share plan in the layout pa.h gives: groups of two or more sequences
    whose tables begin with the same block, sharing the longest run of
    leading entries they hold alike before each member's last token."""
    B, maxb = tables.shape
    plan = np.zeros(2 + 8 * B, np.int32)
    plan[0] = 0x31534150
    nblk = [-(-int(n) // bs) for n in lens]
    for b in range(B):  # the cache-policy hint: entries another table holds
        others = {int(x) for c in range(B) if c != b for x in tables[c, :nblk[c]]}
        k = 0
        while k < nblk[b] and int(tables[b, k]) in others:
            k += 1
        plan[2 + b] = k
    plan[2 + B:2 + 2 * B] = -1
    keys = {}
    for b in range(B):
        if lens[b] > bs and plan[2 + b] >= 1:
            keys.setdefault(int(tables[b, 0]), []).append(b)
    ng = placed = 0
    for members in keys.values():
        if len(members) < 2:
            continue
        k = min((int(lens[b]) - 1) // bs for b in members)
        j = 0
        while j < k and all(tables[b, j] == tables[members[0], j] for b in members):
            j += 1
        if j == 0:
            continue
        plan[2 + 4 * B + ng] = len(members)
        plan[2 + 5 * B + ng] = j
        plan[2 + 7 * B + ng] = placed
        for r, b in enumerate(members):
            plan[2 + B + b] = ng
            plan[2 + 2 * B + b] = r
            plan[2 + 3 * B + b] = j
            plan[2 + 6 * B + placed] = b
            placed += 1
        ng += 1
    plan[1] = ng
    return plan


def _case(path, B, H, G, W, max_len, seed, groups=(), plan_kind="real"):
    """Seeded lengths (zero and one-token sequences included) and tables that
    place every sequence's blocks at random in a pool with spare blocks.
    groups: (first, count, blocks) runs of sequences whose tables begin with
    the same `blocks` blocks (their lengths past them).  plan_kind: "real"
    (the plan of those tables), "hint" (cache-policy counts only, some past
    the tables, no groups) or "garbage" (every word but the magic random)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, max_len + 1, size=B).astype(np.int32)
    lens[0] = 0
    lens[-1] = 1
    for first, count, blocks in groups:
        lens[first:first + count] = np.maximum(lens[first:first + count], blocks * 16 + 1)
    nblk = [-(-int(n) // 16) for n in lens]
    maxb = max(max(nblk), 1)
    NB = sum(nblk) + 7
    perm = rng.permutation(NB).astype(np.int32)
    tables = np.full((B, maxb), -1, np.int32)
    slots = np.full(B, -1, np.int32)
    pos = 0
    for b, k in enumerate(nblk):
        tables[b, :k] = perm[pos:pos + k]
        pos += k
    for first, count, blocks in groups:
        tables[first + 1:first + count, :blocks] = tables[first, :blocks]
    for b in range(B):
        if lens[b] > 0:
            t = lens[b] - 1
            slots[b] = tables[b, t // 16] * 16 + t % 16
    if plan_kind == "garbage":
        plan = rng.integers(-5, B + 6, size=2 + 8 * B).astype(np.int32)
        plan[0] = 0x31534150
        plan[1] = rng.integers(0, B // 2 + 1)
    else:
        plan = _plan(tables, lens)
        if plan_kind == "hint":
            plan[1] = 0
            plan[2:2 + B] = [(i * 37) % 41 for i in range(B)]
    with open(path, "wb") as f:
        f.write(np.array([B, maxb, NB, H, G, 128, W, maxb * 16], np.int32).tobytes())
        f.write(lens.tobytes())
        f.write(tables.tobytes())
        f.write(slots.tobytes())
        f.write(plan.tobytes())
    return plan


def _run(exe, path, mode, stage=None):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1")
    args = [str(exe), str(path), str(mode)] + ([] if stage is None else [str(stage)])
    return subprocess.run(args, capture_output=True, text=True, timeout=900, env=env)


@pytest.mark.parametrize("B,H,G,W,mode", [
    (9, 8, 4, 64, 0),      # W a multiple of 32: the per-XCD run placement
    (9, 8, 4, 64, 1),      # the hint, counts past the tables included
    (70, 2, 2, 60, 0),     # more than 64 sequences; W not a multiple of 32
    (5, 4, 8, 1000, 0),    # more waves than tiles: idle runs
])
def test_kernels_stay_in_bounds(sim, B, H, G, W, mode):
    d, exe = sim
    path = d / f"case_{B}_{H}_{G}_{W}_{mode}.bin"
    _case(path, B, H, G, W, max_len=300, seed=B * 1000 + W,
          plan_kind="hint" if mode else "real")
    r = _run(exe, path, mode)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "unwritten 0 of" in r.stdout and "NaN 0" in r.stdout


@pytest.mark.parametrize("stage", [
    0,      # every result stored at once
    2352,   # room for one partial state and its records: stored often before the end
    1200,   # an acc image does not fit: stored at once beside held m, l and records
])
@pytest.mark.parametrize("mode", [1, 2])
def test_held_results_are_all_stored(sim, stage, mode):
    """With a share plan, a run's outputs, partial states, segment records
    and appended tokens go through the wave's LDS area until the run ends (or
    until it is full): with areas too small for some records and too small
    for more than one piece, every output is still written, the merge still
    reads only written slots, and every store (the token's scattered V
    values included) stays inside its buffer."""
    d, exe = sim
    path = d / f"stage_{stage}_{mode}.bin"
    groups = ((1, 20, 5), (21, 10, 3)) if mode == 2 else ()
    _case(path, 40, 2, 4, 64, max_len=300, seed=40 * 7 + 64, groups=groups,
          plan_kind="real" if mode == 2 else "hint")
    r = _run(exe, path, mode, stage)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "unwritten 0 of" in r.stdout and "NaN 0" in r.stdout


@pytest.mark.parametrize("B,H,G,W,groups,rows", [
    # two groups, one cut into two rows (SPR = 16 at G = 4), and loners;
    # 8 runs per XCD: 4 to the rows, 4 to the sequences
    (40, 2, 4, 64, ((1, 20, 5), (21, 10, 3)), True),
    # more than 64 sequences, G = 8 (8 members a row)
    (70, 2, 8, 96, ((0, 30, 4), (40, 12, 2)), True),
    # a group whose shared blocks are most of each member; more waves than units
    (12, 2, 16, 512, ((0, 12, 12),), True),
    # W not a multiple of 32: no rows, the plan only hints (the merge takes
    # the plan's branch all the same)
    (70, 2, 8, 60, ((0, 30, 4), (40, 12, 2)), False),
    # more than 256 sequences: the split's lookups loop over the tables
    (300, 2, 4, 64, ((3, 100, 3), (150, 40, 2)), True),
    # more than 64 groups: the same
    (140, 1, 4, 64, tuple((2 * i, 2, 1 + i % 3) for i in range(66)), True),
])
def test_prefix_rows_stay_in_bounds(sim, B, H, G, W, groups, rows):
    """Prefix rows in the balanced split: every piece of a row and of the
    members' own tiles stays in its buffers, every output is written, and
    the merge reads only slots some run wrote."""
    d, exe = sim
    path = d / f"prefix_{B}_{H}_{G}_{W}.bin"
    plan = _case(path, B, H, G, W, max_len=300, seed=B * 7 + W, groups=groups)
    assert plan[1] == len(groups)
    r = _run(exe, path, 2)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "unwritten 0 of" in r.stdout and "NaN 0" in r.stdout
    # with rows, every member of every group has a slot per row piece, on
    # every head
    members = sum(c for _, c, _ in groups)
    written = int(r.stdout.split("row slots")[1])
    if rows:
        assert written >= members * H, r.stdout
    else:
        assert written == 0, r.stdout


@pytest.mark.parametrize("seed", [1, 2])
def test_garbage_plan_stays_in_bounds(sim, seed):
    """A plan that does not belong to the tables gives unspecified outputs,
    but no access outside the buffers (AddressSanitizer would stop the run)."""
    d, exe = sim
    path = d / f"garbage_{seed}.bin"
    _case(path, 40, 2, 4, 64, max_len=300, seed=seed, groups=((0, 20, 5),),
          plan_kind="garbage")
    r = _run(exe, path, 2)
    assert r.returncode in (0, 3), (r.stdout + r.stderr)[-3000:]
    assert "unwritten 0 of" in r.stdout, r.stdout


@pytest.fixture(scope="module")
def sim_append(tmp_path_factory):
    if not os.path.exists(CLANG):
        pytest.skip("no ROCm clang++ to build the lane simulator")
    d = tmp_path_factory.mktemp("lanesim_append")
    src = d / "src"
    src.mkdir()
    for f in ("device.hpp", "append.hpp", "append.hip"):
        text = open(os.path.join(CSRC, f)).read()
        for space in (1, 3, 4):
            text = text.replace(f"__attribute__((address_space({space})))", "")
        (src / f).write_text(text)
    exe = d / "sim_append"
    subprocess.check_call([CLANG, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                           "-I", SIM, "-I", str(src), "-I", os.path.join(ROOT, "include"),
                           "-x", "c++", os.path.join(SIM, "sim_append.cpp"), "-o", str(exe),
                           "-lpthread"])
    return d, exe


def _prefill_slots(lens, held, tile_shift, seed, spoil=0):
    """Slots of one append call that writes lens[i] tokens to sequence i,
    which already holds held[i] tokens, the sequences' blocks placed at
    random in a pool with spare blocks; `spoil` entries are then set to -1 or
    past the pool (skipped by the kernels)."""
    rng = np.random.default_rng(seed)
    bs = 16 << tile_shift
    need = [-(-(h + n) // bs) for h, n in zip(held, lens)]
    NB = sum(need) + 5
    perm = rng.permutation(NB)
    slots, pos = [], 0
    for h, n, k in zip(held, lens, need):
        blocks = perm[pos:pos + k]
        pos += k
        slots += [int(blocks[t // bs]) * bs + t % bs for t in range(h, h + n)]
    slots = np.array(slots, np.int32)
    for i in rng.choice(len(slots), size=spoil, replace=False):
        slots[i] = -1 if rng.random() < 0.5 else NB * bs + int(rng.integers(0, 50))
    return slots, NB


@pytest.mark.parametrize("kv,tile_shift,case", [
    (0, 0, "fresh"), (0, 0, "continued"), (0, 1, "spoiled"),
    (1, 1, "fresh"), (1, 0, "continued"), (0, 0, "step"), (1, 1, "step"),
])
def test_tile_append_matches_token_append(sim_append, kv, tile_shift, case):
    """The whole-tile append writes exactly the bytes of the per-token one:
    ragged sequences, so complete tiles start at any place in the token
    array and cross 16-entry windows; sequences that continue mid-tile (their
    first tile is partial and goes token by token); entries skipped for a
    slot outside the pool, which break the tile they fall in; a decode step
    (one token for each of 70 sequences: no complete tile, every entry
    written on its own)."""
    d, exe = sim_append
    if case == "step":
        rng = np.random.default_rng(7 + kv)
        lens = [1] * 70
        held = [int(h) for h in rng.integers(0, 300, size=70)]
    else:
        lens = [17, 70, 3, 64, 33, 20]
        held = [0] * len(lens) if case != "continued" else [5, 16, 31, 7, 0, 12]
    slots, NB = _prefill_slots(lens, held, tile_shift, seed=tile_shift * 10 + kv,
                               spoil=5 if case == "spoiled" else 0)
    path = d / f"app_{kv}_{tile_shift}_{case}.bin"
    with open(path, "wb") as f:
        f.write(np.array([len(slots), 2, NB, tile_shift, kv], np.int32).tobytes())
        f.write(slots.tobytes())
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([str(exe), str(path)], capture_output=True, text=True, timeout=900, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "differing 0 " in r.stdout
