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
the work split, the run placement, the slot arithmetic and the token store to
stay inside their buffers for shapes the GPU tests do not reach, such as a
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


def _case(path, B, H, G, W, max_len, seed):
    """Seeded lengths (zero and one-token sequences included) and tables that
    place every sequence's blocks at random in a pool with spare blocks."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, max_len + 1, size=B).astype(np.int32)
    lens[0] = 0
    lens[-1] = 1
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
        if lens[b] > 0:
            t = lens[b] - 1
            slots[b] = tables[b, t // 16] * 16 + t % 16
    with open(path, "wb") as f:
        f.write(np.array([B, maxb, NB, H, G, 128, W, maxb * 16], np.int32).tobytes())
        f.write(lens.tobytes())
        f.write(tables.tobytes())
        f.write(slots.tobytes())


@pytest.mark.parametrize("B,H,G,W,hint", [
    (9, 8, 4, 64, 0),      # W a multiple of 32: the per-XCD run placement
    (9, 8, 4, 64, 40),     # the hint, counts past the tables included
    (70, 2, 2, 60, 0),     # more than 64 sequences; W not a multiple of 32
    (5, 4, 8, 1000, 0),    # more waves than tiles: idle runs
])
def test_kernels_stay_in_bounds(sim, B, H, G, W, hint):
    d, exe = sim
    path = d / f"case_{B}_{H}_{G}_{W}_{hint}.bin"
    _case(path, B, H, G, W, max_len=300, seed=B * 1000 + W)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([str(exe), str(path), str(hint)], capture_output=True, text=True,
                       timeout=600, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "unwritten 0 of" in r.stdout and "NaN 0" in r.stdout
