"""Inputs that make the decode kernels' online softmax rescale its running
state by a factor strictly between 0 and 1, and a CPU model of the kernels'
per-range update used to show that these inputs catch a rescale left out.

With N(0,1) data and scale 1/sqrt(d), a tile's scores never exceed the
running max by many units after the first tile, so the rescale of a lazy
online softmax (the running max moves only when a tile's max beats it by
more than a threshold) only ever runs with a factor of exactly 0.  Here the
scores are planted instead: q puts a fixed weight c_h on dimension 0 (plus
small noise), and dimension 0 of each K row picks the token's level:

    base    K0 ~ 0.5 N(0,1)     score ~ 0            V ~ N(0,1)
    L1      K0 = 16             score ~ 16 c_h/8     V = 1 + (d % 4) / 4
    L2      K0 = 26             score ~ 26 c_h/8     V = -(1 + (d % 3) / 2)
    L3      K0 = 36             score ~ 36 c_h/8     V = 0.5 + (d % 2) / 4

(scores in log2 units; c_h = 8, 7, 9, 6 for the four heads of a group, so the
steps between levels are 10.2, 8.9, 11.5 and 7.7 units: three heads rescale,
the fourth accumulates weights up to 2^7.7 without one).  Every planted value
is exact in bf16, fp16 and E4M3 at scale 1.

Sequences (lengths at decode; the last token is the step's appended one):
  0  L1 plateau from tile 1, one L2 token in tile ts0, base after it;
     ts0 is the last tile of a 512-token partition (so also of a 64-token
     one) and not the first tile of its balanced run for either KV head;
  1  the same with ts1 the last tile of a balanced run for KV head 0;
  2  the reverse: one L2 token in tile 1, then the L1 plateau, the appended
     token L1 too (later tiles sit below the running max);
  3  L1 plateau, one L2 token mid-sequence, and the appended token at L3: the
     rescale happens in the sequence's last tile, the one the appending
     decode patches in registers.
The plateau is thousands of tokens long, so the running sum a rescale
multiplies is large: a rescale left out changes the output by O(1).

No arithmetic of the method lives here except in `lazy_model`, which restates
the kernels' update (not the oracle's) to show the inputs' sensitivity.
"""
import math

import numpy as np

HKV, G, D = 2, 4, 128
HQ = HKV * G
COEF = (8.0, 7.0, 9.0, 6.0)
K_LEVEL = {"L1": 16.0, "L2": 26.0, "L3": 36.0}
LENS = (40007, 30011, 25003, 33013)  # tokens at decode, appended token included
TILE = 16
LAZY = 8.0  # the kernels' rescale threshold, log2 units


def v_level(level):
    d = np.arange(D)
    if level == "L1":
        return 1.0 + (d % 4) * 0.25
    if level == "L2":
        return -(1.0 + (d % 3) * 0.5)
    return 0.5 + (d % 2) * 0.25


def tiles(n):
    return -(-n // TILE)


def balanced_runs(lens, W):
    """(T, R, Th, seg_start(g, b)) of the balanced split: head-major segments,
    R = min(T, W) runs of tiles [i T / R, (i + 1) T / R)."""
    Th = sum(tiles(n) for n in lens)
    T = Th * HKV
    R = min(T, W)
    before = np.concatenate([[0], np.cumsum([tiles(n) for n in lens])])

    def seg_start(g, b):
        return g * Th + int(before[b])
    return T, R, Th, seg_start


def run_of(x, T, R):
    return ((x + 1) * R - 1) // T


def is_run_first(x, T, R):
    return x == run_of(x, T, R) * T // R


def is_run_last(x, T, R):
    return x + 1 == (run_of(x, T, R) + 1) * T // R


def spike_tiles(W):
    """Tiles holding the L2 token of sequences 0, 1 and 3 for a balanced split
    over W runs (see the module docstring)."""
    T, R, _, seg = balanced_runs(LENS, W)
    mid0 = tiles(LENS[0]) // 2
    ts0 = mid0 - mid0 % 32 + 31
    while any(is_run_first(seg(g, 0) + ts0, T, R) for g in range(HKV)):
        ts0 += 32
    ts1 = tiles(LENS[1]) // 2
    while not (is_run_last(seg(0, 1) + ts1, T, R) and
               not is_run_first(seg(1, 1) + ts1, T, R)):
        ts1 += 1
    ts3 = tiles(LENS[3]) // 2 + 5
    return ts0, ts1, ts3


def layout(W):
    """Per sequence, the level of every token ("base", "L1", "L2", "L3")."""
    ts0, ts1, ts3 = spike_tiles(W)
    out = []
    for b, n in enumerate(LENS):
        lv = np.array(["base"] * n, dtype=object)
        if b in (0, 1):
            ts = ts0 if b == 0 else ts1
            lv[TILE:TILE * ts] = "L1"
            lv[TILE * ts + 5] = "L2"
        elif b == 2:
            lv[20] = "L2"
            lv[21:] = "L1"
        else:
            lv[TILE:] = "L1"
            lv[TILE * ts3 + 9] = "L2"
            lv[n - 1] = "L3"
        out.append(lv)
    return out


def build(W, seed=77):
    """Float32 values (exact in every 16-bit dtype and in E4M3 where planted):
    k_pre, v_pre [sum(n - 1)][HKV][D] in sequence order, k_new, v_new
    [B][HKV][D] (each sequence's last token), q [B][HQ][D], and the levels."""
    rng = np.random.default_rng(seed)
    lv = layout(W)
    ks, vs = [], []
    for b, n in enumerate(LENS):
        K = (rng.standard_normal((n, HKV, D)) * np.float32(1.0)).astype(np.float32)
        V = rng.standard_normal((n, HKV, D)).astype(np.float32)
        K[:, :, 0] = (rng.standard_normal((n, HKV)) * 0.5).astype(np.float32)
        for name in ("L1", "L2", "L3"):
            sel = lv[b] == name
            K[sel, :, 0] = K_LEVEL[name]
            V[sel, :, :] = v_level(name)[None, None, :]
        ks.append(K)
        vs.append(V)
    k_pre = np.concatenate([K[:-1] for K in ks])
    v_pre = np.concatenate([V[:-1] for V in vs])
    k_new = np.stack([K[-1] for K in ks])
    v_new = np.stack([V[-1] for V in vs])
    q = (rng.standard_normal((len(LENS), HQ, D)) * 0.02).astype(np.float32)
    for h in range(HQ):
        q[:, h, 0] = COEF[h % G]
    return dict(k_pre=k_pre, v_pre=v_pre, k_new=k_new, v_new=v_new, q=q, levels=lv)


def ranges(mode, n, g, b, W):
    """Token ranges [t0, t1) of segment (KV head g, sequence b) that the
    decode's work items cover in a launch mode: 0 (one item), a partition
    size, or "balanced"."""
    if mode == 0:
        return [(0, n)]
    if mode != "balanced":
        return [(p, min(p + mode, n)) for p in range(0, n, mode)]
    T, R, _, seg = balanced_runs(LENS, W)
    s0, nt = seg(g, b), tiles(n)
    out = []
    x = s0
    while x < s0 + nt:
        i = run_of(x, T, R)
        end = min((i + 1) * T // R, s0 + nt)
        out.append(((x - s0) * TILE, min((end - s0) * TILE, n)))
        x = end
    return out


def lazy_model(q, K, V, rngs, scale, drop_l=False, drop_acc=False):
    """The kernels' per-range update, in fp64, then the exact merge of the
    ranges.  q [G][D]; K, V [n][D] (stored values); rngs: token ranges.
    Per 16-token tile: scores in log2 units; if any head's tile max beats its
    running max by more than LAZY, every head moves its max to
    max(running, tile max) and multiplies its sum and accumulator by
    2^(old - new); then weights 2^(s - max) are added.  drop_l / drop_acc
    leave out one of the two multiplications (the planted mistakes)."""
    c = scale * math.log2(math.e)
    parts = []
    for t0, t1 in rngs:
        m = np.full(G, -3.0e38)
        l = np.zeros(G)
        acc = np.zeros((G, D))
        for a in range(t0, t1, TILE):
            e = min(a + TILE, t1)
            s = (q @ K[a:e].T) * c  # [G][tokens]
            bm = s.max(axis=1)
            if np.any(bm > m + LAZY):
                mn = np.maximum(m, bm)
                alpha = np.exp2(m - mn)
                m = mn
                if not drop_l:
                    l = l * alpha
                if not drop_acc:
                    acc = acc * alpha[:, None]
            p = np.exp2(s - m[:, None])
            l = l + p.sum(axis=1)
            acc = acc + p @ V[a:e]
        parts.append((m, l, acc))
    M = np.max([p[0] for p in parts], axis=0)
    L = sum(np.exp2(p[0] - M) * p[1] for p in parts)
    A = sum(np.exp2(p[0] - M)[:, None] * p[2] for p in parts)
    return A / L[:, None]
