"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against what the pages or the mathematics fix:
brute force on tiny inputs, a library attention routine, closed forms,
invariances, the pages' worked numbers (tests/golden/), and library number
format conversions.  They run on the CPU only.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests import bruteforce
from tests.cases import BS, random_case, random_storage, v_shape

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def run_oracle(c, **over):
    args = dict(num_q_heads=c["Hq"], num_kv_heads=c["Hkv"], head_dim=c["D"], block_size=c["bs"],
                num_blocks=c["NB"], q_dtype=c["q_dtype"], kv_dtype=c["kv_dtype"],
                scale=c["scale"])
    args.update(over)
    return oracle.decode(c["q"], c["k"], c["v"], c["tables"], c["lens"], **args)


def run_brute(c, **over):
    args = dict(num_q_heads=c["Hq"], num_kv_heads=c["Hkv"], head_dim=c["D"], block_size=c["bs"],
                q_dtype=c["q_dtype"], kv_dtype=c["kv_dtype"], scale=c["scale"])
    args.update(over)
    return bruteforce.attention(c["q"], c["k"], c["v"], c["tables"], c["lens"], **args)


# -- attention math ------------------------------------------------------------
@pytest.mark.parametrize("q_dtype,kv_dtype,Hq,Hkv,D", [
    ("f32", "f32", 4, 4, 64),
    ("f32", "f32", 8, 2, 32),
    ("bf16", "bf16", 8, 2, 128),
    ("f16", "f16", 3, 3, 64),
    ("bf16", "e4m3", 8, 1, 64),
    ("f16", "e4m3", 4, 2, 64),
])
def test_oracle_matches_bruteforce(q_dtype, kv_dtype, Hq, Hkv, D):
    for seed in range(3):
        c = random_case(seed, Hq=Hq, Hkv=Hkv, D=D, q_dtype=q_dtype, kv_dtype=kv_dtype, B=4)
        ks, vs = (0.037, 0.021) if kv_dtype == "e4m3" else (1.0, 1.0)
        o = run_oracle(c, k_scale=ks, v_scale=vs)
        r = run_brute(c, k_scale=ks, v_scale=vs)
        np.testing.assert_allclose(o, r, rtol=1e-12, atol=1e-13)


def test_oracle_matches_torch_sdpa():
    """Library routine: scaled_dot_product_attention in fp64 on the gathered
    contiguous K/V, with the KV heads repeated for the query groups."""
    c = random_case(11, B=3, Hq=8, Hkv=2, D=64, q_dtype="f32", kv_dtype="f32")
    o = run_oracle(c)
    G = c["Hq"] // c["Hkv"]
    kv = torch.from_numpy(c["k"]).double()
    vv = torch.from_numpy(bruteforce.v_token_major(c["v"], c["Hkv"], c["D"], BS, 4)).double()
    for b, n in enumerate(c["lens"]):
        n = int(n)
        blocks = c["tables"][b][: -(-n // BS)]
        K = torch.cat([kv[p].permute(1, 0, 2) for p in blocks])[:n]  # [n][Hkv][D]
        V = torch.cat([vv[p].permute(1, 0, 2) for p in blocks])[:n]
        K = K.permute(1, 0, 2).repeat_interleave(G, dim=0)  # [Hq][n][D]
        V = V.permute(1, 0, 2).repeat_interleave(G, dim=0)
        q = torch.from_numpy(c["q"][b]).double()[:, None, :]  # [Hq][1][D]
        ref = torch.nn.functional.scaled_dot_product_attention(q, K, V, scale=c["scale"])
        np.testing.assert_allclose(o[b], ref[:, 0, :].numpy(), rtol=1e-12, atol=1e-13)


def test_single_token_returns_its_value_row():
    """n = 1: the softmax has one weight, 1, so out = v_scale * V_0 exactly."""
    c = random_case(3, B=2, Hq=4, Hkv=2, D=64, lens=[1, 1], q_dtype="bf16", kv_dtype="e4m3")
    o = run_oracle(c, k_scale=0.5, v_scale=0.25)
    vv = bruteforce.v_token_major(bruteforce.decode_storage(c["v"], "e4m3"), 2, 64, BS, 1)
    for b in range(2):
        for h in range(4):
            np.testing.assert_array_equal(o[b, h], vv[c["tables"][b][0], h // 2, 0, :] * 0.25)


def test_zero_query_gives_mean_of_values():
    """q = 0: all scores equal, so out is the plain mean of the V rows."""
    c = random_case(4, B=2, Hq=2, Hkv=2, D=16, lens=[37, 5])
    c["q"][:] = 0.0
    o = run_oracle(c)
    vv = bruteforce.v_token_major(c["v"].astype(np.float64), 2, 16, BS, 4)
    for b, n in enumerate(c["lens"]):
        rows = [vv[c["tables"][b][t // BS], :, t % BS, :] for t in range(n)]
        np.testing.assert_allclose(o[b], np.mean(rows, axis=0), rtol=1e-13, atol=1e-14)


def test_constant_values_and_constant_keys():
    """All V rows equal c => out = c.  All K rows equal => uniform weights."""
    c = random_case(5, B=2, Hq=4, Hkv=1, D=16, lens=[40, 17])
    cvec = np.linspace(-1, 1, 16).astype(np.float32)
    v_const = bruteforce.v_from_token_major(
        np.broadcast_to(cvec, (c["NB"], 1, BS, 16)).astype(np.float32), 4)
    o = run_oracle(dict(c, v=v_const))
    for b in range(2):
        np.testing.assert_allclose(o[b], np.broadcast_to(cvec, (4, 16)), rtol=1e-13, atol=1e-14)
    k_const = np.empty_like(c["k"])
    k_const[:] = 0.3
    o = run_oracle(dict(c, k=k_const))
    vv = bruteforce.v_token_major(c["v"].astype(np.float64), 1, 16, BS, 4)
    for b, n in enumerate(c["lens"]):
        mean = np.mean([vv[c["tables"][b][t // BS], 0, t % BS, :] for t in range(n)], axis=0)
        np.testing.assert_allclose(o[b], np.broadcast_to(mean, (4, 16)), rtol=1e-12, atol=1e-13)


def test_zero_length_gives_zero_row():
    c = random_case(6, B=3, Hq=2, Hkv=2, D=16, lens=[0, 20, 0])
    o = run_oracle(c)
    assert np.all(o[0] == 0) and np.all(o[2] == 0) and np.any(o[1] != 0)


def test_gqa_equals_mha_with_repeated_kv_heads():
    """dev.to §2 Example 2: GQA query heads share one KV head; repeating each
    KV head G times into an MHA cache must not change any output."""
    c = random_case(7, B=3, Hq=8, Hkv=2, D=32, q_dtype="bf16", kv_dtype="bf16")
    o = run_oracle(c)
    G = 4
    k_mha = np.ascontiguousarray(np.repeat(c["k"], G, axis=1))
    v_mha = np.ascontiguousarray(np.repeat(c["v"], G, axis=1))
    o2 = run_oracle(dict(c, k=k_mha, v=v_mha, Hkv=8))
    np.testing.assert_array_equal(o, o2)


def test_block_permutation_invariance():
    """Moving physical blocks and remapping the tables changes nothing, bit for
    bit (dev.to §4: any free block can hold any logical block)."""
    c = random_case(8, B=4, Hq=4, Hkv=2, D=32, q_dtype="f16", kv_dtype="f16", extra_blocks=9)
    o = run_oracle(c)
    perm = np.random.default_rng(99).permutation(c["NB"])  # old id p -> new id perm[p]
    k2 = np.empty_like(c["k"])
    v2 = np.empty_like(c["v"])
    k2[perm] = c["k"]
    v2[perm] = c["v"]
    t2 = np.where(c["tables"] >= 0, perm[np.maximum(c["tables"], 0)], -1).astype(np.int32)
    o2 = run_oracle(dict(c, k=k2, v=v2, tables=t2))
    np.testing.assert_array_equal(o, o2)


def test_shared_prefix_equals_duplicated_blocks():
    """dev.to §5: block tables that point at the same prompt blocks give the
    same result as private copies of those blocks."""
    rng = np.random.default_rng(12)
    Hq, Hkv, D, NB = 4, 2, 32, 20
    k = random_storage(rng, (NB, Hkv, BS, D), "bf16")
    v = random_storage(rng, (NB, Hkv, D, BS), "bf16")
    q = random_storage(rng, (3, Hq, D), "bf16")
    shared = [[0, 1, 5, -1], [0, 1, 6, 7], [0, 1, 8, -1]]
    lens = [40, 60, 33]
    # duplicated: copy blocks 0 and 1 into 10/11 and 12/13 for sequences 1 and 2
    k2, v2 = k.copy(), v.copy()
    for src, dst in [(0, 10), (1, 11), (0, 12), (1, 13)]:
        k2[dst] = k[src]
        v2[dst] = v[src]
    dup = [[0, 1, 5, -1], [10, 11, 6, 7], [12, 13, 8, -1]]
    common = dict(num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=BS, num_blocks=NB,
                  q_dtype="bf16", kv_dtype="bf16", scale=0.125)
    o1 = oracle.decode(q, k, v, np.array(shared), lens, **common)
    o2 = oracle.decode(q, k2, v2, np.array(dup), lens, **common)
    np.testing.assert_array_equal(o1, o2)


def test_page_addressing_example():
    """dev.to §4 figure: logical blocks 0/1/2 (tokens 0-15, 16-31, 32-47) in
    physical blocks 84/12/903.  Token t must be read from block
    table[t // 16] at offset t % 16: a cache whose only finite values sit in
    exactly those slots reproduces contiguous attention over them."""
    ex = _golden("devto_block_table_example.json")
    table = [e["physical"] for e in ex["logical_blocks"]]
    assert ex["block_size"] == BS
    NB, Hkv, D, n = 904, 1, 16, 48
    rng = np.random.default_rng(5)
    Kc = rng.standard_normal((n, D)).astype(np.float32)
    Vc = rng.standard_normal((n, D)).astype(np.float32)
    q = rng.standard_normal((1, 1, D)).astype(np.float32)
    k = np.full((NB, Hkv, BS, D), np.nan, dtype=np.float32)
    v_tok = np.full((NB, Hkv, BS, D), np.nan, dtype=np.float32)
    for e in ex["logical_blocks"]:
        for t in range(e["first_token"], e["last_token"] + 1):
            k[e["physical"], 0, t - e["first_token"], :] = Kc[t]
            v_tok[e["physical"], 0, t - e["first_token"], :] = Vc[t]
    v = bruteforce.v_from_token_major(v_tok, 4)
    o = oracle.decode(q, k, v, np.array([table]), [n], num_q_heads=1, num_kv_heads=1,
                      head_dim=D, block_size=BS, num_blocks=NB, q_dtype="f32",
                      kv_dtype="f32", scale=0.5)
    s = Kc.astype(np.float64) @ q[0, 0].astype(np.float64) * 0.5
    w = np.exp(s - s.max())
    ref = (w[:, None] * Vc).sum(0) / w.sum()
    np.testing.assert_allclose(o[0, 0], ref, rtol=1e-13, atol=1e-14)


# -- sizes ---------------------------------------------------------------------
def test_kv_bytes_per_token_matches_page_examples():
    g = _golden("devto_kv_sizes.json")
    for ex in g["examples"]:
        bpt = oracle.kv_bytes_per_token(ex["layers"], ex["kv_heads"], ex["head_dim"],
                                        ex["elem_bytes"])
        assert bpt == ex["bytes_per_token"]
        assert bpt * ex["tokens"] == ex["per_sequence_MiB"] * 2**20
        assert bpt * ex["tokens"] * ex["users"] == ex["total_MiB"] * 2**20
    # FP8 halves it (dev.to §6 "Enable FP8 KV Cache": 2 bytes -> 1 byte)
    assert oracle.kv_bytes_per_token(32, 8, 128, 1) * 2 == 131072
    assert 26_843_545_600 == oracle.kv_bytes_per_token(40, 40, 128, 2) * 4096 * 8


# -- number formats ------------------------------------------------------------
def test_e4m3_decode_against_ocp_table_and_torch():
    g = _golden("ocp_e4m3_values.json")
    for e in g["codes"]:
        v = oracle.e4m3_to_double(e["code"])
        if e["value"] == "nan":
            assert math.isnan(v)
        else:
            assert v == e["value"] and math.copysign(1, v) == math.copysign(1, e["value"])
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([oracle.e4m3_to_double(c) for c in range(256)])
    np.testing.assert_array_equal(np.isnan(mine), np.isnan(lib))
    ok = ~np.isnan(lib)
    np.testing.assert_array_equal(mine[ok], lib[ok])


def test_e4m3_encode_rounding_and_saturation():
    vals = np.array([oracle.e4m3_to_double(c) for c in range(0x7F)])  # 0 .. 448
    # exact values encode to themselves
    for c in range(0x7F):
        assert oracle.e4m3_from_float(vals[c]) == c
        assert oracle.e4m3_from_float(-vals[c]) == (c | 0x80)
    # midpoints tie to the even code; nudged midpoints go to the nearer side
    for c in range(0x7E):
        mid = np.float32((vals[c] + vals[c + 1]) / 2)
        assert float(mid) == (vals[c] + vals[c + 1]) / 2  # exact in fp32
        want = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_from_float(mid) == want, (c, mid)
        assert oracle.e4m3_from_float(np.nextafter(mid, np.float32(0))) == c
        assert oracle.e4m3_from_float(np.nextafter(mid, np.float32(1e9))) == c + 1
    # saturation at 448, NaN kept
    for x in [448.0, 449.0, 463.9, 464.0, 1e6, np.inf]:
        assert oracle.e4m3_from_float(x) == 0x7E
        assert oracle.e4m3_from_float(-x) == 0xFE
    assert oracle.e4m3_from_float(np.nan) & 0x7F == 0x7F
    # agreement with torch's cast wherever torch does not overflow (|x| < 464)
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1, 30, 150)])
    x = x[np.abs(x) < 460].astype(np.float32)
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = np.array([oracle.e4m3_from_float(v) for v in x], dtype=np.uint8)
    np.testing.assert_array_equal(mine, lib)


def test_f16_and_bf16_decoders_against_library():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    lib16 = bits.view(np.float16).astype(np.float64)
    libbf = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    for i in range(0, 65536, 7):  # every 7th code keeps the test fast; all exponents covered
        a = oracle.f16_to_double(i)
        b = oracle.bf16_to_double(i)
        assert (math.isnan(a) and math.isnan(lib16[i])) or a == lib16[i], i
        assert (math.isnan(b) and math.isnan(libbf[i])) or b == libbf[i], i
    for i in [0, 1, 0x3FF, 0x400, 0x7BFF, 0x7C00, 0x7C01, 0x8000, 0x8001, 0xFBFF, 0xFC00]:
        a = oracle.f16_to_double(i)
        assert (math.isnan(a) and math.isnan(lib16[i])) or a == lib16[i], i


# -- append ------------------------------------------------------------------
@pytest.mark.parametrize("kv_dtype,in_dtype", [("f32", "f32"), ("bf16", "bf16"),
                                               ("f16", "f16"), ("e4m3", "bf16"),
                                               ("e4m3", "f16")])
@pytest.mark.parametrize("bs", [16, 64])
def test_append_writes_exact_slots_only(kv_dtype, in_dtype, bs):
    """Each token lands in its slot and nowhere else.  The V column of offset
    o is found through bruteforce.v_token_major applied to the storage
    positions."""
    rng = np.random.default_rng(21)
    NB, Hkv, D = 12, 3, 64
    slots = np.array([5, bs * 11 + bs - 1, -1, 33, bs * 4, 2, 100, bs * 7 + bs // 2 + 13],
                     dtype=np.int32)
    T = len(slots)
    eb = oracle.ELEM_BYTES[kv_dtype]
    sentinel = {1: np.uint8(0xFF), 2: np.uint16(0xFFFF), 4: np.float32(np.nan)}[eb]
    k = np.full((NB, Hkv, bs, D), sentinel)
    v = np.full(v_shape(NB, Hkv, D, bs), sentinel)

    vpos = bruteforce.v_token_major(np.arange(v.size).reshape(v.shape), Hkv, D, bs, eb)

    def vcol(a, blk, off):
        return a.reshape(-1)[vpos[blk, :, off, :]]

    k_new = random_storage(rng, (T, Hkv, D), in_dtype)
    v_new = random_storage(rng, (T, Hkv, D), in_dtype)
    ks, vs = 0.011, 0.007
    oracle.cache_append(k_new, v_new, k, v, slots, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                        num_blocks=NB, kv_dtype=kv_dtype, in_dtype=in_dtype,
                        k_scale=ks, v_scale=vs)
    written_k = np.zeros(k.shape, bool)
    written_v = np.zeros(v.shape, bool)
    kin = bruteforce.decode_storage(k_new, in_dtype).reshape(T, Hkv, D)
    vin = bruteforce.decode_storage(v_new, in_dtype).reshape(T, Hkv, D)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        blk, off = divmod(int(s), bs)
        written_k[blk, :, off, :] = True
        written_v.reshape(-1)[vpos[blk, :, off, :]] = True
        if kv_dtype == in_dtype:
            np.testing.assert_array_equal(k[blk, :, off, :], k_new[t])
            np.testing.assert_array_equal(vcol(v, blk, off), v_new[t])
        else:
            # torch's cast agrees with the saturating RNE encoder below 464
            xk = torch.from_numpy((kin[t] .astype(np.float32) * np.float32(1.0 / np.float32(ks)))
                                  .astype(np.float32))
            xv = torch.from_numpy((vin[t].astype(np.float32) * np.float32(1.0 / np.float32(vs)))
                                  .astype(np.float32))
            xk = xk.clamp(-448, 448)
            xv = xv.clamp(-448, 448)
            np.testing.assert_array_equal(k[blk, :, off, :],
                                          xk.to(torch.float8_e4m3fn).view(torch.uint8).numpy())
            np.testing.assert_array_equal(vcol(v, blk, off),
                                          xv.to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    k_bytes = k.view(np.uint8).reshape(k.shape + (eb,))
    v_bytes = v.view(np.uint8).reshape(v.shape + (eb,))
    assert np.all(k_bytes[~written_k] == 0xFF) if eb != 4 else np.all(np.isnan(k[~written_k]))
    assert np.all(v_bytes[~written_v] == 0xFF) if eb != 4 else np.all(np.isnan(v[~written_v]))


def test_append_then_decode_reads_new_token():
    """dev.to §1: append the new token's K/V, then attend over the stored
    history including it.  A huge key on the new token makes its value row
    dominate the output."""
    c = random_case(31, B=1, Hq=1, Hkv=1, D=16, lens=[20], extra_blocks=0)
    n = 20
    slot = int(c["tables"][0][(n - 1) // BS]) * BS + (n - 1) % BS
    knew = (c["q"][0] * 50.0).astype(np.float32)
    vnew = np.arange(16, dtype=np.float32)[None, :]
    oracle.cache_append(knew, vnew.reshape(1, 1, 16), c["k"], c["v"], np.array([slot]),
                        num_kv_heads=1, head_dim=16, block_size=BS, num_blocks=c["NB"],
                        kv_dtype="f32", in_dtype="f32")
    o = run_oracle(c)
    np.testing.assert_allclose(o[0, 0], np.arange(16), atol=1e-6)


# -- block sizes -----------------------------------------------------------------
@pytest.mark.parametrize("bs", [32, 64, 256])
@pytest.mark.parametrize("q_dtype,kv_dtype,Hq,Hkv,D", [("f32", "f32", 4, 2, 32),
                                                     ("bf16", "e4m3", 8, 2, 64)])
def test_block_size_variants_match_bruteforce(bs, q_dtype, kv_dtype, Hq, Hkv, D):
    """Blocks of more than 16 tokens (the pages also name 32, and 256 or more
    per page): the oracle against the brute force, which restates the cache
    layout with its own numpy reshapes.  Lengths span several blocks and end
    inside one."""
    for seed in range(2):
        c = random_case(200 + seed, bs=bs, B=3, Hq=Hq, Hkv=Hkv, D=D, q_dtype=q_dtype,
                        kv_dtype=kv_dtype, max_len=3 * bs + 7)
        ks, vs = (0.037, 0.021) if kv_dtype == "e4m3" else (1.0, 1.0)
        np.testing.assert_allclose(run_oracle(c, k_scale=ks, v_scale=vs),
                                   run_brute(c, k_scale=ks, v_scale=vs), rtol=1e-12, atol=1e-13)


def test_block_size_is_storage_only():
    """The same token rows, appended into pools of 16-, 32-, 64- and 256-token
    blocks under random placements, decode to the same bits: the block size
    changes where a row is stored, not what is computed."""
    rng = np.random.default_rng(41)
    Hq, Hkv, D = 4, 2, 32
    lens = np.array([1, 17, 300, 64], dtype=np.int32)
    rows_k = [random_storage(rng, (n, Hkv, D), "bf16") for n in lens]
    rows_v = [random_storage(rng, (n, Hkv, D), "bf16") for n in lens]
    q = random_storage(rng, (len(lens), Hq, D), "bf16")
    outs = []
    for bs in (16, 32, 64, 256):
        nblk = [-(-int(n) // bs) for n in lens]
        NB = sum(nblk) + 3
        perm = rng.permutation(NB)
        tables = np.full((len(lens), max(nblk)), -1, dtype=np.int32)
        k = np.zeros((NB, Hkv, bs, D), np.uint16)
        v = np.zeros(v_shape(NB, Hkv, D, bs), np.uint16)
        pos = 0
        for b, n in enumerate(lens):
            tables[b, :nblk[b]] = perm[pos:pos + nblk[b]]
            pos += nblk[b]
            t = np.arange(n)
            slots = (tables[b][t // bs] * bs + t % bs).astype(np.int32)
            oracle.cache_append(rows_k[b], rows_v[b], k, v, slots, num_kv_heads=Hkv, head_dim=D,
                                block_size=bs, num_blocks=NB, kv_dtype="bf16", in_dtype="bf16")
        outs.append(oracle.decode(q, k, v, tables, lens, num_q_heads=Hq, num_kv_heads=Hkv,
                                  head_dim=D, block_size=bs, num_blocks=NB, q_dtype="bf16",
                                  kv_dtype="bf16", scale=0.125))
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])


def test_block_size_must_be_a_multiple_of_16():
    c = random_case(3, B=1, lens=[5])
    with pytest.raises(ValueError, match=r"\(-3\)"):
        run_oracle(c, block_size=8)


# -- sliding window ----------------------------------------------------------------
@pytest.mark.parametrize("bs", [16, 64])
@pytest.mark.parametrize("q_dtype,kv_dtype", [("f32", "f32"), ("bf16", "e4m3")])
def test_window_matches_bruteforce(bs, q_dtype, kv_dtype):
    """Window starts anywhere in [0, n] (the first kept block partly cut,
    whole blocks cut, one token left, nothing left): the oracle against the
    brute force, which slices the gathered rows."""
    for seed in range(3):
        c = random_case(300 + seed, bs=bs, B=6, Hq=4, Hkv=2, D=64, q_dtype=q_dtype,
                        kv_dtype=kv_dtype, max_len=4 * bs)
        n = c["lens"]
        rng = np.random.default_rng(seed)
        starts = np.array([0, n[1], n[2] - 1, n[3] // 2, rng.integers(0, n[4] + 1),
                           min(bs + 3, n[5])], dtype=np.int32)
        ks, vs = (0.037, 0.021) if kv_dtype == "e4m3" else (1.0, 1.0)
        np.testing.assert_allclose(run_oracle(c, k_scale=ks, v_scale=vs, seq_starts=starts),
                                   run_brute(c, k_scale=ks, v_scale=vs, seq_starts=starts),
                                   rtol=1e-12, atol=1e-13)


def test_window_equals_a_sequence_holding_only_the_window():
    """Leaving tokens 0..w-1 out gives the same bits as a table whose blocks
    hold only tokens w..n-1 (appended from offset 0 in new blocks)."""
    bs, Hq, Hkv, D = 16, 4, 2, 32
    rng = np.random.default_rng(51)
    n, w = 150, 37
    rows_k = random_storage(rng, (n, Hkv, D), "bf16")
    rows_v = random_storage(rng, (n, Hkv, D), "bf16")
    q = random_storage(rng, (1, Hq, D), "bf16")
    NB = 40
    k = np.zeros((NB, Hkv, bs, D), np.uint16)
    v = np.zeros(v_shape(NB, Hkv, D, bs), np.uint16)
    perm = rng.permutation(NB)
    full = perm[:-(-n // bs)]
    part = perm[20:20 + -(-(n - w) // bs)]
    common = dict(num_kv_heads=Hkv, head_dim=D, block_size=bs, num_blocks=NB, kv_dtype="bf16",
                  in_dtype="bf16")
    t = np.arange(n)
    oracle.cache_append(rows_k, rows_v, k, v, (full[t // bs] * bs + t % bs).astype(np.int32),
                        **common)
    t = np.arange(n - w)
    oracle.cache_append(np.ascontiguousarray(rows_k[w:]), np.ascontiguousarray(rows_v[w:]), k, v,
                        (part[t // bs] * bs + t % bs).astype(np.int32), **common)
    args = dict(num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs, num_blocks=NB,
                q_dtype="bf16", kv_dtype="bf16", scale=0.125)
    a = oracle.decode(q, k, v, full[None, :].astype(np.int32), [n], seq_starts=[w], **args)
    b = oracle.decode(q, k, v, part[None, :].astype(np.int32), [n - w], **args)
    np.testing.assert_array_equal(a, b)


def test_window_closed_forms():
    """One token in the window: its V row exactly.  An empty window: zeros.
    A start outside [0, n]: an error."""
    c = random_case(61, B=2, Hq=2, Hkv=1, D=16, lens=[40, 40])
    vv = bruteforce.v_token_major(bruteforce.decode_storage(c["v"], "f32"), 1, 16, BS, 4)
    o = run_oracle(c, seq_starts=[39, 40])
    t = 39
    np.testing.assert_allclose(o[0, 0], vv[c["tables"][0][t // BS], 0, t % BS], rtol=0, atol=0)
    np.testing.assert_array_equal(o[1], 0.0)
    for bad in ([41, 0], [-1, 0]):
        with pytest.raises(ValueError, match=r"\(-1\)"):
            run_oracle(c, seq_starts=bad)
