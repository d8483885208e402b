"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of oracle/pa_oracle.c (a dropped term,
a wrong sign, index or layout, a wrong exponent bias, a wrong tie rule),
builds it with gcc, and runs the pin suite against that build through
PA_ORACLE_LIB.  The suite must fail for every mutant.  CPU only.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "pa_oracle.c")

MUTANTS = {
    "gqa_head_mapping": ("int g = h / G;", "int g = h % d->num_kv_heads;"),
    "k_tile_transposed": ("* c->block_size + o) * c->head_dim + d;",
                          "* c->head_dim + d) * c->block_size + o;"),
    "v_tile_token_major": ("return tile * 16 * c->head_dim + piece * 4 * p + (size_t)((d / 16) % p) * 4 + u % 4;",
                           "return (tile * 16 + u) * c->head_dim + d;"),
    "v_piece_lane_order": ("(size_t)(u / 4) * 16 + d % 16;", "(size_t)(d % 16) * 4 + u / 4;"),
    "v_piece_dims_adjacent": ("+ (size_t)((d / 16) % p) * 4 + u % 4;",
                              "+ (size_t)(u % 4) * p + (d / 16) % p;"),
    # the same at 16-token blocks: only the larger-block pins can catch it
    "v_subtile_order": ("* (c->block_size / 16) + o / 16;",
                        "* (c->block_size / 16) + (o / 16 + 1) % (c->block_size / 16);"),
    "scale_dropped": ("s[t] = J->scale * dot;", "s[t] = dot;"),
    "softmax_sign": ("s[t] = exp(s[t] - m);", "s[t] = exp(m - s[t]);"),
    "normaliser_dropped": ("out_row[i] /= Z;", "out_row[i] /= 1.0;"),
    "block_index_mod": ("int64_t blk = table[t / d->block_size];",
                        "int64_t blk = table[(t / d->block_size) / 2];"),
    "offset_in_block": ("int o = (int)(t % d->block_size);",
                        "int o = (int)((t + 1) % d->block_size);"),
    "last_token_skipped": ("for (int64_t t = w; t < n; ++t) {\n        int64_t blk",
                           "for (int64_t t = w; t < n - 1; ++t) {\n        int64_t blk"),
    "window_start_ignored": ("int64_t w = J->seq_starts ? J->seq_starts[b] : 0;",
                             "int64_t w = 0;"),
    "window_start_off_by_one": ("int64_t w = J->seq_starts ? J->seq_starts[b] : 0;",
                                "int64_t w = J->seq_starts ? J->seq_starts[b] - (b > 0) : 0;"),
    "k_scale_dropped": ("k_index(&c, blk, g, o, i)) * J->k_scale;", "k_index(&c, blk, g, o, i));"),
    "v_scale_dropped": ("v_index(&c, blk, g, o, i)) * J->v_scale;", "v_index(&c, blk, g, o, i));"),
    "q_decoded_as_kv": ("qv[i] = orc_load(d->q_dtype", "qv[i] = orc_load(d->kv_dtype"),
    "e4m3_bias": ("mag = ldexp(1.0 + (double)m / 8.0, e - 7);",
                  "mag = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "e4m3_subnormal_scale": ("mag = ldexp((double)m / 8.0, 1 - 7);",
                             "mag = ldexp((double)m / 8.0, -7);"),
    "e4m3_ties_to_odd": ("c = (lo & 1) == 0 ? lo : hi;", "c = (lo & 1) == 1 ? lo : hi;"),
    "e4m3_no_saturation": ("if (a >= 448.0)\n        return sign | 0x7E;",
                           "if (a >= 464.0)\n        return sign | 0x7F;"),
    "f16_bias": ("mag = ldexp(1.0 + (double)m / 1024.0, e - 15);",
                 "mag = ldexp(1.0 + (double)m / 1024.0, e - 14);"),
    "append_v_with_k_layout": ("store_elem(c, J->v_cache, v_index(", "store_elem(c, J->v_cache, k_index("),
    "bytes_per_token_no_factor_2": ("return (uint64_t)(2 * layers", "return (uint64_t)(1 * layers"),
}


def _run_mutant(name, tmp):
    find, repl = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(find) >= 1, f"mutant {name}: pattern not found"
    mutated = src.replace(find, repl)
    c_path = os.path.join(tmp, f"{name}.c")
    so_path = os.path.join(tmp, f"{name}.so")
    with open(c_path, "w") as f:
        f.write(mutated)
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-shared", "-fPIC", "-o", so_path, c_path,
                           "-lm", "-lpthread"])
    env = dict(os.environ, PA_ORACLE_LIB=so_path)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode


def test_every_planted_mistake_fails_a_pin():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max_workers=6) as ex:
            codes = dict(zip(MUTANTS, ex.map(lambda n: _run_mutant(n, tmp), MUTANTS)))
    survivors = [n for n, rc in codes.items() if rc == 0]
    assert not survivors, f"pins did not catch: {survivors}"


def test_unmutated_copy_passes(tmp_path):
    """Control: the same harness with the real source passes."""
    so = tmp_path / "orig.so"
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-shared", "-fPIC", "-o", str(so), SRC,
                           "-lm", "-lpthread"])
    env = dict(os.environ, PA_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
