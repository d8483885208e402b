"""CPU oracle for paged-KV decode and cache append -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the GPU library: the arithmetic lives
in pa_oracle.c (fp64, built with gcc, no HIP) and the allocator policy model
in alloc_model.py.

Functions take numpy arrays holding the raw storage bytes of each tensor
(float32, or uint16 for fp16/bf16, or uint8 for E4M3) plus a dtype name, so
the oracle decodes every stored value itself.
"""
import ctypes
import os
import subprocess

import numpy as np

from . import alloc_model  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DTYPES = {"f32": 0, "f16": 1, "bf16": 2, "e4m3": 3}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1}


def build(force=True):
    """Compile pa_oracle.c with gcc into liboracle.so next to it."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
                           "-o", tmp, _SRC, "-lm", "-lpthread"])
    os.replace(tmp, _LIB)
    return _LIB


class _CacheDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("in_dtype", ctypes.c_int32)]


class _DecodeDesc(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("q_dtype", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        # PA_ORACLE_LIB names another build of pa_oracle.c; the mutation tests
        # use it to check that the pins catch planted mistakes.
        path = os.environ.get("PA_ORACLE_LIB")
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        lib.orc_e4m3_to_double.restype = ctypes.c_double
        lib.orc_e4m3_to_double.argtypes = [ctypes.c_uint8]
        lib.orc_f16_to_double.restype = ctypes.c_double
        lib.orc_f16_to_double.argtypes = [ctypes.c_uint16]
        lib.orc_bf16_to_double.restype = ctypes.c_double
        lib.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.orc_e4m3_from_float.restype = ctypes.c_uint8
        lib.orc_e4m3_from_float.argtypes = [ctypes.c_float]
        lib.orc_kv_bytes_per_token.restype = ctypes.c_uint64
        lib.orc_kv_bytes_per_token.argtypes = [ctypes.c_int64] * 4
        lib.orc_cache_append.restype = ctypes.c_int
        lib.orc_cache_append.argtypes = [ctypes.POINTER(_CacheDesc), P, P, P, P, P,
                                         ctypes.c_int32, ctypes.c_float, ctypes.c_float]
        lib.orc_decode.restype = ctypes.c_int
        lib.orc_decode.argtypes = [ctypes.POINTER(_DecodeDesc), P, P, P, P, P, P,
                                   ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                   P, ctypes.c_int64, P, ctypes.c_int]
        _lib = lib
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check_storage(a, dtype):
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "contiguous numpy array expected"
    assert a.dtype.itemsize == ELEM_BYTES[dtype], (a.dtype, dtype)


# -- number formats ------------------------------------------------------
def e4m3_to_double(code):
    return _load().orc_e4m3_to_double(int(code) & 0xFF)


def f16_to_double(bits):
    return _load().orc_f16_to_double(int(bits) & 0xFFFF)


def bf16_to_double(bits):
    return _load().orc_bf16_to_double(int(bits) & 0xFFFF)


def e4m3_from_float(x):
    return _load().orc_e4m3_from_float(float(np.float32(x)))


def kv_bytes_per_token(layers, kv_heads, head_dim, elem_bytes):
    return int(_load().orc_kv_bytes_per_token(layers, kv_heads, head_dim, elem_bytes))


# -- append --------------------------------------------------------------
def cache_append(k_new, v_new, k_cache, v_cache, slot_mapping, *, num_kv_heads, head_dim,
                 block_size, num_blocks, kv_dtype, in_dtype, k_scale=1.0, v_scale=1.0):
    """Writes the new tokens into k_cache / v_cache (numpy storage arrays) in place.

    K cache is [blocks][Hkv][bs][D]; V cache [blocks][Hkv][bs/16][16 D]: tiles
    of 16 tokens (bs a multiple of 16) in which, with p = 4 / element bytes,
    each 16-byte piece holds p dims (16 apart) of 4 consecutive tokens, D a
    multiple of 16 p (the element index is in pa_oracle.c); k_new / v_new are
    [T][Hkv][D]."""
    _check_storage(k_new, in_dtype)
    _check_storage(v_new, in_dtype)
    _check_storage(k_cache, kv_dtype)
    _check_storage(v_cache, kv_dtype)
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int32)
    T = slots.shape[0]
    assert k_new.size == T * num_kv_heads * head_dim
    assert k_cache.size == num_blocks * num_kv_heads * block_size * head_dim
    desc = _CacheDesc(num_blocks, block_size, num_kv_heads, head_dim, DTYPES[kv_dtype],
                      DTYPES[in_dtype])
    rc = _load().orc_cache_append(ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                  _ptr(v_cache), _ptr(slots), T, float(k_scale), float(v_scale))
    if rc != 0:
        raise ValueError(f"oracle cache_append failed ({rc})")


# -- decode --------------------------------------------------------------
def decode(q, k_cache, v_cache, block_tables, seq_lens, *, num_q_heads, num_kv_heads,
           head_dim, block_size, num_blocks, q_dtype, kv_dtype, scale, k_scale=1.0,
           v_scale=1.0, rows=None, nthreads=0, seq_starts=None):
    """fp64 attention output, [B][Hq][D] (or [len(rows)][D] for a row list).

    rows: optional iterable of (b, h) pairs to compute.  seq_starts: optional
    [B] window starts (tokens before them are left out; start = length gives
    a zero row)."""
    _check_storage(q, q_dtype)
    _check_storage(k_cache, kv_dtype)
    _check_storage(v_cache, kv_dtype)
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B = lens.shape[0]
    assert tables.ndim == 2 and tables.shape[0] == B
    assert q.size == B * num_q_heads * head_dim
    starts = None
    if seq_starts is not None:
        starts = np.ascontiguousarray(seq_starts, dtype=np.int32)
        assert starts.shape == (B,)
    desc = _DecodeDesc(B, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       tables.shape[1], DTYPES[q_dtype], DTYPES[kv_dtype])
    if rows is None:
        row_ids = None
        nrows = B * num_q_heads
        out = np.zeros((B, num_q_heads, head_dim), dtype=np.float64)
    else:
        row_ids = np.ascontiguousarray([b * num_q_heads + h for (b, h) in rows], dtype=np.int32)
        nrows = row_ids.shape[0]
        out = np.zeros((nrows, head_dim), dtype=np.float64)
    rc = _load().orc_decode(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                            _ptr(tables), _ptr(lens), None if starts is None else _ptr(starts),
                            float(scale), float(k_scale),
                            float(v_scale), None if row_ids is None else _ptr(row_ids),
                            nrows, _ptr(out), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle decode failed ({rc})")
    return out
