"""Python binding of libpa (paged KV cache + PagedAttention decode on MI355X).

Argument marshalling only: every function forwards to the C entry point of
the same name in libpa.so (declared in include/pa.h), passing tensor data
pointers, sizes and the current HIP stream.  All computation happens in the
library's HIP kernels and host allocator.  Importing this package fails if
libpa.so has not been built (python paged_kv_cache_255_amd/build.py).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python paged_kv_cache_255_amd/build.py`")

# The callers hand the library device pointers and streams of torch's HIP
# runtime, so the library must run on that same runtime.  torch ships its own
# libamdhip64.so.7; once torch is loaded, the dynamic loader resolves libpa's
# dependency of that name to it.  Loading libpa first would bring in a second
# HIP runtime (the system one), which then finds no free device and knows none
# of torch's allocations.
import torch  # noqa: E402,F401  (must precede the CDLL below)

_lib = ctypes.CDLL(LIB_PATH)

# pa_status
OK, ERR_INVALID_ARG, ERR_OUT_OF_BLOCKS, ERR_CAPACITY, ERR_UNSUPPORTED, ERR_HIP = range(6)
STATUS_NAMES = {0: "PA_OK", 1: "PA_ERR_INVALID_ARG", 2: "PA_ERR_OUT_OF_BLOCKS",
                3: "PA_ERR_CAPACITY", 4: "PA_ERR_UNSUPPORTED", 5: "PA_ERR_HIP"}
# pa_dtype
F32, F16, BF16, FP8_E4M3 = 0, 1, 2, 3
DTYPE_CODES = {"f32": F32, "f16": F16, "bf16": BF16, "e4m3": FP8_E4M3}
DTYPE_BYTES = {F32: 4, F16: 2, BF16: 2, FP8_E4M3: 1}
# kernel choice and partitioning
KERNEL_AUTO, KERNEL_VALU, KERNEL_MFMA = 0, 1, 2
PARTITION_NONE, PARTITION_BALANCED = 0, -1
NOALLOC_SCRATCH_BYTES = 16 << 20  # PA_NOALLOC_SCRATCH_BYTES
SHARE_PLAN_MAGIC = 0x31534150      # PA_SHARE_PLAN_MAGIC


def share_plan_words(nseq):
    """PA_SHARE_PLAN_WORDS: int32 words of a share plan for nseq sequences."""
    return 2 + 8 * nseq


class PaError(RuntimeError):
    def __init__(self, status, where):
        msg = _lib.pa_last_error().decode()
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class PoolConfig(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_layers", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("kv_dtype", ctypes.c_int),
                ("shuffle_seed", ctypes.c_uint64), ("num_host_blocks", ctypes.c_int32)]


class PoolStats(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("free_blocks", ctypes.c_int32),
                ("used_blocks", ctypes.c_int32), ("shared_blocks", ctypes.c_int32),
                ("live_seqs", ctypes.c_int32), ("cached_blocks", ctypes.c_int32),
                ("swapped_seqs", ctypes.c_int32), ("free_host_blocks", ctypes.c_int32),
                ("logical_tokens", ctypes.c_int64), ("mapped_blocks", ctypes.c_int64),
                ("tail_slack_tokens", ctypes.c_int64)]


class KvDesc(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32), ("q_dtype", ctypes.c_int),
                ("kv_dtype", ctypes.c_int), ("kernel", ctypes.c_int32)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_PI32 = ctypes.POINTER(ctypes.c_int32)
_SIGS = {
    "pa_block_pool_init": (ctypes.c_int, [ctypes.POINTER(PoolConfig), ctypes.POINTER(_P)]),
    "pa_block_pool_destroy": (None, [_P]),
    "pa_kv_bytes_per_token": (ctypes.c_uint64, [_P]),
    "pa_block_bytes": (ctypes.c_uint64, [_P]),
    "pa_seq_create": (ctypes.c_int, [_P, _PI32]),
    "pa_seq_append_slots": (ctypes.c_int, [_P, _I32, _I32, _P]),
    "pa_seq_append_slots_batch": (ctypes.c_int, [_P, _P, _I32, _I32, _P]),
    "pa_seq_fork": (ctypes.c_int, [_P, _I32, _PI32]),
    "pa_seq_free": (ctypes.c_int, [_P, _I32]),
    "pa_seq_length": (ctypes.c_int, [_P, _I32, _PI32]),
    "pa_block_refcount": (ctypes.c_int, [_P, _I32, _PI32]),
    "pa_export_block_tables": (ctypes.c_int, [_P, _P, _I32, _I32, _P, _P, _P, _P]),
    "pa_seq_slide_window": (ctypes.c_int, [_P, _I32, _I32, _P]),
    "pa_seq_swap_out": (ctypes.c_int, [_P, _I32, _P, _I32, _P]),
    "pa_seq_swap_in": (ctypes.c_int, [_P, _I32, _P, _I32, _P]),
    "pa_swap_blocks": (ctypes.c_int, [_P, _P, _P, _P, _I32, _P, _I32, _I32,
                                      ctypes.POINTER(KvDesc), _P]),
    "pa_pool_get_stats": (ctypes.c_int, [_P, ctypes.POINTER(PoolStats)]),
    "pa_cache_append": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, ctypes.POINTER(KvDesc),
                                       ctypes.c_float, ctypes.c_float, _P]),
    "pa_decode_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(KvDesc), _I32, _I32, _I32]),
    "pa_decode_balanced_waves": (_I32, [ctypes.POINTER(KvDesc)]),
    "pa_decode": (ctypes.c_int, [_P, _P, _P, _P, _I32, _P, _P, _P, _I32, _I32, ctypes.c_float,
                                 ctypes.c_float, ctypes.c_float, _P, _P, ctypes.c_size_t, _I32,
                                 ctypes.POINTER(KvDesc), _P]),
    "pa_decode_partials": (ctypes.c_int, [_P, _P, _P, _P, _I32, _P, _P, _P, _I32, _I32,
                                          ctypes.c_float, ctypes.c_float, ctypes.c_float, _P, _P,
                                          ctypes.c_size_t, _I32, ctypes.POINTER(KvDesc), _P]),
    "pa_decode_merge": (ctypes.c_int, [_P, _P, _I32, _I32, _I32, _P, _P, ctypes.c_size_t, _I32,
                                       ctypes.POINTER(KvDesc), _P]),
    "pa_export_share_plan": (ctypes.c_int, [_P, _P, _I32, _P]),
    "pa_decode_append": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _I32, _I32,
                                        ctypes.c_float, ctypes.c_float, ctypes.c_float, _P, _P,
                                        ctypes.c_size_t, _I32, _P, _P]),
    "pa_pool_take_copies": (ctypes.c_int, [_P, _P, _I32, _P]),
    "pa_prefix_register": (ctypes.c_int, [_P, _I32, _P, _I32, _P]),
    "pa_prefix_match": (ctypes.c_int, [_P, _I32, _P, _I32, _P]),
    "pa_prefix_evict": (ctypes.c_int, [_P, _I32, _P]),
    "pa_copy_blocks": (ctypes.c_int, [_P, _P, _P, _I32, _P, _P]),
    "pa_decode_append_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P,
                                                _I32, _I32, ctypes.c_float, ctypes.c_float,
                                                ctypes.c_float, _P, _I32, _P, _P]),
    "pa_read_probe": (ctypes.c_int, [_P, ctypes.c_size_t, _I32, _I32, _I32, _I32, _P, _P]),
    "pa_last_error": (ctypes.c_char_p, []),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


def _check(status, where):
    if status != OK:
        raise PaError(status, where)


def _addr(x):
    """Data address of a torch tensor, a numpy array, an int or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    return x.data_ptr()


def _i32_array(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# ---- block pool ------------------------------------------------------------
class Pool:
    """Owns a pa_pool handle; destroyed with the object."""

    def __init__(self, handle, config):
        self.handle = handle
        self.config = config
        # held here: module globals may already be None when a pool is
        # collected at interpreter exit
        self._destroy = _lib.pa_block_pool_destroy

    def __del__(self):
        if getattr(self, "handle", None):
            self._destroy(self.handle)
            self.handle = None


def pa_block_pool_init(num_blocks, num_kv_heads, head_dim, kv_dtype, num_layers=1,
                       block_size=16, shuffle_seed=0, num_host_blocks=0):
    cfg = PoolConfig(num_blocks, block_size, num_layers, num_kv_heads, head_dim,
                     DTYPE_CODES.get(kv_dtype, kv_dtype), shuffle_seed, num_host_blocks)
    h = _P()
    _check(_lib.pa_block_pool_init(ctypes.byref(cfg), ctypes.byref(h)), "pa_block_pool_init")
    return Pool(h.value, cfg)


def pa_block_pool_destroy(pool):
    if pool.handle:
        _lib.pa_block_pool_destroy(pool.handle)
        pool.handle = None


def pa_kv_bytes_per_token(pool):
    return int(_lib.pa_kv_bytes_per_token(pool.handle))


def pa_block_bytes(pool):
    return int(_lib.pa_block_bytes(pool.handle))


def pa_seq_create(pool):
    sid = _I32()
    _check(_lib.pa_seq_create(pool.handle, ctypes.byref(sid)), "pa_seq_create")
    return sid.value


def pa_seq_append_slots(pool, seq, ntok):
    slots = np.empty(max(ntok, 1), dtype=np.int32)
    _check(_lib.pa_seq_append_slots(pool.handle, seq, ntok, slots.ctypes.data),
           "pa_seq_append_slots")
    return slots[:ntok]


def pa_seq_append_slots_batch(pool, seqs, ntok, slots_out=None):
    """slots_out: optional int32 buffer (numpy / pinned tensor) of len(seqs)*ntok."""
    seqs = _i32_array(seqs)
    out = slots_out if slots_out is not None else np.empty(max(len(seqs) * ntok, 1), np.int32)
    _check(_lib.pa_seq_append_slots_batch(pool.handle, seqs.ctypes.data, len(seqs), ntok,
                                          _addr(out)), "pa_seq_append_slots_batch")
    return out if slots_out is not None else out[:len(seqs) * ntok]


def pa_seq_fork(pool, parent):
    c = _I32()
    _check(_lib.pa_seq_fork(pool.handle, parent, ctypes.byref(c)), "pa_seq_fork")
    return c.value


def pa_seq_free(pool, seq):
    _check(_lib.pa_seq_free(pool.handle, seq), "pa_seq_free")


def pa_seq_length(pool, seq):
    n = _I32()
    _check(_lib.pa_seq_length(pool.handle, seq, ctypes.byref(n)), "pa_seq_length")
    return n.value


def pa_block_refcount(pool, block):
    r = _I32()
    _check(_lib.pa_block_refcount(pool.handle, block, ctypes.byref(r)), "pa_block_refcount")
    return r.value


def pa_export_block_tables(pool, seqs, max_blocks, tables_out=None, lens_out=None,
                           starts_out=None, with_starts=False, shared_out=None,
                           with_shared=False):
    """Returns (tables [nseq][max_blocks] int32, lens [nseq] int32), then the
    window starts [nseq] with with_starts (or starts_out), then the leading
    shared-block counts [nseq] with with_shared (or shared_out); pass
    preallocated buffers (numpy or pinned tensors) to fill them in place."""
    seqs = _i32_array(seqs)
    t = tables_out if tables_out is not None else np.empty((len(seqs), max_blocks), np.int32)
    n = lens_out if lens_out is not None else np.empty(len(seqs), np.int32)
    w = starts_out
    if w is None and with_starts:
        w = np.empty(len(seqs), np.int32)
    sh = shared_out
    if sh is None and with_shared:
        sh = np.empty(len(seqs), np.int32)
    _check(_lib.pa_export_block_tables(pool.handle, seqs.ctypes.data, len(seqs), max_blocks,
                                       _addr(t), _addr(n), _addr(w), _addr(sh)),
           "pa_export_block_tables")
    out = (t, n)
    if w is not None:
        out += (w,)
    if sh is not None:
        out += (sh,)
    return out


def pa_export_share_plan(pool, seqs, out=None):
    """The share plan of resident sequences `seqs` (pa.h layout): int32
    [share_plan_words(len(seqs))], into `out` (numpy or pinned tensor) when
    given.  Pass it to the decode calls as seq_shared, on the device."""
    seqs = _i32_array(seqs)
    words = share_plan_words(len(seqs))
    plan = out if out is not None else np.empty(words, np.int32)
    if isinstance(plan, np.ndarray):
        ok = plan.dtype == np.int32 and plan.flags.c_contiguous and plan.size >= words
    else:
        import torch
        ok = (plan.dtype == torch.int32 and plan.device.type == "cpu" and plan.is_contiguous()
              and plan.numel() >= words)
    if not ok:
        raise ValueError(f"out must be a contiguous host int32 buffer of >= {words} words")
    _check(_lib.pa_export_share_plan(pool.handle, seqs.ctypes.data, len(seqs), _addr(plan)),
           "pa_export_share_plan")
    return plan


def pa_seq_slide_window(pool, seq, window):
    """Keeps the last `window` positions in the window; returns the blocks
    released."""
    n = _I32()
    _check(_lib.pa_seq_slide_window(pool.handle, seq, window, ctypes.byref(n)),
           "pa_seq_slide_window")
    return n.value


def _swap(fn, name, pool, seq):
    n = _I32()
    st = fn(pool.handle, seq, None, 0, ctypes.byref(n))
    if st != ERR_CAPACITY or n.value == 0:
        _check(st, name)
        return np.zeros((0, 2), dtype=np.int32)
    pairs = np.empty((n.value, 2), dtype=np.int32)
    _check(fn(pool.handle, seq, pairs.ctypes.data, n.value, ctypes.byref(n)), name)
    return pairs


def pa_seq_swap_out(pool, seq):
    """Swaps seq out; returns int32 [n][2] pairs (device block, host block)."""
    return _swap(_lib.pa_seq_swap_out, "pa_seq_swap_out", pool, seq)


def pa_seq_swap_in(pool, seq):
    """Swaps seq back in; returns int32 [n][2] pairs (host block, device block)."""
    return _swap(_lib.pa_seq_swap_in, "pa_seq_swap_in", pool, seq)


def pa_pool_get_stats(pool):
    st = PoolStats()
    _check(_lib.pa_pool_get_stats(pool.handle, ctypes.byref(st)), "pa_pool_get_stats")
    return {f: getattr(st, f) for f, _ in PoolStats._fields_}


def pa_pool_take_copies(pool):
    """The queued copy-on-write block copies as an int32 array [n][2] of
    (source, destination); clears the queue."""
    n = _I32()
    st = _lib.pa_pool_take_copies(pool.handle, None, 0, ctypes.byref(n))
    if n.value == 0:
        _check(st, "pa_pool_take_copies")
        return np.zeros((0, 2), dtype=np.int32)
    pairs = np.empty((n.value, 2), dtype=np.int32)
    _check(_lib.pa_pool_take_copies(pool.handle, pairs.ctypes.data, n.value, ctypes.byref(n)),
           "pa_pool_take_copies")
    return pairs


def _tokens(tokens):
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    return t, (t.ctypes.data if t.size else None)


def pa_prefix_register(pool, seq, tokens):
    """Caches the full blocks of seq's first len(tokens) tokens; returns the
    number of blocks newly cached."""
    t, ptr = _tokens(tokens)
    n = _I32()
    _check(_lib.pa_prefix_register(pool.handle, seq, ptr, t.size, ctypes.byref(n)),
           "pa_prefix_register")
    return n.value


def pa_prefix_match(pool, seq, tokens):
    """Maps the cached full blocks matching tokens into the empty seq;
    returns the tokens they hold."""
    t, ptr = _tokens(tokens)
    n = _I32()
    _check(_lib.pa_prefix_match(pool.handle, seq, ptr, t.size, ctypes.byref(n)),
           "pa_prefix_match")
    return n.value


def pa_prefix_evict(pool, max_blocks):
    n = _I32()
    _check(_lib.pa_prefix_evict(pool.handle, max_blocks, ctypes.byref(n)), "pa_prefix_evict")
    return n.value


# ---- kernels ---------------------------------------------------------------
def kv_desc(num_q_heads, num_kv_heads, head_dim, num_blocks, q_dtype, kv_dtype,
            block_size=16, kernel=KERNEL_AUTO):
    return KvDesc(num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                  DTYPE_CODES.get(q_dtype, q_dtype), DTYPE_CODES.get(kv_dtype, kv_dtype), kernel)


def _check_tensor(t, name, nbytes=None):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if nbytes is not None and t.numel() * t.element_size() != nbytes:
        raise ValueError(f"{name}: expected {nbytes} bytes, got {t.numel() * t.element_size()}")


def _check_i32(t, name, numel=None):
    """An int32 device tensor (the library reads these as int32_t arrays: a
    wider integer type would be misread, not rejected, on the device)."""
    import torch
    if t.dtype != torch.int32:
        raise ValueError(f"{name} must be torch.int32, got {t.dtype}")
    _check_tensor(t, name, None if numel is None else numel * 4)


def _check_tables(block_tables, B):
    """block_tables: int32 [num_seqs][max_blocks_per_seq], contiguous."""
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs][max_blocks_per_seq]")
    _check_i32(block_tables, "block_tables", B * block_tables.shape[1])


def _check_lens_tables(seq_lens, block_tables, B):
    """Types and shapes of both first, then where they live."""
    import torch
    for t, nm in [(seq_lens, "seq_lens"), (block_tables, "block_tables")]:
        if t.dtype != torch.int32:
            raise ValueError(f"{nm} must be torch.int32, got {t.dtype}")
    _check_tables(block_tables, B)
    _check_i32(seq_lens, "seq_lens", B)


def pa_cache_append(k, v, k_cache, v_cache, slot_mapping, desc, k_scale=1.0, v_scale=1.0,
                    stream=None):
    T = slot_mapping.numel()
    _check_i32(slot_mapping, "slot_mapping", T)
    qb, kb = DTYPE_BYTES[desc.q_dtype], DTYPE_BYTES[desc.kv_dtype]
    row = desc.num_kv_heads * desc.head_dim
    cache_bytes = desc.num_blocks * desc.block_size * row * kb
    for t, nm in [(k, "k"), (v, "v")]:
        _check_tensor(t, nm, T * row * qb)
    for t, nm in [(k_cache, "k_cache"), (v_cache, "v_cache")]:
        _check_tensor(t, nm, cache_bytes)
    _check(_lib.pa_cache_append(_addr(k), _addr(v), _addr(k_cache), _addr(v_cache),
                                _addr(slot_mapping), T, ctypes.byref(desc), k_scale, v_scale,
                                _stream(stream)), "pa_cache_append")


def pa_copy_blocks(k_cache, v_cache, pairs, desc, stream=None):
    """pairs: device int32 tensor [n][2] of (source, destination) blocks."""
    kb = DTYPE_BYTES[desc.kv_dtype]
    cache_bytes = desc.num_blocks * desc.block_size * desc.num_kv_heads * desc.head_dim * kb
    for t, nm in [(k_cache, "k_cache"), (v_cache, "v_cache")]:
        _check_tensor(t, nm, cache_bytes)
    n = pairs.shape[0] if pairs.dim() == 2 else 0
    if n:
        _check_i32(pairs, "pairs", n * 2)
    _check(_lib.pa_copy_blocks(_addr(k_cache), _addr(v_cache), _addr(pairs) if n else None, n,
                               ctypes.byref(desc), _stream(stream)), "pa_copy_blocks")


def pa_swap_blocks(k_cache, v_cache, host_k, host_v, pairs, desc, to_host, stream=None):
    """host_k, host_v: pinned host tensors of whole blocks laid out like the
    caches; pairs: device int32 tensor [n][2] as pa_seq_swap_out / _in gave."""
    kb = DTYPE_BYTES[desc.kv_dtype]
    block = desc.block_size * desc.num_kv_heads * desc.head_dim * kb
    for t, nm in [(k_cache, "k_cache"), (v_cache, "v_cache")]:
        _check_tensor(t, nm, desc.num_blocks * block)
    hb = host_k.numel() * host_k.element_size()
    if (host_k.is_cuda or host_v.is_cuda or not host_k.is_pinned() or not host_v.is_pinned()
            or hb % block or host_v.numel() * host_v.element_size() != hb):
        raise ValueError("host_k / host_v must be pinned host tensors of whole blocks")
    n = pairs.shape[0] if pairs.dim() == 2 else 0
    if n:
        _check_i32(pairs, "pairs", n * 2)
    _check(_lib.pa_swap_blocks(_addr(k_cache), _addr(v_cache), _addr(host_k), _addr(host_v),
                               hb // block, _addr(pairs) if n else None, n, int(bool(to_host)),
                               ctypes.byref(desc), _stream(stream)), "pa_swap_blocks")


def pa_decode_balanced_waves(desc):
    """Runs of a balanced launch of this shape on the current device (0 if
    the shape does not take the balanced mode)."""
    return int(_lib.pa_decode_balanced_waves(ctypes.byref(desc)))


def pa_decode_workspace_bytes(desc, num_seqs, max_seq_len, partition_size):
    return int(_lib.pa_decode_workspace_bytes(ctypes.byref(desc), num_seqs, max_seq_len,
                                              partition_size))


def _per_seq(x, name, B):
    if x is None:
        return None
    _check_i32(x, name, B)
    return _addr(x)


def _starts(seq_starts, B):
    return _per_seq(seq_starts, "seq_starts", B)


def _plan(seq_shared, B):
    """seq_shared: the batch's share plan (pa_export_share_plan), an int32
    device tensor of share_plan_words(B) words, or None."""
    if seq_shared is None:
        return None
    _check_i32(seq_shared, "seq_shared", share_plan_words(B))
    return _addr(seq_shared)


def pa_decode(q, k_cache, v_cache, block_tables, seq_lens, max_seq_len, scale, out, desc,
              k_scale=1.0, v_scale=1.0, workspace=None, partition_size=PARTITION_NONE,
              stream=None, seq_starts=None, seq_shared=None):
    B = seq_lens.numel()
    _check_lens_tables(seq_lens, block_tables, B)
    qb, kb = DTYPE_BYTES[desc.q_dtype], DTYPE_BYTES[desc.kv_dtype]
    qrow = desc.num_q_heads * desc.head_dim
    cache_bytes = desc.num_blocks * desc.block_size * desc.num_kv_heads * desc.head_dim * kb
    _check_tensor(q, "q", B * qrow * qb)
    _check_tensor(out, "out", B * qrow * qb)
    for t, nm in [(k_cache, "k_cache"), (v_cache, "v_cache")]:
        _check_tensor(t, nm, cache_bytes)
    ws_bytes = 0
    if workspace is not None:
        _check_tensor(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.pa_decode(_addr(q), _addr(k_cache), _addr(v_cache), _addr(block_tables),
                          block_tables.shape[1], _addr(seq_lens), _starts(seq_starts, B),
                          _plan(seq_shared, B), B, max_seq_len, scale, k_scale, v_scale, _addr(out), _addr(workspace),
                          ws_bytes, partition_size, ctypes.byref(desc), _stream(stream)),
           "pa_decode")


def pa_decode_append(q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables, seq_lens,
                     max_seq_len, scale, out, desc, k_scale=1.0, v_scale=1.0, workspace=None,
                     partition_size=PARTITION_NONE, stream=None, seq_starts=None,
                     seq_shared=None):
    B = seq_lens.numel()
    _check_lens_tables(seq_lens, block_tables, B)
    qb, kb = DTYPE_BYTES[desc.q_dtype], DTYPE_BYTES[desc.kv_dtype]
    qrow = desc.num_q_heads * desc.head_dim
    krow = desc.num_kv_heads * desc.head_dim
    cache_bytes = desc.num_blocks * desc.block_size * desc.num_kv_heads * desc.head_dim * kb
    _check_tensor(q, "q", B * qrow * qb)
    _check_tensor(out, "out", B * qrow * qb)
    _check_tensor(k_new, "k_new", B * krow * qb)
    _check_tensor(v_new, "v_new", B * krow * qb)
    _check_i32(slot_mapping, "slot_mapping", B)
    for t, nm in [(k_cache, "k_cache"), (v_cache, "v_cache")]:
        _check_tensor(t, nm, cache_bytes)
    ws_bytes = 0
    if workspace is not None:
        _check_tensor(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.pa_decode_append(_addr(q), _addr(k_new), _addr(v_new), _addr(slot_mapping),
                                 _addr(k_cache), _addr(v_cache), _addr(block_tables),
                                 block_tables.shape[1], _addr(seq_lens), _starts(seq_starts, B),
                                 _plan(seq_shared, B), B, max_seq_len, scale, k_scale, v_scale, _addr(out),
                                 _addr(workspace), ws_bytes, partition_size, ctypes.byref(desc),
                                 _stream(stream)), "pa_decode_append")


def pa_decode_append_noalloc(q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables,
                             seq_lens, max_seq_len, scale, out, desc, k_scale=1.0, v_scale=1.0,
                             partition_size=PARTITION_NONE, stream=None, seq_starts=None,
                             seq_shared=None):
    """pa_decode_append with the partial states in the library's per-GPU
    scratch instead of a caller workspace (see pa.h)."""
    B = seq_lens.numel()
    _check_lens_tables(seq_lens, block_tables, B)
    qb, kb = DTYPE_BYTES[desc.q_dtype], DTYPE_BYTES[desc.kv_dtype]
    qrow = desc.num_q_heads * desc.head_dim
    krow = desc.num_kv_heads * desc.head_dim
    cache_bytes = desc.num_blocks * desc.block_size * desc.num_kv_heads * desc.head_dim * kb
    _check_tensor(q, "q", B * qrow * qb)
    _check_tensor(out, "out", B * qrow * qb)
    _check_tensor(k_new, "k_new", B * krow * qb)
    _check_tensor(v_new, "v_new", B * krow * qb)
    _check_i32(slot_mapping, "slot_mapping", B)
    for t, nm in [(k_cache, "k_cache"), (v_cache, "v_cache")]:
        _check_tensor(t, nm, cache_bytes)
    _check(_lib.pa_decode_append_noalloc(
        _addr(q), _addr(k_new), _addr(v_new), _addr(slot_mapping), _addr(k_cache),
        _addr(v_cache), _addr(block_tables), block_tables.shape[1], _addr(seq_lens),
        _starts(seq_starts, B), _plan(seq_shared, B), B, max_seq_len, scale,
        k_scale, v_scale, _addr(out), partition_size, ctypes.byref(desc), _stream(stream)),
        "pa_decode_append_noalloc")


def pa_decode_partials(q, k_cache, v_cache, block_tables, seq_lens, max_seq_len, scale, out,
                       desc, workspace, partition_size, k_scale=1.0, v_scale=1.0, stream=None,
                       seq_starts=None, seq_shared=None):
    """The first launch of a partitioned pa_decode.  In the balanced mode it
    writes the rows of the (sequence, KV head) segments one work item covers
    whole to `out`; pa_decode_merge writes the others."""
    B = seq_lens.numel()
    _check_lens_tables(seq_lens, block_tables, B)
    qb, kb = DTYPE_BYTES[desc.q_dtype], DTYPE_BYTES[desc.kv_dtype]
    qrow = desc.num_q_heads * desc.head_dim
    cache_bytes = desc.num_blocks * desc.block_size * desc.num_kv_heads * desc.head_dim * kb
    _check_tensor(q, "q", B * qrow * qb)
    _check_tensor(out, "out", B * qrow * qb)
    for t, nm in [(k_cache, "k_cache"), (v_cache, "v_cache")]:
        _check_tensor(t, nm, cache_bytes)
    _check_tensor(workspace, "workspace")
    _check(_lib.pa_decode_partials(_addr(q), _addr(k_cache), _addr(v_cache), _addr(block_tables),
                                   block_tables.shape[1], _addr(seq_lens),
                                   _starts(seq_starts, B), _plan(seq_shared, B),
                                   B, max_seq_len, scale,
                                   k_scale, v_scale, _addr(out), _addr(workspace),
                                   workspace.numel() * workspace.element_size(), partition_size,
                                   ctypes.byref(desc), _stream(stream)), "pa_decode_partials")


def pa_decode_merge(seq_lens, max_blocks_per_seq, max_seq_len, out, desc, workspace,
                    partition_size, stream=None, seq_shared=None):
    B = seq_lens.numel()
    qrow = desc.num_q_heads * desc.head_dim
    _check_i32(seq_lens, "seq_lens", B)
    _check_tensor(workspace, "workspace")
    _check_tensor(out, "out", B * qrow * DTYPE_BYTES[desc.q_dtype])
    _check(_lib.pa_decode_merge(_addr(seq_lens), _plan(seq_shared, B), B, max_blocks_per_seq,
                                max_seq_len, _addr(out),
                                _addr(workspace), workspace.numel() * workspace.element_size(),
                                partition_size, ctypes.byref(desc), _stream(stream)),
           "pa_decode_merge")


def pa_read_probe(buf, loads_in_flight, workgroups, sink, nontemporal=True, one_per_cu=True,
                  stream=None):
    """One read of the whole device tensor `buf` (see pa.h); sink: a device
    tensor of at least 4 bytes."""
    _check_tensor(buf, "buf")
    _check_tensor(sink, "sink")
    if sink.numel() * sink.element_size() < 4:
        raise ValueError("sink must hold at least 4 bytes")
    _check(_lib.pa_read_probe(_addr(buf), buf.numel() * buf.element_size(), loads_in_flight,
                              workgroups, int(bool(nontemporal)), int(bool(one_per_cu)),
                              _addr(sink), _stream(stream)), "pa_read_probe")


def pa_last_error():
    return _lib.pa_last_error().decode()
