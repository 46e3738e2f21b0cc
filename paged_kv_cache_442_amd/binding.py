"""Thin ctypes binding over ``libpa.so`` (C ABI in ``include/pa.h``).

Functions carry the C names and only marshal arguments: torch tensors become
device pointers, the current torch stream becomes the ``hipStream_t``, host arrays
become numpy buffers.  Every step of the computation runs in the library; if the
library is missing the first call raises, there is no fallback.
"""

import contextlib
import ctypes
import os

import numpy as np

F32, F16, BF16, FP8_E4M3 = 0, 1, 2, 3

PA_OK, PA_E_INVAL, PA_E_NOMEM, PA_E_HIP, PA_E_UNSUPPORTED, PA_E_RANGE = 0, -1, -2, -3, -4, -5

# PA_LIB_PATH selects another build of the same library (the default is the in-tree one).
LIB_PATH = os.environ.get("PA_LIB_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                         "libpa.so")
# The debug build: the same library with the caller's slot and copy-pair preconditions
# checked before each launch.
DEBUG_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa_debug.so")

_lib = None


class PAError(RuntimeError):
    def __init__(self, code, message):
        super().__init__("%s (code %d)" % (message, code))
        self.code = code


class PoolDesc(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("kv_dtype", ctypes.c_int32)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_PI32 = ctypes.POINTER(ctypes.c_int32)
_PI64 = ctypes.POINTER(ctypes.c_int64)
_DECODE_ARGS = [_P, _I32, _P, _I32, _I32, _P, _I32, _P, _I32, ctypes.c_float, _I32, _P, _P,
                _I64, _P]

_SIGNATURES = {
    "pa_block_bytes": (_I64, [ctypes.POINTER(PoolDesc)]),
    "pa_pool_bytes": (_I64, [ctypes.POINTER(PoolDesc)]),
    "pa_alloc_pool": (ctypes.c_int, [ctypes.POINTER(PoolDesc), _P, _I64, _PI32, ctypes.POINTER(_P)]),
    "pa_free_pool": (ctypes.c_int, [_P]),
    "pa_pool_layer_ptrs": (ctypes.c_int, [_P, _I32, ctypes.POINTER(_P), ctypes.POINTER(_P)]),
    "pa_pool_set_kv_scales": (ctypes.c_int, [_P, _I32, ctypes.c_float, ctypes.c_float]),
    "pa_seq_new": (ctypes.c_int, [_P, _PI32]),
    "pa_seq_append": (ctypes.c_int, [_P, _I32, _I32, _PI64, _PI32, _I32, _PI32]),
    "pa_seq_append_batch": (ctypes.c_int, [_P, _PI32, _I32, _PI32, _PI64, _PI32, _I32, _PI32]),
    "pa_seq_fork": (ctypes.c_int, [_P, _I32, _PI32]),
    "pa_seq_free": (ctypes.c_int, [_P, _I32]),
    "pa_seq_length": (ctypes.c_int, [_P, _I32, _PI32]),
    "pa_export_block_tables": (ctypes.c_int, [_P, _PI32, _I32, _I32, _PI32, _PI32]),
    "pa_block_refcount": (ctypes.c_int, [_P, _I32, _PI32]),
    "pa_num_free_blocks": (ctypes.c_int, [_P, _PI32]),
    "pa_export_free_stack": (ctypes.c_int, [_P, _PI32, _I32, _PI32]),
    "pa_reshape_and_cache": (ctypes.c_int, [_P, _I32, _P, _P, _P, _I32, _P]),
    "pa_copy_blocks": (ctypes.c_int, [_P, _P, _I32, _P]),
    "pa_decode_workspace_bytes": (_I64, [_P, _I32, _I32, _I32, _I32]),
    "pa_decode_default_partition": (_I32, [_P, _I32]),
    "pa_decode": (ctypes.c_int, _DECODE_ARGS),
    "pa_decode_plan": (ctypes.c_int, _DECODE_ARGS),
    "pa_decode_partitions": (ctypes.c_int, _DECODE_ARGS),
    "pa_decode_reduce": (ctypes.c_int, _DECODE_ARGS),
    "pa_cache_and_decode": (ctypes.c_int, [_P, _I32, _P, _P, _P, _I32] + _DECODE_ARGS[2:]),
    "pa_cache_and_decode_plan": (ctypes.c_int, [_P, _I32, _P, _P, _P, _I32] + _DECODE_ARGS[2:]),
    "pa_cache_and_decode_window": (ctypes.c_int, [_P, _I32, _P, _P, _P, _I32, _P, _I32, _I32, _P,
                                                  _I32, _P, _I32, _I32, ctypes.c_float, _I32, _P,
                                                  _P, _I64, _P]),
    "pa_prefill_workspace_bytes": (_I64, [_P, _I32, _I32, _I32]),
    "pa_prefill_part_keys": (_I32, []),
    "pa_prefill_chunked": (ctypes.c_int, [_P, _I32, _P, _I32, _I32, _P, _I32, _P, _I32, _P, _I32,
                                          _I32, ctypes.c_float, _P, _P, _I64, _P]),
    "pa_decode_window": (ctypes.c_int, [_P, _I32, _P, _I32, _I32, _P, _I32, _P, _I32, _I32,
                                        ctypes.c_float, _I32, _P, _P, _I64, _P]),
    "pa_seq_release_before": (ctypes.c_int, [_P, _I32, _I32, _PI32]),
    "pa_pool_enable_prefix_caching": (ctypes.c_int, [_P]),
    "pa_seq_new_prefix": (ctypes.c_int, [_P, _PI32, _I32, _PI32, _PI32]),
    "pa_seq_append_tokens": (ctypes.c_int, [_P, _I32, _PI32, _I32, _PI64, _PI32, _I32, _PI32]),
    "pa_seq_append_batch_tokens": (ctypes.c_int, [_P, _PI32, _I32, _PI32, _PI32, _PI64, _PI32, _I32,
                                                  _PI32]),
    "pa_block_state": (ctypes.c_int, [_P, _I32, _PI32]),
    "pa_export_evictable": (ctypes.c_int, [_P, _PI32, _I32, _PI32]),
    "pa_swap_space_bytes": (_I64, [ctypes.POINTER(PoolDesc), _I32]),
    "pa_pool_set_swap_space": (ctypes.c_int, [_P, _I32]),
    "pa_seq_swap_out": (ctypes.c_int, [_P, _PI32, _I32, _PI32, _I32, _PI32]),
    "pa_seq_swap_in": (ctypes.c_int, [_P, _PI32, _I32, _PI32, _I32, _PI32]),
    "pa_seq_swapped": (ctypes.c_int, [_P, _I32, _PI32]),
    "pa_host_block_refcount": (ctypes.c_int, [_P, _I32, _PI32]),
    "pa_export_host_free_stack": (ctypes.c_int, [_P, _PI32, _I32, _PI32]),
    "pa_swap_blocks": (ctypes.c_int, [_P, _P, _I64, _P, _I32, _I32, _P]),
    "pa_static_scratch_bytes": (_I64, []),
    "pa_cache_and_decode_static": (ctypes.c_int, [_P, _I32, _P, _P, _P, _I32, _P, _I32, _I32, _P,
                                                  _I32, _P, _I32, ctypes.c_float, _I32, _P, _P]),
    "pa_check_slots": (ctypes.c_int, [_PI64, _I32, _I64]),
    "pa_check_copy_pairs": (ctypes.c_int, [_PI32, _I32, _I32]),
    "pa_debug_build": (_I32, []),
    "pa_last_error": (ctypes.c_char_p, []),
}


def bind(path):
    """A ctypes handle on the build of the library at ``path``, every prototype set;
    raises if it has not been built."""
    if not os.path.exists(path):
        raise RuntimeError("%s is not built; run __graft_entry__.build()" % path)
    handle = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


def lib():
    """The library every call below goes to: ``libpa.so``, loaded once (or the build
    selected by ``using_library``)."""
    global _lib
    if _lib is None:
        _lib = bind(LIB_PATH)
    return _lib


@contextlib.contextmanager
def using_library(path):
    """Route the calls made inside the block to another build of the library (e.g. the
    debug build); pools created there are freed by the build that created them."""
    global _lib
    saved = lib()
    _lib = bind(path)
    try:
        yield _lib
    finally:
        _lib = saved


def _check(rc):
    if rc < 0:
        raise PAError(int(rc), lib().pa_last_error().decode())
    return rc


def _i32p(a):
    return a.ctypes.data_as(_PI32)


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, dtype=None, name="tensor"):
    """Device pointer of a contiguous GPU tensor (checked on the host)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must have dtype %s, not %s" % (name, dtype, t.dtype))
    return ctypes.c_void_p(t.data_ptr())


def torch_dtype(kv_dtype):
    """dtype of the rows and queries the library takes for a cache of ``kv_dtype`` (an
    FP8 cache takes bf16 and quantizes on the way in)."""
    import torch
    return {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16,
            FP8_E4M3: torch.bfloat16}[kv_dtype]


class Pool:
    """A ``pa_pool*`` plus the caller-owned device tensor backing it (kept alive here)."""

    def __init__(self, handle, desc, storage):
        self.handle = handle
        self.desc = desc
        self.storage = storage
        self.owner = lib()  # the build that created the pool frees it

    @property
    def num_blocks(self):
        return self.desc.num_blocks

    @property
    def block_size(self):
        return self.desc.block_size

    def __del__(self):
        if getattr(self, "handle", None) and getattr(self, "owner", None) is not None:
            self.owner.pa_free_pool(self.handle)
            self.handle = None


def make_desc(num_layers, num_blocks, block_size, num_kv_heads, head_dim, kv_dtype):
    return PoolDesc(num_layers, num_blocks, block_size, num_kv_heads, head_dim, kv_dtype)


def pa_block_bytes(desc):
    return _check(lib().pa_block_bytes(ctypes.byref(desc)))


def pa_pool_bytes(desc):
    return _check(lib().pa_pool_bytes(ctypes.byref(desc)))


def pa_alloc_pool(desc, storage=None, initial_free_order=None):
    """Bind ``storage`` (a GPU tensor of at least ``pa_pool_bytes`` bytes) or, with
    ``storage=None``, build a host-only pool (manager only)."""
    order = None
    if initial_free_order is not None:
        order = np.ascontiguousarray(initial_free_order, dtype=np.int32)
        if order.shape != (desc.num_blocks,):
            raise ValueError("initial_free_order must have num_blocks entries")
    if storage is None:
        base, nbytes = None, 0
    else:
        base = _dev(storage, name="storage")
        nbytes = storage.numel() * storage.element_size()
    out = ctypes.c_void_p()
    _check(lib().pa_alloc_pool(ctypes.byref(desc), base, nbytes,
                               None if order is None else _i32p(order), ctypes.byref(out)))
    return Pool(out, desc, storage)


def pa_free_pool(pool):
    if pool.handle:
        _check(pool.owner.pa_free_pool(pool.handle))
        pool.handle = None


def pa_debug_build():
    return int(lib().pa_debug_build())


def pa_check_slots(slots, num_slots):
    """Host check that the slots of one cache write are distinct (raises PAError)."""
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    buf = slots if len(slots) else np.zeros(1, np.int64)
    _check(lib().pa_check_slots(buf.ctypes.data_as(_PI64), len(slots), int(num_slots)))


def pa_check_copy_pairs(pairs, num_blocks):
    """Host check of one copy call's (src, dst) pairs: distinct destinations, none also a
    source (raises PAError)."""
    pairs = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    buf = pairs if len(pairs) else np.zeros((1, 2), np.int32)
    _check(lib().pa_check_copy_pairs(_i32p(buf), len(pairs), int(num_blocks)))


def pa_pool_layer_ptrs(pool, layer):
    k, v = ctypes.c_void_p(), ctypes.c_void_p()
    _check(lib().pa_pool_layer_ptrs(pool.handle, layer, ctypes.byref(k), ctypes.byref(v)))
    return k.value, v.value


def pa_pool_set_kv_scales(pool, layer, k_scale, v_scale):
    _check(lib().pa_pool_set_kv_scales(pool.handle, layer, float(k_scale), float(v_scale)))


def pa_seq_new(pool):
    s = ctypes.c_int32()
    _check(lib().pa_seq_new(pool.handle, ctypes.byref(s)))
    return s.value


def pa_seq_append(pool, seq, n_tokens):
    """Returns ``(slots int64[n], cow_pairs list of (src, dst))``."""
    slots = np.zeros(max(1, n_tokens), dtype=np.int64)
    pairs = np.zeros(2, dtype=np.int32)
    n_cow = ctypes.c_int32()
    _check(lib().pa_seq_append(pool.handle, seq, n_tokens, slots.ctypes.data_as(_PI64),
                               _i32p(pairs), 1, ctypes.byref(n_cow)))
    return slots[:n_tokens], [(int(pairs[0]), int(pairs[1]))] if n_cow.value else []


def pa_seq_append_batch(pool, seqs, n_tokens=None):
    """Returns ``(slots int64[sum n], cow_pairs list of (src, dst))`` for the whole batch."""
    seqs = np.ascontiguousarray(seqs, dtype=np.int32)
    counts = np.ones(len(seqs), np.int32) if n_tokens is None else \
        np.ascontiguousarray(n_tokens, dtype=np.int32)
    total = int(counts.sum())
    slots = np.zeros(max(1, total), dtype=np.int64)
    cap = max(1, len(seqs))
    pairs = np.zeros(2 * cap, dtype=np.int32)
    n_cow = ctypes.c_int32()
    _check(lib().pa_seq_append_batch(pool.handle, _i32p(seqs), len(seqs),
                                     None if n_tokens is None else _i32p(counts),
                                     slots.ctypes.data_as(_PI64), _i32p(pairs), cap,
                                     ctypes.byref(n_cow)))
    return slots[:total], [(int(pairs[2 * i]), int(pairs[2 * i + 1])) for i in range(n_cow.value)]


def pa_seq_append_tokens(pool, seq, tokens):
    """``pa_seq_append`` with the tokens' ids; returns ``(slots, cow_pairs)``."""
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    n = len(tokens)
    slots = np.zeros(max(1, n), dtype=np.int64)
    pairs = np.zeros(2, dtype=np.int32)
    n_cow = ctypes.c_int32()
    _check(lib().pa_seq_append_tokens(pool.handle, seq, _i32p(tokens), n, slots.ctypes.data_as(_PI64),
                                      _i32p(pairs), 1, ctypes.byref(n_cow)))
    return slots[:n], [(int(pairs[0]), int(pairs[1]))] if n_cow.value else []


def pa_seq_append_batch_tokens(pool, seqs, tokens, n_tokens=None):
    """``pa_seq_append_batch`` with the ids of every appended token, back to back."""
    seqs = np.ascontiguousarray(seqs, dtype=np.int32)
    counts = np.ones(len(seqs), np.int32) if n_tokens is None else \
        np.ascontiguousarray(n_tokens, dtype=np.int32)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    total = int(counts.sum())
    if len(tokens) != total:
        raise ValueError("one token id per appended token")
    slots = np.zeros(max(1, total), dtype=np.int64)
    tok = tokens if total else np.zeros(1, np.int32)
    cap = max(1, len(seqs))
    pairs = np.zeros(2 * cap, dtype=np.int32)
    n_cow = ctypes.c_int32()
    _check(lib().pa_seq_append_batch_tokens(pool.handle, _i32p(seqs), len(seqs),
                                            None if n_tokens is None else _i32p(counts), _i32p(tok),
                                            slots.ctypes.data_as(_PI64), _i32p(pairs), cap,
                                            ctypes.byref(n_cow)))
    return slots[:total], [(int(pairs[2 * i]), int(pairs[2 * i + 1])) for i in range(n_cow.value)]


def pa_pool_enable_prefix_caching(pool):
    _check(lib().pa_pool_enable_prefix_caching(pool.handle))


def pa_seq_new_prefix(pool, prompt):
    """Returns ``(seq, n_cached_tokens)``."""
    prompt = np.ascontiguousarray(prompt, dtype=np.int32)
    buf = prompt if len(prompt) else np.zeros(1, np.int32)
    s, c = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().pa_seq_new_prefix(pool.handle, _i32p(buf), len(prompt), ctypes.byref(s),
                                   ctypes.byref(c)))
    return s.value, c.value


BLOCK_FREE_EMPTY, BLOCK_IN_USE, BLOCK_FREE_CACHED = 0, 1, 2


def pa_block_state(pool, block):
    st = ctypes.c_int32()
    _check(lib().pa_block_state(pool.handle, block, ctypes.byref(st)))
    return st.value


def pa_export_evictable(pool):
    cap = pool.num_blocks
    out = np.zeros(max(1, cap), dtype=np.int32)
    n = ctypes.c_int32()
    _check(lib().pa_export_evictable(pool.handle, _i32p(out), cap, ctypes.byref(n)))
    return out[:n.value]


def pa_swap_space_bytes(desc, host_blocks):
    return _check(lib().pa_swap_space_bytes(ctypes.byref(desc), host_blocks))


def pa_pool_set_swap_space(pool, host_blocks):
    _check(lib().pa_pool_set_swap_space(pool.handle, host_blocks))
    pool.num_host_blocks = host_blocks


def _swap(fn, pool, seqs):
    seqs = np.ascontiguousarray(seqs, dtype=np.int32)
    cap = max(1, getattr(pool, "num_host_blocks", 0), pool.num_blocks)
    pairs = np.zeros(2 * cap, dtype=np.int32)
    n = ctypes.c_int32()
    _check(fn(pool.handle, _i32p(seqs if len(seqs) else np.zeros(1, np.int32)), len(seqs),
              _i32p(pairs), cap, ctypes.byref(n)))
    return [(int(pairs[2 * i]), int(pairs[2 * i + 1])) for i in range(n.value)]


def pa_seq_swap_out(pool, seqs):
    """Returns the (device block, host block) pairs to copy."""
    return _swap(lib().pa_seq_swap_out, pool, seqs)


def pa_seq_swap_in(pool, seqs):
    """Returns the (host block, device block) pairs to copy."""
    return _swap(lib().pa_seq_swap_in, pool, seqs)


def pa_seq_swapped(pool, seq):
    out = ctypes.c_int32()
    _check(lib().pa_seq_swapped(pool.handle, seq, ctypes.byref(out)))
    return bool(out.value)


def pa_host_block_refcount(pool, host_block):
    rc = ctypes.c_int32()
    _check(lib().pa_host_block_refcount(pool.handle, host_block, ctypes.byref(rc)))
    return rc.value


def pa_export_host_free_stack(pool):
    cap = max(1, getattr(pool, "num_host_blocks", 0))
    out = np.zeros(cap, dtype=np.int32)
    n = ctypes.c_int32()
    _check(lib().pa_export_host_free_stack(pool.handle, _i32p(out), cap, ctypes.byref(n)))
    return out[:n.value]


def pa_swap_blocks(pool, host, pairs, to_host, stream=None):
    """host: pinned CPU tensor (the swap space); pairs: GPU int32 ``[n][2]``."""
    import torch
    if host.device.type != "cpu" or not host.is_pinned():
        raise ValueError("the swap space must be a pinned CPU tensor")
    n = pairs.shape[0] if pairs.numel() else 0
    _check(lib().pa_swap_blocks(pool.handle, ctypes.c_void_p(host.data_ptr()),
                                host.numel() * host.element_size(),
                                _dev(pairs, torch.int32, "pairs") if n else None, n,
                                1 if to_host else 0, _stream(stream)))


def pa_seq_fork(pool, parent):
    c = ctypes.c_int32()
    _check(lib().pa_seq_fork(pool.handle, parent, ctypes.byref(c)))
    return c.value


def pa_seq_free(pool, seq):
    _check(lib().pa_seq_free(pool.handle, seq))


def pa_seq_length(pool, seq):
    n = ctypes.c_int32()
    _check(lib().pa_seq_length(pool.handle, seq, ctypes.byref(n)))
    return n.value


def pa_export_block_tables(pool, seqs, max_blocks):
    seqs = np.ascontiguousarray(seqs, dtype=np.int32)
    tables = np.zeros((max(1, len(seqs)), max(1, max_blocks)), dtype=np.int32)
    ctx = np.zeros(max(1, len(seqs)), dtype=np.int32)
    _check(lib().pa_export_block_tables(pool.handle, _i32p(seqs), len(seqs), max_blocks,
                                        _i32p(tables), _i32p(ctx)))
    return tables[:len(seqs), :max_blocks], ctx[:len(seqs)]


def pa_block_refcount(pool, block):
    rc = ctypes.c_int32()
    _check(lib().pa_block_refcount(pool.handle, block, ctypes.byref(rc)))
    return rc.value


def pa_num_free_blocks(pool):
    n = ctypes.c_int32()
    _check(lib().pa_num_free_blocks(pool.handle, ctypes.byref(n)))
    return n.value


def pa_export_free_stack(pool):
    cap = pool.num_blocks
    out = np.zeros(max(1, cap), dtype=np.int32)
    n = ctypes.c_int32()
    _check(lib().pa_export_free_stack(pool.handle, _i32p(out), cap, ctypes.byref(n)))
    return out[:n.value]


def pa_reshape_and_cache(pool, layer, k, v, slots, stream=None):
    """k, v: GPU ``[n][H_kv][d]`` in the pool dtype; slots: GPU int64 ``[n]``."""
    import torch
    dt = torch_dtype(pool.desc.kv_dtype)
    n = slots.numel()
    if k.shape[0] != n or v.shape != k.shape:
        raise ValueError("k, v and slots disagree on the token count")
    _check(lib().pa_reshape_and_cache(pool.handle, layer, _dev(k, dt, "k"), _dev(v, dt, "v"),
                                      _dev(slots, torch.int64, "slots"), n, _stream(stream)))


def pa_copy_blocks(pool, pairs, stream=None):
    """pairs: GPU int32 ``[n][2]`` of (src, dst)."""
    import torch
    n = pairs.shape[0] if pairs.numel() else 0
    _check(lib().pa_copy_blocks(pool.handle, _dev(pairs, torch.int32, "pairs") if n else None, n,
                                _stream(stream)))


def pa_decode_default_partition(pool, num_q_heads):
    return _check(lib().pa_decode_default_partition(pool.handle, num_q_heads))


def pa_decode_workspace_bytes(pool, num_seqs, num_q_heads, max_context, partition_tokens=0):
    return _check(lib().pa_decode_workspace_bytes(pool.handle, num_seqs, num_q_heads, max_context,
                                                  partition_tokens))


def _decode(fn, pool, layer, q, block_tables, context_lens, max_context, scale, out, workspace,
            partition_tokens, stream):
    import torch
    S, H_q = q.shape[0], q.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(fn(pool.handle, layer, _dev(q, torch_dtype(pool.desc.kv_dtype), "q"), S, H_q,
              _dev(block_tables, torch.int32, "block_tables"), block_tables.shape[1],
              _dev(context_lens, torch.int32, "context_lens"), max_context, float(scale),
              partition_tokens, _dev(out, torch.float32, "out"),
              None if workspace is None else _dev(workspace, name="workspace"), ws_bytes,
              _stream(stream)))


def pa_decode(pool, layer, q, block_tables, context_lens, max_context, scale, out, workspace,
              partition_tokens=0, stream=None):
    """q: GPU ``[S][H_q][d]`` pool dtype; out: GPU fp32 ``[S][H_q][d]``."""
    _decode(lib().pa_decode, pool, layer, q, block_tables, context_lens, max_context, scale, out,
            workspace, partition_tokens, stream)


def pa_decode_plan(pool, layer, q, block_tables, context_lens, max_context, scale, out, workspace,
                   partition_tokens=0, stream=None):
    _decode(lib().pa_decode_plan, pool, layer, q, block_tables, context_lens, max_context, scale,
            out, workspace, partition_tokens, stream)


def pa_decode_partitions(pool, layer, q, block_tables, context_lens, max_context, scale, out,
                         workspace, partition_tokens=0, stream=None):
    _decode(lib().pa_decode_partitions, pool, layer, q, block_tables, context_lens, max_context,
            scale, out, workspace, partition_tokens, stream)


def pa_decode_reduce(pool, layer, q, block_tables, context_lens, max_context, scale, out,
                     workspace, partition_tokens=0, stream=None):
    _decode(lib().pa_decode_reduce, pool, layer, q, block_tables, context_lens, max_context,
            scale, out, workspace, partition_tokens, stream)


def _cache_and_decode(fn, pool, layer, k, v, slots, q, block_tables, context_lens, max_context,
                      scale, out, workspace, partition_tokens, stream):
    import torch
    dt = torch_dtype(pool.desc.kv_dtype)
    n = slots.numel()
    if k.shape[0] != n or v.shape != k.shape:
        raise ValueError("k, v and slots disagree on the token count")
    S, H_q = q.shape[0], q.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(fn(pool.handle, layer, _dev(k, dt, "k"), _dev(v, dt, "v"),
              _dev(slots, torch.int64, "slots"), n, _dev(q, dt, "q"), S, H_q,
              _dev(block_tables, torch.int32, "block_tables"), block_tables.shape[1],
              _dev(context_lens, torch.int32, "context_lens"), max_context, float(scale),
              partition_tokens, _dev(out, torch.float32, "out"),
              None if workspace is None else _dev(workspace, name="workspace"), ws_bytes,
              _stream(stream)))


def pa_cache_and_decode(pool, layer, k, v, slots, q, block_tables, context_lens, max_context,
                        scale, out, workspace, partition_tokens=0, stream=None):
    """``pa_reshape_and_cache(k, v, slots)`` then ``pa_decode(q, ...)``, in three launches."""
    _cache_and_decode(lib().pa_cache_and_decode, pool, layer, k, v, slots, q, block_tables,
                      context_lens, max_context, scale, out, workspace, partition_tokens, stream)


def pa_static_scratch_bytes():
    return int(lib().pa_static_scratch_bytes())


def pa_cache_and_decode_static(pool, layer, k, v, slots, q, block_tables, context_lens,
                               max_context, scale, out, partition_tokens=0, stream=None):
    """``pa_cache_and_decode`` with the library's own static workspace (no allocation)."""
    import torch
    dt = torch_dtype(pool.desc.kv_dtype)
    n = slots.numel()
    if k.shape[0] != n or v.shape != k.shape:
        raise ValueError("k, v and slots disagree on the token count")
    S, H_q = q.shape[0], q.shape[1]
    _check(lib().pa_cache_and_decode_static(
        pool.handle, layer, _dev(k, dt, "k"), _dev(v, dt, "v"), _dev(slots, torch.int64, "slots"), n,
        _dev(q, dt, "q"), S, H_q, _dev(block_tables, torch.int32, "block_tables"),
        block_tables.shape[1], _dev(context_lens, torch.int32, "context_lens"), max_context,
        float(scale), partition_tokens, _dev(out, torch.float32, "out"), _stream(stream)))


def pa_cache_and_decode_plan(pool, layer, k, v, slots, q, block_tables, context_lens, max_context,
                             scale, out, workspace, partition_tokens=0, stream=None):
    _cache_and_decode(lib().pa_cache_and_decode_plan, pool, layer, k, v, slots, q, block_tables,
                      context_lens, max_context, scale, out, workspace, partition_tokens, stream)


def pa_cache_and_decode_window(pool, layer, k, v, slots, q, block_tables, context_lens, max_context,
                               window, scale, out, workspace, partition_tokens=0, stream=None):
    """``pa_reshape_and_cache(k, v, slots)`` then ``pa_decode_window(q, ...)``, in three
    launches."""
    import torch
    dt = torch_dtype(pool.desc.kv_dtype)
    n = slots.numel()
    if k.shape[0] != n or v.shape != k.shape:
        raise ValueError("k, v and slots disagree on the token count")
    S, H_q = q.shape[0], q.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pa_cache_and_decode_window(
        pool.handle, layer, _dev(k, dt, "k"), _dev(v, dt, "v"), _dev(slots, torch.int64, "slots"), n,
        _dev(q, dt, "q"), S, H_q, _dev(block_tables, torch.int32, "block_tables"),
        block_tables.shape[1], _dev(context_lens, torch.int32, "context_lens"), max_context, window,
        float(scale), partition_tokens, _dev(out, torch.float32, "out"),
        None if workspace is None else _dev(workspace, name="workspace"), ws_bytes, _stream(stream)))


def pa_prefill_part_keys():
    return _check(lib().pa_prefill_part_keys())


def pa_prefill_workspace_bytes(pool, num_rows, num_q_heads, max_context):
    return _check(lib().pa_prefill_workspace_bytes(pool.handle, num_rows, num_q_heads, max_context))


def pa_prefill_chunked(pool, layer, q, query_start, block_tables, context_lens, max_context,
                       max_query_len, scale, out, workspace=None, stream=None):
    """q: GPU ``[R][H_q][d]`` pool dtype; query_start: GPU int32 ``[S+1]``; out: GPU fp32
    ``[R][H_q][d]``; workspace: GPU uint8 tensor of ``pa_prefill_workspace_bytes`` bytes
    (None when that is 0)."""
    import torch
    R, H_q = q.shape[0], q.shape[1]
    S = query_start.numel() - 1
    ws, ws_bytes = (None, 0) if workspace is None else \
        (_dev(workspace, torch.uint8, "workspace"), workspace.numel())
    _check(lib().pa_prefill_chunked(pool.handle, layer, _dev(q, torch_dtype(pool.desc.kv_dtype), "q"),
                                    R, H_q, _dev(query_start, torch.int32, "query_start"), S,
                                    _dev(block_tables, torch.int32, "block_tables"),
                                    block_tables.shape[1],
                                    _dev(context_lens, torch.int32, "context_lens"), max_context,
                                    max_query_len, float(scale), _dev(out, torch.float32, "out"),
                                    ws, ws_bytes, _stream(stream)))


def pa_decode_window(pool, layer, q, block_tables, context_lens, max_context, window, scale, out,
                     workspace, partition_tokens=0, stream=None):
    """Decode over each sequence's last ``window`` tokens (0 = all)."""
    import torch
    S, H_q = q.shape[0], q.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pa_decode_window(pool.handle, layer, _dev(q, torch_dtype(pool.desc.kv_dtype), "q"), S,
                                  H_q, _dev(block_tables, torch.int32, "block_tables"),
                                  block_tables.shape[1], _dev(context_lens, torch.int32, "context_lens"),
                                  max_context, window, float(scale), partition_tokens,
                                  _dev(out, torch.float32, "out"),
                                  None if workspace is None else _dev(workspace, name="workspace"),
                                  ws_bytes, _stream(stream)))


def pa_seq_release_before(pool, seq, token):
    n = ctypes.c_int32()
    _check(lib().pa_seq_release_before(pool.handle, seq, token, ctypes.byref(n)))
    return n.value

