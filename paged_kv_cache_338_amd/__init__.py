"""Python binding of the paged KV cache library (libpa.so, gfx950).

Argument marshalling only: every computation runs in the library's HIP
kernels or its C++ allocator.  PyTorch supplies device memory and streams.
The functions keep the C names (``pa_cache_append``, ``pa_decode``,
``pa_copy_blocks``, ...); ``Allocator`` wraps the ``pa_allocator_*`` /
``pa_seq_*`` calls of one allocator handle.

The library must be built (``python -m paged_kv_cache_338_amd._build``);
there is no fallback: a missing library raises ``LibraryNotBuilt``.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

# PA_LIBRARY may name another build of the same library (the sanitized host
# build, libpa_sanitize.so); it must exist like the default one.
LIB_PATH = os.environ.get("PA_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libpa.so")

PA_OK = 0
PA_ERR_INVALID_ARGUMENT = 1
PA_ERR_OUT_OF_BLOCKS = 2
PA_ERR_UNKNOWN_SEQ = 3
PA_ERR_UNSUPPORTED = 4
PA_ERR_DEVICE = 5
PA_F32 = 0
PA_BF16 = 1
PA_F16 = 2
PA_TUNE_DECODE_WORKGROUPS = 1
PA_TUNE_PREFILL_KEY_TILES = 2
PA_TUNE_DECODE_KV_CACHED = 3

STATUS_NAMES = {PA_ERR_INVALID_ARGUMENT: "INVALID_ARGUMENT", PA_ERR_OUT_OF_BLOCKS: "OUT_OF_BLOCKS",
                PA_ERR_UNKNOWN_SEQ: "UNKNOWN_SEQ", PA_ERR_UNSUPPORTED: "UNSUPPORTED",
                PA_ERR_DEVICE: "DEVICE"}


class LibraryNotBuilt(RuntimeError):
    pass


class PagedAttentionError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.status_name = STATUS_NAMES.get(status, str(status))


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


_c = ctypes
_P = _c.c_void_p
_I32 = _c.c_int32
_I64 = _c.c_int64
_PI32 = _c.POINTER(_c.c_int32)
_PI64 = _c.POINTER(_c.c_int64)
_PDESC = _c.POINTER(CacheDesc)

# name -> (restype, argtypes); mirrors include/pa.h
SIGNATURES = {
    "pa_abi_version": (_I32, []),
    "pa_set_tuning": (_I32, [_I32, _I32]),
    "pa_get_tuning": (_I32, [_I32, _PI32]),
    "pa_status_string": (_c.c_char_p, [_I32]),
    "pa_last_error": (_c.c_char_p, []),
    "pa_supported": (_I32, [_PDESC, _I32]),
    "pa_cache_append": (_I32, [_P, _P, _P, _I32, _P, _P, _PDESC, _P]),
    "pa_copy_blocks": (_I32, [_P, _I32, _P, _P, _PDESC, _P]),
    "pa_decode": (_I32, [_P, _P, _P, _P, _I32, _P, _I32, _I32, _c.c_float, _P, _I32, _PDESC,
                         _P, _c.c_size_t, _P]),
    "pa_decode_workspace_size": (_I32, [_PDESC, _I32, _I32, _I32, _c.POINTER(_c.c_size_t)]),
    "pa_decode_append": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _P, _I32, _I32, _c.c_float, _P,
                                _I32, _PDESC, _P, _c.c_size_t, _P]),
    "pa_decode_noalloc": (_I32, [_P, _P, _P, _P, _I32, _P, _I32, _I32, _c.c_float, _P, _I32,
                                 _PDESC, _P]),
    "pa_prefill": (_I32, [_P, _P, _P, _P, _I32, _P, _P, _I32, _I32, _I32, _c.c_float, _P, _I32,
                          _PDESC, _P]),
    "pa_prefill_split": (_I32, [_P, _P, _P, _P, _I32, _P, _P, _I32, _I32, _I32, _c.c_float, _P,
                                _I32, _PDESC, _P, _c.c_size_t, _P]),
    "pa_prefill_split_workspace_size": (_I32, [_PDESC, _I32, _I32, _I32, _I32,
                                               _c.POINTER(_c.c_size_t)]),
    "pa_allocator_create": (_I32, [_I32, _I32, _PI32, _c.POINTER(_P)]),
    "pa_allocator_destroy": (None, [_P]),
    "pa_seq_create": (_I32, [_P, _I64]),
    "pa_seq_fork": (_I32, [_P, _I64, _I64]),
    "pa_seq_reserve": (_I32, [_P, _PI64, _PI32, _I32, _PI64, _PI32, _I32, _PI32]),
    "pa_seq_free": (_I32, [_P, _I64]),
    "pa_build_block_tables": (_I32, [_P, _PI64, _I32, _I32, _PI32, _PI32]),
    "pa_allocator_num_free": (_I32, [_P]),
    "pa_allocator_free_list": (_I32, [_P, _PI32, _I32, _PI32]),
    "pa_block_refcount": (_I32, [_P, _I32, _PI32]),
    "pa_seq_block_table": (_I32, [_P, _I64, _PI32, _I32, _PI32]),
    "pa_seq_num_tokens": (_I32, [_P, _I64, _PI32]),
    "pa_swap_blocks": (_I32, [_P, _I32, _P, _P, _I32, _P, _P, _I32, _PDESC, _P]),
    "pa_allocator_add_host_pool": (_I32, [_P, _I32, _PI32]),
    "pa_seq_swap_out": (_I32, [_P, _I64, _PI32, _I32, _PI32]),
    "pa_seq_swap_in": (_I32, [_P, _I64, _PI32, _I32, _PI32]),
    "pa_seq_is_swapped": (_I32, [_P, _I64, _PI32]),
    "pa_allocator_num_free_host": (_I32, [_P]),
    "pa_allocator_host_free_list": (_I32, [_P, _PI32, _I32, _PI32]),
    "pa_allocator_enable_prefix_cache": (_I32, [_P]),
    "pa_seq_match_prefix": (_I32, [_P, _I64, _PI32, _I32, _PI32]),
    "pa_allocator_num_cached": (_I32, [_P]),
    "pa_allocator_cached_list": (_I32, [_P, _PI32, _I32, _PI32]),
    "pa_block_prefix_key": (_I32, [_P, _I32, _PI32, _c.POINTER(_c.c_uint64)]),
}

_lib = None


def load_library():
    """Loads libpa.so once and declares every exported function."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryNotBuilt(f"{LIB_PATH} is missing: run python -m paged_kv_cache_338_amd._build")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status):
    if status != PA_OK:
        raise PagedAttentionError(status, load_library().pa_last_error().decode())


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


# ------------------------------------------------------------------ device
def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype == torch.float16:
        return PA_F16
    raise TypeError(f"unsupported dtype {t.dtype}")


def cache_desc(k_cache):
    """Descriptor of a pool tensor shaped [num_blocks, H_kv, block_size, D]."""
    if k_cache.dim() != 4:
        raise ValueError("pool must be [num_blocks, num_kv_heads, block_size, head_dim]")
    nb, h, bs, d = k_cache.shape
    return CacheDesc(nb, bs, h, d, _dtype_code(k_cache))


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _addressable(t, name):
    """A device tensor, or pinned host memory the GPU reads and writes."""
    if not (t.is_cuda or t.is_pinned()):
        raise ValueError(f"{name} must be a device tensor or pinned host memory")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _same_pool(k_cache, v_cache):
    if k_cache.shape != v_cache.shape or k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache must have the same shape and dtype")


def pa_set_tuning(key, value):
    """Sets a process-wide tuning knob (0 = the library's choice)."""
    _check(load_library().pa_set_tuning(int(key), int(value)))


def pa_get_tuning(key):
    v = ctypes.c_int32(0)
    _check(load_library().pa_get_tuning(int(key), ctypes.byref(v)))
    return v.value


class tuning:
    """Context manager: sets a tuning knob and restores its previous value."""

    def __init__(self, key, value):
        self.key, self.value = key, value

    def __enter__(self):
        self.old = pa_get_tuning(self.key)
        pa_set_tuning(self.key, self.value)
        return self

    def __exit__(self, *exc):
        pa_set_tuning(self.key, self.old)


def pa_supported(desc, num_q_heads):
    return load_library().pa_supported(ctypes.byref(desc), num_q_heads) == PA_OK


def pa_cache_append(k, v, slot_mapping, k_cache, v_cache, stream=None):
    """Writes k[t], v[t] ([T, H_kv, D]) to slot_mapping[t] (int64, <0 = skip)."""
    torch = _torch()
    _same_pool(k_cache, v_cache)
    desc = cache_desc(k_cache)
    T = slot_mapping.numel()
    if slot_mapping.dtype != torch.int64:
        raise TypeError("slot_mapping must be int64")
    want = (T, k_cache.shape[1], k_cache.shape[3])
    if tuple(k.shape) != want or tuple(v.shape) != want:
        raise ValueError(f"k and v must be {want}")
    if k.dtype != k_cache.dtype or v.dtype != k_cache.dtype:
        raise TypeError("k/v dtype must match the pool")
    if T == 0:
        return
    _check(load_library().pa_cache_append(
        _dev(k, "k"), _dev(v, "v"), _dev(slot_mapping, "slot_mapping"), T,
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), ctypes.byref(desc), _stream(stream)))


def pa_copy_blocks(src_dst_pairs, k_cache, v_cache, stream=None):
    """Copies block src -> dst of both pools for each row of int32 [P, 2]."""
    torch = _torch()
    _same_pool(k_cache, v_cache)
    desc = cache_desc(k_cache)
    if src_dst_pairs.dtype != torch.int32:
        raise TypeError("src_dst_pairs must be int32")
    P = src_dst_pairs.numel() // 2
    if src_dst_pairs.numel() != 2 * P:
        raise ValueError("src_dst_pairs must be [P, 2]")
    if P == 0:
        return
    _check(load_library().pa_copy_blocks(
        _dev(src_dst_pairs, "src_dst_pairs"), P, _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), ctypes.byref(desc), _stream(stream)))


def pa_swap_blocks(src_dst_pairs, src_k, src_v, dst_k, dst_v, stream=None):
    """Moves block src of (src_k, src_v) to block dst of (dst_k, dst_v) for each
    row of int32 [P, 2]; either pool pair may be pinned host memory."""
    prepare_swap_blocks(src_dst_pairs, src_dst_pairs.numel() // 2, src_k, src_v, dst_k, dst_v,
                        stream)()


def prepare_swap_blocks(src_dst_pairs, num_pairs, src_k, src_v, dst_k, dst_v, stream=None):
    """pa_swap_blocks over the first num_pairs rows of a fixed pair buffer."""
    torch = _torch()
    _same_pool(src_k, src_v)
    _same_pool(dst_k, dst_v)
    if src_k.shape[1:] != dst_k.shape[1:] or src_k.dtype != dst_k.dtype:
        raise ValueError("source and destination pools differ in block geometry or dtype")
    if src_dst_pairs.dtype != torch.int32 or src_dst_pairs.numel() < 2 * int(num_pairs):
        raise ValueError("src_dst_pairs must be int32 [P, 2] with at least num_pairs rows")
    desc = cache_desc(dst_k)
    lib = load_library()
    args = (_addressable(src_dst_pairs, "src_dst_pairs"), int(num_pairs),
            _addressable(src_k, "src_k"), _addressable(src_v, "src_v"), src_k.shape[0],
            _addressable(dst_k, "dst_k"), _addressable(dst_v, "dst_v"), dst_k.shape[0],
            ctypes.byref(desc), _stream(stream))
    return PreparedCall(lib.pa_swap_blocks, args, (src_dst_pairs, src_k, src_v, dst_k, dst_v,
                                                   desc))


def pa_decode_workspace_size(desc, num_seqs, num_q_heads, max_blocks_per_seq):
    n = ctypes.c_size_t(0)
    _check(load_library().pa_decode_workspace_size(ctypes.byref(desc), num_seqs, num_q_heads,
                                                   max_blocks_per_seq, ctypes.byref(n)))
    return n.value


def decode_workspace(k_cache, num_seqs, num_q_heads, max_blocks_per_seq):
    """Allocates (with torch) a zero-filled workspace sized for pa_decode; one
    workspace serves any number of ordered calls (each leaves it ready for
    the next)."""
    torch = _torch()
    n = pa_decode_workspace_size(cache_desc(k_cache), num_seqs, num_q_heads, max_blocks_per_seq)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=k_cache.device)


def pa_decode(q, k_cache, v_cache, block_tables, context_lens, block_size, scale, out,
              workspace=None, stream=None):
    """out[b, h] = softmax(scale * q[b, h] K_b^T) V_b with K_b/V_b read through
    block_tables[b] (int32 [B, max_blocks]); context_lens int32 [B]."""
    torch = _torch()
    _same_pool(k_cache, v_cache)
    desc = cache_desc(k_cache)
    if q.dim() != 3 or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q and out must be [B, H_q, D] of one shape")
    B, H_q, D = q.shape
    if D != desc.head_dim or q.dtype != k_cache.dtype or out.dtype != k_cache.dtype:
        raise ValueError("q/out must match the pool's head_dim and dtype")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.numel() != B:
        raise ValueError("block_tables must be [B, max_blocks] and context_lens [B]")
    maxb = block_tables.shape[1]
    if workspace is None:
        workspace = decode_workspace(k_cache, B, H_q, maxb)
        if stream is not None and stream != torch.cuda.current_stream():
            # The temporary is freed on return: keep the caching allocator
            # from reusing it before the kernels on `stream` are done.
            workspace.record_stream(stream)
    _check(load_library().pa_decode(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_tables, "block_tables"), maxb, _dev(context_lens, "context_lens"), B,
        int(block_size), float(scale), _dev(out, "out"), H_q, ctypes.byref(desc),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return out


def _check_new_rows(new_k, new_v, k_cache, B):
    shape = (B, k_cache.shape[1], k_cache.shape[3])
    for name, t in (("new_k", new_k), ("new_v", new_v)):
        if tuple(t.shape) != shape or t.dtype != k_cache.dtype:
            raise ValueError(f"{name} must be [B, H_kv, D] = {list(shape)} of the pool's dtype")


def pa_decode_append(q, new_k, new_v, k_cache, v_cache, block_tables, context_lens, block_size,
                     scale, out, workspace=None, stream=None):
    """Writes new_k[b] / new_v[b] ([B, H_kv, D]) at position context_lens[b] - 1
    of sequence b (its slot from block_tables), then decodes as pa_decode,
    in one kernel launch."""
    torch = _torch()
    _same_pool(k_cache, v_cache)
    desc = cache_desc(k_cache)
    if q.dim() != 3 or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q and out must be [B, H_q, D] of one shape")
    B, H_q, D = q.shape
    if D != desc.head_dim or q.dtype != k_cache.dtype or out.dtype != k_cache.dtype:
        raise ValueError("q/out must match the pool's head_dim and dtype")
    _check_new_rows(new_k, new_v, k_cache, B)
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.numel() != B:
        raise ValueError("block_tables must be [B, max_blocks] and context_lens [B]")
    maxb = block_tables.shape[1]
    if workspace is None:
        workspace = decode_workspace(k_cache, B, H_q, maxb)
        if stream is not None and stream != torch.cuda.current_stream():
            workspace.record_stream(stream)
    prepare_decode_append(q, new_k, new_v, k_cache, v_cache, block_tables, context_lens,
                          block_size, scale, out, workspace, stream)()
    return out


def pa_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, block_size, scale, out,
                      stream=None):
    """pa_decode with the library's own per-GPU workspace (no allocation)."""
    torch = _torch()
    _same_pool(k_cache, v_cache)
    desc = cache_desc(k_cache)
    if q.dim() != 3 or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q and out must be [B, H_q, D] of one shape")
    B, H_q, D = q.shape
    if D != desc.head_dim or q.dtype != k_cache.dtype or out.dtype != k_cache.dtype:
        raise ValueError("q/out must match the pool's head_dim and dtype")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.numel() != B:
        raise ValueError("block_tables must be [B, max_blocks] and context_lens [B]")
    _check(load_library().pa_decode_noalloc(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_tables, "block_tables"), block_tables.shape[1],
        _dev(context_lens, "context_lens"), B, int(block_size), float(scale), _dev(out, "out"),
        H_q, ctypes.byref(desc), _stream(stream)))
    return out


def pa_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, block_size, scale,
               out, stream=None):
    """Causal multi-query attention through the block tables: sequence b's
    query rows are q[query_start[b]:query_start[b + 1]] (its last n_b cache
    positions), each attending to the cache up to its own position.
    q, out [T, H_q, D] bf16; block_tables int32 [B, max_blocks]; context_lens
    int32 [B]; query_start int32 [B + 1]."""
    prepare_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, block_size,
                    scale, out, stream)()
    return out


def pa_prefill_split_workspace_size(desc, num_seqs, num_q_heads, num_query_tokens,
                                    max_blocks_per_seq):
    n = ctypes.c_size_t(0)
    _check(load_library().pa_prefill_split_workspace_size(
        ctypes.byref(desc), num_seqs, num_q_heads, num_query_tokens, max_blocks_per_seq,
        ctypes.byref(n)))
    return n.value


def prefill_split_workspace(k_cache, num_seqs, num_q_heads, num_query_tokens,
                            max_blocks_per_seq):
    """Allocates (with torch) a workspace sized for pa_prefill_split on this
    shape (at least 256 bytes; it needs no initialisation)."""
    torch = _torch()
    n = pa_prefill_split_workspace_size(cache_desc(k_cache), num_seqs, num_q_heads,
                                        num_query_tokens, max_blocks_per_seq)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=k_cache.device)


def pa_prefill_split(q, k_cache, v_cache, block_tables, context_lens, query_start, block_size,
                     scale, out, workspace=None, stream=None):
    """pa_prefill with the key range of long query blocks split over several
    workgroups and merged (for few query tokens against long contexts);
    allocates the workspace with torch when none is given."""
    if workspace is None:
        workspace = prefill_split_workspace(k_cache, context_lens.numel(), q.shape[1], q.shape[0],
                                            block_tables.shape[1])
        if stream is not None and stream != _torch().cuda.current_stream():
            workspace.record_stream(stream)
    prepare_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, block_size,
                    scale, out, stream, workspace=workspace)()
    return out


def prepare_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, block_size,
                    scale, out, stream=None, workspace=None):
    """pa_prefill (or pa_prefill_split, when a workspace tensor is given) with
    its arguments checked and fixed (see pa_prefill)."""
    torch = _torch()
    _same_pool(k_cache, v_cache)
    desc = cache_desc(k_cache)
    if q.dim() != 3 or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q and out must be [T, H_q, D] of one shape")
    T, H_q, D = q.shape
    if D != desc.head_dim or q.dtype != k_cache.dtype or out.dtype != k_cache.dtype:
        raise ValueError("q/out must match the pool's head_dim and dtype")
    if (block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32
            or query_start.dtype != torch.int32):
        raise TypeError("block_tables, context_lens and query_start must be int32")
    B = context_lens.numel()
    if block_tables.dim() != 2 or block_tables.shape[0] != B or query_start.numel() != B + 1:
        raise ValueError("block_tables must be [B, max_blocks] and query_start [B + 1]")
    lib = load_library()
    args = (_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
            _dev(block_tables, "block_tables"), block_tables.shape[1],
            _dev(context_lens, "context_lens"), _dev(query_start, "query_start"), B, T,
            int(block_size), ctypes.c_float(scale), _dev(out, "out"), H_q, ctypes.byref(desc))
    keep = (q, k_cache, v_cache, block_tables, context_lens, query_start, out, desc)
    if workspace is None:
        return PreparedCall(lib.pa_prefill, args + (_stream(stream),), keep)
    args += (_dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
             _stream(stream))
    return PreparedCall(lib.pa_prefill_split, args, keep + (workspace,))


# --------------------------------------------------------------- allocator
class Allocator:
    """One pa_allocator handle (host; not thread-safe)."""

    def __init__(self, num_blocks, block_size, free_order=None):
        lib = load_library()
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        h = ctypes.c_void_p()
        if free_order is None:
            _check(lib.pa_allocator_create(self.num_blocks, self.block_size, None, ctypes.byref(h)))
        else:
            fo = np.ascontiguousarray(free_order, dtype=np.int32)
            if fo.size != self.num_blocks:
                raise ValueError("free_order must have num_blocks entries")
            _check(lib.pa_allocator_create(self.num_blocks, self.block_size, _ptr(fo, ctypes.c_int32),
                                           ctypes.byref(h)))
        self._h = h
        self._lib = lib

    def close(self):
        if self._h:
            self._lib.pa_allocator_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def seq_create(self, seq_id):
        _check(self._lib.pa_seq_create(self._h, int(seq_id)))

    def seq_fork(self, parent, child):
        _check(self._lib.pa_seq_fork(self._h, int(parent), int(child)))

    def seq_free(self, seq_id):
        _check(self._lib.pa_seq_free(self._h, int(seq_id)))

    def seq_reserve(self, seq_ids, n_new, cow_cap=None, out=None):
        """Returns (slot_mapping int64 [sum n_new], cow_pairs int32 [P, 2])."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64).reshape(-1)
        ns = np.ascontiguousarray(n_new, dtype=np.int32).reshape(-1)
        if ids.size != ns.size:
            raise ValueError("seq_ids and n_new differ in length")
        total = int(ns.sum()) if ns.size else 0
        cap = ids.size if cow_cap is None else int(cow_cap)
        slots = np.empty(max(total, 1), dtype=np.int64) if out is None else out
        pairs = np.empty((max(cap, 1), 2), dtype=np.int32)
        npairs = ctypes.c_int32(0)
        _check(self._lib.pa_seq_reserve(self._h, _ptr(ids, ctypes.c_int64), _ptr(ns, ctypes.c_int32),
                                        ids.size, _ptr(slots, ctypes.c_int64),
                                        _ptr(pairs, ctypes.c_int32), cap, ctypes.byref(npairs)))
        return slots[:total], pairs[:npairs.value]

    def build_block_tables(self, seq_ids, max_blocks, tables_out=None, lens_out=None):
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64).reshape(-1)
        tables = np.empty((ids.size, max_blocks), np.int32) if tables_out is None else tables_out
        lens = np.empty(ids.size, np.int32) if lens_out is None else lens_out
        _check(self._lib.pa_build_block_tables(self._h, _ptr(ids, ctypes.c_int64), ids.size,
                                               int(max_blocks), _ptr(tables, ctypes.c_int32),
                                               _ptr(lens, ctypes.c_int32)))
        return tables, lens

    def num_free(self):
        return self._lib.pa_allocator_num_free(self._h)

    def free_list(self):
        n = self.num_free()
        out = np.empty(max(n, 1), np.int32)
        ln = ctypes.c_int32(0)
        _check(self._lib.pa_allocator_free_list(self._h, _ptr(out, ctypes.c_int32), out.size,
                                                ctypes.byref(ln)))
        return out[:ln.value].tolist()

    def refcount(self, block):
        v = ctypes.c_int32(0)
        _check(self._lib.pa_block_refcount(self._h, int(block), ctypes.byref(v)))
        return v.value

    def seq_block_table(self, seq_id):
        ln = ctypes.c_int32(0)
        self._lib.pa_seq_block_table(self._h, int(seq_id), None, 0, ctypes.byref(ln))
        out = np.empty(max(ln.value, 1), np.int32)
        _check(self._lib.pa_seq_block_table(self._h, int(seq_id), _ptr(out, ctypes.c_int32),
                                            out.size, ctypes.byref(ln)))
        return out[:ln.value].tolist()

    def seq_num_tokens(self, seq_id):
        v = ctypes.c_int32(0)
        _check(self._lib.pa_seq_num_tokens(self._h, int(seq_id), ctypes.byref(v)))
        return v.value

    # ---------------------------------------------------------- host pool
    def add_host_pool(self, num_host_blocks, free_order=None):
        if free_order is None:
            _check(self._lib.pa_allocator_add_host_pool(self._h, int(num_host_blocks), None))
        else:
            fo = np.ascontiguousarray(free_order, dtype=np.int32)
            if fo.size != int(num_host_blocks):
                raise ValueError("free_order must have num_host_blocks entries")
            _check(self._lib.pa_allocator_add_host_pool(self._h, int(num_host_blocks),
                                                        _ptr(fo, ctypes.c_int32)))

    def _swap(self, fn, seq_id):
        ln = ctypes.c_int32(0)
        self._lib.pa_seq_block_table(self._h, int(seq_id), None, 0, ctypes.byref(ln))
        pairs = np.empty((max(ln.value, 1), 2), np.int32)
        n = ctypes.c_int32(0)
        _check(fn(self._h, int(seq_id), _ptr(pairs, ctypes.c_int32), pairs.shape[0],
                  ctypes.byref(n)))
        return pairs[:n.value]

    def seq_swap_out(self, seq_id):
        """Returns int32 [n, 2] (device block, host block) pairs."""
        return self._swap(self._lib.pa_seq_swap_out, seq_id)

    def seq_swap_in(self, seq_id):
        """Returns int32 [n, 2] (host block, device block) pairs."""
        return self._swap(self._lib.pa_seq_swap_in, seq_id)

    # -------------------------------------------------------- prefix cache
    def enable_prefix_cache(self):
        _check(self._lib.pa_allocator_enable_prefix_cache(self._h))

    def match_prefix(self, seq_id, tokens):
        """Registers the tokens of an empty sequence; returns the cached tokens taken."""
        t = np.ascontiguousarray(tokens, dtype=np.int32).reshape(-1)
        n = ctypes.c_int32(0)
        _check(self._lib.pa_seq_match_prefix(self._h, int(seq_id),
                                             _ptr(t, ctypes.c_int32) if t.size else None, t.size,
                                             ctypes.byref(n)))
        return n.value

    def num_cached(self):
        return self._lib.pa_allocator_num_cached(self._h)

    def cached_list(self):
        n = self.num_cached()
        out = np.empty(max(n, 1), np.int32)
        ln = ctypes.c_int32(0)
        _check(self._lib.pa_allocator_cached_list(self._h, _ptr(out, ctypes.c_int32), out.size,
                                                  ctypes.byref(ln)))
        return out[:ln.value].tolist()

    def block_key(self, block):
        """The prefix-cache key a block holds, or None."""
        c = ctypes.c_int32(0)
        k = ctypes.c_uint64(0)
        _check(self._lib.pa_block_prefix_key(self._h, int(block), ctypes.byref(c), ctypes.byref(k)))
        return k.value if c.value else None

    def seq_is_swapped(self, seq_id):
        v = ctypes.c_int32(0)
        _check(self._lib.pa_seq_is_swapped(self._h, int(seq_id), ctypes.byref(v)))
        return bool(v.value)

    def num_free_host(self):
        return self._lib.pa_allocator_num_free_host(self._h)

    def host_free_list(self):
        n = self.num_free_host()
        out = np.empty(max(n, 1), np.int32)
        ln = ctypes.c_int32(0)
        _check(self._lib.pa_allocator_host_free_list(self._h, _ptr(out, ctypes.c_int32), out.size,
                                                     ctypes.byref(ln)))
        return out[:ln.value].tolist()


# ------------------------------------------------------- prepared launches
class PreparedCall:
    """A device call whose arguments were checked and marshalled once.

    Calling it re-issues the same C call (same tensors, same stream) with no
    Python-side work beyond the ctypes call, for launch-bound loops.  The
    tensors must stay alive and keep their storage while it is used.
    """

    def __init__(self, fn, args, keep):
        self._fn = fn
        self._args = args
        self._keep = keep  # tensors whose storage the call points at

    def __call__(self):
        st = self._fn(*self._args)
        if st != PA_OK:
            _check(st)


def prepare_decode(q, k_cache, v_cache, block_tables, context_lens, block_size, scale, out,
                   workspace, stream=None):
    """pa_decode with its arguments fixed (see pa_decode)."""
    _same_pool(k_cache, v_cache)
    desc = cache_desc(k_cache)
    B, H_q, _ = q.shape
    maxb = block_tables.shape[1]
    lib = load_library()
    args = (_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
            _dev(block_tables, "block_tables"), maxb, _dev(context_lens, "context_lens"), B,
            int(block_size), ctypes.c_float(scale), _dev(out, "out"), H_q, ctypes.byref(desc),
            _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
            _stream(stream))
    return PreparedCall(lib.pa_decode, args, (q, k_cache, v_cache, block_tables, context_lens,
                                              out, workspace, desc))


def prepare_decode_append(q, new_k, new_v, k_cache, v_cache, block_tables, context_lens,
                          block_size, scale, out, workspace, stream=None):
    """pa_decode_append with its arguments fixed (see pa_decode_append)."""
    _same_pool(k_cache, v_cache)
    desc = cache_desc(k_cache)
    B, H_q, _ = q.shape
    _check_new_rows(new_k, new_v, k_cache, B)
    maxb = block_tables.shape[1]
    lib = load_library()
    args = (_dev(q, "q"), _dev(new_k, "new_k"), _dev(new_v, "new_v"), _dev(k_cache, "k_cache"),
            _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables"), maxb,
            _dev(context_lens, "context_lens"), B, int(block_size), ctypes.c_float(scale),
            _dev(out, "out"), H_q, ctypes.byref(desc), _dev(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _stream(stream))
    return PreparedCall(lib.pa_decode_append, args, (q, new_k, new_v, k_cache, v_cache,
                                                     block_tables, context_lens, out, workspace,
                                                     desc))


def prepare_cache_append(k, v, slot_mapping, k_cache, v_cache, stream=None):
    """pa_cache_append with its arguments fixed (see pa_cache_append)."""
    _same_pool(k_cache, v_cache)
    desc = cache_desc(k_cache)
    lib = load_library()
    args = (_dev(k, "k"), _dev(v, "v"), _dev(slot_mapping, "slot_mapping"), slot_mapping.numel(),
            _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), ctypes.byref(desc),
            _stream(stream))
    return PreparedCall(lib.pa_cache_append, args, (k, v, slot_mapping, k_cache, v_cache, desc))


def prepare_copy_blocks(src_dst_pairs, num_pairs, k_cache, v_cache, stream=None):
    """pa_copy_blocks over the first num_pairs rows of a fixed pair buffer."""
    _same_pool(k_cache, v_cache)
    desc = cache_desc(k_cache)
    lib = load_library()
    args = (_dev(src_dst_pairs, "src_dst_pairs"), int(num_pairs), _dev(k_cache, "k_cache"),
            _dev(v_cache, "v_cache"), ctypes.byref(desc), _stream(stream))
    return PreparedCall(lib.pa_copy_blocks, args, (src_dst_pairs, k_cache, v_cache, desc))
