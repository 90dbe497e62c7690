"""Paged KV-cache attention for one MI355X (gfx950): Python binding.

Thin ctypes marshalling over the C ABI in ``include/pa.h`` (``libpa.so``, built
in-tree by ``paged_kv_cache_455_amd._build``).  Every step of the path runs in
the HIP kernels; PyTorch only provides device memory and the current stream.
There is no CPU fallback: without the built library every call raises.

Entry points (same names as the C ABI): ``pa_slot_mapping``,
``kv_cache_write``, ``kv_cache_write_quant``, ``kv_block_copy``, ``pa_decode``,
``pa_decode_append``, ``pa_prefill_chunk``,
``pa_decode_workspace_size``, ``pa_prefill_workspace_size``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "KVPool", "PA_POOL_SHARED_BLOCKS", "PagedAttentionError", "BlockManager", "kv_swap",
    "DecodeStepGraph", "library_path", "load_library",
    "pa_slot_mapping", "kv_cache_write", "kv_cache_write_quant", "kv_block_copy", "pa_decode",
    "pa_decode_append", "pa_prefill_chunk",
    "pa_decode_workspace_size", "pa_prefill_workspace_size", "PA_DTYPE",
    "pa_check_tables", "pa_check_slots", "pa_check_copy_pairs", "PA_CHECK",
]

_HERE = os.path.dirname(os.path.abspath(__file__))

PA_F32, PA_F16, PA_BF16, PA_FP8_E4M3, PA_I8 = 0, 1, 2, 3, 4
PA_DTYPE = {
    torch.float32: PA_F32,
    torch.float16: PA_F16,
    torch.bfloat16: PA_BF16,
    torch.uint8: PA_FP8_E4M3,          # E4M3FN bit patterns
    torch.float8_e4m3fn: PA_FP8_E4M3,
    torch.int8: PA_I8,
}
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace too small", 4: "HIP error",
           5: "no free block"}


class PagedAttentionError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn}: {_STATUS.get(status, status)}: {detail}")
        self.status = status


class _Pool(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int64), ("num_kv_heads", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
        ("flags", ctypes.c_int32),
    ]


_c = ctypes
_SIGS = {
    "pa_version": (_c.c_char_p, []),
    "pa_status_string": (_c.c_char_p, [_c.c_int]),
    "pa_last_error": (_c.c_char_p, []),
    "pa_slot_mapping": (_c.c_int, [_c.c_void_p, _c.c_int32, _c.c_int32, _c.c_void_p, _c.c_void_p,
                                   _c.c_int32, _c.c_int32, _c.c_void_p, _c.c_void_p]),
    "kv_cache_write": (_c.c_int, [_c.POINTER(_Pool), _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                  _c.c_int32, _c.c_void_p]),
    "kv_block_copy": (_c.c_int, [_c.POINTER(_Pool), _c.c_void_p, _c.c_int32, _c.c_void_p]),
    "kv_cache_write_quant": (_c.c_int, [_c.POINTER(_Pool), _c.c_void_p, _c.c_void_p, _c.c_int32,
                                        _c.c_void_p, _c.c_int32, _c.c_void_p]),
    "pa_decode_workspace_size": (_c.c_size_t, [_c.c_int32] * 5),
    "pa_decode": (_c.c_int, [_c.POINTER(_Pool), _c.c_void_p, _c.c_int32, _c.c_void_p, _c.c_void_p,
                             _c.c_int32, _c.c_void_p, _c.c_int32, _c.c_int32, _c.c_int32,
                             _c.c_float, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "pa_decode_append": (_c.c_int, [_c.POINTER(_Pool), _c.c_void_p, _c.c_int32, _c.c_void_p,
                                    _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int32,
                                    _c.c_void_p, _c.c_void_p, _c.c_int32, _c.c_int32, _c.c_int32,
                                    _c.c_float, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "pa_decode_append_noalloc": (_c.c_int, [_c.POINTER(_Pool), _c.c_void_p, _c.c_int32,
                                            _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                            _c.c_int32, _c.c_void_p, _c.c_void_p, _c.c_int32,
                                            _c.c_int32, _c.c_int32, _c.c_float, _c.c_void_p]),
    "pa_noalloc_scratch_bytes": (_c.c_size_t, []),
    "pa_stream_read": (_c.c_int, [_c.c_void_p, _c.c_size_t, _c.c_void_p, _c.c_void_p]),
    "pa_prefill_workspace_size": (_c.c_size_t, [_c.c_int32] * 8),
    "pa_check_tables": (_c.c_int, [_c.POINTER(_Pool), _c.c_void_p, _c.c_int32, _c.c_void_p,
                                   _c.c_void_p, _c.c_int32, _c.c_int32, _c.c_void_p, _c.c_void_p]),
    "pa_check_slots": (_c.c_int, [_c.POINTER(_Pool), _c.c_void_p, _c.c_int32, _c.c_void_p,
                                  _c.c_void_p]),
    "pa_check_copy_pairs": (_c.c_int, [_c.POINTER(_Pool), _c.c_void_p, _c.c_int32, _c.c_void_p,
                                       _c.c_void_p]),
    "pa_bm_create": (_c.c_void_p, [_c.c_int32, _c.c_int32, _c.c_int32]),
    "pa_bm_num_free_host": (_c.c_int32, [_c.c_void_p]),
    "pa_bm_swap_out": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_void_p]),
    "pa_bm_swap_in": (_c.c_int, [_c.c_void_p, _c.c_int64]),
    "pa_bm_lru": (_c.c_int, [_c.c_void_p, _c.c_void_p]),
    "pa_bm_blocks": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_void_p, _c.c_void_p, _c.c_int32,
                                _c.c_void_p]),
    "pa_bm_swaps": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_int32, _c.c_void_p, _c.c_void_p,
                               _c.c_int32, _c.c_void_p]),
    "kv_swap": (_c.c_int, [_c.POINTER(_Pool), _c.POINTER(_Pool), _c.c_void_p, _c.c_int32,
                           _c.c_void_p]),
    "pa_decode_step_graph": (_c.c_int, [_c.POINTER(_Pool), _c.c_void_p, _c.c_int32, _c.c_void_p,
                                        _c.c_void_p, _c.c_int32, _c.c_void_p, _c.c_void_p,
                                        _c.c_int32, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                        _c.c_int32, _c.c_int32, _c.c_int32, _c.c_float,
                                        _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "pa_graph_launch": (_c.c_int, [_c.c_void_p, _c.c_void_p]),
    "pa_graph_destroy": (None, [_c.c_void_p]),
    "pa_bm_destroy": (None, [_c.c_void_p]),
    "pa_bm_num_free": (_c.c_int32, [_c.c_void_p]),
    "pa_bm_refcount": (_c.c_int32, [_c.c_void_p, _c.c_int32]),
    "pa_bm_add": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_void_p, _c.c_int32, _c.c_void_p]),
    "pa_bm_fork": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_int64]),
    "pa_bm_append": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_void_p, _c.c_int32]),
    "pa_bm_release": (_c.c_int, [_c.c_void_p, _c.c_int64]),
    "pa_bm_step": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_int32, _c.c_int32, _c.c_void_p,
                              _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int32, _c.c_void_p]),
    "pa_prefill_chunk": (_c.c_int, [_c.POINTER(_Pool), _c.c_void_p, _c.c_int32, _c.c_void_p,
                                    _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int32, _c.c_int32,
                                    _c.c_int32, _c.c_int32, _c.c_int32, _c.c_int32, _c.c_float,
                                    _c.c_void_p, _c.c_size_t, _c.c_void_p]),
}

_LIB: Optional[ctypes.CDLL] = None


def library_path() -> str:
    return os.environ.get("PA_LIBRARY", os.path.join(_HERE, "libpa.so"))


def load_library() -> ctypes.CDLL:
    """Load ``libpa.so``; raise if it has not been built (no fallback exists)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library {path} is not built; run "
                           "`python -m paged_kv_cache_455_amd._build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        # a library built from part of the sources (the sanitized host-only build)
        # lacks some entry points: calling one of those raises AttributeError
        fn = getattr(lib, name, None)
        if fn is None:
            continue
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def _check(fn: str, status: int):
    if status != 0:
        detail = load_library().pa_last_error().decode(errors="replace")
        raise PagedAttentionError(fn, status, detail)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the HIP library must be contiguous")
    return t.data_ptr()


def _stream(t: torch.Tensor, stream=None) -> Optional[int]:
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return torch.cuda.current_stream(t.device).cuda_stream


def _dt(t: torch.Tensor) -> int:
    try:
        return PA_DTYPE[t.dtype]
    except KeyError:
        raise ValueError(f"unsupported dtype {t.dtype}") from None


PA_POOL_SHARED_BLOCKS = 1


class KVPool:
    """Device K/V pools ``[num_blocks][num_kv_heads][16][head_dim]`` (+ scales).

    ``shared_blocks=True`` declares that some physical blocks appear in several
    sequences' block tables (prefix sharing); decode then reads tiles with cached
    loads instead of streaming them (``PA_POOL_SHARED_BLOCKS``).
    """

    def __init__(self, k: torch.Tensor, v: torch.Tensor, k_scale: Optional[torch.Tensor] = None,
                 v_scale: Optional[torch.Tensor] = None, shared_blocks: bool = False):
        if k.shape != v.shape or k.dim() != 4 or k.dtype != v.dtype:
            raise ValueError("k and v pools must share one 4-d shape and dtype")
        self.k, self.v, self.k_scale, self.v_scale = k, v, k_scale, v_scale
        nb, hkv, bs, d = k.shape
        flags = PA_POOL_SHARED_BLOCKS if shared_blocks else 0
        self._s = _Pool(_ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale), nb, hkv, bs, d, _dt(k),
                        flags)

    @property
    def num_kv_heads(self) -> int:
        return int(self.k.shape[1])

    @property
    def head_dim(self) -> int:
        return int(self.k.shape[3])

    def ref(self):
        return ctypes.byref(self._s)


def pa_slot_mapping(block_tables, query_start_loc, seq_lens, num_tokens: int, out=None, stream=None,
                    block_size: int = 16):
    lib = load_library()
    if out is None:
        out = torch.empty(num_tokens, dtype=torch.int64, device=block_tables.device)
    S = int(seq_lens.shape[0])
    _check("pa_slot_mapping", lib.pa_slot_mapping(
        _ptr(block_tables), int(block_tables.shape[1]), int(block_size), _ptr(query_start_loc),
        _ptr(seq_lens), S, int(num_tokens), _ptr(out), _stream(block_tables, stream)))
    return out


def kv_cache_write(pool: KVPool, k_new, v_new, slot_mapping, stream=None):
    lib = load_library()
    _check("kv_cache_write", lib.kv_cache_write(
        pool.ref(), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), int(slot_mapping.shape[0]),
        _stream(pool.k, stream)))


def kv_cache_write_quant(pool: KVPool, k_new, v_new, slot_mapping, stream=None):
    """Quantise new K/V rows (f32/f16/bf16) into a 1-byte pool, keeping its scales."""
    lib = load_library()
    if k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must share a dtype")
    _check("kv_cache_write_quant", lib.kv_cache_write_quant(
        pool.ref(), _ptr(k_new), _ptr(v_new), _dt(k_new), _ptr(slot_mapping),
        int(slot_mapping.shape[0]), _stream(pool.k, stream)))


def kv_block_copy(pool: KVPool, src_dst, stream=None):
    lib = load_library()
    _check("kv_block_copy", lib.kv_block_copy(
        pool.ref(), _ptr(src_dst), int(src_dst.shape[0]), _stream(pool.k, stream)))


def kv_swap(dst: KVPool, src: KVPool, src_dst, stream=None):
    """Copy blocks src -> dst between two pools of one geometry; either pool may
    live in pinned host memory (``pin_memory=True``), src_dst too."""
    lib = load_library()
    dev = dst.k if dst.k.is_cuda else src.k
    _check("kv_swap", lib.kv_swap(dst.ref(), src.ref(), _ptr(src_dst), int(src_dst.shape[0]),
                                  _stream(dev, stream)))


def pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len) -> int:
    return int(load_library().pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads,
                                                       head_dim, max_context_len))


def pa_prefill_workspace_size(num_seqs, num_q_tokens, num_q_heads, num_kv_heads, head_dim,
                              max_query_len, max_seq_len, kv_dtype=PA_F16) -> int:
    if not isinstance(kv_dtype, int):
        kv_dtype = PA_DTYPE[kv_dtype]
    return int(load_library().pa_prefill_workspace_size(num_seqs, num_q_tokens, num_q_heads,
                                                        num_kv_heads, head_dim, max_query_len,
                                                        max_seq_len, kv_dtype))


def _workspace(nbytes: int, device, workspace):
    if nbytes == 0:
        return workspace
    if workspace is None or workspace.numel() * workspace.element_size() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return workspace


def pa_decode(pool: KVPool, q, block_tables, context_lens, max_context_len: int, scale: float,
              out=None, workspace=None, stream=None):
    lib = load_library()
    S, hq, _ = q.shape
    if out is None:
        out = torch.empty_like(q)
    need = pa_decode_workspace_size(S, hq, pool.num_kv_heads, pool.head_dim, max_context_len)
    workspace = _workspace(need, q.device, workspace)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pa_decode", lib.pa_decode(
        pool.ref(), _ptr(q), _dt(q), _ptr(out), _ptr(block_tables), int(block_tables.shape[1]),
        _ptr(context_lens), int(S), int(hq), int(max_context_len), float(scale),
        _ptr(workspace), wbytes, _stream(q, stream)))
    return out


def pa_decode_append(pool: KVPool, q, k_new, v_new, block_tables, context_lens,
                     max_context_len: int, scale: float, out=None, slot_mapping=None,
                     workspace=None, stream=None):
    """Decode with the new rows' cache write fused in: equals pa_slot_mapping (row s at
    position context_lens[s] - 1), kv_cache_write (kv_cache_write_quant for fp8/int8
    pools, whose new rows come in q's dtype) and pa_decode in that order.
    ``slot_mapping`` (int64 [num_seqs]), when given, receives the slots."""
    lib = load_library()
    S, hq, _ = q.shape
    if out is None:
        out = torch.empty_like(q)
    need = pa_decode_workspace_size(S, hq, pool.num_kv_heads, pool.head_dim, max_context_len)
    workspace = _workspace(need, q.device, workspace)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pa_decode_append", lib.pa_decode_append(
        pool.ref(), _ptr(q), _dt(q), _ptr(k_new), _ptr(v_new), _ptr(out), _ptr(block_tables),
        int(block_tables.shape[1]), _ptr(context_lens), _ptr(slot_mapping), int(S), int(hq),
        int(max_context_len), float(scale), _ptr(workspace), wbytes, _stream(q, stream)))
    return out


def pa_decode_append_noalloc(pool: KVPool, q, k_new, v_new, block_tables, context_lens,
                             max_context_len: int, scale: float, out, slot_mapping=None,
                             stream=None):
    """pa_decode_append with its scratch in the library's static device array: no
    workspace argument and nothing allocated, here or in the library (``out`` must be
    given).  Calls that overlap on one GPU share that array and race."""
    lib = load_library()
    S, hq, _ = q.shape
    _check("pa_decode_append_noalloc", lib.pa_decode_append_noalloc(
        pool.ref(), _ptr(q), _dt(q), _ptr(k_new), _ptr(v_new), _ptr(out), _ptr(block_tables),
        int(block_tables.shape[1]), _ptr(context_lens), _ptr(slot_mapping), int(S), int(hq),
        int(max_context_len), float(scale), _stream(q, stream)))
    return out


def pa_stream_read(src, sink, stream=None):
    """One streaming read of ``src`` (a 16-byte aligned device tensor) folded into the
    device uint32 ``sink``: the achievable HBM read rate, timed beside the path."""
    lib = load_library()
    _check("pa_stream_read", lib.pa_stream_read(_ptr(src), src.numel() * src.element_size(),
                                                _ptr(sink), _stream(src, stream)))


def pa_noalloc_scratch_bytes() -> int:
    return int(load_library().pa_noalloc_scratch_bytes())


def pa_prefill_chunk(pool: KVPool, q, query_start_loc, seq_lens, block_tables, max_query_len: int,
                     max_seq_len: int, scale: float, out=None, workspace=None, stream=None):
    lib = load_library()
    T, hq, _ = q.shape
    S = int(seq_lens.shape[0])
    if out is None:
        out = torch.empty_like(q)
    need = pa_prefill_workspace_size(S, T, hq, pool.num_kv_heads, pool.head_dim, max_query_len,
                                     max_seq_len, pool.k.dtype)
    workspace = _workspace(need, q.device, workspace)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pa_prefill_chunk", lib.pa_prefill_chunk(
        pool.ref(), _ptr(q), _dt(q), _ptr(out), _ptr(query_start_loc), _ptr(seq_lens),
        _ptr(block_tables), int(block_tables.shape[1]), S, int(T), int(hq), int(max_query_len),
        int(max_seq_len), float(scale), _ptr(workspace), wbytes, _stream(q, stream)))
    return out


# bits of the input checks' flags word (include/pa.h PA_CHECK_*)
PA_CHECK = {"len": 1, "block": 2, "qsl": 4, "slot": 8, "slot_dup": 16, "pair": 32}


def _flags(device, flags):
    if flags is None:
        flags = torch.zeros(1, dtype=torch.int32, device=device)
    return flags


def pa_check_tables(pool: KVPool, block_tables, seq_lens, max_seq_len: int, query_start_loc=None,
                    flags=None, stream=None):
    """OR PA_CHECK_* bits for bad lengths, table ids or query starts into ``flags``
    (int32 [1] on the device, zeroed here when not given); read it after a sync."""
    lib = load_library()
    flags = _flags(block_tables.device, flags)
    _check("pa_check_tables", lib.pa_check_tables(
        pool.ref(), _ptr(block_tables), int(block_tables.shape[1]), _ptr(seq_lens),
        _ptr(query_start_loc), int(seq_lens.shape[0]), int(max_seq_len), _ptr(flags),
        _stream(block_tables, stream)))
    return flags


def pa_check_slots(pool: KVPool, slot_mapping, flags=None, stream=None):
    lib = load_library()
    flags = _flags(slot_mapping.device, flags)
    _check("pa_check_slots", lib.pa_check_slots(
        pool.ref(), _ptr(slot_mapping), int(slot_mapping.shape[0]), _ptr(flags),
        _stream(slot_mapping, stream)))
    return flags


def pa_check_copy_pairs(pool: KVPool, src_dst, flags=None, stream=None):
    lib = load_library()
    flags = _flags(src_dst.device, flags)
    _check("pa_check_copy_pairs", lib.pa_check_copy_pairs(
        pool.ref(), _ptr(src_dst), int(src_dst.shape[0]), _ptr(flags), _stream(src_dst, stream)))
    return flags


class DecodeStepGraph:
    """A decode step captured once and replayed (``pa_decode_step_graph``): slot
    mapping, the new K/V rows' write and the decode, over the tensors given
    here.  ``replay()`` reads their contents at that time, so refresh q, k_new,
    v_new, block_tables and context_lens in place between replays.  The tensors
    are held here so they outlive the graph."""

    def __init__(self, pool: KVPool, q, k_new, v_new, block_tables, context_lens,
                 max_context_len: int, scale: float, out=None):
        lib = load_library()
        self._lib = lib
        S, hq, _ = q.shape
        self.out = torch.empty_like(q) if out is None else out
        self.slots = torch.empty(S, dtype=torch.int64, device=q.device)
        self.qsl = torch.arange(S + 1, dtype=torch.int32, device=q.device)
        need = pa_decode_workspace_size(S, hq, pool.num_kv_heads, pool.head_dim, max_context_len)
        self.workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        self._keep = (pool, q, k_new, v_new, block_tables, context_lens)
        h = ctypes.c_void_p()
        _check("pa_decode_step_graph", lib.pa_decode_step_graph(
            pool.ref(), _ptr(q), _dt(q), _ptr(k_new), _ptr(v_new), _dt(k_new), _ptr(self.out),
            _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens), _ptr(self.qsl),
            _ptr(self.slots), int(S), int(hq), int(max_context_len), float(scale),
            _ptr(self.workspace), int(need), ctypes.byref(h)))
        self._h = h

    def replay(self, stream=None):
        _check("pa_graph_launch", self._lib.pa_graph_launch(self._h, _stream(self.out, stream)))
        return self.out

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._lib.pa_graph_destroy(h)
            self._h = None


class BlockManager:
    """Host block manager of the C ABI (``pa_bm_*``): allocation, prefix cache,
    reference counts, copy-on-write and the per-step host arrays.  Marshalling
    only; the bookkeeping runs in the library."""

    def __init__(self, num_blocks: int, num_host_blocks: int = 0, block_size: int = 16):
        lib = load_library()
        self._lib = lib
        self._h = lib.pa_bm_create(int(num_blocks), int(num_host_blocks), int(block_size))
        if not self._h:
            raise PagedAttentionError("pa_bm_create", 1, "bad block counts or out of memory")
        self.num_blocks = int(num_blocks)
        self.num_host_blocks = int(num_host_blocks)
        self.block_size = int(block_size)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._lib.pa_bm_destroy(h)
            self._h = None

    @staticmethod
    def _ints(xs):
        import numpy as np
        a = np.ascontiguousarray(np.asarray(xs, dtype=np.int32))
        return a, a.ctypes.data_as(ctypes.c_void_p)

    def num_free(self) -> int:
        return int(self._lib.pa_bm_num_free(self._h))

    def num_free_host(self) -> int:
        return int(self._lib.pa_bm_num_free_host(self._h))

    def swap_out(self, req: int) -> int:
        """Move the blocks ``req`` holds alone to host slots; returns how many."""
        moved = ctypes.c_int32(0)
        _check("pa_bm_swap_out", self._lib.pa_bm_swap_out(self._h, int(req), ctypes.byref(moved)))
        return int(moved.value)

    def swap_in(self, req: int):
        _check("pa_bm_swap_in", self._lib.pa_bm_swap_in(self._h, int(req)))

    def lru(self) -> int:
        r = ctypes.c_int64(0)
        _check("pa_bm_lru", self._lib.pa_bm_lru(self._h, ctypes.byref(r)))
        return int(r.value)

    def blocks(self, req: int, max_blocks: int = 4096):
        """(device_blocks, host_slots) of ``req``'s logical blocks, -1 where absent."""
        import numpy as np
        dev = np.zeros(max_blocks, dtype=np.int32)
        host = np.zeros(max_blocks, dtype=np.int32)
        n = ctypes.c_int32(0)
        vp = lambda x: x.ctypes.data_as(ctypes.c_void_p)
        _check("pa_bm_blocks", self._lib.pa_bm_blocks(self._h, int(req), vp(dev), vp(host),
                                                      int(max_blocks), ctypes.byref(n)))
        return dev[:n.value].copy(), host[:n.value].copy()

    def swaps(self, max_pairs: int = 4096):
        """Queued (out_pairs, in_pairs): out (device block, host slot), in (host
        slot, device block); to run before the next step's copies."""
        import numpy as np
        out = np.zeros((max(max_pairs, 1), 2), dtype=np.int32)
        inn = np.zeros((max(max_pairs, 1), 2), dtype=np.int32)
        no, ni = ctypes.c_int32(0), ctypes.c_int32(0)
        vp = lambda x: x.ctypes.data_as(ctypes.c_void_p)
        _check("pa_bm_swaps", self._lib.pa_bm_swaps(self._h, vp(out), int(max_pairs),
                                                    ctypes.byref(no), vp(inn), int(max_pairs),
                                                    ctypes.byref(ni)))
        return out[:no.value].copy(), inn[:ni.value].copy()

    def refcount(self, block: int) -> int:
        return int(self._lib.pa_bm_refcount(self._h, int(block)))

    def add(self, req: int, tokens) -> int:
        """Register a request's prompt; returns the number of leading prompt tokens
        already held by shared cached blocks."""
        a, p = self._ints(tokens)
        cached = ctypes.c_int32(0)
        _check("pa_bm_add", self._lib.pa_bm_add(self._h, int(req), p, int(a.size),
                                                ctypes.byref(cached)))
        return int(cached.value)

    def fork(self, parent: int, child: int):
        _check("pa_bm_fork", self._lib.pa_bm_fork(self._h, int(parent), int(child)))

    def append(self, req: int, tokens):
        a, p = self._ints(tokens)
        _check("pa_bm_append", self._lib.pa_bm_append(self._h, int(req), p, int(a.size)))

    def release(self, req: int):
        _check("pa_bm_release", self._lib.pa_bm_release(self._h, int(req)))

    def step(self, reqs, max_blocks_per_seq: int, max_pairs: int = 1024):
        """Host arrays of one step; each request's query rows are its tokens not
        yet written.  Returns (block_tables [n][mb], seq_lens [n],
        query_start_loc [n+1], copy_pairs [P][2]) as numpy int32 arrays."""
        import numpy as np
        n = len(reqs)
        r = np.ascontiguousarray(np.asarray(reqs, dtype=np.int64))
        bt = np.zeros((n, max_blocks_per_seq), dtype=np.int32)
        lens = np.zeros(n, dtype=np.int32)
        qsl = np.zeros(n + 1, dtype=np.int32)
        pairs = np.zeros((max(max_pairs, 1), 2), dtype=np.int32)
        npairs = ctypes.c_int32(0)
        vp = lambda x: x.ctypes.data_as(ctypes.c_void_p)
        _check("pa_bm_step", self._lib.pa_bm_step(
            self._h, vp(r), n, int(max_blocks_per_seq), vp(bt), vp(lens), vp(qsl), vp(pairs),
            int(max_pairs), ctypes.byref(npairs)))
        return bt, lens, qsl, pairs[:npairs.value].copy()
