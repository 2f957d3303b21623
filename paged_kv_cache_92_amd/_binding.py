"""ctypes binding of libpkv.so: argument marshalling only.

Every computation runs in the library's HIP kernels; this module checks
tensor dtypes/devices/shapes, passes raw device pointers and torch's current
HIP stream, and turns a non-OK status into ``PkvError``.  There is no
fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpkv.so")

PKV_F32, PKV_F16, PKV_BF16, PKV_FP8_E4M3 = 0, 1, 2, 3
_TORCH_TO_PKV = {torch.float32: PKV_F32, torch.float16: PKV_F16, torch.bfloat16: PKV_BF16,
                 torch.float8_e4m3fn: PKV_FP8_E4M3}
_STATUS = {0: "OK", 1: "INVALID", 2: "UNSUPPORTED", 3: "WORKSPACE", 4: "HIP"}

EXPORTED = ("pkv_reshape_and_cache", "pkv_copy_blocks", "pkv_decode_workspace_bytes",
            "pkv_paged_decode", "pkv_paged_decode_window", "pkv_paged_decode_append",
            "pkv_paged_decode_noalloc",
            "pkv_paged_prefill", "pkv_paged_mixed",
            "pkv_gather_kv",
            "pkv_validate_host",
            "pkv_last_error", "pkv_version")


class PkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"pkv {_STATUS.get(status, status)}: {message}")
        self.status = status


class PkvCacheDesc(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("num_blocks", ctypes.c_int64), ("num_kv_heads", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("model_dtype", ctypes.c_int32),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
        cp = ctypes.POINTER(PkvCacheDesc)
        L.pkv_reshape_and_cache.argtypes = [cp, vp, vp, vp, i64, vp]
        L.pkv_copy_blocks.argtypes = [cp, vp, i64, vp]
        L.pkv_decode_workspace_bytes.argtypes = [cp, i32, i32, i32, i32]
        L.pkv_decode_workspace_bytes.restype = sz
        L.pkv_paged_decode.argtypes = [cp, vp, i32, vp, i32, vp, i32, vp, i32, i32, f32, i32, vp, sz, vp]
        L.pkv_paged_decode_noalloc.argtypes = [cp, vp, i32, vp, i32, vp, i32, vp, i32, i32, f32, i32,
                                               vp]
        L.pkv_paged_decode_window.argtypes = [cp, vp, i32, vp, i32, vp, i32, vp, i32, i32, i32, f32, i32,
                                              vp, sz, vp]
        L.pkv_paged_decode_append.argtypes = [cp, vp, vp, vp, i32, vp, i32, vp, i32, vp, i32, i32, i32,
                                              f32, i32, vp, sz, vp]
        L.pkv_paged_prefill.argtypes = [cp, vp, i32, vp, i32, vp, vp, vp, i32, i32, i32, i32, f32, vp]
        L.pkv_paged_mixed.argtypes = [cp, vp, i32, vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, f32,
                                      i32, vp, sz, vp]
        L.pkv_gather_kv.argtypes = [cp, vp, vp, vp, i32, vp, vp, i32, i32, vp]
        L.pkv_validate_host.argtypes = [vp, i64, vp, i32, vp, i32, i64, i32, i32]
        L.pkv_last_error.restype = ctypes.c_char_p
        L.pkv_version.restype = ctypes.c_char_p
        for name in ("pkv_reshape_and_cache", "pkv_copy_blocks", "pkv_paged_decode",
                     "pkv_paged_decode_window", "pkv_paged_decode_append",
                     "pkv_paged_decode_noalloc", "pkv_paged_prefill", "pkv_paged_mixed", "pkv_gather_kv", "pkv_validate_host"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise PkvError(status, lib().pkv_last_error().decode())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev_ptr(t: torch.Tensor | None, name: str, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _need_rows(t, rows: int, name: str, width: int | None = None):
    """The kernels read ``rows`` rows of ``t`` (and ``width`` columns per row when given):
    a shorter tensor would be read past its end, so it is refused here."""
    if t.dim() < 1 or t.shape[0] < rows:
        raise ValueError(f"{name} has {t.shape[0] if t.dim() else 0} rows, the call reads {rows}")
    if width is not None and (t.dim() != 2 or t.shape[1] != width):
        raise ValueError(f"{name} must be [n][{width}], got {tuple(t.shape)}")


class PagedKVCache:
    """One layer's paged K/V pool in HBM.

    ``k_pool`` is [num_blocks][num_kv_heads][head_dim/X][block_size][X] with
    X = 64 bytes / element size (key rows cut into 64-byte pieces, the
    block's pieces of one dimension range adjacent) and ``v_pool`` is
    [num_blocks][num_kv_heads][head_dim][block_size] (value tile
    dimension-major).

    ``dtype`` is the pools' element type; ``model_dtype`` the type of the
    key/value rows written, the queries and the outputs (``dtype`` itself,
    except for a ``torch.float8_e4m3fn`` cache: float16 or bfloat16, with
    per-tensor ``k_scale`` / ``v_scale``: stored code = x / scale).
    """

    def __init__(self, num_blocks, num_kv_heads, block_size, head_dim, dtype=torch.float16,
                 device="cuda", k_pool=None, v_pool=None, model_dtype=None, k_scale=1.0,
                 v_scale=1.0):
        self.num_blocks = int(num_blocks)
        self.num_kv_heads = int(num_kv_heads)
        self.block_size = int(block_size)
        self.head_dim = int(head_dim)
        self.dtype = dtype
        if dtype not in _TORCH_TO_PKV:
            raise ValueError(f"unsupported dtype {dtype}")
        self.model_dtype = dtype if model_dtype is None else model_dtype
        if self.model_dtype not in _TORCH_TO_PKV:
            raise ValueError(f"unsupported model dtype {self.model_dtype}")
        self.k_scale = float(k_scale)
        self.v_scale = float(v_scale)
        x = 64 // torch.tensor([], dtype=dtype).element_size()
        if self.head_dim % x:
            raise ValueError(f"head_dim must be a multiple of {x}")
        kshape = (self.num_blocks, self.num_kv_heads, self.head_dim // x, self.block_size, x)
        vshape = (self.num_blocks, self.num_kv_heads, self.head_dim, self.block_size)
        self.k_pool = k_pool if k_pool is not None else torch.empty(kshape, dtype=dtype, device=device)
        self.v_pool = v_pool if v_pool is not None else torch.empty(vshape, dtype=dtype, device=device)
        if tuple(self.k_pool.shape) != kshape or tuple(self.v_pool.shape) != vshape:
            raise ValueError("pool shapes do not match the geometry")
        for t in (self.k_pool, self.v_pool):
            if t.dtype != dtype or not t.is_contiguous():
                raise ValueError("pools must be contiguous and of the cache dtype")

    def desc(self) -> PkvCacheDesc:
        return PkvCacheDesc(self.k_pool.data_ptr(), self.v_pool.data_ptr(), self.num_blocks,
                            self.num_kv_heads, self.block_size, self.head_dim,
                            _TORCH_TO_PKV[self.dtype], _TORCH_TO_PKV[self.model_dtype],
                            self.k_scale, self.v_scale)

    def nbytes(self) -> int:
        return self.k_pool.nbytes + self.v_pool.nbytes


def reshape_and_cache(cache: PagedKVCache, key, value, slot_mapping):
    """Scatter key/value [T][Hkv][d] into the slots named by slot_mapping (int64 [T], <0 skips)."""
    T = slot_mapping.shape[0]
    if T and (tuple(key.shape) != (T, cache.num_kv_heads, cache.head_dim)
              or tuple(value.shape) != tuple(key.shape)):
        raise ValueError("key/value must be [T][num_kv_heads][head_dim]")
    d = cache.desc()
    _check(lib().pkv_reshape_and_cache(ctypes.byref(d), _dev_ptr(key, "key", cache.model_dtype),
                                       _dev_ptr(value, "value", cache.model_dtype),
                                       _dev_ptr(slot_mapping, "slot_mapping", torch.int64), T,
                                       _stream()))


def copy_blocks(cache: PagedKVCache, src_dst):
    """Copy whole blocks: src_dst int32 [n][2] of (src, dst)."""
    n = src_dst.shape[0]
    _need_rows(src_dst, n, "src_dst", width=2)
    d = cache.desc()
    _check(lib().pkv_copy_blocks(ctypes.byref(d), _dev_ptr(src_dst, "src_dst", torch.int32), n,
                                 _stream()))


PARTITION_AUTO = -1   # partition_size: balanced split over the resident workgroups


def decode_workspace_bytes(cache: "PagedKVCache", num_seqs, num_q_heads, max_context_len,
                           partition_size):
    d = cache.desc()
    return int(lib().pkv_decode_workspace_bytes(ctypes.byref(d), int(num_seqs), int(num_q_heads),
                                                int(max_context_len), int(partition_size)))


def _out(q, out, out_dtype):
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    elif out_dtype is not None and out.dtype != out_dtype:
        raise ValueError("out does not have out_dtype")
    if out.dtype not in _TORCH_TO_PKV:
        raise ValueError(f"unsupported output dtype {out.dtype}")
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have the shape of q")
    return out


def paged_decode(cache: PagedKVCache, q, block_tables, context_lens, max_context_len, scale=None,
                 partition_size=0, out=None, workspace=None, out_dtype=None, sliding_window=0):
    """Decode attention: q [S][Hq][d] -> out [S][Hq][d] over each sequence's paged cache.

    ``out_dtype`` is the model dtype (default: the fp32 result rounded once) or
    torch.float32 (the fp32 result itself).  ``sliding_window`` > 0 attends to
    each sequence's last ``sliding_window`` tokens only (pkv_paged_decode_window)."""
    S, Hq, dq = q.shape
    if dq != cache.head_dim:
        raise ValueError("q head_dim does not match the cache")
    _need_rows(block_tables, S, "block_tables")
    _need_rows(context_lens, S, "context_lens")
    if scale is None:
        scale = 1.0 / math.sqrt(cache.head_dim)
    out = _out(q, out, out_dtype)
    need = decode_workspace_bytes(cache, S, Hq, max_context_len, partition_size)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev_ptr(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.nbytes if workspace is not None else 0
    d = cache.desc()
    args = [ctypes.byref(d), _dev_ptr(out, "out"), _TORCH_TO_PKV[out.dtype],
            _dev_ptr(q, "q", cache.model_dtype), Hq,
            _dev_ptr(block_tables, "block_tables", torch.int32), block_tables.shape[1],
            _dev_ptr(context_lens, "context_lens", torch.int32), S, int(max_context_len)]
    tail = [float(scale), int(partition_size), ws_ptr, ws_bytes, _stream()]
    if sliding_window:
        _check(lib().pkv_paged_decode_window(*args, int(sliding_window), *tail))
    else:
        _check(lib().pkv_paged_decode(*args, *tail))
    return out


def paged_decode_noalloc(cache: PagedKVCache, q, block_tables, context_lens, max_context_len,
                         scale=None, partition_size=0, out=None, out_dtype=None):
    """``paged_decode`` with the split partials in the library's static device scratch
    (pkv_paged_decode_noalloc): no workspace is allocated.  ``out`` is still the caller's."""
    S, Hq, dq = q.shape
    if dq != cache.head_dim:
        raise ValueError("q head_dim does not match the cache")
    _need_rows(block_tables, S, "block_tables")
    _need_rows(context_lens, S, "context_lens")
    if scale is None:
        scale = 1.0 / math.sqrt(cache.head_dim)
    out = _out(q, out, out_dtype)
    d = cache.desc()
    _check(lib().pkv_paged_decode_noalloc(
        ctypes.byref(d), _dev_ptr(out, "out"), _TORCH_TO_PKV[out.dtype],
        _dev_ptr(q, "q", cache.model_dtype), Hq, _dev_ptr(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev_ptr(context_lens, "context_lens", torch.int32), S,
        int(max_context_len), float(scale), int(partition_size), _stream()))
    return out


def paged_decode_append(cache: PagedKVCache, key, value, q, block_tables, context_lens,
                        max_context_len, scale=None, partition_size=0, out=None, workspace=None,
                        out_dtype=None, sliding_window=0):
    """Append each sequence's new token (key/value [S][Hkv][d]) at position L-1 of its block
    table and decode, in one launch: the same cache and output as ``reshape_and_cache`` with
    those slots followed by ``paged_decode``."""
    S, Hq, dq = q.shape
    if dq != cache.head_dim:
        raise ValueError("q head_dim does not match the cache")
    if (tuple(key.shape) != (S, cache.num_kv_heads, cache.head_dim)
            or tuple(value.shape) != tuple(key.shape)):
        raise ValueError("key/value must be [S][num_kv_heads][head_dim]")
    _need_rows(block_tables, S, "block_tables")
    _need_rows(context_lens, S, "context_lens")
    if scale is None:
        scale = 1.0 / math.sqrt(cache.head_dim)
    out = _out(q, out, out_dtype)
    need = decode_workspace_bytes(cache, S, Hq, max_context_len, partition_size)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev_ptr(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.nbytes if workspace is not None else 0
    d = cache.desc()
    _check(lib().pkv_paged_decode_append(
        ctypes.byref(d), _dev_ptr(key, "key", cache.model_dtype),
        _dev_ptr(value, "value", cache.model_dtype), _dev_ptr(out, "out"), _TORCH_TO_PKV[out.dtype],
        _dev_ptr(q, "q", cache.model_dtype), Hq, _dev_ptr(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev_ptr(context_lens, "context_lens", torch.int32), S,
        int(max_context_len), int(sliding_window), float(scale), int(partition_size), ws_ptr,
        ws_bytes, _stream()))
    return out


def paged_prefill(cache: PagedKVCache, q, query_start_loc, context_lens, block_tables,
                  max_query_len, max_context_len, scale=None, out=None, out_dtype=None):
    """Causal chunked prefill: q [Tq][Hq][d] rows of each sequence's last chunk -> out [Tq][Hq][d]."""
    Tq, Hq, dq = q.shape
    if dq != cache.head_dim:
        raise ValueError("q head_dim does not match the cache")
    if scale is None:
        scale = 1.0 / math.sqrt(cache.head_dim)
    out = _out(q, out, out_dtype)
    S = context_lens.shape[0]
    _need_rows(block_tables, S, "block_tables")
    _need_rows(query_start_loc, S + 1, "query_start_loc")
    d = cache.desc()
    _check(lib().pkv_paged_prefill(ctypes.byref(d), _dev_ptr(out, "out"), _TORCH_TO_PKV[out.dtype],
                                   _dev_ptr(q, "q", cache.model_dtype), Hq,
                                   _dev_ptr(query_start_loc, "query_start_loc", torch.int32),
                                   _dev_ptr(context_lens, "context_lens", torch.int32),
                                   _dev_ptr(block_tables, "block_tables", torch.int32),
                                   block_tables.shape[1], S, int(max_query_len),
                                   int(max_context_len), float(scale), _stream()))
    return out


def paged_mixed(cache: PagedKVCache, q, query_start_loc, context_lens, block_tables,
                num_decode_seqs, max_query_len, max_context_len, scale=None, partition_size=0,
                out=None, workspace=None, out_dtype=None):
    """One step over decode rows and prefill-chunk rows: q [rows][Hq][d] -> out.

    Sequences ``0 .. num_decode_seqs-1`` hold one query row each (rows
    ``0 .. num_decode_seqs-1``); the rest are chunks placed by
    ``query_start_loc`` (absolute rows).  ``partition_size`` and
    ``workspace`` apply to the decode sequences."""
    Tq, Hq, dq = q.shape
    if dq != cache.head_dim:
        raise ValueError("q head_dim does not match the cache")
    if scale is None:
        scale = 1.0 / math.sqrt(cache.head_dim)
    out = _out(q, out, out_dtype)
    S = context_lens.shape[0]
    nd = int(num_decode_seqs)
    _need_rows(block_tables, S, "block_tables")
    if S > nd:
        _need_rows(query_start_loc, S + 1, "query_start_loc")
    need = decode_workspace_bytes(cache, nd, Hq, max_context_len, partition_size) if nd else 0
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev_ptr(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.nbytes if workspace is not None else 0
    d = cache.desc()
    _check(lib().pkv_paged_mixed(ctypes.byref(d), _dev_ptr(out, "out"), _TORCH_TO_PKV[out.dtype],
                                 _dev_ptr(q, "q", cache.model_dtype), Hq,
                                 _dev_ptr(query_start_loc, "query_start_loc", torch.int32),
                                 _dev_ptr(context_lens, "context_lens", torch.int32),
                                 _dev_ptr(block_tables, "block_tables", torch.int32),
                                 block_tables.shape[1], S, nd, int(max_query_len),
                                 int(max_context_len), float(scale), int(partition_size), ws_ptr,
                                 ws_bytes, _stream()))
    return out


def gather_kv(cache: PagedKVCache, block_tables, context_lens, cu_context_lens, total_tokens,
              max_context_len):
    """Debug gather: contiguous token-major (K, V), each [sum L][Hkv][d]."""
    S = context_lens.shape[0]
    _need_rows(block_tables, S, "block_tables")
    _need_rows(cu_context_lens, S + 1, "cu_context_lens")
    shape = (int(total_tokens), cache.num_kv_heads, cache.head_dim)
    dev = cache.k_pool.device
    k = torch.empty(shape, dtype=cache.dtype, device=dev)
    v = torch.empty(shape, dtype=cache.dtype, device=dev)
    d = cache.desc()
    _check(lib().pkv_gather_kv(ctypes.byref(d), _dev_ptr(k, "k_out"), _dev_ptr(v, "v_out"),
                               _dev_ptr(block_tables, "block_tables", torch.int32),
                               block_tables.shape[1],
                               _dev_ptr(context_lens, "context_lens", torch.int32),
                               _dev_ptr(cu_context_lens, "cu_context_lens", torch.int32),
                               context_lens.shape[0], int(max_context_len), _stream()))
    return k, v


def _host_ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def validate_host(num_blocks, block_size, slot_mapping=None, block_tables=None, context_lens=None,
                  max_context_len=0):
    """Check the device-side contract on host (numpy) copies; raises PkvError on a violation.
    ``max_context_len`` > 0 also checks every length against it."""
    sm = None if slot_mapping is None else np.ascontiguousarray(slot_mapping, dtype=np.int64)
    bt = None if block_tables is None else np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = None if context_lens is None else np.ascontiguousarray(context_lens, dtype=np.int32)
    _check(lib().pkv_validate_host(_host_ptr(sm), 0 if sm is None else sm.shape[0], _host_ptr(bt),
                                   0 if bt is None else bt.shape[1], _host_ptr(cl),
                                   0 if cl is None else cl.shape[0], int(num_blocks),
                                   int(block_size), int(max_context_len)))


def version() -> str:
    return lib().pkv_version().decode()
