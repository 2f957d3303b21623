"""CPU oracle for the paged KV-cache hot path — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never uses it and the
two share no code: the oracle is plain C (``pkv_oracle.c``) that decodes the
raw fp16/bf16/fp32 bits itself and computes in fp64, reached through ctypes
with numpy arrays.

Arrays carry raw element bits: ``float32`` for fp32 and ``uint16`` for fp16
and bf16, with the dtype code (0 fp32, 1 fp16, 2 bf16) passed alongside.
Pools use the library's documented layout: K ``[num_blocks][H][d/X][B][X]``
with X = 64 bytes / element size, V ``[num_blocks][H][d][B]``;
slot = block * B + offset.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, worked examples from the pages, invariants and special cases).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pkv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, F16, BF16, FP8 = 0, 1, 2, 3
_STORAGE = {F32: np.float32, F16: np.uint16, BF16: np.uint16, FP8: np.uint8}

_ERRORS = {-1: "bad argument", -2: "index out of range", -3: "duplicate destination", -4: "out of memory"}


class OracleError(RuntimeError):
    pass


def build(extra_flags: tuple[str, ...] = (), out_path: str | None = None,
          src: str | None = None) -> str:
    """Compile the oracle with gcc into a shared library and return its path."""
    out = out_path or _LIB_PATH
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", *extra_flags, src or _SRC, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def use_library(path: str | None):
    """Point the wrappers at another build of the oracle (None: the default one).

    Used by the mutation tests, which compile deliberately broken copies."""
    global _lib
    _lib = None
    if path is not None:
        _load(path)


def _load(path: str | None = None) -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if path is None and not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(path or _LIB_PATH)
        vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        f64 = ctypes.c_double
        lib.oracle_reshape_and_cache.argtypes = [vp, vp, i32, i64, i32, i32, i32, vp, vp, vp, i64]
        lib.oracle_reshape_and_cache_fp8.argtypes = [vp, vp, i32, f32, f32, i64, i32, i32, i32, vp, vp,
                                                     vp, i64]
        lib.oracle_copy_blocks.argtypes = [vp, vp, i32, i64, i32, i32, i32, vp, i64]
        lib.oracle_gather_kv.argtypes = [vp, vp, i32, i64, i32, i32, i32, vp, i32, vp, i32, vp, vp]
        lib.oracle_paged_attention_rows.argtypes = [vp, vp, i32, i32, f64, f64, i64, i32, i32, i32, vp,
                                                   i32, vp, i32, vp, i32, vp, vp, i64, i32, f32, vp]
        lib.oracle_paged_decode.argtypes = [vp, vp, i32, i32, f64, f64, i64, i32, i32, i32, vp, i32, vp,
                                            i32, vp, i32, i32, f32, vp]
        lib.oracle_paged_prefill.argtypes = [vp, vp, i32, i32, f64, f64, i64, i32, i32, i32, vp, i32, vp,
                                             vp, vp, i32, i32, f32, vp]
        lib.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_double.restype = ctypes.c_double
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_double.restype = ctypes.c_double
        lib.oracle_fp8_to_double.argtypes = [ctypes.c_uint8]
        lib.oracle_fp8_to_double.restype = ctypes.c_double
        lib.oracle_fp8_from_float.argtypes = [ctypes.c_float]
        lib.oracle_fp8_from_float.restype = ctypes.c_uint8
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what}: {_ERRORS.get(rc, rc)}")


def _geom(k_pool: np.ndarray, v_pool: np.ndarray, dtype: int):
    if k_pool.ndim != 5 or k_pool.shape[4] != 64 // np.dtype(_STORAGE[dtype]).itemsize:
        raise OracleError(f"K pool shape {k_pool.shape} is not [nb][H][d/X][B][X]")
    nb, H, nc, B, x = k_pool.shape
    d = nc * x
    if v_pool.shape != (nb, H, d, B):
        raise OracleError(f"V pool shape {v_pool.shape} does not match K pool {k_pool.shape}")
    if k_pool.dtype != _STORAGE[dtype] or v_pool.dtype != _STORAGE[dtype]:
        raise OracleError("pool storage does not match dtype")
    return nb, H, B, d


def reshape_and_cache(k_pool, v_pool, dtype, key, value, slots, in_dtype=None, k_scale=1.0,
                      v_scale=1.0):
    """Scatter key/value [T][H][d] into the pools (in place) at ``slots`` [T] (int64, <0 = skip).

    ``dtype`` is the pools' dtype; for an FP8 cache, key/value are ``in_dtype``
    (F16 or BF16) bits and are quantised with the per-tensor scales."""
    nb, H, B, d = _geom(k_pool, v_pool, dtype)
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    key = np.ascontiguousarray(key)
    value = np.ascontiguousarray(value)
    T = slots.shape[0]
    assert key.shape == (T, H, d) and value.shape == (T, H, d)
    if dtype == FP8:
        _check(_load().oracle_reshape_and_cache_fp8(_ptr(k_pool), _ptr(v_pool), in_dtype,
                                                    float(k_scale), float(v_scale), nb, H, B, d,
                                                    _ptr(key), _ptr(value), _ptr(slots), T),
               "reshape_and_cache")
        return
    _check(_load().oracle_reshape_and_cache(_ptr(k_pool), _ptr(v_pool), dtype, nb, H, B, d,
                                            _ptr(key), _ptr(value), _ptr(slots), T),
           "reshape_and_cache")


def copy_blocks(k_pool, v_pool, dtype, src_dst):
    """Copy whole blocks (K and V tiles of every head) for each (src, dst) row of ``src_dst``."""
    nb, H, B, d = _geom(k_pool, v_pool, dtype)
    sd = np.ascontiguousarray(src_dst, dtype=np.int32).reshape(-1, 2)
    _check(_load().oracle_copy_blocks(_ptr(k_pool), _ptr(v_pool), dtype, nb, H, B, d, _ptr(sd),
                                      sd.shape[0]), "copy_blocks")


def gather_kv(k_pool, v_pool, dtype, block_tables, context_lens):
    """Bitwise reassembly: returns (K, V), each [sum L][H][d] in the cache's storage type."""
    nb, H, B, d = _geom(k_pool, v_pool, dtype)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    total = int(ctx.sum())
    k_out = np.zeros((total, H, d), dtype=_STORAGE[dtype])
    v_out = np.zeros((total, H, d), dtype=_STORAGE[dtype])
    _check(_load().oracle_gather_kv(_ptr(k_pool), _ptr(v_pool), dtype, nb, H, B, d, _ptr(bt),
                                    bt.shape[1], _ptr(ctx), ctx.shape[0], _ptr(k_out), _ptr(v_out)),
           "gather_kv")
    return k_out, v_out


def paged_attention_rows(k_pool, v_pool, dtype, q, block_tables, context_lens, row_seq, row_pos,
                         scale, q_dtype=None, k_scale=1.0, v_scale=1.0, window=0):
    """fp64 attention for query rows q [n][Hq][d] at (row_seq[r], row_pos[r]); returns [n][Hq][d].

    q is in ``q_dtype`` (default: the cache dtype; F16/BF16 over an FP8 cache,
    whose entries read as code * k_scale / code * v_scale).  ``window`` > 0:
    each row attends to its last ``window`` positions only."""
    nb, Hkv, B, d = _geom(k_pool, v_pool, dtype)
    q = np.ascontiguousarray(q)
    n, Hq, dq = q.shape
    assert dq == d
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    rs = np.ascontiguousarray(row_seq, dtype=np.int32)
    rp = np.ascontiguousarray(row_pos, dtype=np.int32)
    out = np.zeros((n, Hq, d), dtype=np.float64)
    qd = dtype if q_dtype is None else q_dtype
    _check(_load().oracle_paged_attention_rows(_ptr(k_pool), _ptr(v_pool), dtype, qd, float(k_scale),
                                               float(v_scale), nb, Hkv, B, d,
                                               _ptr(q), Hq, _ptr(bt), bt.shape[1], _ptr(ctx),
                                               ctx.shape[0], _ptr(rs), _ptr(rp), n, int(window),
                                               float(scale), _ptr(out)), "paged_attention_rows")
    return out


def paged_decode(k_pool, v_pool, dtype, q, block_tables, context_lens, scale, q_dtype=None,
                 k_scale=1.0, v_scale=1.0, window=0):
    """fp64 decode output [S][Hq][d]: each sequence's query over all its ctx tokens (its
    last ``window`` tokens when ``window`` > 0)."""
    nb, Hkv, B, d = _geom(k_pool, v_pool, dtype)
    q = np.ascontiguousarray(q)
    S, Hq, _ = q.shape
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    out = np.zeros((S, Hq, d), dtype=np.float64)
    qd = dtype if q_dtype is None else q_dtype
    _check(_load().oracle_paged_decode(_ptr(k_pool), _ptr(v_pool), dtype, qd, float(k_scale),
                                       float(v_scale), nb, Hkv, B, d, _ptr(q), Hq,
                                       _ptr(bt), bt.shape[1], _ptr(ctx), S, int(window), float(scale),
                                       _ptr(out)), "paged_decode")
    return out


def paged_prefill(k_pool, v_pool, dtype, q, query_start_loc, context_lens, block_tables, scale,
                  q_dtype=None, k_scale=1.0, v_scale=1.0):
    """fp64 chunked-prefill output [Tq][Hq][d] (causal over history + chunk)."""
    nb, Hkv, B, d = _geom(k_pool, v_pool, dtype)
    q = np.ascontiguousarray(q)
    Tq, Hq, _ = q.shape
    qsl = np.ascontiguousarray(query_start_loc, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    assert qsl[-1] == Tq
    out = np.zeros((Tq, Hq, d), dtype=np.float64)
    qd = dtype if q_dtype is None else q_dtype
    _check(_load().oracle_paged_prefill(_ptr(k_pool), _ptr(v_pool), dtype, qd, float(k_scale),
                                        float(v_scale), nb, Hkv, B, d, _ptr(q), Hq,
                                        _ptr(qsl), _ptr(ctx), _ptr(bt), bt.shape[1], ctx.shape[0],
                                        float(scale), _ptr(out)), "paged_prefill")
    return out


def f16_to_double(bits: int) -> float:
    return _load().oracle_f16_to_double(bits)


def bf16_to_double(bits: int) -> float:
    return _load().oracle_bf16_to_double(bits)


def fp8_to_double(bits: int) -> float:
    return _load().oracle_fp8_to_double(bits)


def fp8_from_float(x: float) -> int:
    """E4M3 code of an fp32 value (nearest, ties to even; saturating at +-448)."""
    return int(_load().oracle_fp8_from_float(x))


def decode_values(arr: np.ndarray, dtype: int) -> np.ndarray:
    """fp64 values of a raw-bits array, decoded element by element by the C decoder."""
    flat = np.ascontiguousarray(arr).reshape(-1)
    if dtype == F32:
        return flat.astype(np.float64).reshape(arr.shape)
    f = {F16: f16_to_double, BF16: bf16_to_double, FP8: fp8_to_double}[dtype]
    return np.array([f(int(b)) for b in flat], dtype=np.float64).reshape(arr.shape)
