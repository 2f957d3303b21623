"""Drive the CPU oracle through a workload (test-side helper)."""
from __future__ import annotations

import os

import numpy as np

import oracle


def key_rows(k):
    """K pool [nb][H][d/X][B][X] as [nb][H][B][d] (a copy): element (blk, h, off, e)."""
    nb, H, nc, B, x = k.shape
    return k.transpose(0, 1, 3, 2, 4).reshape(nb, H, B, nc * x)


def fill_pools(wl, include_step=True):
    """Oracle pools after the workload's setup ops (and, by default, the step's scatter)."""
    k, v = wl.empty_pools()
    ops = list(wl.setup) + ([wl.step_scatter] if include_step and wl.step_scatter else [])
    for op in ops:
        if op.kind == "scatter":
            oracle.reshape_and_cache(k, v, wl.cache_dtype, op.key, op.value, op.slots,
                                     in_dtype=wl.dtype, k_scale=wl.k_scale, v_scale=wl.v_scale)
        else:
            oracle.copy_blocks(k, v, wl.cache_dtype, op.pairs)
    return k, v


def _kv(wl):
    return dict(q_dtype=wl.dtype, k_scale=wl.k_scale, v_scale=wl.v_scale)


def reference_output(wl, k, v):
    """fp64 oracle output of the workload's attention step over pools k, v."""
    if wl.mode == "decode":
        return oracle.paged_decode(k, v, wl.cache_dtype, wl.q, wl.block_tables, wl.context_lens,
                                   wl.scale, window=wl.window, **_kv(wl))
    return oracle.paged_prefill(k, v, wl.cache_dtype, wl.q, wl.query_start_loc, wl.context_lens,
                                wl.block_tables, wl.scale, **_kv(wl))


def oracle_threads():
    """Threads for row-parallel oracle calls (the C entry points run without the
    interpreter lock and share no state): the host's cores, at most 16."""
    return max(1, min(16, os.cpu_count() or 1))


def sampled_rows(wl, k, v, rows, threads=None):
    """fp64 oracle output for selected query rows only (all heads), the rows
    spread over a thread pool."""
    rows = np.asarray(rows, dtype=np.int64)
    n = oracle_threads() if threads is None else threads
    if n > 1 and rows.size > 1:
        from concurrent.futures import ThreadPoolExecutor
        parts = [p for p in np.array_split(rows, min(n * 4, rows.size)) if p.size]
        with ThreadPoolExecutor(max_workers=n) as pool:
            outs = list(pool.map(lambda p: _rows(wl, k, v, p), parts))
        return np.concatenate(outs, axis=0)
    return _rows(wl, k, v, rows)


def _rows(wl, k, v, rows):
    if wl.mode == "decode":
        seq = rows
        pos = wl.context_lens[rows] - 1
    else:
        qsl = wl.query_start_loc
        seq = np.searchsorted(qsl, rows, side="right") - 1
        qlen = qsl[seq + 1] - qsl[seq]
        pos = wl.context_lens[seq] - qlen + (rows - qsl[seq])
    return oracle.paged_attention_rows(k, v, wl.cache_dtype, wl.q[rows], wl.block_tables,
                                       wl.context_lens, seq, pos, wl.scale, window=wl.window,
                                       **_kv(wl))
