"""Drive a synthetic workload through libpkv: host arrays -> device -> library calls.

Used by the benchmark, the smoke check and the GPU tests.  Every computation
is a library call; this module only uploads inputs and sequences the calls.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _binding as pkv
from . import workloads as W

TORCH_DTYPE = {W.F32: torch.float32, W.F16: torch.float16, W.BF16: torch.bfloat16,
               W.FP8: torch.float8_e4m3fn}
NAN_BITS = {W.F32: None, W.F16: 0x7E00, W.BF16: 0x7FC0, W.FP8: 0x7F}


def to_device(bits: np.ndarray, dtype: int, device="cuda") -> torch.Tensor:
    """Raw-bits numpy array -> device tensor of the cache dtype (same bits)."""
    if dtype == W.F32:
        return torch.from_numpy(np.ascontiguousarray(bits)).to(device)
    if dtype == W.FP8:
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.uint8)).to(device).view(torch.float8_e4m3fn)
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device)
    return t.view(TORCH_DTYPE[dtype])


def bits_of(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> raw-bits numpy array (float32, uint16, or uint8 for 8-bit floats)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def values_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def new_cache(wl, device="cuda") -> pkv.PagedKVCache:
    cd = wl.cache_dtype
    cache = pkv.PagedKVCache(wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim,
                             TORCH_DTYPE[cd], device=device, model_dtype=TORCH_DTYPE[wl.dtype],
                             k_scale=wl.k_scale, v_scale=wl.v_scale)
    if cd == W.F32:
        cache.k_pool.fill_(float("nan"))
        cache.v_pool.fill_(float("nan"))
    elif cd == W.FP8:
        cache.k_pool.view(torch.uint8).fill_(NAN_BITS[cd])
        cache.v_pool.view(torch.uint8).fill_(NAN_BITS[cd])
    else:
        cache.k_pool.view(torch.int16).fill_(NAN_BITS[cd])
        cache.v_pool.view(torch.int16).fill_(NAN_BITS[cd])
    return cache


class DeviceWorkload:
    """Device copies of a workload's integer inputs and query."""

    def __init__(self, wl, device="cuda"):
        self.wl = wl
        self.block_tables = torch.from_numpy(wl.block_tables).to(device)
        self.context_lens = torch.from_numpy(wl.context_lens).to(device)
        self.q = to_device(wl.q, wl.dtype, device)
        self.qsl = None if wl.query_start_loc is None else torch.from_numpy(wl.query_start_loc).to(device)
        self._qsl_tail = None
        self.ops = []
        for op in wl.setup:
            self.ops.append(self._dev_op(op, device))
        self.step = self._dev_op(wl.step_scatter, device)

    def _dev_op(self, op, device):
        if op.kind == "scatter":
            return ("scatter", to_device(op.key, self.wl.dtype, device),
                    to_device(op.value, self.wl.dtype, device), torch.from_numpy(op.slots).to(device))
        return ("copy", torch.from_numpy(np.ascontiguousarray(op.pairs, dtype=np.int32)).to(device))

    def apply(self, cache, op):
        if op[0] == "scatter":
            pkv.reshape_and_cache(cache, op[1], op[2], op[3])
        else:
            pkv.copy_blocks(cache, op[1])

    def fill(self, cache):
        for op in self.ops:
            self.apply(cache, op)

    def attend(self, cache, partition_size=None, out=None, workspace=None, out_dtype=None):
        wl = self.wl
        if wl.mode == "decode":
            ps = wl.partition_size if partition_size is None else partition_size
            return pkv.paged_decode(cache, self.q, self.block_tables, self.context_lens,
                                    wl.max_context_len, scale=wl.scale, partition_size=ps, out=out,
                                    workspace=workspace, out_dtype=out_dtype,
                                    sliding_window=wl.window)
        qlens = np.diff(wl.query_start_loc)
        if wl.mode == "mixed":
            nd = int(wl.info["num_decode_seqs"])
            ps = wl.partition_size if partition_size is None else partition_size
            return pkv.paged_mixed(cache, self.q, self.qsl, self.context_lens, self.block_tables,
                                   nd, int(qlens[nd:].max(initial=0)), wl.max_context_len,
                                   scale=wl.scale, partition_size=ps, out=out,
                                   workspace=workspace, out_dtype=out_dtype)
        return pkv.paged_prefill(cache, self.q, self.qsl, self.context_lens, self.block_tables,
                                 int(qlens.max()), wl.max_context_len, scale=wl.scale, out=out,
                                 out_dtype=out_dtype)

    def append_attend(self, cache, partition_size=None, out=None, workspace=None, out_dtype=None):
        """The decode step's scatter and attention as one appending call (the
        step's key/value rows are one per sequence, for position L-1)."""
        wl = self.wl
        assert wl.mode == "decode"
        _, key, value, _ = self.step
        ps = wl.partition_size if partition_size is None else partition_size
        return pkv.paged_decode_append(cache, key, value, self.q, self.block_tables,
                                       self.context_lens, wl.max_context_len, scale=wl.scale,
                                       partition_size=ps, out=out, workspace=workspace,
                                       out_dtype=out_dtype, sliding_window=wl.window)

    def attend_split(self, cache, how, out, workspace=None):
        """A mixed step served another way, for comparison: ``"sequential"`` is
        a decode call then a prefill call on one stream, ``"unified"`` one
        prefill call over every row (a decode row as a chunk of one);
        ``"decode"`` and ``"prefill"`` run one part alone."""
        wl = self.wl
        assert wl.mode == "mixed"
        nd = int(wl.info["num_decode_seqs"])
        qlens = np.diff(wl.query_start_loc)
        if how == "unified":
            return pkv.paged_prefill(cache, self.q, self.qsl, self.context_lens, self.block_tables,
                                     int(qlens.max()), wl.max_context_len, scale=wl.scale, out=out)
        assert how in ("sequential", "decode", "prefill")
        if how != "prefill":
            pkv.paged_decode(cache, self.q[:nd], self.block_tables[:nd], self.context_lens[:nd],
                             wl.max_context_len, scale=wl.scale, partition_size=wl.partition_size,
                             out=out[:nd], workspace=workspace)
        if how != "decode":
            base = int(wl.query_start_loc[nd])
            if self._qsl_tail is None:
                self._qsl_tail = self.qsl[nd:] - base
            pkv.paged_prefill(cache, self.q[base:], self._qsl_tail, self.context_lens[nd:],
                              self.block_tables[nd:], int(qlens[nd:].max()), wl.max_context_len,
                              scale=wl.scale, out=out[base:])
        return out

    def run(self, cache, partition_size=None):
        """Setup, then one step: scatter the new tokens and attend."""
        self.fill(cache)
        self.apply(cache, self.step)
        return self.attend(cache, partition_size=partition_size)
