#!/usr/bin/env python3
"""Benchmark of the paged KV-cache hot path on one MI355X.

Default workload: LLaMA-2-13B-shaped single-layer decode (64 sequences,
contexts U[128, 2048], 40 heads, head_dim 128, block_size 16, fp16 KV, pool
1.1x the need with shuffled blocks).  One step = the reshape_and_cache
scatter of the 64 new tokens + paged decode attention over every sequence's
whole cache (+ the split-KV reduce when partitioned).  Inputs are resident
in HBM before timing; two identical pool copies alternate between steps so
the 256 MiB Infinity Cache cannot serve a step from the previous one.

`value` comes from K steps timed back to back with nothing between them; the
roofline's per-launch duration from K further steps with timing events around
each attention call.  The default run also measures, in the same process,
the tiny fp32 decode (launch-bound; its roofline fraction is reported, not
tuned for), long-context split-KV decode, GQA decode at block sizes 16 and 32
and chunked prefill, each under `extra_configs` with its own roofline and a
short CPU oracle sample.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}   # dense


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def make_workload(name, partition, block_size=16, placement="shuffled"):
    from paged_kv_cache_92_amd import workloads as W
    if name == "llama13b":
        wl = W.llama13b_decode_f16(B=block_size, placement=placement)
        desc = "llama2-13b-shaped single-layer paged decode, fp16 KV"
        if block_size != 16 or placement != "shuffled":
            desc += f" (block {block_size}, {placement} blocks)"
    elif name == "llama13b_fp8":
        wl = W.llama13b_decode_fp8()
        desc = ("llama2-13b-shaped single-layer paged decode, fp8 e4m3 KV cache "
                "(per-tensor scales, fp16 queries)")
    elif name == "long_split":
        wl = W.long_context_split_f16()
        desc = "long-context split-KV paged decode, fp16 KV"
    elif name in ("gqa16", "gqa32"):
        wl = W.gqa_decode_bf16(B=16 if name == "gqa16" else 32)
        desc = f"GQA 32q/8kv paged decode, bf16 KV, block {wl.block_size}"
    elif name == "prefill":
        wl = W.chunked_prefill_bf16()
        desc = "chunked causal prefill over paged cache with shared prefixes, bf16"
    elif name == "sliding":
        wl = W.sliding_window_gqa_bf16()
        desc = ("mistral-7b-shaped sliding-window paged decode (window 4096, 32q/8kv heads, "
                "L ~ U[1024, 16384], blocks before each window released), bf16")
    elif name == "mixed":
        wl = W.mixed_step_f16()
        desc = ("llama2-13b-shaped step batching 64 decode rows with two 512-row prefill chunks "
                "in one call, fp16")
    elif name == "tiny":
        wl = W.tiny_decode_f32()
        desc = "tiny paged decode, fp32"
    else:
        raise SystemExit(f"unknown config {name}")
    if partition is not None and wl.mode in ("decode", "mixed"):
        wl.partition_size = partition
    return wl, desc


def attention_flops(wl):
    import numpy as np
    d, Hq = wl.head_dim, wl.num_q_heads
    if wl.mode == "decode":
        L = wl.context_lens.astype(np.int64)
        if wl.window > 0:
            L = np.minimum(L, wl.window)
        return float(L.sum()) * Hq * d * 4
    qsl = wl.query_start_loc
    total = 0
    for s in range(wl.S):
        ql = int(qsl[s + 1] - qsl[s])
        h = int(wl.context_lens[s]) - ql
        # rows at positions h .. h+ql-1 attend to p+1 keys each
        total += ql * (h + 1) + ql * (ql - 1) // 2
    return float(total) * Hq * d * 4


def kernel_source_sha():
    """First 16 hex digits of sha256 over the HIP sources, headers and C++ API, in name order."""
    import glob
    import hashlib
    csrc = os.path.join(ROOT, "paged_kv_cache_92_amd", "csrc")
    h = hashlib.sha256()
    for pat in ("*.hip", "*.h", "*.cpp"):
        for f in sorted(glob.glob(os.path.join(csrc, pat))):
            with open(f, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(config):
    """HBM bytes per launch of the dominant kernel, from the committed rocprofv3 counter runs.

    None unless the counters were taken on the kernel sources as they are now."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    e = t.get(config)
    if e is None or t.get("source_sha") != kernel_source_sha():
        return None
    return int(round(e["fetch_bytes"] + e["write_bytes"]))


def read_probe_gbps(torch, gib=4, reps=5, tile=4096, waves=65536):
    """Read ceiling of the memory system for the decode kernels' access pattern: 4 KiB tiles in
    random order, non-temporal 16-byte loads (paged_kv_cache_92_amd/probe).  GB/s."""
    import ctypes

    import numpy as np

    from paged_kv_cache_92_amd.build import PROBE_LIB
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"{PROBE_LIB} is not built: run __graft_entry__.build() first")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.pkv_probe_read_tiles.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    nbytes = gib << 30
    ntiles = nbytes // tile
    tpw = ntiles // waves
    used = waves * tpw
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    perm = np.random.default_rng(0).permutation(used).astype(np.int32)
    assert 0 <= perm.min() and perm.max() < ntiles
    idx = torch.from_numpy(perm).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def run():
        rc = lib.pkv_probe_read_tiles(ctypes.c_void_p(buf.data_ptr()), ctypes.c_void_p(idx.data_ptr()),
                                      tile, waves, tpw, ctypes.c_void_p(sink.data_ptr()), stream)
        if rc != 0:
            raise RuntimeError(f"read probe launch failed ({rc})")
    run()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        run()
    b.record()
    torch.cuda.synchronize()
    return used * tile / (a.elapsed_time(b) * 1e-3 / reps) / 1e9


def cache_ops(torch, pkv, steps):
    """Block copy (copy-on-write) and slot scatter timed alone, at the chunked-prefill pool shape
    (32 KV heads, block 16, head_dim 128, bf16: 128 KiB per block and tensor).  Bytes moved count
    every element read and written once."""
    import numpy as np
    H, B, d, nb = 32, 16, 128, 4096
    cache = pkv.PagedKVCache(nb, H, B, d, torch.bfloat16)
    cache.k_pool.view(torch.int16).random_()
    cache.v_pool.view(torch.int16).random_()
    rng = np.random.default_rng(11)
    res = {}

    def timed(fn):
        fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / steps

    blk = H * B * d * 2
    for n in (64, 1024):
        ids = rng.permutation(nb)[:2 * n].astype(np.int32)
        pairs = torch.from_numpy(np.stack([ids[:n], ids[n:]], axis=1).copy()).cuda()
        us = timed(lambda: pkv.copy_blocks(cache, pairs))
        moved = n * 2 * blk * 2
        res[f"copy_blocks_{n}_pairs"] = {"us": round(us, 2), "bytes": moved,
                                         "GBps": round(moved / us / 1e3, 1),
                                         "frac": round(moved / us / 1e3 / HBM_PEAK_GBS, 4)}
    # A plain device copy of 2 GiB for comparison (reads and writes 2 GiB each).
    src = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    us = timed(lambda: dst.copy_(src))
    res["device_copy_2GiB"] = {"us": round(us, 2), "bytes": 2 * (2 << 30),
                               "GBps": round(2 * (2 << 30) / us / 1e3, 1),
                               "frac": round(2 * (2 << 30) / us / 1e3 / HBM_PEAK_GBS, 4)}
    del src, dst
    for T, kind in ((4096, "chunk"), (64, "decode")):
        key = torch.randn(T, H, d, device="cuda").to(torch.bfloat16)
        value = torch.randn(T, H, d, device="cuda").to(torch.bfloat16)
        if kind == "chunk":      # one 4096-token run of consecutive slots
            slots = np.arange(T, dtype=np.int64) + 7 * B
        else:                    # one token in each of 64 scattered blocks
            slots = rng.permutation(nb)[:T].astype(np.int64) * B + rng.integers(0, B, size=T)
        sl = torch.from_numpy(slots).cuda()
        us = timed(lambda: pkv.reshape_and_cache(cache, key, value, sl))
        moved = T * H * d * 2 * 2 * 2
        res[f"scatter_{T}_{kind}"] = {"us": round(us, 2), "bytes": moved,
                                      "GBps": round(moved / us / 1e3, 1),
                                      "frac": round(moved / us / 1e3 / HBM_PEAK_GBS, 4)}
    return res


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _all_cores(calls, cores):
    """Wall time of the same oracle calls spread over `cores` threads (the oracle's C
    entry points run without the interpreter lock and keep no shared state)."""
    from concurrent.futures import ThreadPoolExecutor
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=cores) as pool:
        list(pool.map(lambda f: f(), calls))
    return time.perf_counter() - t0


def cpu_baseline(wl, budget_s):
    """The oracle as it stands on a bounded sample of the same input: one thread, then the
    same sample over all host cores (up to 16 threads)."""
    import numpy as np

    import oracle
    k, v = wl.empty_pools()
    for op in wl.setup + [wl.step_scatter]:
        if op.kind == "scatter":
            oracle.reshape_and_cache(k, v, wl.cache_dtype, op.key, op.value, op.slots,
                                     in_dtype=wl.dtype, k_scale=wl.k_scale, v_scale=wl.v_scale)
        else:
            oracle.copy_blocks(k, v, wl.cache_dtype, op.pairs)
    elt = {0: 4, 1: 2, 2: 2, 3: 1}[wl.cache_dtype]
    kv = dict(q_dtype=wl.dtype, k_scale=wl.k_scale, v_scale=wl.v_scale)
    cores = max(1, min(16, os.cpu_count() or 1))
    t0 = time.perf_counter()
    n = 0
    kv_bytes = 0
    if wl.mode == "decode":
        def seq(i):
            return lambda: oracle.paged_attention_rows(
                k, v, wl.cache_dtype, wl.q[i:i + 1], wl.block_tables, wl.context_lens, [i],
                [int(wl.context_lens[i]) - 1], wl.scale, window=wl.window, **kv)
        while n < wl.S and (time.perf_counter() - t0) < budget_s:
            seq(n)()
            L = int(wl.context_lens[n])
            kv_bytes += (min(L, wl.window) if wl.window else L) * 2 * wl.num_kv_heads * wl.head_dim * elt
            n += 1
        el = time.perf_counter() - t0
        el_all = _all_cores([seq(i) for i in range(n)], cores)
        return {"value": round(kv_bytes / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                "tokens_per_s": round(n / el, 3),
                "all_cores": {"value": round(kv_bytes / el_all / 1e9, 4), "cores": cores,
                              "tokens_per_s": round(n / el_all, 3)},
                "cpu_model": _cpu_model(),
                "sample": f"decode of the first {n} of {wl.S} sequences (all {wl.num_q_heads} heads): "
                          f"block-table reassembly + fp64 softmax attention, {el:.1f} s wall on 1 "
                          f"thread, {el_all:.1f} s on {cores}"}
    qsl = wl.query_start_loc
    flops = 0.0

    def row(r):
        s_ = int(np.searchsorted(qsl, r, side="right") - 1)
        pos = int(wl.context_lens[s_] - (qsl[s_ + 1] - qsl[s_]) + (r - qsl[s_]))
        return pos, lambda: oracle.paged_attention_rows(
            k, v, wl.cache_dtype, wl.q[r:r + 1], wl.block_tables, wl.context_lens, [s_], [pos],
            wl.scale, **kv)
    while n < qsl[-1] and (time.perf_counter() - t0) < budget_s:
        pos, call = row(n)
        call()
        flops += (pos + 1) * wl.num_q_heads * wl.head_dim * 4
        n += 1
    el = time.perf_counter() - t0
    el_all = _all_cores([row(r)[1] for r in range(n)], cores)
    common = {"kind": "oracle", "cores": 1, "cpu_model": _cpu_model()}
    if wl.mode == "mixed":
        return {"value": round(n / el, 3), "unit": "rows/s", **common,
                "all_cores": {"value": round(n / el_all, 3), "cores": cores},
                "sample": f"first {n} query rows of {int(qsl[-1])} (decode rows first, all "
                          f"{wl.num_q_heads} heads), {el:.1f} s wall on 1 thread, {el_all:.1f} s on "
                          f"{cores}"}
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", **common,
            "all_cores": {"value": round(flops / el_all / 1e12, 6), "cores": cores},
            "sample": f"first {n} query rows of {int(qsl[-1])} (all {wl.num_q_heads} heads), "
                      f"{el:.1f} s wall on 1 thread, {el_all:.1f} s on {cores}"}


EXTRA_CONFIGS = ("tiny", "long_split", "gqa16", "gqa32", "prefill")


def gemm_probe_tflops(torch, n=16384, reps=20):
    """Dense bf16 matrix-product rate this GPU sustains in practice: one n x n x n product
    y = x w^T (torch.nn.functional.linear: both operands contiguous along the reduced
    dimension, the library's fastest layout here) repeated back to back.  TFLOP/s.  A
    calibration of what the matrix cores deliver under load, beside the nominal peak; not
    part of the path."""
    import torch.nn.functional as F
    g = torch.Generator(device="cuda").manual_seed(0)
    x = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
    w = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
    for _ in range(3):
        c = F.linear(x, w)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(reps):
        c = F.linear(x, w)
    t1.record()
    torch.cuda.synchronize()
    sec = t0.elapsed_time(t1) * 1e-3 / reps
    del x, w, c
    return 2.0 * n ** 3 / sec / 1e12


def run_config(torch, pkv, name, args, cpu_budget, read_probe, fused=False, kv_cache="model",
               block_size=16, placement="shuffled", partition=None):
    """One workload: generate, upload two pool copies, time the step, report its roofline.

    Two timed loops over the same inputs, each bracketed by one pair of events (an event
    pair around every call would cost the stream a few microseconds per call): K whole steps
    (the new tokens' scatter, then the attention call) back to back give ms_per_step and
    value; K attention calls back to back give the roofline's per-launch duration."""
    import numpy as np

    from paged_kv_cache_92_amd.runner import DeviceWorkload, new_cache

    t0 = time.time()
    wl, desc = make_workload(name, partition, block_size, placement)
    if kv_cache == "fp8" and wl.cache_dtype != 3:
        from paged_kv_cache_92_amd import workloads as W
        wl.kv_dtype, wl.k_scale, wl.v_scale = W.FP8, 0.0135, 0.0135
        desc += ", stored as fp8 e4m3 codes (per-tensor scales)"
    if fused and wl.mode != "decode":
        raise SystemExit("--step fused applies to decode workloads")
    log(f"[bench] generated {wl.name} in {time.time() - t0:.1f}s "
        f"(pool {wl.num_blocks} blocks, KV {wl.kv_bytes() / 1e9:.3f} GB)")

    # Two identical device copies of the cache; steps alternate between them.
    copies = []
    for i in range(2):
        dw = DeviceWorkload(wl)
        cache = new_cache(wl)
        dw.fill(cache)
        copies.append((dw, cache))
    torch.cuda.synchronize()
    log(f"[bench] uploaded and filled 2 x {copies[0][1].nbytes() / 1e9:.2f} GB pools")

    dw0 = copies[0][0]
    out = torch.empty_like(dw0.q)
    ws = None
    if wl.mode in ("decode", "mixed"):
        nd = wl.S if wl.mode == "decode" else int(wl.info["num_decode_seqs"])
        need = pkv.decode_workspace_bytes(copies[0][1], nd, wl.num_q_heads, wl.max_context_len,
                                          wl.partition_size)
        if need:
            ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def attend(i):
        dw, cache = copies[i % 2]
        if fused:
            dw.append_attend(cache, out=out, workspace=ws)
        else:
            dw.attend(cache, out=out, workspace=ws)

    def step(i):
        if not fused:
            dw, cache = copies[i % 2]
            dw.apply(cache, dw.step)
        attend(i)

    def timed(fn, n):
        """Average ms of n calls fn(0) .. fn(n-1), back to back, after a synchronisation."""
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for i in range(n):
            fn(i)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / n

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps done")

    # Throughput: K whole steps back to back.
    ms_step = timed(step, args.steps)
    # Per-launch duration of the attention call: K calls back to back (for the
    # appending call the step is that call).
    attn_avg = timed(attend, args.steps)
    log(f"[bench] {args.steps} steps: {ms_step * 1e3:.1f} us/step; attention call "
        f"{attn_avg * 1e3:.1f} us avg")

    ways = {}
    if wl.mode == "mixed":
        # The same step served other ways, attention only, same alternation.
        for how in ("sequential", "unified", "decode", "prefill"):
            def split_call(i, how=how):
                dw, cache = copies[i % 2]
                dw.attend_split(cache, how, out, workspace=ws)
            for i in range(args.warmup):
                split_call(i)
            ways[how] = timed(split_call, args.steps)
            log(f"[bench] {how}: {ways[how] * 1e3:.1f} us avg")

    dt = {0: "f32", 1: "f16", 2: "bf16", 3: "fp8_e4m3"}[wl.cache_dtype]
    # The products run in the model dtype (an 8-bit cache is widened to it).
    mdt = {0: "f32", 1: "f16", 2: "bf16"}[wl.dtype]
    kv = wl.kv_bytes()
    flops = attention_flops(wl)
    res = {
        "metric": "paged decode effective KV GB/s (% of HBM peak) + decode tokens/s, 13B shape",
        "ms_per_step": round(ms_step, 5), "dtype": dt,
    }
    if wl.mode == "decode":
        gbs_step = kv / (ms_step * 1e-3) / 1e9
        gbs_attn = kv / (attn_avg * 1e-3) / 1e9
        res.update({
            "value": round(gbs_step, 2), "unit": "GB/s",
            "pct_hbm_peak": round(100 * gbs_step / HBM_PEAK_GBS, 2),
            "decode_tokens_per_s": round(wl.S / (ms_step * 1e-3), 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs_attn, 2), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs_attn / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic(name),
                         "kernel": "paged decode (partial + reduce when split)" if not fused
                         else "appending paged decode (partial + reduce when split)",
                         "algorithmic_bytes_per_launch": kv,
                         "avg_launch_us": round(attn_avg * 1e3, 2)},
        })
        if read_probe:
            probe = read_probe_gbps(torch)
            res["roofline"]["read_probe_GBps"] = round(probe, 1)
            res["roofline"]["frac_of_read_probe"] = round(gbs_attn / probe, 4)
            log(f"[bench] read-ceiling probe: {probe:.0f} GB/s (decode call at "
                f"{100 * gbs_attn / probe:.1f}% of it)")
        if name.startswith("llama13b"):
            res["decode_tokens_per_s_40_layer_attention_only"] = round(wl.S / (40 * ms_step * 1e-3), 1)
        else:
            res["metric"] = "paged decode effective KV GB/s (% of HBM peak)"
        if wl.window:
            res["metric"] = "sliding-window paged decode effective KV GB/s (window tokens only)"
    elif wl.mode == "mixed":
        nd = int(wl.info["num_decode_seqs"])
        rows = int(wl.query_start_loc[-1])
        elt = {0: 4, 1: 2, 2: 2, 3: 1}[wl.cache_dtype]
        dec_bytes = int(wl.context_lens[:nd].astype(np.int64).sum()) * 2 * wl.num_kv_heads * \
            wl.head_dim * elt
        pre_flops = attention_flops(wl) - float(wl.context_lens[:nd].astype(np.int64).sum()) * \
            wl.num_q_heads * wl.head_dim * 4
        # KV bytes of the chunk rows' contexts: the step reads them too.
        pre_kv_bytes = int(wl.context_lens[nd:].astype(np.int64).sum()) * 2 * wl.num_kv_heads * \
            wl.head_dim * elt
        # Lower bound of the step: decode KV at HBM peak and chunk products at
        # MFMA peak, overlapped perfectly; the larger of the two names the bound.
        t_hbm = dec_bytes / (HBM_PEAK_GBS * 1e9)
        t_mfma = pre_flops / (MFMA_PEAK_TFLOPS[mdt] * 1e12)
        # The same bound with the chunks' KV bytes added to the HBM side.
        t_hbm_all = (dec_bytes + pre_kv_bytes) / (HBM_PEAK_GBS * 1e9)
        bound = "hbm" if t_hbm >= t_mfma else "mfma"
        t_attn = attn_avg * 1e-3
        res["metric"] = "mixed decode + chunked-prefill step: query rows/s (one call)"
        res.update({
            "value": round(rows / (ms_step * 1e-3), 1), "unit": "rows/s",
            "roofline": {"bound": bound,
                         "achieved": round(dec_bytes / t_attn / 1e9, 2) if bound == "hbm"
                         else round(pre_flops / t_attn / 1e12, 2),
                         "peak": HBM_PEAK_GBS if bound == "hbm" else MFMA_PEAK_TFLOPS[mdt],
                         "unit": "GB/s" if bound == "hbm" else "TFLOP/s",
                         "frac": round(max(t_hbm, t_mfma) / t_attn, 4),
                         "traffic": measured_traffic(name),
                         "kernel": "mixed step (decode kernel and prefill kernel at once)",
                         "algorithmic_bytes_decode": dec_bytes,
                         "algorithmic_flops_prefill": pre_flops,
                         "algorithmic_bytes_prefill_kv": pre_kv_bytes,
                         "frac_with_prefill_kv": round(max(t_hbm_all, t_mfma) / t_attn, 4),
                         "avg_launch_us": round(attn_avg * 1e3, 2)},
            "mixed": {"one_call_us": round(attn_avg * 1e3, 2),
                      "sequential_calls_us": round(ways["sequential"] * 1e3, 2),
                      "unified_prefill_kernel_us": round(ways["unified"] * 1e3, 2),
                      "decode_part_alone_us": round(ways["decode"] * 1e3, 2),
                      "prefill_part_alone_us": round(ways["prefill"] * 1e3, 2),
                      "decode_rows": nd, "chunk_rows": rows - nd},
        })
    else:
        tf_step = flops / (ms_step * 1e-3) / 1e12
        tf_attn = flops / (attn_avg * 1e-3) / 1e12
        res.update({
            "value": round(tf_step, 2), "unit": "TFLOP/s",
            "roofline": {"bound": "mfma", "achieved": round(tf_attn, 2), "peak": MFMA_PEAK_TFLOPS[mdt],
                         "unit": "TFLOP/s", "frac": round(tf_attn / MFMA_PEAK_TFLOPS[mdt], 4),
                         "traffic": measured_traffic(name), "kernel": "paged prefill",
                         "algorithmic_flops_per_launch": flops,
                         "avg_launch_us": round(attn_avg * 1e3, 2)},
        })
        if read_probe:
            # A calibration beside the measurement: if the library product fails,
            # the line is still reported, with the probe's fields null.
            try:
                gp = gemm_probe_tflops(torch)
            except RuntimeError as e:
                log(f"[bench] dense bf16 product probe failed: {e}")
                gp = None
            res["roofline"]["gemm_probe_TFLOPs"] = None if gp is None else round(gp, 1)
            res["roofline"]["frac_of_gemm_probe"] = None if gp is None else round(tf_attn / gp, 4)
            if gp is not None:
                log(f"[bench] dense bf16 product probe: {gp:.0f} TFLOP/s (prefill call at "
                    f"{100 * tf_attn / gp:.1f}% of it)")
        res["metric"] = "chunked prefill attention TFLOP/s (% of MFMA peak)"
    res["config"] = {"workload": desc, "seqs": wl.S, "q_heads": wl.num_q_heads,
                     "kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
                     "block_size": wl.block_size, "pool_blocks": wl.num_blocks,
                     "placement": placement,
                     "step": ("fused" if fused else "scatter+decode") if wl.mode == "decode" else None,
                     "total_context_tokens": int(wl.context_lens.sum()),
                     "sliding_window": wl.window or None,
                     "partition_size": wl.partition_size if wl.mode != "prefill" else None,
                     "kv_bytes": kv, "attention_flops": flops}
    if cpu_budget > 0:
        log("[bench] timing the CPU oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(wl, cpu_budget)
    del copies, out, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="llama13b",
                    choices=["llama13b", "llama13b_fp8", "long_split", "gqa16", "gqa32", "prefill",
                             "mixed", "sliding", "tiny"])
    ap.add_argument("--partition", type=int, default=None,
                    help="split-KV partition size in tokens (default: the workload's)")
    ap.add_argument("--block-size", type=int, default=16, choices=[8, 16, 32],
                    help="block size of the llama13b workload (paging-overhead sweep)")
    ap.add_argument("--placement", default="shuffled", choices=["shuffled", "contiguous"],
                    help="physical block order of the llama13b workload (paging-overhead sweep)")
    ap.add_argument("--kv-cache", default="model", choices=["model", "fp8"],
                    help="fp8: store the workload's cache as E4M3 codes (scales 0.0135)")
    ap.add_argument("--step", default="scatter+decode", choices=["scatter+decode", "fused"],
                    help="decode workloads: fused = one appending call that writes the new "
                         "tokens' K/V and attends (timed as the attention launch)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--extra-cpu-budget", type=float, default=3.0,
                    help="seconds of oracle work for each extra configuration")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="default run: skip the tiny, long-split, GQA and prefill configurations")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--read-probe-gib", type=int, default=0,
                    help="only run the HBM read-ceiling probe over this many GiB of random 4 KiB tiles")
    ap.add_argument("--cache-ops", action="store_true",
                    help="only time the block copy and the slot scatter alone (prefill pool shape)")
    ap.add_argument("--no-read-probe", action="store_true",
                    help="skip the ceiling probes after the timed steps (decode: HBM reads of random "
                         "4 KiB tiles; prefill: a dense bf16 matrix product)")
    ap.add_argument("--gemm-probe", action="store_true",
                    help="only time the dense bf16 matrix-product probe (16384^3, torch.nn.functional.linear)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_92_amd as pkv

    torch.cuda.set_device(0)
    if args.copy_probe_mib:
        # A copy of known size: reads and writes exactly n bytes per launch.
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": args.steps}), flush=True)
        return
    if args.cache_ops:
        print(json.dumps({"cache_ops": cache_ops(torch, pkv, args.steps), "steps": args.steps,
                          "peak_GBps": HBM_PEAK_GBS}), flush=True)
        return
    if args.gemm_probe:
        gp = gemm_probe_tflops(torch, reps=args.steps)
        print(json.dumps({"gemm_probe_TFLOPs": round(gp, 1), "n": 16384, "dtype": "bf16",
                          "launches": args.steps}), flush=True)
        return
    if args.read_probe_gib:
        g = read_probe_gbps(torch, gib=args.read_probe_gib, reps=args.steps)
        print(json.dumps({"read_probe_GBps": round(g, 1), "tile_bytes": 4096,
                          "bytes": args.read_probe_gib << 30, "launches": args.steps}), flush=True)
        return
    pkv.lib()
    if args.config != "llama13b" and (args.block_size != 16 or args.placement != "shuffled"):
        raise SystemExit("--block-size/--placement apply to the llama13b workload only")
    fused = args.step == "fused"
    res = {"metric": None, "value": None, "unit": None, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": None, "data": "synthetic"}
    main_res = run_config(torch, pkv, args.config, args,
                          0.0 if args.no_cpu_baseline else args.cpu_budget,
                          not args.no_read_probe, fused=fused, kv_cache=args.kv_cache,
                          block_size=args.block_size, placement=args.placement,
                          partition=args.partition)
    res.update(main_res)
    # The default run also measures the other configurations' hot paths, each
    # with its own roofline, in this process.
    default_sweep = (args.config == "llama13b" and args.block_size == 16 and args.placement == "shuffled"
                     and args.kv_cache == "model" and not fused and args.partition is None)
    if default_sweep and not args.no_extras:
        extras = {}
        for name in EXTRA_CONFIGS:
            log(f"[bench] configuration {name}")
            extras[name] = run_config(torch, pkv, name, args,
                                      0.0 if args.no_cpu_baseline else args.extra_cpu_budget,
                                      name == "prefill" and not args.no_read_probe)
        res["extra_configs"] = extras
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
