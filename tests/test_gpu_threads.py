"""Calls from several host threads at once, each on its own stream.

The library keeps per-device state behind locks (occupancy figures, LDS size,
the mixed call's side stream and two events per caller stream); the kernels
share nothing but read-only inputs.  Every thread's result must equal, bit for bit, the
same call made alone.
"""
import threading

import numpy as np
import pytest
import torch

from paged_kv_cache_92_amd import workloads as W
from tests.gpu_run import DeviceWorkload, bits_of, new_cache
from tests.test_gpu_mixed import _mixed

pytestmark = pytest.mark.gpu


def test_concurrent_calls_on_separate_streams():
    wls = [
        # wavefront kernel, balanced schedule
        W.make_decode("thr_a", 401, lambda rng: [1, 17, 100, 255, 700], Hq=8, Hkv=8, d=128, B=16,
                      dtype=W.F16, max_context_len=1024, partition_size=-1),
        # matrix-core kernel, fixed partitions + reduce
        W.make_decode("thr_b", 402, lambda rng: [3, 64, 513, 1000], Hq=16, Hkv=2, d=128, B=16,
                      dtype=W.BF16, max_context_len=1024, partition_size=256),
        # decode rows on the side stream, chunk rows on the caller's
        _mixed(W.BF16, 128, 16, 4, partition_size=-1, seed=403),
        _mixed(W.F16, 64, 32, 2, partition_size=64, seed=404),
    ]
    jobs = []
    for wl in wls:
        dw = DeviceWorkload(wl)
        cache = new_cache(wl)
        dw.fill(cache)
        dw.apply(cache, dw.step)
        jobs.append((dw, cache))
    refs = [bits_of(dw.attend(cache, out_dtype=torch.float32)) for dw, cache in jobs]
    torch.cuda.synchronize()

    rounds = 25
    start = threading.Barrier(len(jobs))
    errors = []

    def worker(i):
        dw, cache = jobs[i]
        stream = torch.cuda.Stream()
        try:
            with torch.cuda.stream(stream):
                for r in range(rounds):
                    start.wait(timeout=60)
                    got = dw.attend(cache, out_dtype=torch.float32)
                    stream.synchronize()
                    if not np.array_equal(bits_of(got), refs[i]):
                        errors.append(f"job {i} round {r}: result differs from the call made alone")
                        return
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append(f"job {i}: {e!r}")
            start.abort()

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
